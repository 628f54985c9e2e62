"""GPU parity of document masks (packed sequences: each query sees only its own
document, which starts at raw position lo) for the MXFP4 indexer and the FP8
CSA / HCA attention, against the oracle's masked selection and attention; and
a zero bound bit-identical to no mask."""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import attention as OA
from oracle import codecs
from oracle import compress as OC
from oracle import indexer as OI
from tests._common import check_attention, np_

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mods():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_hca_amd as H
    from long_context_attention_hca_amd import workloads as W
    return H, W


def _split_dec(st):
    return OC.decode({k: np_(v) for k, v in st.items()}, "split")


@pytest.mark.parametrize("k", [64, 1024])
def test_document_masks_index_and_attention(mods, k):
    """One sequence of 8192 raw positions packing five documents (starts 0, 1234, 3001, 5120 and
    7777: on and off the m and m' grids); queries at a document's start, just after it, past the
    first HCA entry, mid-document and at its end; k = 64 (selection within long documents)
    and k = 1024 (whole short documents, padded)."""
    H, W = mods
    _say(f"document masks k={k}")
    L, m, w, mp, Wn, dn, dr, Hh = 8192, 4, 8, 128, 128, 448, 64, 16
    D = dn + dr
    n_c, n_h = L // m, L // mp
    starts = [0, 1234, 3001, 5120, 7777]
    ends = starts[1:] + [L]
    qpos, qlo = [], []
    for s0, e0 in zip(starts, ends):
        for t in sorted({s0, s0 + 1, s0 + 7, s0 + 130, (s0 + e0) // 2, e0 - 1}):
            if s0 <= t < e0:
                qpos.append(t)
                qlo.append(s0)
    nq = len(qpos)
    g = synth.generator(1016)
    kp, ks = synth.mxfp4_rows(g, n_c, 64)
    qp, qs = synth.mxfp4_rows(g, nq * 4, 64)
    wi = synth.normal(g, (nq, 4), std=0.125)
    cs, hs, ws_ = (synth.split_entries(g, n, dn, dr) for n in (n_c, n_h, L))
    q = synth.bf16_bits(synth.normal(g, (nq, Hh, D))).view(torch.bfloat16)
    dev = "cuda"
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device=dev)
    zero, q_seq, q_pos, q_lo = i64([0]), torch.zeros(nq, dtype=torch.int32, device=dev), i64(qpos), i64(qlo)
    ws = W.Workspace(dev)
    st = lambda d: H.Store.split(d["nope"].to(dev), d["scale"].to(dev), d["rope"].to(dev))
    csa_st, hca_st, win_st = st(cs), st(hs), st(ws_)
    scale = 1.0 / D ** 0.5

    def run(lo):
        idx = W.index_topk(qp.view(nq, 4, 32).to(dev), wi.to(dev), kp.to(dev), zero, q_seq, q_pos, n_c, m, k, ws,
                           q_idx_scale=qs.view(nq, 4, 2).to(dev), k_idx_scale=ks.to(dev), q_lo=lo, w=w)
        oc, lc = W.csa_attn(q.to(dev), csa_st, zero, idx, win_st, zero, zero, Wn, q_seq, q_pos, scale, ws,
                            o_dtype=torch.float32, q_lo=lo)
        oh, lh = W.hca_attn(q.to(dev), hca_st, zero, mp, n_h, win_st, zero, zero, Wn, q_seq, q_pos, scale, ws,
                            o_dtype=torch.float32, q_lo=lo)
        torch.cuda.synchronize()
        return [np_(x) for x in (idx, oc, lc, oh, lh)]

    masked = run(q_lo)
    plain, zeros = run(None), run(torch.zeros(nq, dtype=torch.int64, device=dev))
    for a_, b_ in zip(plain, zeros):
        assert np.array_equal(a_, b_), "a zero bound differs from no mask"
    _say("oracle")
    keys = codecs.decode_mxfp4(np_(kp), np_(ks))
    csa_dec, hca_dec, win_dec = _split_dec(cs), _split_dec(hs), _split_dec(ws_)
    qpn, qsn = np_(qp).reshape(nq, 4, 32), np_(qs).reshape(nq, 4, 2)
    qd = q.float().double().numpy()
    idx, oc, lc, oh, lh = masked
    for i, (t, lo) in enumerate(zip(qpos, qlo)):
        nv = OI.n_visible(t, m)
        s = OI.scores_mxfp4(codecs.decode_mxfp4(qpn[i], qsn[i]), np_(wi[i]), keys[:max(nv, 1)])
        ref = OI.topk_among(s, OI.visible_entries(t, m, w, lo, nv), k)
        assert np.array_equal(idx[i], ref), f"query {i} (t={t}, lo={lo}): index sets differ"
        ro, rl = OA.csa(qd[i], t, csa_dec, ref, win_dec, Wn, scale, lo=lo)
        check_attention(oc[i], lc[i], ro, rl, "low", f"csa query {i} t={t} lo={lo}")
        ro, rl = OA.hca(qd[i], t, hca_dec, mp, win_dec, Wn, scale, lo=lo)
        check_attention(oh[i], lh[i], ro, rl, "low", f"hca query {i} t={t} lo={lo}")


def test_document_masks_many_queries(mods):
    """300 queries with 64 heads over the same packed sequence take the many-query kernels (the
    4-query scorer and the row-owning attention) with document masks: runs of consecutive
    positions inside each document (blocks of 4 queries with one start row) and runs across
    document boundaries (blocks whose queries' visible keys start at different rows). Every
    query's index set is checked; attention on a sample."""
    H, W = mods
    _say("document masks, many queries")
    L, m, w, mp, Wn, dn, dr, Hh, k = 8192, 4, 8, 128, 128, 448, 64, 64, 64
    D = dn + dr
    n_c, n_h = L // m, L // mp
    starts = [0, 1234, 3001, 5120, 7777]
    ends = starts[1:] + [L]
    qpos = []
    for s0, e0 in zip(starts, ends):
        qpos += list(range(s0, min(s0 + 50, e0)))           # from the document's start
        qpos += list(range(max(e0 - 11, s0), min(e0 + 10, L)))  # across its end (3 blocks mixed)
    qpos = sorted(set(qpos))[:300]
    qlo = [max(s for s in starts if s <= t) for t in qpos]
    nq = len(qpos)
    assert nq >= 256
    g = synth.generator(1018)
    kp, ks = synth.mxfp4_rows(g, n_c, 64)
    qp, qs = synth.mxfp4_rows(g, nq * 4, 64)
    wi = synth.normal(g, (nq, 4), std=0.125)
    cs, hs, ws_ = (synth.split_entries(g, n, dn, dr) for n in (n_c, n_h, L))
    q = synth.bf16_bits(synth.normal(g, (nq, Hh, D))).view(torch.bfloat16)
    dev = "cuda"
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device=dev)
    zero, q_seq, q_pos, q_lo = i64([0]), torch.zeros(nq, dtype=torch.int32, device=dev), i64(qpos), i64(qlo)
    ws = W.Workspace(dev)
    st = lambda d: H.Store.split(d["nope"].to(dev), d["scale"].to(dev), d["rope"].to(dev))
    csa_st, hca_st, win_st = st(cs), st(hs), st(ws_)
    scale = 1.0 / D ** 0.5
    idx = W.index_topk(qp.view(nq, 4, 32).to(dev), wi.to(dev), kp.to(dev), zero, q_seq, q_pos, n_c, m, k, ws,
                       q_idx_scale=qs.view(nq, 4, 2).to(dev), k_idx_scale=ks.to(dev), q_lo=q_lo, w=w)
    oc, lc = W.csa_attn(q.to(dev), csa_st, zero, idx, win_st, zero, zero, Wn, q_seq, q_pos, scale, ws,
                        o_dtype=torch.float32, q_lo=q_lo)
    oh, lh = W.hca_attn(q.to(dev), hca_st, zero, mp, n_h, win_st, zero, zero, Wn, q_seq, q_pos, scale, ws,
                        o_dtype=torch.float32, q_lo=q_lo)
    torch.cuda.synchronize()
    idx, oc, lc, oh, lh = (np_(x) for x in (idx, oc, lc, oh, lh))
    _say("oracle")
    keys = codecs.decode_mxfp4(np_(kp), np_(ks))
    csa_dec, hca_dec, win_dec = _split_dec(cs), _split_dec(hs), _split_dec(ws_)
    qpn, qsn = np_(qp).reshape(nq, 4, 32), np_(qs).reshape(nq, 4, 2)
    qd = q.float().double().numpy()
    sample = set(range(0, nq, 7)) | {0, nq - 1}
    for i, (t, lo) in enumerate(zip(qpos, qlo)):
        nv = OI.n_visible(t, m)
        s = OI.scores_mxfp4(codecs.decode_mxfp4(qpn[i], qsn[i]), np_(wi[i]), keys[:max(nv, 1)])
        ref = OI.topk_among(s, OI.visible_entries(t, m, w, lo, nv), k)
        assert np.array_equal(idx[i], ref), f"query {i} (t={t}, lo={lo}): index sets differ"
        if i in sample:
            ro, rl = OA.csa(qd[i], t, csa_dec, ref, win_dec, Wn, scale, lo=lo)
            check_attention(oc[i], lc[i], ro, rl, "low", f"csa query {i} t={t} lo={lo}")
            ro, rl = OA.hca(qd[i], t, hca_dec, mp, win_dec, Wn, scale, lo=lo)
            check_attention(oh[i], lh[i], ro, rl, "low", f"hca query {i} t={t} lo={lo}")
