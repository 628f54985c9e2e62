"""The deferred split-K merge: csa_sparse_mqa_attn_partials / hca_dense_mqa_attn_partials
followed by one mqa_attn_merge give the same o and lse bits as the undeferred calls, for two
calls merged in one launch (HCA over 8192 + 128 entries and CSA over 1024 + 128, both split),
for one call alone, with a call that was not split (it writes its output itself), and with
the fp32 vector path."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mods():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_hca_amd as m
    from long_context_attention_hca_amd import workloads
    return m, workloads


def _case(H, n_h, n_c, k, W, nq=4, seed=71, dn=448, dr=64, f32=False):
    g = synth.generator(seed)
    D = dn + dr
    dev = "cuda"
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device=dev)
    if f32:
        mk = lambda n: {"data": synth.normal(g, (n, D))}
    else:
        mk = lambda n: synth.split_entries(g, n, dn, dr)
    hs, cs, ws_ = mk(nq * n_h), mk(nq * n_c), mk(nq * W)
    q = synth.normal(g, (nq, H, D))
    q = q.cuda() if f32 else synth.bf16_bits(q).view(torch.bfloat16).cuda()
    idx = torch.stack([torch.randperm(n_c, generator=g)[:k].sort().values for _ in range(nq)]).to(torch.int32)
    L = 128 * n_h
    c = dict(q=q, hca=hs, csa=cs, win=ws_, idx=idx.cuda(), hrb=i64([b * n_h for b in range(nq)]),
             crb=i64([b * n_c for b in range(nq)]), wrb=i64([b * W for b in range(nq)]), wp0=i64([L - W] * nq),
             q_seq=torch.arange(nq, dtype=torch.int32, device=dev), q_pos=i64([L - 1] * nq), W=W, n_h=n_h,
             scale=1.0 / D ** 0.5)
    return c


def _store(m, st, dn=448, dr=64):
    if "nope" in st:
        return m.Store.split(st["nope"].cuda(), st["scale"].cuda(), st["rope"].cuda())
    return m.Store.dense(st["data"].cuda(), dn, dr)


def _run(m, W_, c, defer, f32=False, ws=None):
    # a deferred call's partials live in ws until the merge: the caller keeps ws alive
    ws = ws or W_.Workspace("cuda")
    H = c["q"].shape[1]
    hs, cs, wn = _store(m, c["hca"]), _store(m, c["csa"]), _store(m, c["win"])
    od = torch.float32 if f32 else torch.bfloat16
    h = W_.hca_attn(c["q"], hs, c["hrb"], 128, c["n_h"], wn, c["wrb"], c["wp0"], c["W"], c["q_seq"], c["q_pos"],
                    c["scale"], ws, o_dtype=od, defer=defer)
    s = W_.csa_attn(c["q"], cs, c["crb"], c["idx"], wn, c["wrb"], c["wp0"], c["W"], c["q_seq"], c["q_pos"],
                    c["scale"], ws, o_dtype=od, defer=defer)
    return h, s


def test_two_calls_in_one_merge(mods):
    m, W_ = mods
    c = _case(64, 8192, 4096, 1024, 128)
    (ho, hl), (so, sl) = _run(m, W_, c, defer=False)
    ws = W_.Workspace("cuda")
    (do, dl, hp), (eo, el, sp) = _run(m, W_, c, defer=True, ws=ws)
    assert hp.n_split > 1 and sp.n_split > 1
    m.mqa_attn_merge(sp, hp)
    torch.cuda.synchronize()
    for x, y in ((ho, do), (hl, dl), (so, eo), (sl, el)):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def test_one_call_and_an_unsplit_call(mods):
    """Merging one call alone; and a split call merged with one that was not split (many
    queries over few entries take one block per query and head group)."""
    m, W_ = mods
    c = _case(64, 8192, 4096, 1024, 128, seed=72)
    (ho, hl), _ = _run(m, W_, c, defer=False)
    ws1, ws2 = W_.Workspace("cuda"), W_.Workspace("cuda")
    (do, dl, hp), _ = _run(m, W_, c, defer=True, ws=ws1)
    m.mqa_attn_merge(hp)
    torch.cuda.synchronize()
    assert torch.equal(ho.view(torch.int16), do.view(torch.int16)) and torch.equal(hl, dl)
    u = _case(64, 2, 4096, 64, 8, nq=300, seed=73)
    (uo, ul), _ = _run(m, W_, u, defer=False)
    (vo, vl, up), _ = _run(m, W_, u, defer=True, ws=ws2)
    assert up.n_split == 1
    (do, dl, hp), _ = _run(m, W_, c, defer=True, ws=ws1)
    m.mqa_attn_merge(up, hp)
    torch.cuda.synchronize()
    assert torch.equal(uo.view(torch.int16), vo.view(torch.int16)) and torch.equal(ul, vl)
    assert torch.equal(ho.view(torch.int16), do.view(torch.int16)) and torch.equal(hl, dl)


def test_fp32_vector_path(mods):
    m, W_ = mods
    c = _case(16, 700, 500, 64, 37, nq=3, seed=74, dn=128, dr=64, f32=True)
    (ho, hl), (so, sl) = _run_f32(m, W_, c, defer=False)
    ws = W_.Workspace("cuda")
    (do, dl, hp), (eo, el, sp) = _run_f32(m, W_, c, defer=True, ws=ws)
    assert hp.n_split > 1
    m.mqa_attn_merge(hp, sp)
    torch.cuda.synchronize()
    assert torch.equal(ho, do) and torch.equal(hl, dl) and torch.equal(so, eo) and torch.equal(sl, el)


def _run_f32(m, W_, c, defer, ws=None):
    ws = ws or W_.Workspace("cuda")
    st = lambda d: m.Store.dense(d["data"].cuda(), 128, 64)
    hs, cs, wn = st(c["hca"]), st(c["csa"]), st(c["win"])
    h = W_.hca_attn(c["q"], hs, c["hrb"], 128, c["n_h"], wn, c["wrb"], c["wp0"], c["W"], c["q_seq"], c["q_pos"],
                    c["scale"], ws, o_dtype=torch.float32, defer=defer)
    s = W_.csa_attn(c["q"], cs, c["crb"], c["idx"], wn, c["wrb"], c["wp0"], c["W"], c["q_seq"], c["q_pos"],
                    c["scale"], ws, o_dtype=torch.float32, defer=defer)
    return h, s
