"""GPU parity of whole workloads against the oracle: compression, indexer top-k
and CSA/HCA attention, at sizes the oracle finishes in seconds and at the full
benchmark sizes (sampled where the oracle must go entry by entry)."""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import compress as OC
from oracle import pipeline as OP
from tests._common import (case_numpy, check_attention, check_bf16_entries, check_f32_entries, check_idx,
                           check_split_entries, np_, tie_margin_ok, to_device)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def W():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_attention_hca_amd import workloads
    return workloads


def _tie_free_tiny(seed, **kw):
    for s in range(seed, seed + 10):
        c = synth.tiny_fp32(seed=s, **kw)
        a = case_numpy(c)
        p = c.params
        ok = all(tie_margin_ok(a["q_idx"][i].astype(np.float64), a["w_idx"][i].astype(np.float64),
                               a["k_idx"].astype(np.float64), (int(t) + 1) // p["m"], p["topk"])
                 for i, t in enumerate(a["q_pos"]))
        if ok:
            return c, a
    raise AssertionError("no tie-free draw")


@pytest.mark.parametrize("kw", [dict(), dict(L=1000, n_queries=7, topk=64)])
def test_tiny_fp32_pipeline(W, kw):
    _say(f"tiny_fp32 {kw}")
    c, a = _tie_free_tiny(1001, **kw)
    p = c.params
    ref = OP.tiny_fp32(p, a)
    got = W.tiny_fp32(to_device(c))
    torch.cuda.synchronize()
    check_f32_entries(np_(got["csa"].data), ref["y_csa"], ref["yabs_csa"], "csa entries")
    check_f32_entries(np_(got["hca"].data), ref["y_hca"], ref["yabs_hca"], "hca entries")
    check_idx(np_(got["idx"]), np.stack(ref["idx"]), "top-k")
    check_attention(np_(got["o_csa"]), np_(got["lse_csa"]), np.stack(ref["o_csa"]), np.stack(ref["lse_csa"]),
                    "fp32", "csa attention")
    check_attention(np_(got["o_hca"]), np_(got["lse_hca"]), np.stack(ref["o_hca"]), np.stack(ref["lse_hca"]),
                    "fp32", "hca attention")


def _decode_bf16_case(B, L, topk, dev="cpu"):
    for s in range(1002, 1012):
        c = synth.decode_bf16(seed=s, B=B, L=L, topk=topk, device=dev)
        a = case_numpy(c, keys={"q_idx", "w_idx", "k_idx"})
        n_c = L // 4
        from oracle.codecs import decode_bf16
        if all(tie_margin_ok(decode_bf16(a["q_idx"][b].view(np.uint16)), a["w_idx"][b].astype(np.float64),
                             decode_bf16(a["k_idx"][b * n_c:(b + 1) * n_c].view(np.uint16)), n_c, topk)
               for b in range(B)):
            return c
    raise AssertionError("no tie-free draw")


@pytest.mark.parametrize("B,L,topk,seqs", [(3, 8192, 512, [0, 1, 2]), (8, 131072, 512, [0, 3, 5, 7])])
def test_decode_bf16(W, B, L, topk, seqs):
    _say(f"decode_bf16 B={B} L={L}")
    c = _decode_bf16_case(B, L, topk, dev="cuda" if L > 8192 else "cpu")
    a = case_numpy(c)
    ref = OP.decode_bf16(c.params, a, seqs)
    got = W.decode_bf16(to_device(c))
    torch.cuda.synchronize()
    p = c.params
    n_c, n_h = L // p["m"], L // p["m_prime"]
    idx = np_(got["idx"])
    csa_rows = np_(got["csa"].data)
    hca_rows = np_(got["hca"].data)
    o_c, l_c, o_h, l_h = (np_(got[k]).astype(np.float64) if k.startswith("lse") else
                          np_(got[k].float()) for k in ("o_csa", "lse_csa", "o_hca", "lse_hca"))
    for b in seqs:
        r = ref[b]
        check_idx(idx[b], r["idx"], f"top-k seq {b}")
        sel = [j for j in r["idx"] if j >= 0]
        ys = np.stack([r["csa_y"][j] for j in sel])
        ya = np.stack([r["csa_yabs"][j] for j in sel])
        check_bf16_entries(csa_rows[b * n_c + np.array(sel)], ys, f"csa entries seq {b}", ya)
        check_bf16_entries(hca_rows[b * n_h:(b + 1) * n_h], r["y_hca"], f"hca entries seq {b}", r["yabs_hca"])
        check_attention(o_c[b], l_c[b], r["o_csa"], r["lse_csa"], "low", f"csa attention seq {b}")
        check_attention(o_h[b], l_h[b], r["o_hca"], r["lse_hca"], "low", f"hca attention seq {b}")


def test_decode_bf16_step(W):
    """The timed bf16 decode step (8 sequences at 128K over bf16 stores generated already
    compressed, k = 512): the step with the top-k selection in HCA attention's launch equals,
    bit for bit, the calls one after another, and sampled sequences match the oracle's index,
    CSA and HCA attention computed from the stored rows."""
    from oracle import attention as OA
    from oracle import indexer as OI
    from oracle.codecs import decode_bf16
    B, L, k, seqs = 8, 131072, 512, [0, 3, 5, 7]
    _say(f"decode_bf16 step B={B} L={L}")
    for s in range(1021, 1031):
        c = synth.decode_bf16_caches(seed=s, B=B, L=L, topk=k, device="cuda")
        p = c.params
        n_c = L // p["m"]
        qi = np_(c.t["q_idx"].cpu())
        wi = np_(c.t["w_idx"].cpu()).astype(np.float64)
        ki = np_(c.t["k_idx"].cpu())
        if all(tie_margin_ok(decode_bf16(qi[b].view(np.uint16)), wi[b],
                             decode_bf16(ki[b * n_c:(b + 1) * n_c].view(np.uint16)), n_c, k) for b in seqs):
            break
    else:
        raise AssertionError("no tie-free draw")
    fused = W.DecodeBf16(c, ws=W.Workspace("cuda"))
    serial = W.DecodeBf16(c, ws=W.Workspace("cuda"), fused=False)
    fused.step()
    serial.step()
    torch.cuda.synchronize()
    for name in ("idx", "o_csa", "lse_csa", "o_hca", "lse_hca"):
        x, y = getattr(fused, name), getattr(serial, name)
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), f"fused step differs from the serial calls: {name}"
    mp, Wn = p["m_prime"], p["W"]
    n_h, t = L // mp, L - 1
    scale = 1.0 / np.sqrt(p["D"])
    idx = np_(fused.idx)
    o_c, o_h = np_(fused.o_csa.float()), np_(fused.o_hca.float())
    l_c, l_h = np_(fused.lse_csa), np_(fused.lse_hca)
    csa, hca, win = (np_(c.t[n].cpu()) for n in ("csa_data", "hca_data", "win_data"))
    q = np_(c.t["q"].cpu())
    for b in seqs:
        keys = decode_bf16(ki[b * n_c:(b + 1) * n_c].view(np.uint16))
        n_vis = OI.n_visible(t, p["m"])
        ref_idx = OI.topk(OI.scores(decode_bf16(qi[b].view(np.uint16)), wi[b], keys[:n_vis]), n_vis, k)
        check_idx(idx[b], ref_idx, f"top-k seq {b}")
        rows = decode_bf16(win[b * Wn:(b + 1) * Wn].view(np.uint16))
        window = lambda pos, rows=rows: rows[np.asarray(pos) - (L - Wn)]
        ent = np.zeros((n_c, p["D"]))
        sel = ref_idx[ref_idx >= 0]
        ent[sel] = decode_bf16(csa[b * n_c + sel].view(np.uint16))
        qb = decode_bf16(q[b].view(np.uint16))
        ro, rl = OA.csa(qb, t, ent, ref_idx, window, Wn, scale)
        check_attention(o_c[b], l_c[b], ro, rl, "low", f"csa attention seq {b}")
        ro, rl = OA.hca(qb, t, decode_bf16(hca[b * n_h:(b + 1) * n_h].view(np.uint16)), mp, window, Wn, scale)
        check_attention(o_h[b], l_h[b], ro, rl, "low", f"hca attention seq {b}")


@pytest.mark.parametrize("B,L,seqs", [(3, 1 << 16, [0, 1, 2]), (4, 1 << 20, [0, 1, 2, 3])])
def test_decode_1m(W, B, L, seqs):
    _say(f"decode_1m B={B} L={L}")
    c = synth.decode_1m(seed=1003, B=B, L=L, device="cuda")
    run = W.Decode1M(c)
    run.step()
    torch.cuda.synchronize()
    a = case_numpy(c)
    idx = np_(run.idx)
    o_c, o_h = np_(run.o_csa.float()), np_(run.o_hca.float())
    l_c, l_h = np_(run.lse_csa), np_(run.lse_hca)
    for b in seqs:
        r = OP.decode_1m_query(c.params, a, b)
        check_idx(idx[b], r["idx"], f"top-k seq {b}")
        check_attention(o_c[b], l_c[b], r["o_csa"], r["lse_csa"], "low", f"csa attention seq {b}")
        check_attention(o_h[b], l_h[b], r["o_hca"], r["lse_hca"], "low", f"hca attention seq {b}")


@pytest.mark.parametrize("L", [4096 + 128 * 3, 1 << 20])
def test_compression_split(W, L):
    _say(f"compression L={L}")
    c = synth.compression(seed=1004, L=L, device="cuda")
    csa, hca = W.compress_1m(c)
    torch.cuda.synchronize()
    p = c.params
    m, w, mp, dn, dr = p["m"], p["w"], p["m_prime"], p["d_nope"], p["d_rope"]
    n_c, n_h = L // m, L // mp
    rng = np.random.default_rng(0)
    cj = np.unique(np.concatenate([[0, 1, 2, n_c - 1], rng.integers(0, n_c, 200)]))
    hj = np.unique(np.concatenate([[0, n_h - 1], rng.integers(0, n_h, 12)]))
    from oracle.codecs import decode_bf16
    raw = c.t["raw"]
    for name, js, mm, ww, lg, bias, st in (("csa", cj, m, w, "logits_csa", "bias_csa", csa),
                                           ("hca", hj, mp, mp, "logits_hca", "bias_hca", hca)):
        ys, ya = [], []
        for j in js:
            lo, hi = max(0, j * mm - (ww - mm)), (j + 1) * mm
            x = decode_bf16(np_(raw[lo:hi]).view(np.uint16))
            z = decode_bf16(np_(c.t[lg][lo:hi]).view(np.uint16))
            ys.append(OC.compress(x, z, np_(c.t[bias]), mm, ww, int(j), 1, first_pos=lo)[0])
            ya.append(OC.compress(np.abs(x), z, np_(c.t[bias]), mm, ww, int(j), 1, first_pos=lo)[0])
        ys, ya = np.stack(ys), np.stack(ya)
        check_split_entries(np_(st.data)[js], np_(st.scale)[js], np_(st.rope)[js], ys, dn, f"{name} entries", ya)


@pytest.mark.parametrize("prefixes,chunk,nsample,window", [((4096, 8192, 16384), 512, 24, "bf16"),
                                                            ((4096, 8192, 16384), 512, 24, "split"),
                                                            ((32768, 131072, 262144), 8192, 256, "split")])
def test_chunked_prefill(W, prefixes, chunk, nsample, window):
    _say(f"prefill prefixes={prefixes} chunk={chunk} window={window}")
    c = synth.chunked_prefill(seed=1005, prefixes=prefixes, chunk=chunk, device="cuda")
    a_in = case_numpy(c, keys={"raw", "logits_csa", "logits_hca", "bias_csa", "bias_hca", "csa_nope", "csa_scale",
                               "csa_rope", "hca_nope", "hca_scale", "hca_rope", "k_idx", "k_idx_scale", "q_seq",
                               "q_pos"})
    got = W.chunked_prefill(c, window=window)
    torch.cuda.synchronize()
    p = c.params
    S = p["S"]
    if window == "split":
        # window rows: each entry is its raw row (softmax over one position), so the store must
        # equal the oracle's own split encoding of the raw rows bit for bit
        rows = p["W"] + chunk
        ref = OC.encode(OC.decode({"data": a_in["raw"]}, "bf16"), "split", p["d_nope"], p["d_rope"])
        st = got["win"]
        assert np.array_equal(np_(st.data), ref["nope"]), "window FP8 codes"
        assert np.array_equal(np_(st.scale), ref["scale"]), "window scales"
        assert np.array_equal(np_(st.rope).view(np.uint16), ref["rope"]), "window RoPE bits"
        assert np_(st.data).shape[0] == S * rows
    rng = np.random.default_rng(1)
    picks = []
    for b in range(S):
        base = b * chunk
        if nsample >= 256:
            # the first 64 and last 64 queries of the chunk and 128 strided ones between them
            picks += list(range(base, base + 64)) + list(range(base + chunk - 64, base + chunk))
            picks += list(base + 64 + (np.arange(128) * (chunk - 128)) // 128)
        else:
            picks += [base, base + 1, base + chunk - 1] + list(base + rng.integers(0, chunk, nsample - 3))
    picks = sorted(set(int(x) for x in picks))
    t = c.t
    a = dict(a_in)
    for k in ("q", "q_idx", "q_idx_scale", "w_idx"):
        rows = np_(t[k][picks])
        a[k] = {qi: rows[n] for n, qi in enumerate(picks)}
    chunk_ent = {b: OP.prefill_chunk_entries(p, a, b) for b in range(S)}
    idx = np_(got["idx"])
    m, mp, dn = p["m"], p["m_prime"], p["d_nope"]
    # the chunk's compressed entries
    for b, P in enumerate(prefixes):
        y_c, _, y_h, _, ya_c, ya_h = chunk_ent[b]
        r0 = p["csa_row_begin"][b] + P // m
        rows = np.arange(r0, r0 + chunk // m)
        st = got["csa"]
        check_split_entries(np_(st.data)[rows], np_(st.scale)[rows], np_(st.rope)[rows], y_c, dn, f"csa chunk {b}", ya_c)
        r0 = p["hca_row_begin"][b] + P // mp
        rows = np.arange(r0, r0 + chunk // mp)
        st = got["hca"]
        check_split_entries(np_(st.data)[rows], np_(st.scale)[rows], np_(st.rope)[rows], y_h, dn, f"hca chunk {b}", ya_h)
    o_c, l_c = np_(got["o_csa"][picks].float()), np_(got["lse_csa"][picks])
    o_h, l_h = np_(got["o_hca"][picks].float()), np_(got["lse_hca"][picks])
    memo = {}
    if len(picks) > 100:
        _say(f"oracle over {len(picks)} sampled queries")
    for n, qi in enumerate(picks):
        r = OP.prefill_query(p, a, qi, lambda b: chunk_ent[b][1], lambda b: chunk_ent[b][3],
                             split_window=window == "split", memo=memo)
        check_idx(idx[qi], r["idx"], f"top-k query {qi}")
        check_attention(o_c[n], l_c[n], r["o_csa"], r["lse_csa"], "low", f"csa attention query {qi}")
        check_attention(o_h[n], l_h[n], r["o_hca"], r["lse_hca"], "low", f"hca attention query {qi}")


@pytest.mark.parametrize("raw_dt,layout,scalar", [("bf16", "split", False), ("bf16", "split", True),
                                                  ("bf16", "bf16", True), ("f32", "f32", False), ("f32", "f32", True)])
def test_csa_compress_runs_and_scalar_logits(W, raw_dt, layout, scalar):
    """csa_compress of entries 37 .. 239 from raw rows that begin at entry 37's window (runs of
    consecutive entries end mid-run), with per-channel or one-per-token logits, against the
    oracle on every entry."""
    import long_context_attention_hca_amd as H
    from oracle.codecs import decode_bf16
    _say(f"csa compress {raw_dt} {layout} scalar={scalar}")
    m, w = 4, 8
    dn, dr = (448, 64) if raw_dt == "bf16" else (128, 64)
    D = dn + dr
    e0, n = 37, 203
    first_pos = e0 * m - (w - m)
    rows = (e0 + n) * m - first_pos  # through the last entry's window
    g = synth.generator(1006)
    x = synth.normal(g, (rows, D))
    z = synth.normal(g, (rows, 1 if scalar else D), std=2.0)
    bias = synth.normal(g, (w, D), std=0.5)
    if raw_dt == "bf16":
        xin, zin = synth.bf16_bits(x), synth.bf16_bits(z)
        xd, zd = decode_bf16(np_(xin).view(np.uint16)), decode_bf16(np_(zin).view(np.uint16))
    else:
        xin, zin = x, z
        xd, zd = x.double().numpy(), z.double().numpy()
    code = {"split": H.LAYOUT_SPLIT, "bf16": H.LAYOUT_BF16, "f32": H.LAYOUT_F32}[layout]
    out = W.empty_store(code, n, dn, dr, "cuda")
    H.csa_compress(xin.cuda(), first_pos, zin.cuda(), bias.cuda(), m, w, e0, n, out, scalar_logits=scalar)
    torch.cuda.synchronize()
    b = bias.double().numpy()
    y = OC.compress(xd, zd, b, m, w, e0, n, first_pos=first_pos)
    ya = OC.compress(np.abs(xd), zd, b, m, w, e0, n, first_pos=first_pos)
    if layout == "split":
        check_split_entries(np_(out.data), np_(out.scale), np_(out.rope), y, dn, "csa entries", ya)
    elif layout == "bf16":
        check_bf16_entries(np_(out.data), y, "csa entries", ya)
    else:
        check_f32_entries(np_(out.data), y, ya, "csa entries")
