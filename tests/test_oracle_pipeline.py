"""Pins of the oracle's whole-workload compositions (oracle/pipeline.py) against routes that
share none of its slicing (DeepSeek-V4 page, Method section: CSA and HCA paragraphs, both with
a sliding-window branch; efficiency paragraph for the storage formats).

pipeline.py decides which rows of the packed inputs belong to a query's sequence, which
entries are visible at its position, how a chunk's entries join the prefix, the halo of raw
rows a chunk's compression reads and where a window position sits in the window store. Each
test below rebuilds a query from the whole raw sequence (or from the stores read whole, in
order) and compares:

* decode_1m_query / prefill_query with k >= n_vis: the selection is every visible entry, and
  the output equals textbook attention over the explicitly listed entry rows plus the last W
  raw rows of the sequence;
* prefill_chunk_entries: compressing prefix-halo + chunk equals compressing the whole raw
  sequence on the chunk's entries;
* tiny_fp32 / decode_bf16 with m = w = 1, m' = 1, W = 0 and k >= L: plain causal MQA through
  torch's scaled_dot_product_attention.

An off-by-one in any window base, halo or row map changes a row that the rebuilt route reads,
which the tests show by planting such mistakes in copies of the maps."""
import math

import numpy as np
import torch
import torch.nn.functional as F

import synth
from oracle import attention as A
from oracle import codecs
from oracle import compress as C
from oracle import indexer as I
from oracle import pipeline as OP
from tests._common import case_numpy


def _split_dec(a, prefix, rows):
    st = {"nope": a[f"{prefix}_nope"][rows], "scale": a[f"{prefix}_scale"][rows], "rope": a[f"{prefix}_rope"][rows]}
    return C.decode(st, "split")


def _sdpa_causal(q, X, t, scale):
    """Heads q [h, D] attending causally to rows X[0..t] (K = V = X), torch float64 on the CPU."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, :, None, :]
    K = torch.from_numpy(np.asarray(X[: t + 1], np.float64))
    kt = K[None, None].expand(1, q.shape[0], K.shape[0], K.shape[1])
    o = F.scaled_dot_product_attention(qt, kt, kt, scale=scale)[0, :, 0, :].numpy()
    lse = torch.logsumexp(scale * (torch.from_numpy(np.asarray(q, np.float64)) @ K.T), dim=1).numpy()
    return o, lse


# ---------------------------------------------------------------------------------------------
# decode at long context over precompressed stores


def _decode_case():
    # 2 sequences of 256 positions; every CSA entry is visible to the query at t = L - 1
    return synth.decode_1m(seed=1301, B=2, L=256, heads=4, d_nope=32, d_rope=16, m=4, topk=64, m_prime=16, W=8)


def test_decode_query_with_k_at_least_n_vis_is_dense_attention_over_listed_rows():
    c = _decode_case()
    p, a = c.params, case_numpy(c)
    L, m, mp, W = p["L"], p["m"], p["m_prime"], p["W"]
    n_c, n_h = L // m, L // mp
    scale = 1.0 / math.sqrt(p["D"])
    assert p["topk"] >= n_c
    for b in range(p["B"]):
        r = OP.decode_1m_query(p, a, b)
        assert np.array_equal(r["idx"], np.arange(n_c, dtype=np.int32))
        # the window store holds the sequence's last W positions, in order, in its own W rows
        win = _split_dec(a, "win_csa", slice(b * W, (b + 1) * W))
        ent = _split_dec(a, "csa", slice(b * n_c, (b + 1) * n_c))
        o, lse = A.attend(codecs.decode_bf16(a["q_csa"][b].view(np.uint16)), np.concatenate([ent, win]), scale)
        assert np.allclose(r["o_csa"], o, rtol=0, atol=1e-12) and np.allclose(r["lse_csa"], lse, rtol=0, atol=1e-12)
        win = _split_dec(a, "win_hca", slice(b * W, (b + 1) * W))
        ent = _split_dec(a, "hca", slice(b * n_h, (b + 1) * n_h))
        o, lse = A.attend(codecs.decode_bf16(a["q_hca"][b].view(np.uint16)), np.concatenate([ent, win]), scale)
        assert np.allclose(r["o_hca"], o, rtol=0, atol=1e-12) and np.allclose(r["lse_hca"], lse, rtol=0, atol=1e-12)


def test_decode_query_selection_reads_its_own_sequence_keys():
    # k < n_vis: the set must be the brute-force top-k of the sequence's own keys (rows b * n_c ..),
    # with scores from exact integer dot products of the E2M1 codes times the block scales
    c = synth.decode_1m(seed=1302, B=3, L=512, heads=4, d_nope=32, d_rope=16, m=4, topk=16, m_prime=16, W=8)
    p, a = c.params, case_numpy(c)
    n_c, k = p["L"] // p["m"], p["topk"]
    for b in range(p["B"]):
        r = OP.decode_1m_query(p, a, b)
        q = codecs.decode_mxfp4(a["q_idx"][b], a["q_idx_scale"][b])
        keys = codecs.decode_mxfp4(a["k_idx"][b * n_c:(b + 1) * n_c], a["k_idx_scale"][b * n_c:(b + 1) * n_c])
        w32 = np.asarray(a["w_idx"][b], np.float32)
        s = []
        for j in range(n_c):
            acc = None
            for h in range(q.shape[0]):
                rh = np.float32(max(0.0, float(sum(x * y for x, y in zip(q[h].tolist(), keys[j].tolist())))))
                term = np.float32(w32[h] * rh)
                acc = term if acc is None else np.float32(acc + term)
            s.append(float(acc))
        best = sorted(range(n_c), key=lambda j: (-s[j], j))[:k]
        assert np.array_equal(r["idx"], np.array(sorted(best), dtype=np.int32)), b


# ---------------------------------------------------------------------------------------------
# chunked prefill


def _prefill_full(seed=1303, prefixes=(64, 128), chunk=64, W=16):
    """A chunked-prefill case whose raw rows are cut from whole raw sequences built here: for
    sequence b, positions 0 .. P + chunk - 1 (raw values, compression logits); the case holds
    positions P - W .. P + chunk - 1 of each, as the generator lays them out."""
    c = synth.chunked_prefill(seed=seed, prefixes=prefixes, chunk=chunk, heads=4, d_nope=32, d_rope=16, m=4, w=8,
                              topk=4096, m_prime=16, W=W, device="cpu")
    p = c.params
    rng = np.random.default_rng(seed)
    rows = W + chunk
    full = {}
    for key in ("raw", "logits_csa", "logits_hca"):
        parts = []
        for b, P in enumerate(p["prefixes"]):
            x = rng.normal(size=(P + chunk, p["D"])) * (1.0 if key == "raw" else 0.5)
            bits = synth.bf16_bits(torch.from_numpy(x).float()).numpy()
            full.setdefault(key, []).append(bits)
            parts.append(bits[P - W:])
        c.t[key] = torch.from_numpy(np.concatenate(parts)).contiguous()
        assert c.t[key].shape[0] == p["S"] * rows
    return c, full


def test_prefill_chunk_entries_equal_whole_sequence_compression():
    c, full = _prefill_full()
    p, a = c.params, case_numpy(c)
    m, w, mp, chunk = p["m"], p["w"], p["m_prime"], p["chunk"]
    for b, P in enumerate(p["prefixes"]):
        y_c, _, y_h, _, _, _ = OP.prefill_chunk_entries(p, a, b)
        raw = codecs.decode_bf16(full["raw"][b].view(np.uint16))
        want_c = C.compress(raw, codecs.decode_bf16(full["logits_csa"][b].view(np.uint16)), a["bias_csa"], m, w,
                            P // m, chunk // m)
        want_h = C.compress(raw, codecs.decode_bf16(full["logits_hca"][b].view(np.uint16)), a["bias_hca"], mp, mp,
                            P // mp, chunk // mp)
        assert np.array_equal(y_c, want_c) and np.array_equal(y_h, want_h), b


def _prefill_expected(c, full, qi, split_window):
    """Query qi of the prefill case rebuilt from the whole raw sequence: all visible CSA and HCA
    entries (prefix entries as stored, chunk entries compressed from the whole sequence) and the
    window's raw rows t - W + 1 .. t read straight from the whole sequence."""
    p, a = c.params, case_numpy(c)
    m, w, mp, W, chunk = p["m"], p["w"], p["m_prime"], p["W"], p["chunk"]
    dn, dr = p["d_nope"], p["d_rope"]
    b, t = int(a["q_seq"][qi]), int(a["q_pos"][qi])
    P = p["prefixes"][b]
    raw = codecs.decode_bf16(full["raw"][b].view(np.uint16))
    y_c = C.compress(raw, codecs.decode_bf16(full["logits_csa"][b].view(np.uint16)), a["bias_csa"], m, w, 0,
                     (P + chunk) // m)
    y_h = C.compress(raw, codecs.decode_bf16(full["logits_hca"][b].view(np.uint16)), a["bias_hca"], mp, mp, 0,
                     (P + chunk) // mp)
    crb, hrb = p["csa_row_begin"][b], p["hca_row_begin"][b]
    ent_c = np.concatenate([_split_dec(a, "csa", slice(crb, crb + P // m)),
                            C.decode(C.encode(y_c[P // m:], "split", dn, dr), "split")])
    ent_h = np.concatenate([_split_dec(a, "hca", slice(hrb, hrb + P // mp)),
                            C.decode(C.encode(y_h[P // mp:], "split", dn, dr), "split")])
    win = raw[t - W + 1:t + 1]
    if split_window:
        win = C.decode(C.encode(win, "split", dn, dr), "split")
    q = codecs.decode_bf16(a["q"][qi].view(np.uint16))
    scale = 1.0 / math.sqrt(dn + dr)
    oc = A.attend(q, np.concatenate([ent_c[:(t + 1) // m], win]), scale)
    oh = A.attend(q, np.concatenate([ent_h[:(t + 1) // mp], win]), scale)
    return (t + 1) // m, oc, oh


def test_prefill_query_with_k_at_least_n_vis_is_dense_attention_over_the_whole_sequence():
    c, full = _prefill_full()
    p, a = c.params, case_numpy(c)
    ent = {b: OP.prefill_chunk_entries(p, a, b) for b in range(p["S"])}
    chunk = p["chunk"]
    # first chunk query (its window is all halo but one row), mid-chunk, and the last query of each
    # sequence, both at and off the m and m' grids
    picks = [0, 1, 15, 30, chunk - 1, chunk, chunk + 17, 2 * chunk - 1]
    for split in (False, True):
        for qi in picks:
            r = OP.prefill_query(p, a, qi, lambda b: ent[b][1], lambda b: ent[b][3], split_window=split)
            n_vis, (oc, lc), (oh, lh) = _prefill_expected(c, full, qi, split)
            want = np.full(p["topk"], -1, np.int32)
            want[:n_vis] = np.arange(n_vis)
            assert np.array_equal(r["idx"], want), qi
            assert np.allclose(r["o_csa"], oc, rtol=0, atol=1e-12) and np.allclose(r["lse_csa"], lc, rtol=0, atol=1e-12)
            assert np.allclose(r["o_hca"], oh, rtol=0, atol=1e-12) and np.allclose(r["lse_hca"], lh, rtol=0, atol=1e-12)


def test_a_shifted_window_map_would_be_caught():
    # the rebuilt route is sensitive to the window map: reading positions one row early changes
    # the output by far more than the tolerance used above
    c, full = _prefill_full()
    p, a = c.params, case_numpy(c)
    W, dn, dr = p["W"], p["d_nope"], p["d_rope"]
    qi = p["chunk"] + 17
    b, t = int(a["q_seq"][qi]), int(a["q_pos"][qi])
    raw = codecs.decode_bf16(full["raw"][b].view(np.uint16))
    q = codecs.decode_bf16(a["q"][qi].view(np.uint16))
    scale = 1.0 / math.sqrt(dn + dr)
    o1, _ = A.attend(q, raw[t - W + 1:t + 1], scale)
    o2, _ = A.attend(q, raw[t - W:t], scale)
    assert np.max(np.abs(o1 - o2)) > 1e-3


# ---------------------------------------------------------------------------------------------
# reduction to plain causal MQA: one entry per token (m = w = 1, m' = 1), no window, k >= L


def test_tiny_fp32_pipeline_reduces_to_causal_mqa():
    L = 40
    c = synth.tiny_fp32(seed=1304, L=L, n_queries=5, heads=3, d_nope=8, d_rope=8, m=1, w=1, topk=L, m_prime=1, W=0)
    p, a = c.params, case_numpy(c)
    r = OP.tiny_fp32(p, a)
    X = np.asarray(a["raw"], np.float32).astype(np.float64)
    scale = 1.0 / math.sqrt(p["D"])
    assert np.array_equal(r["y_csa"], X) and np.array_equal(r["y_hca"], X)
    for i, t in enumerate(a["q_pos"].tolist()):
        want = np.full(L, -1, np.int32)
        want[:t + 1] = np.arange(t + 1)
        assert np.array_equal(r["idx"][i], want)
        q = np.asarray(a["q"][i], np.float32).astype(np.float64)
        o, lse = _sdpa_causal(q, X, t, scale)
        for key in ("csa", "hca"):
            assert np.allclose(r[f"o_{key}"][i], o, rtol=0, atol=1e-12), (key, t)
            assert np.allclose(r[f"lse_{key}"][i], lse, rtol=0, atol=1e-12), (key, t)


def test_decode_bf16_pipeline_reduces_to_causal_mqa():
    L = 32
    c = synth.decode_bf16(seed=1305, B=3, L=L, heads=2, d_nope=8, d_rope=8, m=1, w=1, topk=L, n_idx_heads=2,
                          m_prime=1, W=0)
    p, a = c.params, case_numpy(c)
    r = OP.decode_bf16(p, a, range(p["B"]))
    scale = 1.0 / math.sqrt(p["D"])
    for b in range(p["B"]):
        X = codecs.decode_bf16(a["raw"][b * L:(b + 1) * L].view(np.uint16))
        assert np.array_equal(r[b]["idx"], np.arange(L, dtype=np.int32))
        o, lse = _sdpa_causal(codecs.decode_bf16(a["q"][b].view(np.uint16)), X, L - 1, scale)
        for key in ("csa", "hca"):
            assert np.allclose(r[b][f"o_{key}"], o, rtol=0, atol=1e-12), (key, b)
            assert np.allclose(r[b][f"lse_{key}"], lse, rtol=0, atol=1e-12), (key, b)


def test_visibility_counts_of_the_compositions():
    # n_vis(t) = floor((t + 1) / m): the prefill query at the chunk's first position sees the prefix's
    # entries only, one m later exactly one chunk entry more
    c, full = _prefill_full()
    p = c.params
    P, m, mp = p["prefixes"][0], p["m"], p["m_prime"]
    assert I.n_visible(P, m) == P // m and I.n_visible(P + m - 1, m) == P // m + 1
    assert _prefill_expected(c, full, 0, False)[0] == P // m
    assert _prefill_expected(c, full, m - 1, False)[0] == P // m + 1
    assert I.n_visible(P + mp - 1, mp) == P // mp + 1
