"""GPU parity of csa_sparse_mqa_attn / hca_dense_mqa_attn against the oracle on
edge cases, for each store layout (split FP8/bf16, dense bf16, dense fp32): empty
entry sets (o = 0, lse = -inf), W = 0 and W = 1, -1 padding anywhere in idx,
split-K (few queries) and single-block (many queries) launches, fp32 output from
bf16 queries, 16/32/64 heads, a window store in a different layout from the cache."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import attention as OA
from oracle import compress as OC
from tests._common import check_attention, np_

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hca():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_hca_amd as m
    from long_context_attention_hca_amd import workloads
    return m, workloads


def make_store(layout, n, seed, dn=448, dr=64):
    g = synth.generator(seed)
    if layout == "split":
        st = synth.split_entries(g, n, dn, dr)
        dec = OC.decode({k: np_(v) for k, v in st.items()}, "split")
        return st, dec
    v = synth.normal(g, (n, dn + dr))
    if layout == "bf16":
        bits = synth.bf16_bits(v)
        return {"data": bits}, OC.decode({"data": np_(bits).view(np.uint16)}, "bf16")
    return {"data": v}, v.double().numpy()


def to_store(hca_mod, st, dn, dr):
    if "nope" in st:
        return hca_mod.Store.split(st["nope"].cuda(), st["scale"].cuda(), st["rope"].cuda())
    return hca_mod.Store.dense(st["data"].cuda(), dn, dr)


CASES = [
    # cache layout, window layout, q dtype, o dtype, heads, D split
    ("split", "split", "bf16", "bf16", 64, (448, 64)),
    ("split", "split", "bf16", "f32", 16, (448, 64)),
    ("bf16", "bf16", "bf16", "bf16", 32, (448, 64)),
    ("split", "bf16", "bf16", "bf16", 64, (448, 64)),
    ("f32", "f32", "f32", "f32", 16, (128, 64)),
]


@pytest.mark.parametrize("cl,wl,qd,od,H,dims", CASES)
@pytest.mark.parametrize("nq", [3, 300])
def test_attention_layouts_and_edges(hca, cl, wl, qd, od, H, dims, nq):
    m, W_ = hca
    dn, dr = dims
    D = dn + dr
    n_cache, n_win, k, W, mp = 1500, 400, 96, 37, 16
    cache_st, cache_dec = make_store(cl, n_cache, 5, dn, dr)
    win_st, win_dec = make_store(wl, n_win, 6, dn, dr)
    rng = np.random.default_rng(nq)
    # two sequences: cache rows [0, 800) and [800, 1500); window rows 0..199 hold positions
    # 5000.., rows 200..399 positions 300..
    crb, wrb, wp0 = [0, 800], [0, 200], [5000, 300]
    q_seq = rng.integers(0, 2, nq).astype(np.int32)
    q_pos = np.where(q_seq == 0, rng.integers(5000 + W, 5200, nq), rng.integers(300 + W, 500, nq)).astype(np.int64)
    q_pos[0], q_seq[0] = 5000 + W - 1, 0                 # first query: smallest legal position
    idx = np.full((nq, k), -1, np.int32)
    for i in range(nq):
        nvis = 700 if q_seq[i] == 0 else 650
        cnt = rng.integers(0, k + 1)
        sel = rng.choice(nvis, size=cnt, replace=False)
        slots = rng.choice(k, size=cnt, replace=False)   # -1 padding anywhere
        idx[i, slots] = sel
    g = synth.generator(77)
    qf = synth.normal(g, (nq, H, D))
    q = qf if qd == "f32" else qf.bfloat16()
    qdec = q.double().numpy()
    scale = 1.0 / math.sqrt(D)
    dev = "cuda"
    cache = to_store(m, cache_st, dn, dr)
    win = to_store(m, win_st, dn, dr)
    t_seq = torch.tensor(q_seq, device=dev)
    t_pos = torch.tensor(q_pos, device=dev)
    ws = W_.Workspace(dev)
    o_dt = torch.float32 if od == "f32" else torch.bfloat16
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device=dev)
    for Wx in (W, 0, 1):
        o, lse = W_.csa_attn(q.to(dev), cache, i64(crb), torch.tensor(idx, device=dev), win, i64(wrb), i64(wp0), Wx,
                             t_seq, t_pos, scale, ws, o_dtype=o_dt)
        o2, lse2 = W_.hca_attn(q.to(dev), cache, i64(crb), mp, 60, win, i64(wrb), i64(wp0), Wx, t_seq, t_pos, scale,
                               ws, o_dtype=o_dt)
        torch.cuda.synchronize()
        o, lse, o2, lse2 = np_(o.float()), np_(lse), np_(o2.float()), np_(lse2)
        kind = "fp32" if qd == "f32" else "low"
        for i in range(min(nq, 40)):
            b, t = int(q_seq[i]), int(q_pos[i])
            ent = cache_dec[crb[b]:]
            raw = lambda pos, b=b: win_dec[wrb[b] + np.asarray(pos) - wp0[b]]
            ro, rl = OA.csa(qdec[i], t, ent, idx[i], raw, Wx, scale)
            check_attention(o[i], lse[i], ro, rl, kind, f"csa q{i} W={Wx}")
            # HCA: the visible entries are the first min((t+1)//mp, max_visible = 60)
            nv = min((t + 1) // mp, 60)
            ro, rl = OA.attend(qdec[i], np.concatenate([ent[:nv], raw(OA.window_positions(t, Wx))]), scale)
            check_attention(o2[i], lse2[i], ro, rl, kind, f"hca q{i} W={Wx}")


def test_empty_sets_give_zero_and_neg_inf(hca):
    m, W_ = hca
    st, _ = make_store("split", 64, 9)
    cache = to_store(m, st, 448, 64)
    dev = "cuda"
    q = synth.normal(synth.generator(3), (2, 64, 512)).bfloat16().to(dev)
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device=dev)
    ws = W_.Workspace(dev)
    idx = torch.full((2, 32), -1, dtype=torch.int32, device=dev)
    seq = torch.tensor([0, 0], dtype=torch.int32, device=dev)
    pos = torch.tensor([5, 100], dtype=torch.int64, device=dev)
    o, lse = W_.csa_attn(q, cache, i64([0]), idx, cache, i64([0]), i64([0]), 0, seq, pos, 0.05, ws)
    o2, lse2 = W_.hca_attn(q, cache, i64([0]), 128, 64, cache, i64([0]), i64([0]), 0, seq, pos, 0.05, ws)
    torch.cuda.synchronize()
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(o2.float() == 0) and torch.all(torch.isneginf(lse2))


def test_many_splits_and_unaligned_width(hca):
    """fp32 path with D = 27 (rows padded to 28 floats) and about 1000 visible HCA entries:
    more than 16 split-K partials per (query, head) and a width that is not a multiple of 4,
    so the merge runs several load groups and a single-dim tail."""
    m, W_ = hca
    dn, dr, n, H = 21, 6, 1500, 4
    D = dn + dr
    g = synth.generator(91)
    dec = synth.normal(g, (n, D))
    full = torch.zeros(n, D + 1)
    full[:, :D] = dec
    dev = "cuda"
    cache = m.Store.dense(full.to(dev)[:, :D], dn, dr)  # row stride 28 floats
    nq, W, mp, max_vis = 3, 20, 1, 1000
    q_pos = np.array([1199, 1499, 400], np.int64)
    q = synth.normal(synth.generator(92), (nq, H, D))
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device=dev)
    ws = W_.Workspace(dev)
    scale = 1.0 / math.sqrt(D)
    seq = torch.zeros(nq, dtype=torch.int32, device=dev)
    o, lse = W_.hca_attn(q.to(dev), cache, i64([0]), mp, max_vis, cache, i64([0]), i64([0]), W, seq,
                         torch.tensor(q_pos, device=dev), scale, ws)
    torch.cuda.synchronize()
    o, lse = np_(o), np_(lse)
    ent = dec.double().numpy()
    for i in range(nq):
        t = int(q_pos[i])
        nv = min((t + 1) // mp, max_vis)
        rows = np.concatenate([ent[:nv], ent[OA.window_positions(t, W)]])
        ro, rl = OA.attend(q[i].double().numpy(), rows, scale)
        check_attention(o[i], lse[i], ro, rl, "fp32", f"q{i} nv={nv}")


@pytest.mark.parametrize("H", [16, 32])
def test_long_entry_lists(hca, H):
    """CSA with k = 65536 selected entries (the largest k the call accepts; a quarter of the slots
    padded with -1) and HCA over 70000 visible entries, split FP8 stores, 16 heads (one head
    group per block) and 32 (two): long lists give many split-K partials per head (more than one
    merge group)."""
    m, W_ = hca
    n_cache, n_win, W, k = 70000, 256, 128, 65536
    dn, dr = 448, 64
    D = dn + dr
    cache_st, cache_dec = make_store("split", n_cache, 31, dn, dr)
    win_st, win_dec = make_store("split", n_win, 32, dn, dr)
    dev = "cuda"
    cache, win = to_store(m, cache_st, dn, dr), to_store(m, win_st, dn, dr)
    rng = np.random.default_rng(33)
    nq = 2
    q_pos = np.array([n_cache - 1, n_cache - 50], np.int64)  # the window store holds positions 69744 .. 69999
    q_seq = np.zeros(nq, np.int32)
    idx = np.full((nq, k), -1, np.int32)
    for i in range(nq):
        sel = rng.choice(n_cache, size=3 * k // 4, replace=False)
        idx[i, rng.choice(k, size=sel.size, replace=False)] = sel
    g = synth.generator(34)
    q = synth.normal(g, (nq, H, D)).bfloat16()
    qdec = q.double().numpy()
    scale = 1.0 / math.sqrt(D)
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device=dev)
    wp0 = n_cache - n_win
    ws = W_.Workspace(dev)
    o, lse = W_.csa_attn(q.to(dev), cache, i64([0]), torch.tensor(idx, device=dev), win, i64([0]), i64([wp0]), W,
                         torch.tensor(q_seq, device=dev), torch.tensor(q_pos, device=dev), scale, ws,
                         o_dtype=torch.float32)
    o2, lse2 = W_.hca_attn(q.to(dev), cache, i64([0]), 1, n_cache, win, i64([0]), i64([wp0]), W,
                           torch.tensor(q_seq, device=dev), torch.tensor(q_pos, device=dev), scale, ws,
                           o_dtype=torch.float32)
    torch.cuda.synchronize()
    o, lse, o2, lse2 = np_(o), np_(lse), np_(o2), np_(lse2)
    raw = lambda pos: win_dec[np.asarray(pos) - wp0]
    for i in range(nq):
        t = int(q_pos[i])
        ro, rl = OA.csa(qdec[i], t, cache_dec, idx[i], raw, W, scale)
        check_attention(o[i], lse[i], ro, rl, "low", f"csa k=65536 q{i}")
        ro, rl = OA.attend(qdec[i], np.concatenate([cache_dec[:t + 1], raw(OA.window_positions(t, W))]), scale)
        check_attention(o2[i], lse2[i], ro, rl, "low", f"hca {t + 1} visible q{i}")


def test_k_zero_reads_no_index(hca):
    """k == 0 with idx a zero-width view into the middle of a larger int32 tensor (a non-NULL
    pointer, a row stride of 0 slots): CSA attention is the window-only attention, for split and
    bf16 stores."""
    m, W_ = hca
    dev = "cuda"
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device=dev)
    for layout in ("split", "bf16"):
        st, dec = make_store(layout, 300, 41)
        cache = to_store(m, st, 448, 64)
        nq, H, W = 3, 64, 50
        q = synth.normal(synth.generator(42), (nq, H, 512)).bfloat16()
        big = torch.full((nq, 64), 7, dtype=torch.int32, device=dev)

        class ZeroWidthView:
            """idx[:, 20:20] of `big` as the C ABI sees it: k = 0 and a non-NULL pointer into the
            middle of the tensor (torch itself reports NULL for an empty view)."""
            shape = (nq, 0)

            def data_ptr(self):
                return big.data_ptr() + 20 * 4

            def is_contiguous(self):
                return True

        idx = ZeroWidthView()
        seq = torch.zeros(nq, dtype=torch.int32, device=dev)
        pos = torch.tensor([60, 299, 10], dtype=torch.int64, device=dev)
        ws = W_.Workspace(dev)
        o, lse = W_.csa_attn(q.to(dev), cache, i64([0]), idx, cache, i64([0]), i64([0]), W, seq, pos, 0.05, ws)
        torch.cuda.synchronize()
        o, lse = np_(o.float()), np_(lse)
        for i, t in enumerate(pos.tolist()):
            ro, rl = OA.attend(q[i].double().numpy(), dec[OA.window_positions(t, W)], 0.05)
            check_attention(o[i], lse[i], ro, rl, "low", f"{layout} k=0 q{i}")


def test_fp32_sixteen_heads_of_512(hca):
    """The float32 path at its largest documented shape (16 heads of 512: 66,752 bytes of LDS per
    block) with split-K partials (about 2000 visible HCA entries for 2 queries) and a CSA call."""
    m, W_ = hca
    dn, dr, n, H = 448, 64, 2200, 16
    D = dn + dr
    st, dec = make_store("f32", n, 51, dn, dr)
    dev = "cuda"
    cache = to_store(m, st, dn, dr)
    nq, W, mp = 2, 64, 1
    q_pos = np.array([2199, 1500], np.int64)
    q = synth.normal(synth.generator(52), (nq, H, D))
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device=dev)
    ws = W_.Workspace(dev)
    scale = 1.0 / math.sqrt(D)
    seq = torch.zeros(nq, dtype=torch.int32, device=dev)
    pos = torch.tensor(q_pos, device=dev)
    assert m.mqa_attn_workspace(m.F32, nq, H, D, 2000 + W) > 0  # split-K
    o, lse = W_.hca_attn(q.to(dev), cache, i64([0]), mp, 2000, cache, i64([0]), i64([0]), W, seq, pos, scale, ws)
    rng = np.random.default_rng(53)
    idx = np.stack([np.sort(rng.choice(1400, size=300, replace=False)) for _ in range(nq)]).astype(np.int32)
    o2, lse2 = W_.csa_attn(q.to(dev), cache, i64([0]), torch.tensor(idx, device=dev), cache, i64([0]), i64([0]), W,
                           seq, pos, scale, ws)
    torch.cuda.synchronize()
    o, lse, o2, lse2 = np_(o), np_(lse), np_(o2), np_(lse2)
    for i in range(nq):
        t = int(q_pos[i])
        qd = q[i].double().numpy()
        ro, rl = OA.attend(qd, np.concatenate([dec[:min(t + 1, 2000)], dec[OA.window_positions(t, W)]]), scale)
        check_attention(o[i], lse[i], ro, rl, "fp32", f"hca q{i}")
        ro, rl = OA.csa(qd, t, dec, idx[i], dec, W, scale)
        check_attention(o2[i], lse2[i], ro, rl, "fp32", f"csa q{i}")


@pytest.mark.parametrize("nq", [3, 300])
def test_query_blocks_with_one_large_element(hca, nq):
    """Adversarial queries for the FP8 score path, which splits each bf16 query into two FP8 parts
    with one power-of-two scale per 32 dims: every 32-dim block holds one element of magnitude
    ~30-60, the others N(0, 1), and a quarter of them near 1e-3 (below E4M3's normal range under
    the block's scale). bf16 elements at least 2^-14 of their block's maximum are carried exactly
    by the two parts and smaller ones to within 2^-21 of that maximum, so attention must match
    the oracle at the usual tolerance. nq = 3 runs the per-head-group kernel, 300 the 64-head
    prefill kernel."""
    m, W_ = hca
    dev = "cuda"
    n_cache, W, k, mp = 1200, 64, 256, 8
    cache_st, cache_dec = make_store("split", n_cache, 61)
    cache = to_store(m, cache_st, 448, 64)
    g = synth.generator(63)
    H, D = 64, 512
    q = synth.normal(g, (nq, H, D))
    tiny = torch.rand((nq, H, D), generator=g) < 0.25
    q = torch.where(tiny, q * 1e-3, q)
    big_at = torch.randint(0, 32, (nq, H, D // 32), generator=g) + 32 * torch.arange(D // 32)
    big = (30.0 + 30.0 * torch.rand((nq, H, D // 32), generator=g)) * torch.sign(synth.normal(g, (nq, H, D // 32)))
    q.scatter_(2, big_at, big)
    q = q.bfloat16()
    qdec = q.double().numpy()
    rng = np.random.default_rng(64)
    q_pos = rng.integers(W + 200, n_cache, nq).astype(np.int64)
    idx = np.full((nq, k), -1, np.int32)
    for i, t in enumerate(q_pos):
        n = min(k, int(t + 1) // 4)
        idx[i, :n] = np.sort(rng.choice(int(t + 1) // 4, size=n, replace=False))
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device=dev)
    seq = torch.zeros(nq, dtype=torch.int32, device=dev)
    pos = torch.tensor(q_pos, device=dev)
    scale = 1.0 / math.sqrt(D)
    ws = W_.Workspace(dev)
    # the cache rows double as the window store (row p holds raw position p)
    o, lse = W_.csa_attn(q.to(dev), cache, i64([0]), torch.tensor(idx, device=dev), cache, i64([0]), i64([0]), W, seq,
                         pos, scale, ws, o_dtype=torch.float32)
    o2, lse2 = W_.hca_attn(q.to(dev), cache, i64([0]), mp, n_cache, cache, i64([0]), i64([0]), W, seq, pos, scale, ws,
                           o_dtype=torch.float32)
    torch.cuda.synchronize()
    o, lse, o2, lse2 = np_(o), np_(lse), np_(o2), np_(lse2)
    for i in range(min(nq, 24)):
        t = int(q_pos[i])
        ro, rl = OA.csa(qdec[i], t, cache_dec, idx[i], cache_dec, W, scale)
        check_attention(o[i], lse[i], ro, rl, "low", f"csa q{i}")
        nv = (t + 1) // mp
        ro, rl = OA.attend(qdec[i], np.concatenate([cache_dec[:nv], cache_dec[OA.window_positions(t, W)]]), scale)
        check_attention(o2[i], lse2[i], ro, rl, "low", f"hca q{i}")


def test_wide_dense_runs_at_store_end_and_documents(hca):
    """HCA on the 64-head prefill kernel, whose waves take 8 consecutive cache rows as one dense
    run when they are all valid and stage them row by row otherwise: two sequences share one
    split store (rows 0..699 and 700..1356, so the second ends at the store's last row), visible
    counts that end inside a wave's 8 rows, queries that see every row up to the store's end, and
    document starts that shift the first cache row by amounts that are no multiple of 8."""
    m, W_ = hca
    dev = "cuda"
    n0, n1 = 700, 657
    mp, W, H, D = 4, 64, 64, 512
    cache_st, cache_dec = make_store("split", n0 + n1, 71)
    cache = to_store(m, cache_st, 448, 64)
    L = 2816  # window rows of raw positions 0 .. L - 1 for each sequence
    win_st, win_dec = make_store("split", 2 * L, 72)
    win = to_store(m, win_st, 448, 64)
    rng = np.random.default_rng(73)
    nq = 96
    q_seq = np.repeat([0, 1], nq // 2).astype(np.int32)
    t0 = rng.integers(4 * 600, 4 * n0, nq // 2)
    t1 = rng.integers(4 * 500, 4 * n1, nq // 2)
    t1[:4] = [4 * n1 - 1, 4 * n1 - 2, 4 * n1 - 3, 4 * n1 - 4]  # all 657 rows of the last sequence
    q_pos = np.concatenate([t0, t1]).astype(np.int64)
    q_lo = np.zeros(nq, np.int64)
    q_lo[1::2] = rng.integers(1, 1500, nq // 2)
    g = synth.generator(74)
    q = synth.normal(g, (nq, H, D)).bfloat16()
    qdec = q.double().numpy()
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device=dev)
    scale = 1.0 / math.sqrt(D)
    ws = W_.Workspace(dev)
    o, lse = W_.hca_attn(q.to(dev), cache, i64([0, n0]), mp, n0, win, i64([0, L]), i64([0, 0]), W,
                         torch.tensor(q_seq, device=dev), torch.tensor(q_pos, device=dev), scale, ws,
                         o_dtype=torch.float32, q_lo=torch.tensor(q_lo, device=dev))
    torch.cuda.synchronize()
    o, lse = np_(o), np_(lse)
    for i in range(nq):
        b, t, lo = int(q_seq[i]), int(q_pos[i]), int(q_lo[i])
        entries = cache_dec[:n0] if b == 0 else cache_dec[n0:]
        raw = win_dec[b * L:(b + 1) * L]
        ro, rl = OA.hca(qdec[i], t, entries, mp, raw, W, scale, lo)
        check_attention(o[i], lse[i], ro, rl, "low", f"hca q{i} seq {b} t={t} lo={lo}")
