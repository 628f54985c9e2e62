"""GPU parity of lightning_index_topk against the oracle on edge cases: exact
ties (all-equal keys, all-zero scores), fewer visible entries than k, no visible
entry, several sequences, batching forced by a small workspace, 1 and 8 indexer
heads, k = 1 and k = 2048, the path for more than 2^19 visible entries, and the maximum of
2^21 visible entries with k = 2048."""
import numpy as np
import pytest
import torch

import synth
from oracle import codecs
from oracle import indexer as OI
from tests._common import check_idx, np_, tie_margin_ok

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hca():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_hca_amd as m
    return m


def run(hca, q, w, keys, row_begin, q_seq, q_pos, max_visible, m, k, q_scale=None, k_scale=None, ws_bytes=None):
    dev = "cuda"
    nq = q.shape[0]
    out = torch.full((nq, k), -7, dtype=torch.int32, device=dev)
    need = hca.lightning_index_topk_workspace(nq, max_visible, k)
    ws = torch.empty(ws_bytes or need, dtype=torch.uint8, device=dev)
    hca.lightning_index_topk(q.to(dev), w.to(dev), keys.to(dev), torch.tensor(row_begin, dtype=torch.int64, device=dev),
                             torch.tensor(q_seq, dtype=torch.int32, device=dev),
                             torch.tensor(q_pos, dtype=torch.int64, device=dev), max_visible, m, k, out, ws,
                             q_idx_scale=None if q_scale is None else q_scale.to(dev),
                             k_idx_scale=None if k_scale is None else k_scale.to(dev))
    torch.cuda.synchronize()
    return np_(out)


def oracle_mxfp4(q, qs, w, keys, ks, row_begin, q_seq, q_pos, m, k):
    kd = codecs.decode_mxfp4(np_(keys), np_(ks))
    res = []
    for i in range(q.shape[0]):
        b, t = q_seq[i], q_pos[i]
        qd = codecs.decode_mxfp4(np_(q[i]), np_(qs[i]))
        nv = min((t + 1) // m, kd.shape[0] - row_begin[b])
        s = OI.scores_mxfp4(qd, np_(w[i]), kd[row_begin[b]:row_begin[b] + nv])
        res.append(OI.topk(s, nv, k))
    return np.stack(res)


def mx_case(seed, n_keys, nq, H=4):
    g = synth.generator(seed)
    kp, ks = synth.mxfp4_rows(g, n_keys, 64)
    qp, qs = synth.mxfp4_rows(g, nq * H, 64)
    w = synth.normal(g, (nq, H), 0.125)
    return qp.view(nq, H, 32), qs.view(nq, H, 2), w, kp, ks


@pytest.mark.parametrize("H", [1, 4, 8])
@pytest.mark.parametrize("k", [1, 64, 2048])
def test_mxfp4_random(hca, H, k):
    q, qs, w, kp, ks = mx_case(11 + H, 20000, 6, H)
    q_seq, q_pos, rb = [0, 1, 1, 0, 1, 0], [19999, 39999, 4000, 79, 8191 * 4 + 3, 3], [0, 10000]
    keys = torch.cat([kp, kp[:10000]])          # two sequences sharing rows of one key store
    kss = torch.cat([ks, ks[:10000]])
    got = run(hca, q, w, keys, rb, q_seq, q_pos, 20000, 4, k, qs, kss)
    ref = oracle_mxfp4(q, qs, w, keys, kss, rb, q_seq, q_pos, 4, k)
    check_idx(got, ref, f"mxfp4 H={H} k={k}")


@pytest.mark.parametrize("k", [64, 1024])
def test_mxfp4_many_queries_grouped_and_mixed(hca, k):
    """At least 256 queries with 4 indexer heads take the scorer that serves 4 consecutive
    queries per block: their keys are loaded once and scored by one MFMA when the queries' visible
    keys start at the same row, and one query at a time otherwise. Queries 0 .. 199 alternate
    between two sequences in runs of 3 (most blocks mixed), queries 200 .. 300 all belong to
    sequence 0 (uniform blocks) at random positions, some of which see fewer than k entries or
    none; nq = 301 leaves a partial last block."""
    nq = 301
    q, qs, w, kp, ks = mx_case(31, 20000, nq, 4)
    rng = np.random.default_rng(5)
    q_seq = [(i // 3) % 2 if i < 200 else 0 for i in range(nq)]
    q_pos = [int(rng.integers(0, 80000)) for _ in range(nq)]
    for i in (200, 201, 250, 300):
        q_pos[i] = int(rng.integers(0, 4 * k))  # at most k visible entries
    q_pos[202] = 2                               # no visible entry
    rb = [0, 10000]
    keys = torch.cat([kp, kp[:10000]])
    kss = torch.cat([ks, ks[:10000]])
    got = run(hca, q, w, keys, rb, q_seq, q_pos, 20000, 4, k, qs, kss)
    ref = oracle_mxfp4(q, qs, w, keys, kss, rb, q_seq, q_pos, 4, k)
    check_idx(got, ref, f"mxfp4 many queries k={k}")


@pytest.mark.parametrize("k", [1, 1536, 1537])
def test_mxfp4_many_queries_ties(hca, k):
    """Many queries (the streaming selector keeps each query's best keys in a bounded buffer
    that it cuts to k whenever it could overflow) on keys copied from 6 distinct rows, so that
    every score is shared by thousands of entries and the cuts fall inside runs of ties; the
    queries with odd index have negative head weights (their best score is 0, held by most
    entries). k = 1537 is just past what the streaming selector takes and checks the other
    path on the same case. The split calls give the same result."""
    nq, n = 264, 20000
    q, qs, w, kp, ks = mx_case(41, n, nq, 4)
    rng = np.random.default_rng(9)
    pick = torch.from_numpy(rng.integers(0, 6, n))
    kp, ks = kp[pick].contiguous(), ks[pick].contiguous()
    w[1::2] = -w[1::2].abs()
    q_pos = [int(rng.integers(0, 4 * n)) for _ in range(nq)]
    q_pos[5] = 4 * n - 1
    q_pos[6] = 3                                 # no visible entry
    got = run(hca, q, w, kp, [0], [0] * nq, q_pos, n, 4, k, qs, ks)
    ref = oracle_mxfp4(q, qs, w, kp, ks, [0], [0] * nq, q_pos, 4, k)
    check_idx(got, ref, f"many queries, ties, k={k}")
    # with the smallest workspace the call accepts (other paths then batch the queries)
    small = run(hca, q, w, kp, [0], [0] * nq, q_pos, n, 4, k, qs, ks,
                ws_bytes=hca.lightning_index_topk_workspace(1, n, k))
    assert np.array_equal(small, got)
    dev = "cuda"
    a = (q.to(dev), w.to(dev), kp.to(dev), torch.zeros(1, dtype=torch.int64, device=dev),
         torch.zeros(nq, dtype=torch.int32, device=dev), torch.tensor(q_pos, dtype=torch.int64, device=dev), n, 4, k)
    ws = torch.empty(hca.lightning_index_topk_workspace(nq, n, k), dtype=torch.uint8, device=dev)
    two = torch.full((nq, k), -7, dtype=torch.int32, device=dev)
    kw = dict(q_idx_scale=qs.to(dev), k_idx_scale=ks.to(dev))
    hca.lightning_index_topk(*a, two, ws, phase="scores", **kw)
    hca.lightning_index_topk(*a, two, ws, phase="select", **kw)
    torch.cuda.synchronize()
    assert np.array_equal(np_(two), got)


def test_mxfp4_many_queries_long_range(hca):
    """The streaming selector over 2^20 visible entries (2048 tiles of 512 keys, dozens of
    buffer cuts per query): 256 queries made of two distinct queries alternating, so the oracle
    scores two; every row is checked."""
    n, nq, k = 1 << 20, 256, 1024
    q2, qs2, w2, kp, ks = mx_case(51, n, 2, 4)
    q = q2.repeat(nq // 2, 1, 1)
    qs = qs2.repeat(nq // 2, 1, 1)
    w = w2.repeat(nq // 2, 1)
    q_pos = [4 * n - 1, 4 * n - 3001] * (nq // 2)
    got = run(hca, q, w, kp, [0], [0] * nq, q_pos, n, 4, k, qs, ks)
    ref = oracle_mxfp4(q2, qs2, w2, kp, ks, [0], [0, 0], q_pos[:2], 4, k)
    check_idx(got, np.tile(ref, (nq // 2, 1)), "2^20 visible, streaming")


def _fold_sensitive_pairs(n, positive):
    """n cases (w0, w1, a, b): two entries a = (a0, a1) and b = (b0, b1) of E2M1 values whose
    scores w0 relu(x0) + w1 relu(x1), each product and the sum rounded to float32, give
    score(a) >= score(b) (so a, the lower index, wins), while both ways of fusing one product
    into the add (one rounding instead of two) rank b above a. A scorer that contracts the fold
    into a fused multiply-add selects b."""
    f32, f64 = np.float32, np.float64
    grid = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    two = lambda w0, w1, x: f32(f32(w0 * f32(x[0])) + f32(w1 * f32(x[1])))
    fa = lambda w0, w1, x: f32(f64(w0) * x[0] + f64(f32(w1 * f32(x[1]))))
    fb = lambda w0, w1, x: f32(f64(w1) * x[1] + f64(f32(w0 * f32(x[0]))))
    rng = np.random.default_rng(77)
    out = []
    while len(out) < n:
        a, b = rng.choice(grid, 2), rng.choice(grid, 2)
        if a[0] == b[0] or a[1] == b[1] or (positive and max(a.max(), b.max()) == 6.0):
            continue
        w0 = f32(abs(rng.standard_normal()) * 0.125 if positive else rng.standard_normal() * 0.125)
        base = f32(w0 * (a[0] - b[0]) / (b[1] - a[1]))
        if positive and base <= 0:
            continue
        for d in range(-6, 7):
            w1 = (np.array([base], f32).view(np.int32) + d).view(f32)[0]
            if (two(w0, w1, a) >= two(w0, w1, b) and fa(w0, w1, a) < fa(w0, w1, b)
                    and fb(w0, w1, a) < fb(w0, w1, b)):
                out.append((w0, w1, a, b))
                break
    return out


@pytest.mark.parametrize("nq", [8, 264])
@pytest.mark.parametrize("n_fill,k", [(0, 1), (1024, 1025), (1536, 1537)])
def test_mxfp4_score_fold_rounds_each_step(hca, nq, n_fill, k):
    """Every scorer (one query at a time, 4 queries per block, the streaming selector) rounds
    each product and each partial sum of the score to float32, as the oracle's fold does. Query
    i sees its own entries: a and b (entries 0 and 1) of a fold-sensitive case, then n_fill
    entries (6, 6) that outscore both, and k = n_fill + 1 selects all but the loser of a and b.
    Heads 0 and 1 read dims 0 and 1 of the keys; heads 2 and 3 have zero queries and weights."""
    cases = _fold_sensitive_pairs(nq, positive=n_fill > 0)
    code = {v: c for c, v in enumerate([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])}
    nv = n_fill + 2
    keys = np.zeros((nq * nv, 32), np.uint8)
    keys[:, 0] = code[6.0] | (code[6.0] << 4)
    q = np.zeros((nq, 4, 32), np.uint8)
    q[:, 0, 0] = code[1.0]                       # head 0: dim 0
    q[:, 1, 0] = code[1.0] << 4                  # head 1: dim 1
    w = np.zeros((nq, 4), np.float32)
    for i, (w0, w1, a, b) in enumerate(cases):
        keys[i * nv, 0] = code[a[0]] | (code[a[1]] << 4)
        keys[i * nv + 1, 0] = code[b[0]] | (code[b[1]] << 4)
        w[i, :2] = (w0, w1)
    ks = np.full((nq * nv, 2), 127, np.uint8)
    qs = np.full((nq, 4, 2), 127, np.uint8)
    rb = [i * nv for i in range(nq)]
    q_pos = [4 * nv - 1] * nq
    T = torch.from_numpy
    got = run(hca, T(q), T(w), T(keys), rb, list(range(nq)), q_pos, nv, 4, k, T(qs), T(ks))
    want = np.array([0] + list(range(2, nv)), np.int32)
    ref = oracle_mxfp4(T(q), T(qs), T(w), T(keys), T(ks), rb, list(range(nq)), q_pos, 4, k)
    assert (ref == want).all(), "the oracle's fold does not round each step"
    check_idx(got, ref, f"fold nq={nq} k={k}")


def test_mxfp4_all_equal_keys(hca):
    q, qs, w, kp, ks = mx_case(3, 9000, 2)
    kp[:] = kp[0]
    ks[:] = ks[0]
    got = run(hca, q, w, kp, [0], [0, 0], [35999, 20000], 9000, 4, 1024, qs, ks)
    assert (got == np.arange(1024)).all()      # every score ties: the lowest indices win
    check_idx(got, oracle_mxfp4(q, qs, w, kp, ks, [0], [0, 0], [35999, 20000], 4, 1024), "all equal")


def test_mxfp4_zero_scores_dominate(hca):
    # all head weights negative: the best score is 0 (every ReLU off), held by many entries
    q, qs, w, kp, ks = mx_case(4, 30000, 3)
    w = -w.abs()
    got = run(hca, q, w, kp, [0], [0, 0, 0], [119999, 60000, 100], 30000, 4, 1024, qs, ks)
    ref = oracle_mxfp4(q, qs, w, kp, ks, [0], [0, 0, 0], [119999, 60000, 100], 4, 1024)
    check_idx(got, ref, "zero scores")


def test_few_and_no_visible_entries(hca):
    q, qs, w, kp, ks = mx_case(5, 5000, 4)
    q_pos = [2, 3, 4098, 11]                    # n_vis = 0, 1, 1024, 3 with m = 4
    got = run(hca, q, w, kp, [0], [0] * 4, q_pos, 5000, 4, 1024, qs, ks)
    assert (got[0] == -1).all()
    assert got[1, 0] == 0 and (got[1, 1:] == -1).all()
    assert (got[2] == np.arange(1024)).all()
    check_idx(got, oracle_mxfp4(q, qs, w, kp, ks, [0], [0] * 4, q_pos, 4, 1024), "few visible")


def test_small_workspace_batches_queries(hca):
    q, qs, w, kp, ks = mx_case(6, 12000, 7)
    q_pos = [47999 - 1000 * i for i in range(7)]
    one = hca.lightning_index_topk_workspace(1, 12000, 512)
    got = run(hca, q, w, kp, [0], [0] * 7, q_pos, 12000, 4, 512, qs, ks, ws_bytes=one + 100)
    check_idx(got, oracle_mxfp4(q, qs, w, kp, ks, [0], [0] * 7, q_pos, 4, 512), "batched")


def test_more_than_2_19_visible_entries(hca):
    n = 600000
    q, qs, w, kp, ks = mx_case(7, n, 2)
    got = run(hca, q, w, kp, [0], [0, 0], [n - 1, n - 5000], n, 1, 1000, qs, ks)
    check_idx(got, oracle_mxfp4(q, qs, w, kp, ks, [0], [0, 0], [n - 1, n - 5000], 1, 1000), "fallback path")


def test_maximum_visible_entries_and_k(hca):
    """The documented maximum: 2^21 visible entries (2048 score blocks) with k = 2048, beside a
    query that sees fewer entries in the same launch."""
    n = 1 << 21
    q, qs, w, kp, ks = mx_case(8, n, 2)
    q_pos = [n - 1, n - 700001]
    got = run(hca, q, w, kp, [0], [0, 0], q_pos, n, 1, 2048, qs, ks)
    check_idx(got, oracle_mxfp4(q, qs, w, kp, ks, [0], [0, 0], q_pos, 1, 2048), "2^21 visible, k = 2048")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_float_indexer(hca, dtype):
    for seed in range(20, 40):
        g = synth.generator(seed)
        keys = synth.normal(g, (16000, 64))
        q = synth.normal(g, (3, 4, 64))
        w = synth.normal(g, (3, 4), 0.125)
        if dtype == "bf16":
            keys, q = keys.bfloat16().float(), q.bfloat16().float()
        q_pos = [63999, 30000, 9000]
        kd, qd = keys.double().numpy(), q.double().numpy()
        if all(tie_margin_ok(qd[i], w[i].double().numpy(), kd, (q_pos[i] + 1) // 4, 300) for i in range(3)):
            break
    kk = keys if dtype == "f32" else keys.bfloat16()
    qq = q if dtype == "f32" else q.bfloat16()
    got = run(hca, qq, w, kk, [0], [0] * 3, q_pos, 16000, 4, 300)
    ref = np.stack([OI.topk(OI.scores(qd[i], w[i].double().numpy(), kd[:(q_pos[i] + 1) // 4]),
                            (q_pos[i] + 1) // 4, 300) for i in range(3)])
    check_idx(got, ref, dtype)


@pytest.mark.parametrize("dt", ["mxfp4", "f32"])
def test_split_calls_equal_one_call(hca, dt):
    """lightning_index_scores then lightning_index_select (with other GPU work queued between
    them) give the same indices as lightning_index_topk, bit for bit: MXFP4 keys at the
    decode-1M size, and fp32 keys with some queries seeing at most k entries."""
    dev = "cuda"
    g = synth.generator(1018)
    if dt == "mxfp4":
        n, nq, k, m = 1 << 18, 4, 1024, 4
        kp, ks = synth.mxfp4_rows(g, n, 64)
        qp, qs = synth.mxfp4_rows(g, nq * 4, 64)
        q, keys, qsc, ksc = qp.view(nq, 4, 32), kp, qs.view(nq, 4, 2), ks
        q_pos = [4 * n - 1, 4 * n - 1000, 100000, 37]
    else:
        n, nq, k, m = 5000, 6, 64, 4
        q, keys, qsc, ksc = synth.normal(g, (nq, 4, 64)), synth.normal(g, (n, 64)), None, None
        q_pos = [4 * n - 1, 200, 255, 256, 3, 12345]
    w = synth.normal(g, (nq, 4), std=0.125)
    args = lambda: (q.to(dev), w.to(dev), keys.to(dev), torch.zeros(1, dtype=torch.int64, device=dev),
                    torch.zeros(nq, dtype=torch.int32, device=dev), torch.tensor(q_pos, dtype=torch.int64, device=dev),
                    n, m, k)
    ws = torch.empty(hca.lightning_index_topk_workspace(nq, n, k), dtype=torch.uint8, device=dev)
    kw = dict(q_idx_scale=None if qsc is None else qsc.to(dev), k_idx_scale=None if ksc is None else ksc.to(dev))
    one = torch.full((nq, k), -7, dtype=torch.int32, device=dev)
    hca.lightning_index_topk(*args(), one, ws, **kw)
    two = torch.full((nq, k), -7, dtype=torch.int32, device=dev)
    a = args()
    hca.lightning_index_topk(*a, two, ws, phase="scores", **kw)
    junk = torch.randn(1 << 20, device=dev)
    junk.mul_(2.0).add_(1.0)                                # unrelated work between the two halves
    hca.lightning_index_topk(*a, two, ws, phase="select", **kw)
    torch.cuda.synchronize()
    assert torch.equal(one, two)
    assert bool((one >= -1).all())
