"""Pins of the oracle's lightning-indexer scores and top-k: a hand-computed
example, brute-force selection, and exact rational arithmetic for MXFP4."""
from fractions import Fraction

import numpy as np
import torch

from oracle import codecs, indexer as I


def test_scores_hand_computed():
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    w = np.array([1.0, -2.0])
    keys = np.array([[1.0, 1.0], [-1.0, 2.0], [3.0, -1.0], [-1.0, -1.0]])
    # per head: relu(<q_h, k>) = [1,1], [0,2], [3,0], [0,0]
    assert I.scores(q, w, keys).tolist() == [1 - 2, 0 - 4, 3 - 0, 0.0]


def test_visibility_brute_force():
    for m in (1, 2, 4, 128):
        for t in range(0, 600):
            vis = [j for j in range(t + 2) if (j + 1) * m - 1 <= t]
            assert I.n_visible(t, m) == len(vis) and vis == list(range(len(vis)))


def _brute_topk(s, n_vis, k):
    best = sorted(range(n_vis), key=lambda j: (-float(s[j]), j))[:k]
    return sorted(best) + [-1] * (k - min(k, n_vis))


def test_topk_brute_force_with_ties_and_padding():
    rng = np.random.default_rng(0)
    for trial in range(300):
        n = int(rng.integers(0, 80))
        s = rng.integers(-3, 4, size=n).astype(np.float64)       # many exact ties
        n_vis = int(rng.integers(0, n + 1))
        k = int(rng.integers(1, 40))
        assert I.topk(s, n_vis, k).tolist() == _brute_topk(s, n_vis, k)


def test_topk_prefers_lower_index_on_ties():
    assert I.topk(np.array([5.0, 7.0, 7.0, 7.0, 1.0]), 5, 2).tolist() == [1, 2]
    assert I.topk(np.array([0.0, -0.0, 0.0]), 3, 2).tolist() == [0, 1]


def test_mxfp4_scores_exact_and_fold_in_float32():
    rng = np.random.default_rng(1)
    H, d, n = 4, 64, 300
    qp = rng.integers(0, 256, (H, d // 2), dtype=np.uint8)
    qs = rng.integers(125, 128, (H, d // 32), dtype=np.uint8)
    kp = rng.integers(0, 256, (n, d // 2), dtype=np.uint8)
    ks = rng.integers(125, 128, (n, d // 32), dtype=np.uint8)
    q = codecs.decode_mxfp4(qp, qs)
    k = codecs.decode_mxfp4(kp, ks)
    w = (rng.normal(size=H) / 8).astype(np.float32)
    s = I.scores_mxfp4(q, w, k)
    # exact rational dot products
    qf = [[Fraction(float(v)) for v in row] for row in q]
    for j in range(0, n, 7):
        kf = [Fraction(float(v)) for v in k[j]]
        r = [max(Fraction(0), sum(a * b for a, b in zip(qf[h], kf))) for h in range(H)]
        # fold in float32 with torch (separate multiply and add, head order)
        acc = torch.tensor(float(r[0]), dtype=torch.float32) * torch.tensor(w[0])
        for h in range(1, H):
            acc = acc + torch.tensor(float(r[h]), dtype=torch.float32) * torch.tensor(w[h])
        assert float(r[0]) == float(np.float32(float(r[0])))
        assert acc.item() == float(s[j])
    # same set of scores as the float64 definition up to float32 rounding
    assert np.allclose(s, I.scores(q, w, k), rtol=1e-6, atol=1e-6)
