"""Pins of the oracle's document masks (packed sequences: a query sees only its
own document, which starts at raw position lo): no mask at lo <= 0, the
selection under a bound equal to the unmasked selection on the shifted keys,
and masked HCA attention on a packed sequence equal to plain attention on the
document alone."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import compress as C
from oracle import indexer as I


@pytest.mark.parametrize("m,w", [(4, 8), (3, 5), (1, 1)])
def test_no_mask_at_lo_zero(m, w):
    rng = np.random.default_rng(20)
    n = 200
    s = rng.normal(size=n)
    s[50:60] = s[10]                                  # ties
    for t in [0, 5, 100, 799]:
        nv = min(I.n_visible(t, m), n)
        for lo in (0, -7):
            vis = I.visible_entries(t, m, w, lo, n)
            assert np.array_equal(vis, np.arange(nv))
            for k in (1, 16, 300):
                assert np.array_equal(I.topk_among(s, vis, k), I.topk(s, nv, k))


def test_bound_equals_unmasked_selection_on_shifted_keys():
    m, w, n = 4, 8, 400
    rng = np.random.default_rng(21)
    s = np.round(rng.normal(size=n), 1)               # many exact ties
    t = 1599                                          # all 400 entries end by t
    for lo in [1, 4, 5, 37, 400, 1592, 1596]:
        vis = I.visible_entries(t, m, w, lo, n)
        J = vis[0] if len(vis) else n
        # the visible entries are exactly J .. n-1, and J's window is the first one within [lo, t]
        assert np.array_equal(vis, np.arange(J, n))
        assert J * m - (w - m) >= lo and (J == 0 or (J - 1) * m - (w - m) < lo)
        for k in (1, 64, 500):
            shifted = I.topk(s[J:], n - J, k)
            want = np.where(shifted >= 0, shifted + J, -1).astype(np.int32)
            assert np.array_equal(I.topk_among(s, vis, k), want)
    assert np.all(I.topk_among(s, I.visible_entries(100, m, w, 101, n), 8) == -1)


def test_masked_hca_on_packed_sequence_is_attention_on_the_document():
    """Two documents packed in one sequence, the second starting at P (a multiple of m'): the
    HCA entries of the second document are compressed from its own rows only, so masked HCA
    attention of a query in it equals HCA attention on that document alone, positions shifted
    by P."""
    rng = np.random.default_rng(22)
    mp, W, D, P, L = 16, 8, 12, 64, 160
    x, z = rng.normal(size=(L, D)), rng.normal(0, 0.5, (L, D))
    beta = rng.normal(0, 0.1, (mp, D))
    packed = C.compress(x, z, beta, mp, mp, 0, L // mp)
    alone = C.compress(x[P:], z[P:], beta, mp, mp, 0, (L - P) // mp)
    q = rng.normal(size=(3, D))
    for t in [P, P + 5, P + 15, P + 16, L - 1]:
        o1, l1 = A.hca(q, t, packed, mp, x, W, 0.3, lo=P)
        o2, l2 = A.hca(q, t - P, alone, mp, x[P:], W, 0.3)
        assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)
    # and the window never reaches into the first document
    assert A.window_positions(P + 2, W, P).min() == P and len(A.window_positions(P + 2, W, P)) == 3
