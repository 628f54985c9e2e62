"""Pins of the oracle's grouped output projection: brute-force sums on tiny
shapes, one group is a plain matrix product, each group's outputs depend on
its own heads only, and block-diagonal identity weights copy the input."""
import numpy as np

from oracle import projection as P


def test_brute_force_sums():
    rng = np.random.default_rng(30)
    G, N, K, n = 3, 4, 5, 2
    x, w = rng.normal(size=(n, G * K)), rng.normal(size=(G, N, K))
    y = P.grouped_projection(x, w)
    for r in range(n):
        for g in range(G):
            for c in range(N):
                s = 0.0
                for k in range(K):
                    s += x[r, g * K + k] * w[g, c, k]
                assert abs(y[r, g * N + c] - s) <= 1e-12 * (1 + abs(s))


def test_one_group_and_group_locality():
    rng = np.random.default_rng(31)
    x, w = rng.normal(size=(6, 40)), rng.normal(size=(1, 7, 40))
    assert np.allclose(P.grouped_projection(x, w), np.einsum("rk,ck->rc", x, w[0]), rtol=0, atol=1e-12)
    G, N, K = 4, 3, 10
    x, w = rng.normal(size=(5, G * K)), rng.normal(size=(G, N, K))
    y = P.grouped_projection(x, w)
    x2 = x.copy()
    x2[:, 2 * K:3 * K] = rng.normal(size=(5, K))          # change group 2's heads only
    y2 = P.grouped_projection(x2, w)
    same = np.ones(G * N, bool)
    same[2 * N:3 * N] = False
    assert np.array_equal(y[:, same], y2[:, same]) and not np.allclose(y[:, ~same], y2[:, ~same])


def test_identity_weights_copy_the_input():
    rng = np.random.default_rng(32)
    G, K = 4, 6
    x = rng.normal(size=(3, G * K))
    w = np.stack([np.eye(K) for _ in range(G)])
    assert np.array_equal(P.grouped_projection(x, w), x)
