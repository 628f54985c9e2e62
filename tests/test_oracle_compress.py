"""Pins of the oracle's CSA/HCA compression: counts and window membership by
brute force, and closed-form special cases (mean, copy, identity, logistic)."""
import numpy as np
import pytest
from scipy.special import expit

from oracle import compress as C


@pytest.mark.parametrize("m", [1, 2, 4])
@pytest.mark.parametrize("mult", [1, 2])
def test_counts_and_membership_brute_force(m, mult):
    w = mult * m
    for L in range(0, 65):
        # an entry exists once all of its raw positions are present; its last position is (j+1)m-1
        complete = [j for j in range(L + 1) if all(t < L for _, t in C.window(j, m, w))
                    and max(t for _, t in C.window(j, m, w)) == (j + 1) * m - 1]
        assert complete == list(range(C.n_entries(L, m)))
    # every raw position belongs to exactly `mult` entries (away from the tail), each covering w positions
    L = 16 * m
    cover = np.zeros(L, int)
    for j in range(C.n_entries(L, m)):
        pairs = C.window(j, m, w)
        ts = [t for _, t in pairs]
        assert ts == sorted(ts) and len(set(ts)) == len(ts)
        assert [p for p, _ in pairs] == [t - ts[-1] + w - 1 for t in ts]   # p counts from the window start
        for t in ts:
            cover[t] += 1
    assert np.all(cover[: L - (mult - 1) * m] == mult)


def test_hca_windows_partition():
    m = 8
    owner = {}
    for j in range(10):
        for _, t in C.window(j, m, m):
            assert t not in owner
            owner[t] = j
    assert all(owner[t] == t // m for t in range(80))


def _rand(shape, seed):
    return np.random.default_rng(seed).normal(size=shape)


def test_zero_logits_give_mean_of_available_rows():
    L, D, m, w = 40, 6, 4, 8
    x = _rand((L, D), 0)
    y = C.compress(x, np.zeros((L, D)), np.zeros((w, D)), m, w, 0, L // m)
    assert np.allclose(y[0], x[0:4].mean(axis=0), rtol=0, atol=1e-14)    # window truncated at 0
    for j in range(1, L // m):
        assert np.allclose(y[j], x[4 * j - 4: 4 * j + 4].mean(axis=0), rtol=0, atol=1e-14)


def test_one_hot_position_bias_copies_that_row():
    L, D, m, w = 48, 5, 4, 8
    x = _rand((L, D), 1)
    for pstar in range(w):
        beta = np.zeros((w, D))
        beta[pstar] = 800.0          # exp(-800) underflows to exactly 0
        y = C.compress(x, np.zeros((L, D)), beta, m, w, 0, L // m)
        for j in range(1, L // m):
            assert np.array_equal(y[j], x[j * m - (w - m) + pstar])


def test_one_hot_logit_copies_that_token_in_every_window_holding_it():
    L, D, m, w = 32, 3, 4, 8
    x = _rand((L, D), 2)
    tstar = 13
    z = np.zeros((L, D))
    z[tstar] = 800.0
    y = C.compress(x, z, np.zeros((w, D)), m, w, 0, L // m)
    holders = [j for j in range(L // m) if j * m - 4 <= tstar < j * m + 4]
    assert holders == [3, 4]
    for j in holders:
        assert np.array_equal(y[j], x[tstar])


def test_m1_is_identity_and_constant_kv_is_preserved():
    L, D = 20, 4
    x = _rand((L, D), 3)
    y = C.compress(x, _rand((L, D), 4), _rand((1, D), 5), 1, 1, 0, L)
    assert np.array_equal(y, x)
    y2 = C.compress(np.full((64, D), 2.5), _rand((64, D), 6), _rand((8, D), 7), 4, 8, 0, 16)
    assert np.allclose(y2, 2.5, rtol=0, atol=1e-14)


def test_two_position_window_is_logistic():
    a, b = 0.7, -1.3
    x = np.array([[1.0, -2.0], [3.0, 5.0]])
    z = np.array([[a, 0.0], [b, 0.0]])
    beta = np.array([[0.2, 0.0], [0.0, 0.0]])
    y = C.compress(x, z, beta, 2, 2, 0, 1)
    g = expit((a + 0.2) - b)
    assert np.allclose(y[0, 0], g * 1.0 + (1 - g) * 3.0, rtol=1e-15)
    assert np.allclose(y[0, 1], 0.5 * (-2.0) + 0.5 * 5.0, rtol=1e-15)


def test_channels_independent_and_scalar_logits():
    L, D, m, w = 24, 6, 4, 8
    x, z, beta = _rand((L, D), 8), _rand((L, D), 9), _rand((w, D), 10)
    y = C.compress(x, z, beta, m, w, 0, L // m)
    z2 = z.copy()
    z2[:, 2] += _rand(L, 11)
    y2 = C.compress(x, z2, beta, m, w, 0, L // m)
    assert np.array_equal(np.delete(y, 2, axis=1), np.delete(y2, 2, axis=1))
    assert not np.allclose(y[:, 2], y2[:, 2])
    zs = _rand((L, 1), 12)
    assert np.allclose(C.compress(x, zs, beta, m, w, 0, L // m),
                       C.compress(x, np.repeat(zs, D, axis=1), beta, m, w, 0, L // m), atol=1e-15)


def test_offset_runs_match_whole_sequence():
    L, D, m, w = 64, 4, 4, 8
    x, z, beta = _rand((L, D), 13), _rand((L, D), 14), _rand((w, D), 15)
    full = C.compress(x, z, beta, m, w, 0, L // m)
    # entries 5..12 from rows 16.. (halo of w - m rows before entry 5's block)
    part = C.compress(x[16:], z[16:], beta, m, w, 5, 8, first_pos=16)
    assert np.array_equal(part, full[5:13])


def test_pow2_scale_is_the_smallest_power_of_two_covering_448():
    rng = np.random.default_rng(16)
    amax = np.concatenate([np.exp(rng.uniform(-30, 30, 5000)), 448.0 * 2.0 ** np.arange(-20, 20)])
    s = C.pow2_scale(amax)
    e = np.log2(s)
    assert np.array_equal(e, np.round(e))
    assert np.all(amax <= 448 * s) and np.all(amax > 224 * s)
    assert np.array_equal(C.pow2_scale(448.0 * 2.0 ** np.arange(-5, 5)), 2.0 ** np.arange(-5, 5))
    assert C.pow2_scale(np.array([0.0]))[0] == 1.0
    assert C.pow2_scale(np.array([1e-40]))[0] == 2.0 ** -126           # floor: a normal float32


def test_split_encoding_error_within_half_an_ulp():
    rng = np.random.default_rng(17)
    y = rng.normal(size=(200, 512)) * np.exp(rng.uniform(-5, 5, (200, 1)))
    st = C.encode(y, "split", 448, 64)
    dec = C.decode(st, "split")
    s = st["scale"].astype(np.float64)[:, None]
    assert np.max(np.abs(dec[:, :448]) / s) <= 448.0
    # E4M3 spacing at |v|: 2^(floor(log2|v|)-3) for normals, 2^-9 for subnormals (in units of s)
    v = np.abs(y[:, :448]) / s
    ulp = np.where(v < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(v, 1e-300))) - 3))
    assert np.all(np.abs(dec[:, :448] / s - y[:, :448] / s) <= 0.5 * ulp + 1e-12)
    r = np.abs(y[:, 448:])
    assert np.all(np.abs(dec[:, 448:] - y[:, 448:]) <= 2.0 ** (np.floor(np.log2(r)) - 8) + 1e-300)
