"""Pins of the oracle's MXFP4 encoder (OCP Microscaling Formats v1.0: E2M1
elements, E8M0 shared scale 2**(floor(log2 amax) - 2)) and of its decode-step
model (one token appended per step; CSA entry every m tokens, HCA entry every
m' tokens; a window of the last W raw tokens), against brute force, the
format's value table and the bulk compressor."""
import math

import numpy as np
import pytest

from oracle import codecs
from oracle import compress as C
from oracle import decode as DEC


def _nearest_even_code(v):
    """E2M1 code by brute force: the nearest of the 8 magnitudes, ties to the
    even code, saturating at 6; zero magnitude is +0."""
    mags = codecs.decode_e2m1(np.arange(8))
    d = np.abs(abs(v) - mags)
    best = np.flatnonzero(d == d.min())
    c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
    if abs(v) >= 6.0:
        c = 7
    return c | (8 if (v < 0 and c != 0) else 0)


def test_e2m1_encoder_matches_brute_force():
    mags = codecs.decode_e2m1(np.arange(8))
    mids = 0.5 * (mags[:-1] + mags[1:])
    rng = np.random.default_rng(5)
    v = np.concatenate([mags, -mags, mids, -mids, mids + 1e-9, mids - 1e-9, rng.uniform(-9, 9, 4000), [7.9, -100.0]])
    got = codecs.encode_e2m1(v)
    want = np.array([_nearest_even_code(x) for x in v], np.uint8)
    assert np.array_equal(got, want)
    # exact values round-trip; the ties of the format land on the even codes
    assert np.array_equal(codecs.decode_e2m1(codecs.encode_e2m1(mags)), mags)
    assert list(codecs.encode_e2m1(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]))) == [0, 2, 2, 4, 4, 6, 6]


def test_mx_shared_exponent_brackets_amax():
    rng = np.random.default_rng(6)
    a = np.concatenate([np.exp2(rng.uniform(-100, 100, 3000)), np.exp2(np.arange(-120, 120, dtype=np.float64)),
                        np.nextafter(np.exp2(np.arange(-120, 120, dtype=np.float64)), 0)])
    e = codecs.mx_shared_exp(a)
    # scale 2^e with 4 * 2^e <= amax < 8 * 2^e: the block's largest value lands in [4, 8)
    assert np.all(np.ldexp(4.0, e) <= a) and np.all(a < np.ldexp(8.0, e))
    assert all(int(x) == math.floor(math.log2(float(y))) - 2 for x, y in zip(e[:50], a[:50]))
    assert codecs.mx_shared_exp(0.0) == -127 and codecs.mx_shared_exp(2.0 ** -140) == -127


def test_mxfp4_encode_round_trip_and_error_bound():
    rng = np.random.default_rng(7)
    v = rng.normal(0, 1, (300, 64)) * np.exp2(rng.integers(-20, 20, (300, 1)))
    v[0] = 0.0
    v[1, :32] = 0.0
    p, s = codecs.encode_mxfp4(v)
    assert p.shape == (300, 32) and s.shape == (300, 2)
    dec = codecs.decode_mxfp4(p, s)
    # per block: the error is at most half the gap of the grid at the value, i.e. at most
    # 1 * scale for |v| / scale in [4, 6] (gap 2), 0.5 * scale in [2, 4), 0.25 * scale below 2,
    # and v - 6 * scale where it saturates
    blocks, dblocks = v.reshape(300, 2, 32), dec.reshape(300, 2, 32)
    scale = codecs.decode_e8m0(s)[:, :, None]
    r = np.abs(blocks) / scale
    bound = np.where(r >= 6, r - 6, np.where(r >= 4, 1.0, np.where(r >= 2, 0.5, 0.25))) * scale
    assert np.all(np.abs(blocks - dblocks) <= bound + 1e-300)
    assert np.all(dec[0] == 0) and np.all(dec[1, :32] == 0) and s[0, 0] == 0
    # values already on the MXFP4 grid with their own block maximum in [4, 6] * scale re-encode exactly
    codes = rng.integers(0, 16, (50, 64)).astype(np.uint8)
    codes[:, 0] = 7                                    # block maxima 6 * scale
    codes[:, 32] = 6
    sc = rng.integers(100, 150, (50, 2)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    exact = codecs.decode_mxfp4(packed, sc)
    p2, s2 = codecs.encode_mxfp4(exact)
    assert np.array_equal(s2, sc)
    assert np.array_equal(codecs.decode_mxfp4(p2, s2), exact)


@pytest.mark.parametrize("W", [1, 4, 128])
def test_window_layout_holds_the_last_w_positions(W):
    rows = np.full(2 * W, -1)
    for t in range(6 * W + 3):
        for r in DEC.window_rows(t, W):
            rows[r] = t
        lo = max(0, t - W + 1)
        for p in range(lo, t + 1):
            r = DEC.window_row(p, t, W)
            assert 0 <= r < 2 * W and rows[r] == p


@pytest.mark.parametrize("m,w", [(4, 8), (16, 16), (1, 1), (3, 5)])
def test_decode_steps_emit_the_bulk_entries(m, w):
    rng = np.random.default_rng(8)
    L, D = 70, 24
    x, z = rng.normal(size=(L, D)), rng.normal(0, 0.5, (L, D))
    beta = rng.normal(0, 0.1, (w, D))
    got = DEC.run(x, z, beta, m, w, L)
    n = C.n_entries(L, m)
    assert sorted(got) == list(range(n))
    bulk = C.compress(x, z, beta, m, w, 0, n)
    for j in range(n):
        assert np.array_equal(got[j], bulk[j])
    # an entry appears at the step holding its last raw position
    assert [DEC.entries_due(t, m) for t in range(2 * m)] == [None] * (m - 1) + [0] + [None] * (m - 1) + [1]
