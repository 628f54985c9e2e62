"""Storage formats of the path, decoded exactly to float64 and encoded with
round-to-nearest-even (test infrastructure only).

Formats (hyper.ai page for arXiv 2606.19348, section 方法, efficiency
paragraph: BF16 RoPE dimensions, FP8 for the rest, FP4 indexer; the
DeepSeek-V4-Pro model card's "Tensor type" list: F8_E4M3, F8_E8M0):

* FP8 = OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
  infinities; S.1111.111 is NaN; largest finite value 448.
* BF16: the top 16 bits of an IEEE binary32.
* FP4 = OCP E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit;
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* E8M0 block scale: 2**(code - 127); code 255 is NaN.
* MXFP4 block: 32 E2M1 elements sharing one E8M0 scale; two elements per
  byte, element 2i in the low nibble of byte i.

Encoders round to nearest, ties to the even code, and saturate to the
largest finite magnitude. Non-finite inputs are outside the contract.
"""

import numpy as np

E4M3_MAX = 448.0


def _e4m3_magnitude(code):
    e = (code >> 3) & 0xF
    man = code & 0x7
    if e == 0:
        return man * 2.0 ** -9          # subnormal: 0.mmm x 2^(1-7)
    return (1.0 + man / 8.0) * 2.0 ** (e - 7)


def e4m3_table():
    """float64 value of every one of the 256 E4M3FN codes (NaN at 0x7F, 0xFF)."""
    t = np.empty(256)
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            t[c] = np.nan
        else:
            mag = _e4m3_magnitude(c & 0x7F)
            t[c] = -mag if c & 0x80 else mag
    return t


_E4M3 = e4m3_table()


def decode_e4m3(codes):
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def _round_to_grid(mag, grid):
    """Index of the nearest value in the increasing grid (ties -> even index).
    The grid index equals the code for the positive codes of E4M3/BF16."""
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.searchsorted(grid, mag, side="left")
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    dlo = mag - grid[lo]
    dhi = grid[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    return np.where(mag >= grid[-1], len(grid) - 1, idx)


_E4M3_POS = np.array([_e4m3_magnitude(c) for c in range(0x7F)])  # codes 0..126


def encode_e4m3(values):
    """float64 -> E4M3FN codes (uint8), RNE, saturating at +-448."""
    v = np.asarray(values, dtype=np.float64)
    assert np.all(np.isfinite(v)), "non-finite input"
    code = _round_to_grid(np.abs(v), _E4M3_POS).astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 7
    return code | sign


def decode_bf16(bits):
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


_BF16_POS = decode_bf16(np.arange(0x7F80, dtype=np.uint16))  # +0 .. largest finite


def encode_bf16(values):
    """float64 -> bf16 bit patterns (uint16), RNE straight from float64."""
    v = np.asarray(values, dtype=np.float64)
    assert np.all(np.isfinite(v)), "non-finite input"
    code = _round_to_grid(np.abs(v), _BF16_POS).astype(np.uint16)
    return code | (np.signbit(v).astype(np.uint16) << 15)


def encode_f32(values):
    """float64 -> float32, RNE (numpy's conversion)."""
    return np.asarray(values, dtype=np.float64).astype(np.float32)


E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def _e2m1_from_bits(nib):
    """E2M1 nibble -> value from its bit fields (sign, 2-bit exponent with
    bias 1, 1 mantissa bit); used to build and cross-check the table."""
    s = -1.0 if nib & 8 else 1.0
    e = (nib >> 1) & 3
    man = nib & 1
    if e == 0:
        return s * man * 0.5
    return s * (1.0 + man / 2.0) * 2.0 ** (e - 1)


def decode_e2m1(nibbles):
    return E2M1_VALUES[np.asarray(nibbles, dtype=np.uint8) & 0xF]


def decode_e8m0(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    out = np.exp2(c - 127.0)
    return np.where(c == 255, np.nan, out)


def decode_mxfp4(packed, scales, block=32):
    """Packed MXFP4 rows -> float64.

    packed: uint8 [..., d/2] (element 2i in the low nibble of byte i),
    scales: uint8 [..., d/block] E8M0. Returns float64 [..., d].
    """
    packed = np.asarray(packed, dtype=np.uint8)
    lo = packed & 0xF
    hi = packed >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    vals = decode_e2m1(nib)
    d = vals.shape[-1]
    sc = decode_e8m0(scales)
    assert sc.shape[-1] * block == d
    return vals * np.repeat(sc, block, axis=-1)


def mx_shared_exp(amax, emax_elem=2):
    """Shared exponent of an MX block (OCP Microscaling Formats v1.0, the
    conversion of a block of values: the scale is 2**(floor(log2(amax)) -
    emax_elem), with emax_elem = 2 for E2M1, whose largest normal is 1.5 * 2**2).

    Readings of what the spec leaves to the implementation: the exponent is
    clamped below at -127 (the smallest E8M0 scale), and a block of zeros gets
    -127 too. floor(log2(amax)) is taken from frexp, so it is exact."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)                  # amax = mant * 2**ex, mant in [0.5, 1)
    e = np.maximum(ex - 1 - emax_elem, -127)
    return np.where(amax == 0, -127, e).astype(np.int64)


_E2M1_POS = E2M1_VALUES[:8]                 # codes 0..7, increasing


def encode_e2m1(values):
    """float64 -> E2M1 codes (uint8 nibbles), nearest with ties to the even
    code, saturating at +-6. A value that rounds to zero magnitude encodes as
    +0 (code 0), whatever its sign."""
    v = np.asarray(values, dtype=np.float64)
    assert np.all(np.isfinite(v)), "non-finite input"
    code = _round_to_grid(np.abs(v), _E2M1_POS).astype(np.uint8)
    sign = (np.signbit(v) & (code != 0)).astype(np.uint8) << 3
    return code | sign


def encode_mxfp4(values, block=32):
    """float64 [..., d] -> (packed uint8 [..., d/2], E8M0 scales uint8
    [..., d/block]): per block of `block` consecutive values the shared
    exponent of mx_shared_exp, elements encode_e2m1(v / 2**exp), two per
    byte with element 2i in the low nibble of byte i."""
    v = np.asarray(values, dtype=np.float64)
    d = v.shape[-1]
    assert d % block == 0 and d % 2 == 0
    blocks = v.reshape(*v.shape[:-1], d // block, block)
    e = mx_shared_exp(np.abs(blocks).max(axis=-1))
    nib = encode_e2m1(blocks / np.ldexp(1.0, e)[..., None]).reshape(v.shape)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)
