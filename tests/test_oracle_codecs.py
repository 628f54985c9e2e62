"""Pins of the oracle's storage codecs against torch's own dtype conversions
(independent library code) and the format definitions (OCP FP8 E4M3FN, OCP MX
E2M1 / E8M0)."""
import numpy as np
import torch

from oracle import codecs


def test_e4m3_table_matches_torch():
    ours = codecs.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # format facts: largest finite 448, smallest subnormal 2^-9, smallest normal 2^-6
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def _e4m3_midpoints():
    t = codecs.e4m3_table()[:0x7F]
    mids = 0.5 * (t[:-1] + t[1:])
    return np.concatenate([t, mids, t[:-1] + 0.3 * (t[1:] - t[:-1])])


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(0)
    v = np.concatenate([_e4m3_midpoints(), rng.normal(0, 30, 20000), rng.normal(0, 0.01, 5000)])
    v = np.clip(v, -448, 448).astype(np.float32)
    v = np.concatenate([v, -v])
    ours = codecs.encode_e4m3(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # compare values (torch may keep the sign of a zero differently)
    assert np.array_equal(codecs.decode_e4m3(ours), codecs.decode_e4m3(ref))


def test_e4m3_ties_to_even_and_saturation():
    # 1 + 1/16 is halfway between 1.0 (code 0x38) and 1.125 (0x39): even code wins
    assert codecs.encode_e4m3([1.0625])[0] == 0x38
    assert codecs.encode_e4m3([1.1875])[0] == 0x3A
    assert codecs.encode_e4m3([2.0 ** -10])[0] == 0x00        # half the smallest subnormal
    assert codecs.encode_e4m3([3 * 2.0 ** -10])[0] == 0x02
    assert codecs.encode_e4m3([460.0, 1e9, -1e9]).tolist() == [0x7E, 0x7E, 0xFE]


def test_bf16_matches_torch():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.normal(0, 1, 50000), rng.normal(0, 1e-30, 1000),
                        rng.normal(0, 1e30, 1000)]).astype(np.float32)
    ours = codecs.encode_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(codecs.decode_bf16(ref), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy())


def test_e2m1_values_match_format():
    # OCP MX E2M1 magnitudes as the format defines them
    assert codecs.E2M1_VALUES[:8].tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for nib in range(16):
        assert codecs.E2M1_VALUES[nib] == codecs._e2m1_from_bits(nib)
    assert np.all(np.signbit(codecs.E2M1_VALUES[8:]))


def test_e8m0_matches_torch():
    ours = codecs.decode_e8m0(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[:255], ref[:255])


def test_mxfp4_packing_and_scale():
    # byte 0x21: element 0 = low nibble (code 1 = 0.5), element 1 = high nibble (code 2 = 1.0)
    packed = np.zeros((1, 32), np.uint8)
    packed[0, 0] = 0x21
    packed[0, 16] = 0xF7      # elements 32, 33: codes 7 (6.0) and 15 (-6.0)
    scales = np.array([[127 + 3, 127 - 2]], np.uint8)
    v = codecs.decode_mxfp4(packed, scales)
    assert v.shape == (1, 64)
    assert v[0, 0] == 0.5 * 8 and v[0, 1] == 1.0 * 8
    assert v[0, 32] == 6.0 / 4 and v[0, 33] == -6.0 / 4
    assert np.count_nonzero(v) == 4
