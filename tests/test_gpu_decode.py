"""GPU parity of the decode-time state (decode_append: raw ring, window store, an
entry per completed block) and of MXFP4 indexer-key compression, against the
oracle (oracle.decode, oracle.codecs.encode_mxfp4, oracle.compress) and
against the bulk compressors bit for bit."""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import codecs
from oracle import compress as OC
from oracle import decode as OD
from tests._common import EVAL, check_bf16_entries, check_f32_entries, check_split_entries, np_

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mods():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_hca_amd as H
    from long_context_attention_hca_amd import workloads as W
    return H, W


def _bits_f64(t):
    return codecs.decode_bf16(np_(t).view(np.uint16))


def _mx_rows(n, d, seed):
    """Rows whose MXFP4 encoding exercises every rule: normal values over a wide exponent
    range, exact E2M1 ties scaled to the block, zero blocks, saturation, and blocks whose
    exponent clamps at -127 (values in [2^-126, 2^-125))."""
    rng = np.random.default_rng(seed)
    v = rng.normal(size=(n, d)) * np.exp2(rng.integers(-30, 30, (n, 1)))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 4.0])
    for r in range(0, n, 7):                                  # ties, block maximum 4 * 2^k or more
        k = int(rng.integers(-20, 20))
        row = rng.choice(mids, d) * rng.choice([-1.0, 1.0], d)
        row[:: 32] = 4.0
        v[r] = row * 2.0 ** k
    v[3] = 0.0
    v[5, :32] = 0.0
    v[9] = np.exp2(-126.0) * rng.uniform(1.0, 1.9, d) * rng.choice([-1.0, 1.0], d)
    return v


@pytest.mark.parametrize("raw_dt,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_mxfp4_output_is_the_encoder_bit_for_bit(mods, raw_dt, d):
    """With m = w = 1 an entry is its one raw row (a softmax over one position weighs it by
    exactly 1), so the MXFP4 store holds encode_mxfp4 of the raw values: codes and scales
    bit-exact, including ties, zero blocks, saturation and the clamped exponent."""
    H, W = mods
    _say(f"mxfp4 identity {raw_dt} d={d}")
    n = 300
    v = _mx_rows(n, d, 11)
    if raw_dt == "bf16":
        xin = synth.bf16_bits(torch.tensor(v, dtype=torch.float32))
        xd = _bits_f64(xin)
    else:
        xin = torch.tensor(v, dtype=torch.float32)
        xd = xin.double().numpy()
    zin = torch.zeros_like(xin)
    bias = torch.zeros(1, d, dtype=torch.float32)
    out = W.empty_store(H.LAYOUT_MXFP4, n, d, 0, "cuda")
    H.csa_compress(xin.cuda(), 0, zin.cuda(), bias.cuda(), 1, 1, 0, n, out)
    torch.cuda.synchronize()
    p_ref, s_ref = codecs.encode_mxfp4(xd)
    assert np.array_equal(np_(out.rope), s_ref), "E8M0 scales differ"
    bad = np.argwhere(np_(out.data) != p_ref)
    assert len(bad) == 0, f"E2M1 bytes differ at {bad[:6].tolist()}"


def _check_mxfp4_entries(codes, scales, y, yabs, what):
    """Stored MXFP4 entries against float64 entries y: the scale equal to the oracle's (or its
    neighbour where the block maximum lies within 2^-16 of a power of two), and each code one
    that rounding some value within the float32 evaluation allowance of y gives."""
    codes, scales = np.asarray(codes, np.uint8), np.asarray(scales, np.uint8)
    n, d = y.shape
    _, s_ref = codecs.encode_mxfp4(y)
    amax = np.abs(y.reshape(n, d // 32, 32)).max(axis=-1)
    near = np.abs(amax / np.exp2(np.round(np.log2(np.maximum(amax, 1e-300)))) - 1.0) <= 2.0 ** -16
    ds = scales.astype(int) - s_ref.astype(int)
    assert np.all((ds == 0) | (near & (np.abs(ds) == 1))), f"{what}: scale mismatch"
    sc = np.repeat(codecs.decode_e8m0(scales), 32, axis=-1)
    eps = (EVAL * yabs + 2.0 ** -24 * np.abs(y)) / sc
    v = y / sc
    lo = codecs.decode_e2m1(codecs.encode_e2m1(v - eps))
    hi = codecs.decode_e2m1(codecs.encode_e2m1(v + eps))
    nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(n, d)
    got = codecs.decode_e2m1(nib)
    ok = (got >= lo) & (got <= hi)
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} E2M1 codes outside the rounding of y"


@pytest.mark.parametrize("raw_dt,d,layout,scalar", [("bf16", 64, "mxfp4", False), ("bf16", 128, "mxfp4", False),
                                                    ("bf16", 64, "mxfp4", True), ("bf16", 64, "bf16", False),
                                                    ("f32", 64, "f32", False), ("f32", 32, "mxfp4", False)])
def test_narrow_key_compression_vs_oracle(mods, raw_dt, d, layout, scalar):
    """The CSA compressor (m = 4, w = 8) on narrow rows (64-dim indexer keys and neighbours:
    several runs of entries share a wave) into MXFP4, bf16 or float32 rows, 1000 entries (a
    ragged last block), against the oracle's float64 entries (MXFP4: encoded by its MXFP4
    encoder)."""
    H, W = mods
    _say(f"narrow keys {raw_dt} d={d} {layout} scalar={scalar}")
    m, w, n = 4, 8, 1000
    g = synth.generator(1012)
    x = synth.normal(g, (n * m, d))
    z = synth.normal(g, (n * m, 1 if scalar else d), std=0.5)
    bias = synth.normal(g, (w, d), std=0.1)
    if raw_dt == "bf16":
        x, z = synth.bf16_bits(x), synth.bf16_bits(z)
        xd, zd = _bits_f64(x), _bits_f64(z)
    else:
        xd, zd = x.double().numpy(), z.double().numpy()
    code = {"mxfp4": H.LAYOUT_MXFP4, "bf16": H.LAYOUT_BF16, "f32": H.LAYOUT_F32}[layout]
    out = W.empty_store(code, n, d, 0, "cuda")
    H.csa_compress(x.cuda(), 0, z.cuda(), bias.cuda(), m, w, 0, n, out, scalar_logits=scalar)
    torch.cuda.synchronize()
    b = bias.double().numpy()
    y = OC.compress(xd, zd, b, m, w, 0, n)
    ya = OC.compress(np.abs(xd), zd, b, m, w, 0, n)
    if layout == "mxfp4":
        _check_mxfp4_entries(np_(out.data), np_(out.rope), y, ya, "narrow keys")
    elif layout == "bf16":
        check_bf16_entries(np_(out.data), y, "narrow keys", ya)
    else:
        check_f32_entries(np_(out.data), y, ya, "narrow keys")


DECODE_CASES = [
    # m, w, m', W, d_nope, d_rope, d_idx, steps, first step of each sequence (None: idle)
    (4, 8, 128, 128, 448, 64, 64, 300, [0, 37, None]),
    (3, 5, 20, 7, 48, 16, 32, 150, [0, 11, None]),      # m' not a multiple of 8: a short last block
]


@pytest.mark.parametrize("m,w,mp,Wn,dn,dr,di,T,start", DECODE_CASES)
def test_decode_append_equals_bulk_and_oracle(mods, m, w, mp, Wn, dn, dr, di, T, start):
    """Decode steps over a batch of three sequences: sequence 0 from the first step, sequence 1
    from a later one, sequence 2 idle throughout (pos = -1). The CSA, HCA and MXFP4 indexer-key
    entries emitted along the way equal the bulk compressors' bit for bit and the oracle to
    the compression tolerances; the window store and win_pos0 hold the last W tokens (checked
    mid-run and at the end); the idle sequence's rows stay untouched; at D = 512, HCA attention
    through the decode-built window equals attention through a contiguous window bit for bit."""
    H, W = mods
    _say(f"decode m={m} w={w} m'={mp} W={Wn} D={dn}+{dr} d_idx={di}")
    B = 3
    D = dn + dr
    g = synth.generator(1013)
    X = synth.bf16_bits(synth.normal(g, (B, T, D)))
    ZC = synth.bf16_bits(synth.normal(g, (B, T, D), std=0.5))
    ZH = synth.bf16_bits(synth.normal(g, (B, T, D), std=0.5))
    KI = synth.bf16_bits(synth.normal(g, (B, T, di)))
    ZI = synth.bf16_bits(synth.normal(g, (B, T, di), std=0.5))
    bc, bh, bi = synth.normal(g, (w, D), std=0.1), synth.normal(g, (mp, D), std=0.1), synth.normal(g, (w, di), std=0.1)
    st = W.DecodeState(B, T, bc.cuda(), bh.cuda(), bi.cuda(), d_nope=dn, d_rope=dr, d_idx=di, m=m, w=w,
                       m_prime=mp, W=Wn)
    for s_ in (st.csa, st.hca, st.window):
        s_.data.fill_(0x5A)
    st.idx.data.fill_(0x5A)
    Xc, ZCc, ZHc, KIc, ZIc = (a.cuda() for a in (X, ZC, ZH, KI, ZI))
    ar = torch.arange(B, device="cuda")
    win_ident = lambda xs: _encode_rows(H, W, xs, dn, dr)

    def positions(step):
        return [step - s0 if s0 is not None and step >= s0 else -1 for s0 in start]

    _say("decode steps")
    for step in range(T):
        p = positions(step)
        pos = torch.tensor(p, dtype=torch.int64, device="cuda")
        pc = torch.tensor([max(v, 0) for v in p], device="cuda")
        st.step(pos, Xc[ar, pc], ZCc[ar, pc], ZHc[ar, pc], KIc[ar, pc], ZIc[ar, pc])
        if step == T // 2:
            torch.cuda.synchronize()
            _check_window(H, W, st, 0, T // 2, X[0], Wn, dn, dr, "window mid-run")
    torch.cuda.synchronize()
    _say("bulk comparisons")
    for b in range(2):
        L = T - start[b]
        n_c, n_h = L // m, L // mp
        ref = W.empty_store(H.LAYOUT_SPLIT, n_c, dn, dr, "cuda")
        H.csa_compress(Xc[b, :L], 0, ZCc[b, :L], bc.cuda(), m, w, 0, n_c, ref)
        r0 = b * st.n_c
        for f in ("data", "scale", "rope"):
            assert torch.equal(getattr(st.csa, f)[r0:r0 + n_c], getattr(ref, f)), f"csa {f} seq {b}"
        ref = W.empty_store(H.LAYOUT_SPLIT, n_h, dn, dr, "cuda")
        H.hca_compress(Xc[b, :L], 0, ZHc[b, :L], bh.cuda(), mp, 0, n_h, ref)
        r0 = b * st.n_h
        for f in ("data", "scale", "rope"):
            assert torch.equal(getattr(st.hca, f)[r0:r0 + n_h], getattr(ref, f)), f"hca {f} seq {b}"
        ref = W.empty_store(H.LAYOUT_MXFP4, n_c, di, 0, "cuda")
        H.csa_compress(KIc[b, :L], 0, ZIc[b, :L], bi.cuda(), m, w, 0, n_c, ref)
        r0 = b * st.n_c
        assert torch.equal(st.idx.data[r0:r0 + n_c], ref.data) and torch.equal(st.idx.rope[r0:r0 + n_c], ref.rope)
        _check_window(H, W, st, b, L - 1, X[b], Wn, dn, dr, f"window seq {b}")
    # the idle sequence
    for s_, n in ((st.csa, st.n_c), (st.hca, st.n_h)):
        assert bool((s_.data[2 * n:3 * n] == 0x5A).all())
    assert bool((st.window.data[2 * 2 * Wn:] == 0x5A).all()) and int(st.win_pos0[2]) == 0
    # the oracle, sequence 1: its decode-step model and the compression tolerances
    _say("oracle")
    L = T - start[1]
    xd, zcd, zhd = _bits_f64(X[1, :L]), _bits_f64(ZC[1, :L]), _bits_f64(ZH[1, :L])
    got = OD.run(xd, zcd, bc.double().numpy(), m, w, L)
    y = np.stack([got[j] for j in range(L // m)])
    ya = OC.compress(np.abs(xd), zcd, bc.double().numpy(), m, w, 0, L // m)
    r0 = st.n_c
    check_split_entries(np_(st.csa.data[r0:r0 + L // m]), np_(st.csa.scale[r0:r0 + L // m]),
                        np_(st.csa.rope[r0:r0 + L // m]), y, dn, "decode csa vs oracle", ya)
    got = OD.run(xd, zhd, bh.double().numpy(), mp, mp, L)
    y = np.stack([got[j] for j in range(L // mp)])
    ya = OC.compress(np.abs(xd), zhd, bh.double().numpy(), mp, mp, 0, L // mp)
    r0 = st.n_h
    check_split_entries(np_(st.hca.data[r0:r0 + L // mp]), np_(st.hca.scale[r0:r0 + L // mp]),
                        np_(st.hca.rope[r0:r0 + L // mp]), y, dn, "decode hca vs oracle", ya)
    kid, zid = _bits_f64(KI[1, :L]), _bits_f64(ZI[1, :L])
    got = OD.run(kid, zid, bi.double().numpy(), m, w, L)
    y = np.stack([got[j] for j in range(L // m)])
    ya = OC.compress(np.abs(kid), zid, bi.double().numpy(), m, w, 0, L // m)
    r0 = st.n_c
    _check_mxfp4_entries(np_(st.idx.data[r0:r0 + L // m]), np_(st.idx.rope[r0:r0 + L // m]), y, ya,
                         "decode indexer keys vs oracle")
    if D != 512:
        return
    # HCA attention for each sequence's last token: decode-built window vs a contiguous one
    _say("attention through the window")
    Hh = 16
    q = synth.bf16_bits(synth.normal(g, (2, Hh, D))).view(torch.bfloat16).cuda()
    tq = [T - 1 - start[b] for b in range(2)]
    q_pos = torch.tensor(tq, dtype=torch.int64, device="cuda")
    q_seq = torch.arange(2, dtype=torch.int32, device="cuda")
    ws = W.Workspace("cuda")
    o1, l1 = W.hca_attn(q, st.hca, st.hca_row_begin, mp, max(tq) + 1, st.window, st.win_row_begin, st.win_pos0,
                        Wn, q_seq, q_pos, 1.0 / D ** 0.5, ws)
    rows = torch.cat([Xc[b, tq[b] - Wn + 1:tq[b] + 1] for b in range(2)])
    cw = _encode_rows(H, W, rows, dn, dr)
    o2, l2 = W.hca_attn(q, st.hca, st.hca_row_begin, mp, max(tq) + 1, cw,
                        torch.tensor([0, Wn], dtype=torch.int64, device="cuda"),
                        torch.tensor([t - Wn + 1 for t in tq], dtype=torch.int64, device="cuda"),
                        Wn, q_seq, q_pos, 1.0 / D ** 0.5, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _encode_rows(H, W, xs, dn, dr):
    """Split encodings of raw rows (bf16 [n, D] on the GPU) by the compressor with m = w = 1."""
    n, D = xs.shape
    out = W.empty_store(H.LAYOUT_SPLIT, n, dn, dr, "cuda")
    zeros = torch.zeros_like(xs)
    H.csa_compress(xs.contiguous(), 0, zeros, torch.zeros(1, D, dtype=torch.float32, device="cuda"), 1, 1, 0, n,
                   out)
    return out


def _check_window(H, W, st, b, t, Xb, Wn, dn, dr, what):
    """The window rows of sequence b hold the split encodings of positions max(0,t-W+1)..t at
    row win_row_begin + p - win_pos0, and win_pos0 is the oracle's."""
    pos0 = int(st.win_pos0[b])
    assert pos0 == OD.window_pos0(t, Wn), f"{what}: win_pos0 {pos0}"
    lo = max(0, t - Wn + 1)
    ref = _encode_rows(H, W, Xb[lo:t + 1].cuda(), dn, dr)
    torch.cuda.synchronize()
    rb = b * 2 * Wn
    rows = torch.tensor([rb + p - pos0 for p in range(lo, t + 1)], device="cuda")
    for f in ("data", "scale", "rope"):
        assert torch.equal(getattr(st.window, f)[rows], getattr(ref, f)), f"{what}: {f}"
