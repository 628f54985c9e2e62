"""Shared helpers of the test suite: comparisons of GPU results with the oracle
at the tolerances of the path, and case plumbing."""
import numpy as np
import torch

from oracle import codecs, compress, indexer

# Attention tolerances: max |o - o_ref| <= TOL * ||o_ref||_inf, |lse - lse_ref| <= LSE_TOL.
TOL_O = {"fp32": 1e-4, "low": 2e-2}
TOL_LSE = {"fp32": 1e-5, "low": 1e-2}


def np_(t):
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().numpy()
    return np.asarray(t)


def case_numpy(case, keys=None):
    """Host numpy copies of a case's tensors (bf16 stays as int16 bits)."""
    return {k: np_(v) for k, v in case.t.items() if keys is None or k in keys}


def to_device(case, dev="cuda"):
    case.t = {k: v.to(dev) for k, v in case.t.items()}
    return case


def bf16_ulp(y):
    a = np.abs(np.asarray(y, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -133)))
    return 2.0 ** (np.maximum(e, -126) - 7)


def e4m3_ulp(v):
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -20)))
    return np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))


# Compressed entries are computed in float32 on the GPU: besides the stored format's own
# rounding (1 ulp), allow a float32 evaluation error of EVAL * sum_p weight_p * |x_p| (the
# weighted sum of magnitudes, i.e. the entry compressed from |x|), which covers the exp and
# the accumulation of up to a few hundred terms and matters only under cancellation.
EVAL = 2.0 ** -16


def check_f32_entries(gpu, y, yabs, what):
    gpu = np.asarray(gpu, np.float64)
    err = np.abs(gpu - y)
    bound = EVAL * yabs + 2.0 ** -24 * np.abs(y)
    assert np.all(err <= bound), f"{what}: max err {err.max():.3e}"


def check_bf16_entries(gpu_bits, y, what, yabs=None):
    dec = codecs.decode_bf16(np.asarray(gpu_bits).view(np.uint16))
    err = np.abs(dec - y)
    ok = err <= bf16_ulp(y) + (0.0 if yabs is None else EVAL * yabs)
    bad = np.argwhere(~ok)[:6].tolist()
    detail = [(r, c, float(y[r, c]), float(dec[r, c])) for r, c in bad] if y.ndim == 2 else bad
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} elements beyond 1 bf16 ulp (max err {err.max():.3e}) {detail}"


def check_split_entries(nope, scale, rope, y, d_nope, what, yabs):
    """Each stored element within 1 ulp of the stored format (plus the float32 evaluation
    allowance); the power-of-two scale equal to the oracle's unless the oracle's amax/448 lies
    within 2^-20 (relative) of a power of two."""
    nope = np.asarray(nope, np.uint8)
    scale = np.asarray(scale, np.float64)
    y_n, y_r = y[:, :d_nope], y[:, d_nope:]
    amax = np.abs(y_n).max(axis=1)
    s_ref = compress.pow2_scale(amax)
    r = amax / 448.0
    near = np.abs(r / 2.0 ** np.round(np.log2(np.maximum(r, 1e-300))) - 1.0) <= 2.0 ** -20
    same = scale == s_ref
    neighbour = near & ((scale == 2 * s_ref) | (scale == s_ref / 2))
    assert np.all(same | neighbour), f"{what}: scale mismatch in {np.count_nonzero(~(same | neighbour))} rows"
    dec = codecs.decode_e4m3(nope) * scale[:, None]
    v = y_n / scale[:, None]
    tol = np.maximum(e4m3_ulp(v), e4m3_ulp(dec / scale[:, None])) * scale[:, None] + EVAL * yabs[:, :d_nope]
    err = np.abs(dec - y_n)
    ok = err <= tol
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} FP8 elements beyond 1 ulp (max err {err.max():.3e})"
    check_bf16_entries(rope, y_r, what + " rope", yabs[:, d_nope:])


def check_idx(gpu, ref, what):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    bad = np.nonzero((gpu != ref).any(axis=-1))[0] if gpu.ndim == 2 else ([0] if (gpu != ref).any() else [])
    assert len(bad) == 0, f"{what}: index sets differ for rows {list(bad)[:8]}"


def check_attention(o, lse, o_ref, lse_ref, kind, what):
    o = np.asarray(o, np.float64)
    lse = np.asarray(lse, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    lse_ref = np.asarray(lse_ref, np.float64)
    ninf = np.isneginf(lse_ref)
    assert np.array_equal(ninf, np.isneginf(lse)), f"{what}: -inf lse pattern differs"
    scale = max(np.abs(o_ref).max(), 1e-30)
    err = np.abs(o - o_ref).max()
    assert err <= TOL_O[kind] * scale, f"{what}: max|o err| {err:.3e} > {TOL_O[kind]} * {scale:.3e}"
    if (~ninf).any():
        le = np.abs(lse[~ninf] - lse_ref[~ninf]).max()
        assert le <= TOL_LSE[kind], f"{what}: max|lse err| {le:.3e}"


def bf16_tensor_to_f64(t):
    return codecs.decode_bf16(np_(t.view(torch.int16)).view(np.uint16))


def score_error_bounds(q, w, keys):
    """Per-key bound on |float32 score - exact score| for float (fp32/bf16) inputs.

    A head whose exact dot product is below minus its accumulation bound
    (2^-17 * sum_d |q_d k_d|, far above 64 float32 roundings) is clamped to an
    exact 0 by the ReLU on both sides and contributes no error; every other head
    contributes |w_h| times that bound; the float32 fold adds 2^-20 * sum |w_h r_h|."""
    dots = keys @ q.T                                    # [n, H]
    e = 2.0 ** -17 * (np.abs(keys) @ np.abs(q).T)
    active = dots + e >= 0
    r = np.maximum(dots, 0.0)
    return (np.where(active, e, 0.0) @ np.abs(w)) + 2.0 ** -20 * (r @ np.abs(w))


def tie_margin_ok(q, w, keys, n_vis, k):
    """Float inputs: the oracle's top-k set is the only one consistent with the
    float32 error bounds, i.e. every selected score stays above every unselected
    one, except exact ties whose bounds are zero (both sides then see equal
    scores and break the tie by the lower index)."""
    if n_vis <= k:
        return True
    keys = keys[:n_vis]
    s = indexer.scores(q, w, keys)
    eps = score_error_bounds(q, w, keys)
    order = np.lexsort((np.arange(n_vis), -s))
    sel, uns = order[:k], order[k:]
    lo = (s[sel] - eps[sel]).min()
    hi = (s[uns] + eps[uns]).max()
    if lo > hi:
        return True
    T = s[order[k - 1]]
    bad_sel = sel[(s[sel] - eps[sel]) <= hi]
    bad_uns = uns[(s[uns] + eps[uns]) >= lo]
    conflict = np.concatenate([bad_sel, bad_uns])
    return bool(np.all(s[conflict] == T) and np.all(eps[conflict] == 0))
