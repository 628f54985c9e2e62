"""KV compression of CSA and HCA in float64 (test infrastructure only).

Source: hyper.ai page for arXiv 2606.19348 ("DeepSeek-V4"), section 方法
(Method). CSA paragraph: every m tokens are compressed into one entry using
learnable compression weights and a position bias. HCA paragraph: every
m' >> m tokens merge into one entry, without overlapping compression.

Readings of what the pages leave open:

* Weighting: for entry j, channel c and window position p, the weight is a
  softmax over the window positions of (z[t, c] + beta[p, c]), where z is a
  per-token, per-channel compression logit (a column stride of 0 gives one
  logit per token) and beta is the learnable position bias shared by all
  entries. The entry is sum_p weight * x[t, c].
* Window geometry: entry j covers the w raw positions that end at
  (j + 1) * m - 1, i.e. [j*m - (w - m), j*m + m). HCA uses w = m' (no
  overlap); CSA uses w = 2m (overlap, since only HCA is said to be
  non-overlapping). Positions below 0 drop out of the softmax. The number
  of entries of a length-L sequence is floor(L / m): one entry per m
  tokens; a partial tail is left to the sliding window.
* The RoPE dimensions are compressed like the others.
"""

import numpy as np

from . import codecs


def n_entries(L, m):
    """Number of compressed entries of a sequence of L raw tokens."""
    return L // m


def window(j, m, w):
    """(p, t) pairs of entry j: window position p in [0, w) and raw position
    t >= 0 that the position maps to."""
    start = j * m - (w - m)
    return [(p, start + p) for p in range(w) if start + p >= 0]


def compress(x, z, beta, m, w, first_entry, count, first_pos=0):
    """Compressed entries first_entry .. first_entry + count - 1 in float64.

    x: float64 [n_rows, D] raw KV of positions first_pos .. first_pos+n_rows-1
    z: float64 [n_rows, D] or [n_rows, 1] compression logits
    beta: float64 [w, D] position bias
    Returns float64 [count, D].
    """
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    D = x.shape[1]
    out = np.empty((count, D))
    for jj in range(count):
        pairs = window(first_entry + jj, m, w)
        p = np.array([pp for pp, _ in pairs])
        rows = np.array([t for _, t in pairs]) - first_pos
        assert rows.min() >= 0 and rows.max() < x.shape[0], "raw rows missing"
        a = z[rows] + beta[p]                      # [n_p, D] (broadcast if z is [., 1])
        a = a - a.max(axis=0, keepdims=True)
        e = np.exp(a)
        weight = e / e.sum(axis=0, keepdims=True)  # softmax over window positions
        out[jj] = (weight * x[rows]).sum(axis=0)
    return out


def pow2_scale(amax):
    """Smallest power of two s = 2**e with amax <= 448 * s and e >= -126
    (1 where amax == 0).

    Per-entry scale of the FP8 part of a split entry (a reading: the pages
    name FP8 but no scale granularity). The floor keeps s a normal float32."""
    amax = np.asarray(amax, dtype=np.float64)
    mant, ex = np.frexp(amax)                      # amax = mant * 2**ex, mant in [0.5, 1)
    e = np.maximum(ex - 9 + (mant > 0.875), -126)  # 448 = 0.875 * 2**9
    s = np.ldexp(1.0, e)
    return np.where(amax == 0, 1.0, s)


def encode(y, layout, d_nope, d_rope):
    """Encode float64 entries [n, D] into a store.

    layout "f32": {"data": float32 [n, D]}
    layout "bf16": {"data": uint16 [n, D]} (bf16 bits)
    layout "split": {"nope": uint8 E4M3 [n, d_nope], "scale": float32 [n],
                     "rope": uint16 bf16 [n, d_rope]}
    """
    y = np.asarray(y, dtype=np.float64)
    assert y.shape[1] == d_nope + d_rope
    if layout == "f32":
        return {"data": codecs.encode_f32(y)}
    if layout == "bf16":
        return {"data": codecs.encode_bf16(y)}
    assert layout == "split"
    nope = y[:, :d_nope]
    s = pow2_scale(np.abs(nope).max(axis=1) if d_nope else np.zeros(len(y)))
    return {"nope": codecs.encode_e4m3(nope / s[:, None]),
            "scale": s.astype(np.float32),
            "rope": codecs.encode_bf16(y[:, d_nope:])}


def decode(store, layout):
    """Store -> float64 [n, D] (exact)."""
    if layout == "f32":
        return np.asarray(store["data"], dtype=np.float32).astype(np.float64)
    if layout == "bf16":
        return codecs.decode_bf16(store["data"])
    assert layout == "split"
    nope = codecs.decode_e4m3(store["nope"]) * np.asarray(store["scale"], np.float64)[:, None]
    return np.concatenate([nope, codecs.decode_bf16(store["rope"])], axis=1)
