"""Decode-time state of one layer, step by step (test infrastructure only).

Source: hyper.ai page for arXiv 2606.19348 ("DeepSeek-V4"), section 方法
(Method). CSA paragraph: every m tokens are compressed into one entry and a
lightning indexer scores the compressed entries; HCA paragraph: every m'
tokens merge into one entry without overlap; both branches add a sliding
window over the most recent raw tokens.

During decoding one token arrives per step and per sequence. Once the token
at position t is in:
* the CSA store holds entries j < floor((t+1)/m), the HCA store entries
  j < floor((t+1)/m'), the indexer-key store entries j < floor((t+1)/m):
  an entry appears at the step that completes its block of raw positions,
  and its value is that of compressing the whole sequence at once;
* the window store holds the last W raw tokens.

Layout readings (the pages describe no storage layout):
* Raw ring: the last R raw tokens of a sequence (R at least the longest
  compression window), the token at position p in ring row p mod R.
* Window store: each token at position p is written twice, to rows p mod W
  and p mod W + W, and a per-sequence base position
  win_pos0 = W * floor(max(0, t-W+1) / W) makes position p of the window live
  in row p - win_pos0: the last W positions are one contiguous run of rows,
  which the attention calls read through exactly this linear map.
"""

import numpy as np

from . import compress as C


def ring_row(p, R):
    """The raw-ring row that holds position p."""
    return p % R


def window_rows(p, W):
    """The two window-store rows that the token at position p is written to."""
    return p % W, p % W + W


def window_pos0(t, W):
    """Base position of the window store once the token at t is in."""
    return W * (max(0, t - W + 1) // W)


def window_row(p, t, W):
    """Row of the window store holding position p (max(0,t-W+1) <= p <= t)."""
    return p - window_pos0(t, W)


def entries_due(t, m):
    """Entry completed by the token at position t (the step emits it), or None."""
    return (t + 1) // m - 1 if (t + 1) % m == 0 else None


def run(x, z, beta, m, w, steps):
    """Entries emitted while appending positions 0 .. steps-1 one at a time:
    {j: float64 [D]}, each computed at the step that completes it from the
    raw rows the ring holds at that step (positions t-R+1 .. t, R = w)."""
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    R = w
    ring_x = np.zeros((R, x.shape[1]))
    ring_z = np.zeros((R, z.shape[1]))
    out = {}
    for t in range(steps):
        ring_x[ring_row(t, R)] = x[t]
        ring_z[ring_row(t, R)] = z[t]
        j = entries_due(t, m)
        if j is None:
            continue
        lo = max(0, t - R + 1)                 # first position the ring still holds
        rows = [ring_row(p, R) for p in range(lo, t + 1)]
        out[j] = C.compress(ring_x[rows], ring_z[rows], beta, m, w, j, 1, first_pos=lo)[0]
    return out
