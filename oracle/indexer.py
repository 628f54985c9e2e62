"""Lightning indexer: scores and top-k selection (test infrastructure only).

Source: hyper.ai page for arXiv 2606.19348 ("DeepSeek-V4"), section 方法
(Method), CSA paragraph: a lightning indexer selects the top-k compressed KV
entries for core attention; efficiency paragraph: the indexer runs in FP4.

Readings of what the pages leave open:

* Score form: s[j] = sum_h w[h] * max(0, <qI[h], kI[j]>) over the indexer
  heads h, with one indexer key per compressed entry shared by the heads
  and per-query head weights w given as inputs (the form of the lightning
  indexer published with DeepSeek-V3.2; an assumption, not on the pages).
* Causality: entry j is visible at position t iff its last raw position
  (j + 1) * m - 1 is <= t, so n_vis(t) = floor((t + 1) / m).
* Ties go to the lower entry index; when fewer than k entries are visible
  all of them are returned; the selection is returned in ascending entry
  order and padded with -1 up to k.
* Document masks (packed sequences; the pages use sample-level masks in
  pretraining): a query whose document starts at raw position lo sees an
  entry only if every raw position of the entry's window (those >= 0) lies
  in [lo, t]; lo <= 0 is no mask.
* FP4 case: q and keys are MXFP4 (block 32 along the indexer dimension).
  Each per-head dot product is then exact in float32, and the score is
  defined bit-exactly as a float32 fold in head order with separate
  roundings: s = w0*r0; s = s + w_h*r_h for h = 1.. (no fused multiply-add).
"""

import numpy as np


def n_visible(t, m):
    """Compressed entries visible to a query at absolute position t."""
    return (t + 1) // m


def scores(q, w, keys):
    """float64 scores of every key.

    q: [H, d] decoded indexer query, w: [H] head weights, keys: [n, d].
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    r = np.maximum(keys @ q.T, 0.0)              # [n, H]
    return r @ w


def scores_mxfp4(q, w, keys):
    """Bit-exact float32 scores for MXFP4-decoded q [H, d] and keys [n, d]."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    r = np.maximum(keys @ q.T, 0.0)              # exact: dyadic values, small spread
    r32 = r.astype(np.float32)
    assert np.array_equal(r32.astype(np.float64), r), "dot product not exact in float32"
    w32 = np.asarray(w, dtype=np.float32)
    s = r32[:, 0] * w32[0]
    for h in range(1, r32.shape[1]):
        s = s + r32[:, h] * w32[h]               # float32 multiply, then float32 add
    return s


def topk(s, n_vis, k):
    """Indices of the k largest of s[:n_vis] (ties -> lower index), ascending,
    padded with -1 to length k (int32)."""
    s = np.asarray(s)[:n_vis]
    order = np.lexsort((np.arange(n_vis), -s.astype(np.float64)))
    sel = np.sort(order[:min(k, n_vis)])
    out = np.full(k, -1, dtype=np.int32)
    out[:len(sel)] = sel
    return out


def visible_entries(t, m, w, lo, n_entries):
    """Entries a query at t in a document starting at lo may select: those
    whose window's raw positions (the ones >= 0) all lie in [lo, t]."""
    out = []
    for j in range(n_entries):
        pos = [p for p in range(j * m - (w - m), (j + 1) * m) if p >= 0]
        if pos and min(pos) >= max(lo, 0) and max(pos) <= t:
            out.append(j)
    return np.array(out, dtype=np.int64)


def topk_among(s, entries, k):
    """The k entries of `entries` with the largest s (ties -> lower index),
    ascending, padded with -1 to length k (int32)."""
    entries = np.asarray(entries, dtype=np.int64)
    s = np.asarray(s)
    order = np.lexsort((entries, -s[entries].astype(np.float64))) if len(entries) else np.array([], np.int64)
    sel = np.sort(entries[order[:min(k, len(entries))]])
    out = np.full(k, -1, dtype=np.int32)
    out[:len(sel)] = sel
    return out
