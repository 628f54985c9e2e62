"""CSA and HCA core attention with the sliding-window branch, float64
(test infrastructure only).

Source: hyper.ai page for arXiv 2606.19348 ("DeepSeek-V4"), section 方法
(Method). CSA paragraph: core attention is MQA with shared keys and values
over the top-k compressed entries. HCA paragraph: dense attention over all
heavily compressed entries; both mechanisms include a supplementary
sliding-window attention branch that keeps causality and models local
dependencies.

Readings of what the pages leave open:

* Shared keys and values: K = V = the stored entry (all D dims, RoPE dims
  included), shared by all query heads; each head's output has D dims.
* Scale: logits are scale * <q_h, e>, scale = 1/sqrt(D) by default.
* The window branch covers raw positions max(0, t-W+1) .. t of the query's
  sequence. Recent tokens can appear both raw and inside compressed
  entries; nothing is de-duplicated.
* The two branches are combined by log-sum-exp, i.e. one joint softmax over
  the union of compressed entries and window tokens.
* HCA entry j is visible at t iff (j + 1) * m' - 1 <= t.
* Document masks (packed sequences, a query's document starting at raw
  position lo): the window starts at lo at the earliest, and an HCA entry is
  visible only if its window [j m', (j+1) m') starts at or after lo; CSA's
  entries are whatever the (masked) indexer selected. lo <= 0 is no mask.
* An empty entry set gives o = 0 and lse = -inf.
* lse is the natural log of the softmax denominator of the scaled logits.
"""

import numpy as np


def attend(q, E, scale):
    """Softmax attention of heads q [h, D] over entries E [n, D] with K = V = E.

    Returns (o [h, D], lse [h]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    h, D = q.shape
    if E.shape[0] == 0:
        return np.zeros((h, D)), np.full(h, -np.inf)
    logits = scale * (q @ E.T)                   # [h, n]
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx)
    den = p.sum(axis=1, keepdims=True)
    o = (p @ E) / den
    return o, mx[:, 0] + np.log(den[:, 0])


def window_positions(t, W, lo=0):
    """Raw positions of the sliding-window branch of a query at position t
    (in a document starting at lo)."""
    return np.arange(max(0, lo, t - W + 1), t + 1)


def merge(o1, lse1, o2, lse2):
    """Log-sum-exp merge of two partial attentions over disjoint entry sets."""
    lse = np.logaddexp(lse1, lse2)
    w1 = np.where(np.isneginf(lse1), 0.0, np.exp(lse1 - lse))
    w2 = np.where(np.isneginf(lse2), 0.0, np.exp(lse2 - lse))
    return w1[:, None] * o1 + w2[:, None] * o2, lse


def csa(q, t, entries, idx, raw, W, scale, lo=0):
    """CSA core attention of one query.

    q [h, D]; t: absolute position; entries [n, D]: decoded compressed
    entries of the sequence; idx: selected entry indices (-1 = padding);
    raw: callable or array mapping raw positions -> decoded rows [., D]
    (the window store); W: window length.
    """
    idx = np.asarray(idx)
    sel = idx[idx >= 0]
    assert len(np.unique(sel)) == len(sel), "duplicate selection"
    win = _rows(raw, window_positions(t, W, lo))
    E = np.concatenate([np.asarray(entries, np.float64)[sel], win], axis=0)
    return attend(q, E, scale)


def hca(q, t, entries, m_prime, raw, W, scale, lo=0):
    """HCA core attention of one query over all visible heavily compressed
    entries plus the window."""
    n_vis = (t + 1) // m_prime
    entries = np.asarray(entries, np.float64)
    assert n_vis <= entries.shape[0], "visible entries missing from the store"
    vis = [j for j in range(n_vis) if j * m_prime >= lo]
    win = _rows(raw, window_positions(t, W, lo))
    E = np.concatenate([entries[np.array(vis, dtype=np.int64)].reshape(len(vis), entries.shape[1]), win], axis=0)
    return attend(q, E, scale)


def _rows(raw, positions):
    if callable(raw):
        r = np.asarray(raw(positions), np.float64)
        return r if r.ndim == 2 else r.reshape(len(positions), -1)
    return np.asarray(raw, np.float64)[positions]
