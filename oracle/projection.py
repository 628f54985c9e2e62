"""Grouped output projection after core attention, float64 (test
infrastructure only).

Source: hyper.ai page for arXiv 2606.19348 ("DeepSeek-V4"), section 方法
(Method), CSA paragraph: core attention is followed by a grouped output
projection, to manage the computational cost.

Readings of what the page leaves open: the heads are split into G equal
groups of consecutive heads; group g's head outputs, concatenated into one
vector of (h/G)*D values, are multiplied by the group's own weight matrix
W[g] of shape [n_group, (h/G)*D] (out-features by in-features); the G
results are concatenated into the projection's output of G*n_group values.
G and n_group are inputs (the page gives neither).
"""

import numpy as np


def grouped_projection(x, w):
    """x: [n, G*K] (group g = columns g*K .. (g+1)*K - 1); w: [G, N, K].
    Returns y [n, G*N] with y[:, g*N:(g+1)*N] = x[:, g*K:(g+1)*K] @ w[g].T."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    G, N, K = w.shape
    assert x.shape[1] == G * K
    return np.concatenate([x[:, g * K:(g + 1) * K] @ w[g].T for g in range(G)], axis=1)
