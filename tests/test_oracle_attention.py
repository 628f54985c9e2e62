"""Pins of the oracle's CSA/HCA attention: reduction to torch's
scaled_dot_product_attention (an independent library routine) in the
degenerate cases, the window as a ln 2 logit bias on duplicated tokens,
weights summing to one, and log-sum-exp associativity."""
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import attention as A
from oracle import compress as C


def _sdpa(q, K, scale, bias=None):
    """torch SDPA (float64, CPU) of heads q [h, D] over K = V [n, D]; also the lse."""
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(K)[None, None].expand(1, q.shape[0], K.shape[0], K.shape[1])
    mask = None if bias is None else torch.from_numpy(bias)[None, None, None, :]
    o = F.scaled_dot_product_attention(qt, kt, kt, attn_mask=mask, scale=scale)[0, :, 0, :].numpy()
    logits = scale * (torch.from_numpy(q) @ torch.from_numpy(K).T)
    if bias is not None:
        logits = logits + torch.from_numpy(bias)[None]
    return o, torch.logsumexp(logits, dim=1).numpy()


def _setup(L=50, D=8, h=3, seed=0):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(L, D)), rng.normal(size=(h, D)), 1.0 / math.sqrt(D)


def test_csa_reduces_to_causal_mqa():
    x, q, sc = _setup()
    ent = C.compress(x, np.zeros_like(x), np.zeros((1, x.shape[1])), 1, 1, 0, len(x))   # identity
    for t in (0, 7, 49):
        idx = np.arange(t + 1)
        o, lse = A.csa(q, t, ent, np.concatenate([idx, [-1, -1]]), x, 0, sc)
        ro, rl = _sdpa(q, x[: t + 1], sc)
        assert np.allclose(o, ro, atol=1e-13) and np.allclose(lse, rl, atol=1e-13)


def test_hca_reduces_to_causal_mqa():
    x, q, sc = _setup(seed=1)
    for t in (0, 20, 49):
        o, lse = A.hca(q, t, x, 1, x, 0, sc)
        ro, rl = _sdpa(q, x[: t + 1], sc)
        assert np.allclose(o, ro, atol=1e-13) and np.allclose(lse, rl, atol=1e-13)


def test_window_duplicates_recent_tokens():
    # with every token also present as an entry, the window's W most recent tokens count twice:
    # identical to one softmax with a +ln 2 logit bias on positions t-W+1..t
    x, q, sc = _setup(seed=2)
    for t, W in ((30, 5), (3, 10), (49, 1)):
        o, lse = A.hca(q, t, x, 1, x, W, sc)
        bias = np.zeros(t + 1)
        bias[max(0, t - W + 1):] = math.log(2.0)
        ro, rl = _sdpa(q, x[: t + 1], sc, bias)
        assert np.allclose(o, ro, atol=1e-13) and np.allclose(lse, rl, atol=1e-13)


def test_window_alone_before_first_entry():
    x, q, sc = _setup(seed=3)
    t, W, mp = 6, 4, 8                      # no HCA entry is complete yet
    o, lse = A.hca(q, t, np.zeros((0, x.shape[1])), mp, x, W, sc)
    ro, rl = _sdpa(q, x[t - W + 1: t + 1], sc)
    assert np.allclose(o, ro, atol=1e-13) and np.allclose(lse, rl, atol=1e-13)


def test_csa_with_all_entries_selected_is_dense():
    rng = np.random.default_rng(4)
    x, q, sc = _setup(L=64, seed=4)
    ent = C.compress(x, rng.normal(size=x.shape), rng.normal(size=(8, x.shape[1])), 4, 8, 0, 16)
    t = 63
    o1, l1 = A.csa(q, t, ent, rng.permutation(16), x, 9, sc)
    o2, l2 = A.hca(q, t, ent, 4, x, 9, sc)
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


def test_constant_values_and_weights_sum_to_one():
    _, q, sc = _setup(seed=5)
    E = np.tile(np.arange(8.0), (11, 1))
    o, lse = A.attend(q, E, sc)
    assert np.allclose(o, E[0], atol=1e-14)
    assert np.allclose(lse, math.log(11) + sc * (q @ E[0]), atol=1e-13)


def test_lse_merge_of_any_partition():
    rng = np.random.default_rng(6)
    E = rng.normal(size=(30, 8))
    q = rng.normal(size=(4, 8))
    o, lse = A.attend(q, E, 0.3)
    perm = rng.permutation(30)
    parts = np.split(perm, [7, 8, 21])
    acc_o, acc_l = np.zeros_like(o), np.full(4, -np.inf)
    for p in parts + [np.array([], int)]:
        po, pl = A.attend(q, E[p], 0.3)
        acc_o, acc_l = A.merge(acc_o, acc_l, po, pl)
    assert np.allclose(acc_o, o, atol=1e-13) and np.allclose(acc_l, lse, atol=1e-13)


def test_empty_set():
    o, lse = A.attend(np.ones((2, 3)), np.zeros((0, 3)), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_window_store_as_callable_including_empty_window():
    x, q, sc = _setup(seed=7)
    ent = C.compress(x, np.zeros_like(x), np.zeros((1, x.shape[1])), 1, 1, 0, len(x))
    rows = lambda pos: x[np.asarray(pos)]
    for W in (0, 1, 6):
        a = A.csa(q, 30, ent, np.arange(20), rows, W, sc)
        b = A.csa(q, 30, ent, np.arange(20), x, W, sc)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # W = 0 with the first 20 entries only: plain attention over them
    o, lse = A.csa(q, 30, ent, np.arange(20), rows, 0, sc)
    ro, rl = _sdpa(q, x[:20], sc)
    assert np.allclose(o, ro, atol=1e-13) and np.allclose(lse, rl, atol=1e-13)
