"""hca_dense_mqa_attn_noalloc (the entry point for callers that cannot allocate: its split-K
partials live in the library's static device scratch) against hca_dense_mqa_attn with a
caller workspace, through the C ABI: two calls in a row, the second with a smaller input, each
bit-identical to the workspace entry point's output (the same kernels on the same inputs)."""
import math

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _case(seed, nq, H, n_vis, W):
    g = synth.generator(seed)
    dn, dr = 448, 64
    st = synth.split_entries(g, n_vis, dn, dr)
    win = synth.split_entries(g, nq * W, dn, dr)
    q = synth.normal(g, (nq, H, dn + dr)).bfloat16()
    return st, win, q


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_hca_amd as m
    from long_context_attention_hca_amd import workloads
    return m, workloads


def _run(m, W_, seed, nq, H, n_vis, W, mp):
    dev = "cuda"
    st, win_st, q = _case(seed, nq, H, n_vis, W)
    cache = m.Store.split(st["nope"].to(dev), st["scale"].to(dev), st["rope"].to(dev))
    win = m.Store.split(win_st["nope"].to(dev), win_st["scale"].to(dev), win_st["rope"].to(dev))
    q = q.to(dev)
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device=dev)
    L = n_vis * mp
    # every query sees all n_vis entries of the one cache (cache_row_begin 0 for each sequence)
    # and its own W window rows
    seq = torch.arange(nq, dtype=torch.int32, device=dev)
    pos = torch.full((nq,), L - 1, dtype=torch.int64, device=dev)
    crb = i64([0] * nq)
    wrb = i64([b * W for b in range(nq)])
    wp0 = i64([L - W] * nq)
    scale = 1.0 / math.sqrt(512)
    o_ref, lse_ref = W_.hca_attn(q, cache, crb, mp, n_vis, win, wrb, wp0, W, seq, pos, scale, W_.Workspace(dev))
    assert m.mqa_attn_workspace(m.BF16, nq, H, 512, n_vis + W) > 0  # split-K partials in the scratch
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    m.hca_dense_mqa_attn_noalloc(q, cache, crb, mp, n_vis, win, wrb, wp0, W, seq, pos, scale, o, lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_noalloc_matches_workspace_entry_point_twice(lib):
    m, W_ = lib
    print("noalloc call 1: nq=4 H=64 n_vis=8192 W=128", flush=True)
    _run(m, W_, 2101, nq=4, H=64, n_vis=8192, W=128, mp=128)
    print("noalloc call 2: nq=2 H=16 n_vis=700 W=37", flush=True)
    _run(m, W_, 2102, nq=2, H=16, n_vis=700, W=37, mp=16)
