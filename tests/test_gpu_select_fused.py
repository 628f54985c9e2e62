"""The top-k selection enqueued with HCA attention (lightning_index_select_pending +
hca_dense_mqa_attn_partials_select): at the decode configuration (4 sequences at 1M context,
64 heads, split stores, MXFP4 indexer keys, k = 1024) the selection runs in the grid of the FP8
HCA kernel, and the step's top-k, CSA and HCA outputs equal, bit for bit, the calls made one
after another. Also: a query whose indexer weights are all negative (its top-k is a run of
exact-zero ties: the selection's second round), an HCA call with no query (the selection runs alone), an HCA
call on the bf16 store path (the selection's 256-thread variant in the grid of the bf16 MFMA
kernel), and an inactive record (an index call with no query)."""
import ctypes
import sys

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mods():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_hca_amd as m
    from long_context_attention_hca_amd import workloads
    return m, workloads


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x


def _outputs(run):
    return [run.idx, run.o_csa, run.lse_csa, run.o_hca, run.lse_hca]


@pytest.mark.parametrize("seed,negative", [(1003, False), (1003 + 7919, True), (1003 + 3 * 7919, False)])
def test_fused_step_equals_serial_calls(mods, seed, negative):
    m, W_ = mods
    _say(f"fused step seed={seed} negative={negative}")
    c = synth.decode_1m(seed=seed, B=4, L=1 << 20, device="cuda")
    if negative:
        c.t["w_idx"][1] = -c.t["w_idx"][1].abs() - 0.01  # query 1: no score above 0
    fused = W_.Decode1M(c, ws=W_.Workspace("cuda"))
    serial = W_.Decode1M(c, ws=W_.Workspace("cuda"), overlap=False)
    fused.step()
    serial.step()
    torch.cuda.synchronize()
    for name, x, y in zip(("idx", "o_csa", "lse_csa", "o_hca", "lse_hca"), _outputs(fused), _outputs(serial)):
        assert torch.equal(_bits(x), _bits(y)), name
    if negative:  # the top-k: the lowest entries among the many that score exactly 0
        sel = fused.idx[1].cpu()
        assert torch.equal(sel, torch.unique(sel)) and int(sel[-1]) < 262144


def test_selection_beside_no_hca_query_and_inactive_record(mods):
    m, W_ = mods
    _say("selection alone; inactive record")
    c = synth.decode_1m(seed=1009, B=4, L=1 << 18, device="cuda")
    run = W_.Decode1M(c, ws=W_.Workspace("cuda"))
    ref = run.index().clone()
    torch.cuda.synchronize()
    run.idx.fill_(-7)
    run.index(phase="scores")
    sel = run.index(phase="pending")
    t = c.t
    # nq = 0 through the C ABI (torch gives empty tensors a NULL data pointer)
    part = m.AttnPartials()
    assert m._hca_attn_partials_select(m._ptr(run.q_hca), m.BF16, 0, 64, run.hca.c(), m._ptr(run.hrb), run.mp,
                                       run.n_h, run.win_hca.c(), m._ptr(run.wrb), m._ptr(run.wp0), run.W,
                                       m._ptr(t["q_seq"]), m._ptr(t["q_pos"]), None, run.scale, m._ptr(run.o_hca),
                                       m.BF16, m._ptr(run.lse_hca), None, 0, m._stream(None), ctypes.byref(sel),
                                       ctypes.byref(part)) == 0
    torch.cuda.synchronize()
    assert part.nq == 0
    assert torch.equal(run.idx, ref)
    # an index call with no query records an inactive selection: the HCA call is the plain one
    args = list(m._index_call_args(t["q_idx"], t["w_idx"], t["k_idx"], run.crb, t["q_seq"], t["q_pos"], run.n_c,
                                   run.m, run.k, run.idx, run.ws.get("index", 1), t["q_idx_scale"],
                                   t["k_idx_scale"], None, None, None, None))
    args[13] = 0  # nq
    none = m.PendingSelect()
    assert m._index_pending(*args, ctypes.byref(none)) == 0
    ws_a, ws_b = W_.Workspace("cuda"), W_.Workspace("cuda")
    oa, la, pa = W_.hca_attn(run.q_hca, run.hca, run.hrb, run.mp, run.n_h, run.win_hca, run.wrb, run.wp0, run.W,
                             t["q_seq"], t["q_pos"], run.scale, ws_a, defer=True, sel=none)
    ob, lb, pb = W_.hca_attn(run.q_hca, run.hca, run.hrb, run.mp, run.n_h, run.win_hca, run.wrb, run.wp0, run.W,
                             t["q_seq"], t["q_pos"], run.scale, ws_b, defer=True)
    m.mqa_attn_merge(pa, pb)
    torch.cuda.synchronize()
    assert torch.equal(_bits(oa), _bits(ob)) and torch.equal(la, lb)


def test_selection_beside_bf16_hca_store(mods):
    """The HCA call takes the bf16-store kernel, whose 256-thread blocks run the selection's
    256-thread variant in the same grid."""
    m, W_ = mods
    _say("selection beside a bf16-store HCA call")
    c = synth.decode_1m(seed=1013, B=4, L=1 << 18, device="cuda")
    run = W_.Decode1M(c, ws=W_.Workspace("cuda"))
    ref = run.index().clone()
    torch.cuda.synchronize()
    run.idx.fill_(-7)
    g = synth.generator(5)
    n_h, Wn = 512, 128
    hs = synth.bf16_bits(synth.normal(g, (4 * n_h, 512))).view(torch.bfloat16).cuda()
    wn = synth.bf16_bits(synth.normal(g, (4 * Wn, 512))).view(torch.bfloat16).cuda()
    q = synth.bf16_bits(synth.normal(g, (4, 64, 512))).view(torch.bfloat16).cuda()
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device="cuda")
    L = 128 * n_h
    args = (q, m.Store.dense(hs, 448, 64), i64([b * n_h for b in range(4)]), 128, n_h, m.Store.dense(wn, 448, 64),
            i64([b * Wn for b in range(4)]), i64([L - Wn] * 4), Wn, torch.arange(4, dtype=torch.int32, device="cuda"),
            i64([L - 1] * 4), 512 ** -0.5)
    run.index(phase="scores")
    sel = run.index(phase="pending")
    ws_a, ws_b = W_.Workspace("cuda"), W_.Workspace("cuda")
    oa, la, pa = W_.hca_attn(*args, ws_a, defer=True, sel=sel)
    ob, lb, pb = W_.hca_attn(*args, ws_b, defer=True)
    m.mqa_attn_merge(pa, pb)
    torch.cuda.synchronize()
    assert torch.equal(run.idx, ref)
    assert torch.equal(_bits(oa), _bits(ob)) and torch.equal(la, lb)
