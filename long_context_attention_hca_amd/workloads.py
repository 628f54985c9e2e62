"""Runs the hybrid-attention hot path on the GPU for the workloads of the
benchmark and the tests: compression (CSA and HCA), lightning-indexer top-k,
CSA sparse and HCA dense MQA attention.

Every step is a call into libhca.so through the binding; torch only allocates
outputs and workspaces and provides the stream. A workload is described by a
`case` object with `.params` (dict) and `.t` (dict of CUDA tensors), as the
seeded generators in `synth` produce.
"""

import math

import torch

from . import (BF16, DecodeLayer, F32, LAYOUT_BF16, LAYOUT_F32, LAYOUT_MXFP4, LAYOUT_SPLIT, Store, csa_compress,
               csa_sparse_mqa_attn, csa_sparse_mqa_attn_partials, decode_append, hca_compress, hca_dense_mqa_attn,
               hca_dense_mqa_attn_partials, hca_dense_mqa_attn_partials_select, lightning_index_select_pending,
               lightning_index_topk, lightning_index_topk_workspace, mqa_attn_merge, mqa_attn_workspace)


def _i64(vals, dev):
    return torch.tensor(vals, dtype=torch.int64, device=dev)


def empty_store(layout, n, d_nope, d_rope, dev):
    """Zero-filled store of n rows."""
    if layout == LAYOUT_F32:
        return Store.dense(torch.zeros(n, d_nope + d_rope, dtype=torch.float32, device=dev), d_nope, d_rope)
    if layout == LAYOUT_BF16:
        return Store.dense(torch.zeros(n, d_nope + d_rope, dtype=torch.int16, device=dev), d_nope, d_rope)
    if layout == LAYOUT_MXFP4:
        assert d_rope == 0 and d_nope % 32 == 0
        return Store.mxfp4(torch.zeros(n, d_nope // 2, dtype=torch.uint8, device=dev),
                           torch.zeros(n, d_nope // 32, dtype=torch.uint8, device=dev))
    return Store.split(torch.zeros(n, d_nope, dtype=torch.uint8, device=dev),
                       torch.zeros(n, dtype=torch.float32, device=dev),
                       torch.zeros(n, d_rope, dtype=torch.int16, device=dev))


def split_store(t, prefix):
    return Store.split(t[f"{prefix}_nope"], t[f"{prefix}_scale"], t[f"{prefix}_rope"])


class Workspace:
    """Grow-only byte buffers reused across calls (zero-filled when allocated)."""

    def __init__(self, dev):
        self.dev = dev
        self.bufs = {}

    def get(self, name, nbytes):
        b = self.bufs.get(name)
        if b is None or b.numel() < nbytes:
            b = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.dev)
            self.bufs[name] = b
        return b


def index_topk(q_idx, w_idx, k_idx, k_row_begin, q_seq, q_pos, max_visible, m, k, ws, q_idx_scale=None,
               k_idx_scale=None, out=None, q_lo=None, w=None, phase="both", stream=None):
    nq = q_idx.shape[0]
    if out is None:
        out = torch.empty(nq, k, dtype=torch.int32, device=q_idx.device)
    # all queries at once up to 4 GiB of workspace (always for the split phases); beyond that
    # the library batches queries
    need = lightning_index_topk_workspace(nq, max_visible, k)
    one = lightning_index_topk_workspace(1, max_visible, k)
    buf = ws.get("index", need if phase != "both" else min(need, max(one, 4 << 30)))
    if phase == "pending":
        # the selection recorded for hca_attn(..., sel=...), which runs it in its own launch
        return lightning_index_select_pending(q_idx, w_idx, k_idx, k_row_begin, q_seq, q_pos, max_visible, m, k, out,
                                              buf, q_idx_scale=q_idx_scale, k_idx_scale=k_idx_scale, q_lo=q_lo, w=w)
    lightning_index_topk(q_idx, w_idx, k_idx, k_row_begin, q_seq, q_pos, max_visible, m, k, out, buf,
                         q_idx_scale=q_idx_scale, k_idx_scale=k_idx_scale, q_lo=q_lo, w=w, phase=phase,
                         stream=stream)
    return out


def csa_attn(q, cache, cache_row_begin, idx, window, win_row_begin, win_pos0, W, q_seq, q_pos, scale, ws,
             o_dtype=None, o=None, lse=None, q_lo=None, stream=None, defer=False):
    """CSA attention; with defer=True the split-K merge is left for mqa_attn_merge and the
    call's AttnPartials is returned as a third value."""
    nq, H, D = q.shape
    if o is None:
        o = torch.empty(nq, H, D, dtype=o_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(nq, H, dtype=torch.float32, device=q.device)
    qd = F32 if q.dtype == torch.float32 else BF16
    buf = ws.get("csa", mqa_attn_workspace(qd, nq, H, D, idx.shape[1] + W))
    if defer:
        part = csa_sparse_mqa_attn_partials(q, cache, cache_row_begin, idx, window, win_row_begin, win_pos0, W, q_seq,
                                            q_pos, scale, o, lse, buf, q_lo=q_lo, stream=stream)
        return o, lse, part
    csa_sparse_mqa_attn(q, cache, cache_row_begin, idx, window, win_row_begin, win_pos0, W, q_seq, q_pos, scale,
                        o, lse, buf, q_lo=q_lo, stream=stream)
    return o, lse


def hca_attn(q, cache, cache_row_begin, m_prime, max_visible, window, win_row_begin, win_pos0, W, q_seq, q_pos,
             scale, ws, o_dtype=None, o=None, lse=None, q_lo=None, stream=None, defer=False, sel=None):
    """HCA attention; defer as in csa_attn. sel: a PendingSelect (index_topk(..., phase="pending"))
    enqueued with the call (deferred calls only)."""
    nq, H, D = q.shape
    if o is None:
        o = torch.empty(nq, H, D, dtype=o_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(nq, H, dtype=torch.float32, device=q.device)
    qd = F32 if q.dtype == torch.float32 else BF16
    buf = ws.get("hca", mqa_attn_workspace(qd, nq, H, D, max_visible + W))
    if sel is not None and not defer:
        raise ValueError("sel needs defer=True")
    if sel is not None:
        part = hca_dense_mqa_attn_partials_select(q, cache, cache_row_begin, m_prime, max_visible, window,
                                                  win_row_begin, win_pos0, W, q_seq, q_pos, scale, o, lse, sel, buf,
                                                  q_lo=q_lo, stream=stream)
        return o, lse, part
    if defer:
        part = hca_dense_mqa_attn_partials(q, cache, cache_row_begin, m_prime, max_visible, window, win_row_begin,
                                           win_pos0, W, q_seq, q_pos, scale, o, lse, buf, q_lo=q_lo, stream=stream)
        return o, lse, part
    hca_dense_mqa_attn(q, cache, cache_row_begin, m_prime, max_visible, window, win_row_begin, win_pos0, W, q_seq,
                       q_pos, scale, o, lse, buf, q_lo=q_lo, stream=stream)
    return o, lse


class DecodeState:
    """Decode-time compression state of one layer for B sequences of up to max_len positions:
    raw rings of R = max(w, m_prime) rows, the window store (2W rows per sequence), CSA and HCA
    entry stores in `layout` and MXFP4 indexer keys (d_idx > 0). step() appends one token per
    sequence with decode_append; the stores are then what the attention and indexer calls read
    (window through win_row_begin / win_pos0)."""

    def __init__(self, B, max_len, bias_csa, bias_hca, bias_idx=None, d_nope=448, d_rope=64, d_idx=64, m=4, w=8,
                 m_prime=128, W=128, layout=LAYOUT_SPLIT, dev="cuda"):
        D = d_nope + d_rope
        R = max(w, m_prime)
        self.B, self.D, self.d_idx, self.m, self.w, self.m_prime, self.W, self.R = B, D, d_idx, m, w, m_prime, W, R
        self.n_c, self.n_h = max_len // m, max_len // m_prime
        z = lambda n, d: torch.zeros(n, d, dtype=torch.int16, device=dev)
        self.rings = {"x": z(B * R, D), "z_csa": z(B * R, D), "z_hca": z(B * R, D)}
        if d_idx:
            self.rings.update({"k_idx": z(B * R, d_idx), "z_idx": z(B * R, d_idx)})
        self.hca_state = torch.zeros(B, 3, D, dtype=torch.float32, device=dev)
        self.window = empty_store(layout, B * 2 * W, d_nope, d_rope, dev)
        self.win_row_begin = _i64([b * 2 * W for b in range(B)], dev)
        self.win_pos0 = torch.zeros(B, dtype=torch.int64, device=dev)
        self.csa = empty_store(layout, B * max(self.n_c, 1), d_nope, d_rope, dev)
        self.csa_row_begin = _i64([b * max(self.n_c, 1) for b in range(B)], dev)
        self.hca = empty_store(layout, B * max(self.n_h, 1), d_nope, d_rope, dev)
        self.hca_row_begin = _i64([b * max(self.n_h, 1) for b in range(B)], dev)
        self.idx = self.idx_row_begin = None
        if d_idx:
            self.idx = empty_store(LAYOUT_MXFP4, B * max(self.n_c, 1), d_idx, 0, dev)
            self.idx_row_begin = self.csa_row_begin
        self.layer = DecodeLayer(m, w, m_prime, W, R, bias_csa, bias_hca, self.rings, self.hca_state, self.window,
                                 self.win_row_begin, self.win_pos0, self.csa, self.csa_row_begin, self.hca,
                                 self.hca_row_begin, self.idx, self.idx_row_begin, bias_idx)

    def step(self, pos, x, z_csa, z_hca, k_idx=None, z_idx=None, stream=None):
        decode_append(self.layer, pos, x, z_csa, z_hca, k_idx, z_idx, stream=stream)


# ---------------------------------------------------------------------------------------------
# Workloads


def tiny_fp32(case, ws=None):
    """Full pipeline on one fp32 sequence: compress (CSA, HCA), index, attend."""
    p, t = case.params, case.t
    dev = t["raw"].device
    ws = ws or Workspace(dev)
    L, m, w, mp, W, k = p["L"], p["m"], p["w"], p["m_prime"], p["W"], p["topk"]
    dn, dr = p["d_nope"], p["d_rope"]
    n_c, n_h = L // m, L // mp
    csa = empty_store(LAYOUT_F32, n_c, dn, dr, dev)
    hca = empty_store(LAYOUT_F32, n_h, dn, dr, dev)
    csa_compress(t["raw"], 0, t["logits_csa"], t["bias_csa"], m, w, 0, n_c, csa)
    hca_compress(t["raw"], 0, t["logits_hca"], t["bias_hca"], mp, 0, n_h, hca)
    zero = _i64([0], dev)
    idx = index_topk(t["q_idx"], t["w_idx"], t["k_idx"], zero, t["q_seq"], t["q_pos"], n_c, m, k, ws)
    win = Store.dense(t["raw"], dn, dr)
    scale = 1.0 / math.sqrt(dn + dr)
    o_c, l_c = csa_attn(t["q"], csa, zero, idx, win, zero, zero, W, t["q_seq"], t["q_pos"], scale, ws)
    o_h, l_h = hca_attn(t["q"], hca, zero, mp, n_h, win, zero, zero, W, t["q_seq"], t["q_pos"], scale, ws)
    return dict(csa=csa, hca=hca, idx=idx, o_csa=o_c, lse_csa=l_c, o_hca=o_h, lse_hca=l_h)


def decode_bf16(case, ws=None):
    """B decode queries over bf16 KV: compress every sequence's caches (bf16 stores), index, attend."""
    p, t = case.params, case.t
    dev = t["raw"].device
    ws = ws or Workspace(dev)
    B, L, m, w, mp, W, k = p["B"], p["L"], p["m"], p["w"], p["m_prime"], p["W"], p["topk"]
    dn, dr = p["d_nope"], p["d_rope"]
    n_c, n_h = L // m, L // mp
    raw = t["raw"].view(B, L, -1)
    lc = t["logits_csa"].view(B, L, -1)
    lh = t["logits_hca"].view(B, L, -1)
    csa = empty_store(LAYOUT_BF16, B * n_c, dn, dr, dev)
    hca = empty_store(LAYOUT_BF16, B * n_h, dn, dr, dev)
    for b in range(B):
        csa_compress(raw[b], 0, lc[b], t["bias_csa"], m, w, 0, n_c, csa, out_row0=b * n_c)
        hca_compress(raw[b], 0, lh[b], t["bias_hca"], mp, 0, n_h, hca, out_row0=b * n_h)
    crb = _i64([b * n_c for b in range(B)], dev)
    hrb = _i64([b * n_h for b in range(B)], dev)
    wrb = _i64([b * L for b in range(B)], dev)
    wp0 = _i64([0] * B, dev)
    idx = index_topk(t["q_idx"], t["w_idx"], t["k_idx"], crb, t["q_seq"], t["q_pos"], n_c, m, k, ws)
    win = Store.dense(t["raw"], dn, dr)
    scale = 1.0 / math.sqrt(dn + dr)
    q = t["q"].view(torch.bfloat16)
    o_c, l_c = csa_attn(q, csa, crb, idx, win, wrb, wp0, W, t["q_seq"], t["q_pos"], scale, ws)
    o_h, l_h = hca_attn(q, hca, hrb, mp, n_h, win, wrb, wp0, W, t["q_seq"], t["q_pos"], scale, ws)
    return dict(csa=csa, hca=hca, idx=idx, o_csa=o_c, lse_csa=l_c, o_hca=o_h, lse_hca=l_h)


class Decode1M:
    """Decode step over precompressed split-layout caches and MXFP4 indexer keys
    (index + CSA attention for one layer, HCA attention for another), with all
    outputs and workspaces preallocated so that `step()` only enqueues kernels.

    HCA attention does not depend on the indexer. `step()` runs on one stream: the indexer's
    scores, then one launch holding the top-k selection (one block per query) beside HCA
    attention (hca_dense_mqa_attn_partials_select with the selection recorded by
    lightning_index_select_pending), then CSA attention over the selected entries, and one
    mqa_attn_merge launch for both calls' split-K partials. Running HCA attention on a second
    stream instead, forked after the scores and joined before the merge, costs the step the
    latency of two cross-stream waits. Beside the scores, HCA attention and the
    bandwidth-bound scoring slow each other down about as much as they overlap.
    overlap=False runs the index, CSA and HCA calls one after another, undeferred."""

    def __init__(self, case, ws=None, overlap=True):
        p, t = case.params, case.t
        self.case = case
        dev = t["q_csa"].device
        self.ws = ws or Workspace(dev)
        B, L, m, mp, W, k = p["B"], p["L"], p["m"], p["m_prime"], p["W"], p["topk"]
        self.B, self.m, self.mp, self.W, self.k = B, m, mp, W, k
        self.n_c, self.n_h = L // m, L // mp
        self.csa = split_store(t, "csa")
        self.hca = split_store(t, "hca")
        self.win_csa = split_store(t, "win_csa")
        self.win_hca = split_store(t, "win_hca")
        self.crb = _i64([b * self.n_c for b in range(B)], dev)
        self.hrb = _i64([b * self.n_h for b in range(B)], dev)
        self.wrb = _i64([b * W for b in range(B)], dev)
        self.wp0 = _i64([L - W] * B, dev)
        self.q_csa = t["q_csa"].view(torch.bfloat16)
        self.q_hca = t["q_hca"].view(torch.bfloat16)
        self.scale = 1.0 / math.sqrt(p["d_nope"] + p["d_rope"])
        H, D = p["heads"], p["D"]
        self.idx = torch.empty(B, k, dtype=torch.int32, device=dev)
        self.o_csa = torch.empty(B, H, D, dtype=torch.bfloat16, device=dev)
        self.o_hca = torch.empty(B, H, D, dtype=torch.bfloat16, device=dev)
        self.lse_csa = torch.empty(B, H, dtype=torch.float32, device=dev)
        self.lse_hca = torch.empty(B, H, dtype=torch.float32, device=dev)
        # size workspaces up front
        self.ws.get("index", lightning_index_topk_workspace(B, self.n_c, k))
        self.ws.get("csa", mqa_attn_workspace(BF16, B, H, D, k + W))
        self.ws.get("hca", mqa_attn_workspace(BF16, B, H, D, self.n_h + W))
        self.overlap = overlap

    def index(self, stream=None, phase="both"):
        t = self.case.t
        return index_topk(t["q_idx"], t["w_idx"], t["k_idx"], self.crb, t["q_seq"], t["q_pos"], self.n_c, self.m,
                          self.k, self.ws, q_idx_scale=t["q_idx_scale"], k_idx_scale=t["k_idx_scale"], out=self.idx,
                          phase=phase, stream=stream)

    def csa_attention(self, stream=None, defer=False):
        t = self.case.t
        return csa_attn(self.q_csa, self.csa, self.crb, self.idx, self.win_csa, self.wrb, self.wp0, self.W,
                        t["q_seq"], t["q_pos"], self.scale, self.ws, o=self.o_csa, lse=self.lse_csa, stream=stream,
                        defer=defer)

    def hca_attention(self, stream=None, defer=False, sel=None):
        t = self.case.t
        return hca_attn(self.q_hca, self.hca, self.hrb, self.mp, self.n_h, self.win_hca, self.wrb, self.wp0, self.W,
                        t["q_seq"], t["q_pos"], self.scale, self.ws, o=self.o_hca, lse=self.lse_hca, stream=stream,
                        defer=defer, sel=sel)

    def step(self):
        if not self.overlap:
            self.index()
            self.csa_attention()
            self.hca_attention()
            return
        self.index(phase="scores")
        sel = self.index(phase="pending")
        hp = self.hca_attention(defer=True, sel=sel)[2]
        cp = self.csa_attention(defer=True)[2]
        # one launch merges both calls' split-K partials
        mqa_attn_merge(cp, hp)


class DecodeBf16:
    """Decode step over precompressed bf16 stores (dense [n, D] rows) with bf16 indexer keys: index
    (top-k), CSA attention over the selected entries and the window, HCA attention over all
    visible entries and the window; outputs and workspaces preallocated, so that `step()` only
    enqueues kernels. As in Decode1M, `step()` runs on one stream with the top-k selection inside
    HCA attention's launch; fused=False runs the calls one after another."""

    def __init__(self, case, ws=None, fused=True):
        p, t = case.params, case.t
        self.case = case
        dev = t["q"].device
        self.ws = ws or Workspace(dev)
        B, L, m, mp, W, k = p["B"], p["L"], p["m"], p["m_prime"], p["W"], p["topk"]
        dn, dr = p["d_nope"], p["d_rope"]
        self.B, self.m, self.mp, self.W, self.k = B, m, mp, W, k
        self.n_c, self.n_h = L // m, L // mp
        self.csa = Store.dense(t["csa_data"], dn, dr)
        self.hca = Store.dense(t["hca_data"], dn, dr)
        self.win = Store.dense(t["win_data"], dn, dr)
        self.crb = _i64([b * self.n_c for b in range(B)], dev)
        self.hrb = _i64([b * self.n_h for b in range(B)], dev)
        self.wrb = _i64([b * W for b in range(B)], dev)
        self.wp0 = _i64([L - W] * B, dev)
        self.q = t["q"].view(torch.bfloat16)
        self.scale = 1.0 / math.sqrt(dn + dr)
        H, D = p["heads"], dn + dr
        self.idx = torch.empty(B, k, dtype=torch.int32, device=dev)
        self.o_csa = torch.empty(B, H, D, dtype=torch.bfloat16, device=dev)
        self.o_hca = torch.empty(B, H, D, dtype=torch.bfloat16, device=dev)
        self.lse_csa = torch.empty(B, H, dtype=torch.float32, device=dev)
        self.lse_hca = torch.empty(B, H, dtype=torch.float32, device=dev)
        self.ws.get("index", lightning_index_topk_workspace(B, self.n_c, k))
        self.ws.get("csa", mqa_attn_workspace(BF16, B, H, D, k + W))
        self.ws.get("hca", mqa_attn_workspace(BF16, B, H, D, self.n_h + W))
        self.fused = fused

    def index(self, phase="both"):
        t = self.case.t
        return index_topk(t["q_idx"], t["w_idx"], t["k_idx"], self.crb, t["q_seq"], t["q_pos"], self.n_c, self.m,
                          self.k, self.ws, out=self.idx, phase=phase)

    def csa_attention(self):
        t = self.case.t
        return csa_attn(self.q, self.csa, self.crb, self.idx, self.win, self.wrb, self.wp0, self.W, t["q_seq"],
                        t["q_pos"], self.scale, self.ws, o=self.o_csa, lse=self.lse_csa)

    def hca_attention(self):
        t = self.case.t
        return hca_attn(self.q, self.hca, self.hrb, self.mp, self.n_h, self.win, self.wrb, self.wp0, self.W,
                        t["q_seq"], t["q_pos"], self.scale, self.ws, o=self.o_hca, lse=self.lse_hca)

    def step(self):
        t = self.case.t
        sel = None
        if self.fused:
            self.index(phase="scores")
            sel = self.index(phase="pending")
        else:
            self.index()
        _, _, hp = hca_attn(self.q, self.hca, self.hrb, self.mp, self.n_h, self.win, self.wrb, self.wp0, self.W,
                            t["q_seq"], t["q_pos"], self.scale, self.ws, o=self.o_hca, lse=self.lse_hca, defer=True,
                            sel=sel)
        _, _, cp = csa_attn(self.q, self.csa, self.crb, self.idx, self.win, self.wrb, self.wp0, self.W, t["q_seq"],
                            t["q_pos"], self.scale, self.ws, o=self.o_csa, lse=self.lse_csa, defer=True)
        mqa_attn_merge(cp, hp)  # both calls' split-K partials in one launch


def compress_1m(case, out_csa=None, out_hca=None, stream=None):
    """csa_compress + hca_compress of one long bf16 sequence into split-layout stores."""
    p, t = case.params, case.t
    dev = t["raw"].device
    L, m, w, mp = p["L"], p["m"], p["w"], p["m_prime"]
    dn, dr = p["d_nope"], p["d_rope"]
    if out_csa is None:
        out_csa = empty_store(LAYOUT_SPLIT, L // m, dn, dr, dev)
    if out_hca is None:
        out_hca = empty_store(LAYOUT_SPLIT, L // mp, dn, dr, dev)
    csa_compress(t["raw"], 0, t["logits_csa"], t["bias_csa"], m, w, 0, L // m, out_csa, stream=stream)
    hca_compress(t["raw"], 0, t["logits_hca"], t["bias_hca"], mp, 0, L // mp, out_hca, stream=stream)
    return out_csa, out_hca


def chunked_prefill(case, ws=None, window="split"):
    """Chunked prefill for S sequences: compress each chunk into the sequence's
    caches (CSA with a w-m row halo from the prefix), index every chunk query,
    then CSA and HCA attention for all queries.

    window="split": the window rows (the last W prefix rows and the chunk) are
    first written into a split-layout store, the layout the caches and the
    decode window use, by csa_compress with m = w = 1 (a softmax over one
    position is exactly 1, so each entry is its raw row, encoded).
    window="bf16": the attention calls read the raw bf16 rows directly."""
    p, t = case.params, case.t
    dev = t["raw"].device
    ws = ws or Workspace(dev)
    S, chunk, m, w, mp, W, k = p["S"], p["chunk"], p["m"], p["w"], p["m_prime"], p["W"], p["topk"]
    dn, dr = p["d_nope"], p["d_rope"]
    csa, hca = split_store(t, "csa"), split_store(t, "hca")
    rows = W + chunk
    raw = t["raw"].view(S, rows, -1)
    lc = t["logits_csa"].view(S, rows, -1)
    lh = t["logits_hca"].view(S, rows, -1)
    for b, P in enumerate(p["prefixes"]):
        first_pos = P - W
        csa_compress(raw[b], first_pos, lc[b], t["bias_csa"], m, w, P // m, chunk // m, csa,
                     out_row0=p["csa_row_begin"][b] + P // m)
        hca_compress(raw[b], first_pos, lh[b], t["bias_hca"], mp, P // mp, chunk // mp, hca,
                     out_row0=p["hca_row_begin"][b] + P // mp)
    # the per-sequence offsets go to the device once per case (a copy from host lists waits for
    # the stream, which would serialise the calls around it)
    offs = getattr(case, "_device_offsets", None)
    if offs is None:
        offs = tuple(_i64(p[name], dev) for name in ("csa_row_begin", "hca_row_begin", "win_row_begin", "win_pos0"))
        case._device_offsets = offs
    crb, hrb, wrb, wp0 = offs
    max_c = max((P + chunk) // m for P in p["prefixes"])
    max_h = max((P + chunk) // mp for P in p["prefixes"])
    idx = index_topk(t["q_idx"], t["w_idx"], t["k_idx"], crb, t["q_seq"], t["q_pos"], max_c, m, k, ws,
                     q_idx_scale=t["q_idx_scale"], k_idx_scale=t["k_idx_scale"])
    if window == "split":
        win = prefill_window(case, ws)
    elif window == "bf16":
        win = Store.dense(t["raw"], dn, dr)
    else:
        raise ValueError(f"window layout {window!r}")
    scale = 1.0 / math.sqrt(dn + dr)
    q = t["q"].view(torch.bfloat16)
    o_c, l_c = csa_attn(q, csa, crb, idx, win, wrb, wp0, W, t["q_seq"], t["q_pos"], scale, ws)
    o_h, l_h = hca_attn(q, hca, hrb, mp, max_h, win, wrb, wp0, W, t["q_seq"], t["q_pos"], scale, ws)
    return dict(csa=csa, hca=hca, win=win, idx=idx, o_csa=o_c, lse_csa=l_c, o_hca=o_h, lse_hca=l_h)


def prefill_window(case, ws, stream=None):
    """The chunked-prefill window rows of every sequence (positions P - W .. P + chunk - 1, the
    rows of the raw input) written into a split-layout store by csa_compress with m = w = 1:
    zero logits and bias, so every entry is its own raw row, encoded as the caches are."""
    p, t = case.params, case.t
    dev = t["raw"].device
    S, W, chunk = p["S"], p["W"], p["chunk"]
    dn, dr = p["d_nope"], p["d_rope"]
    rows = W + chunk
    raw = t["raw"].view(S, rows, -1)
    win = Store.split(ws.get("win_nope", S * rows * dn).view(torch.uint8)[:S * rows * dn].view(S * rows, dn),
                      ws.get("win_scale", S * rows * 4)[:S * rows * 4].view(torch.float32),
                      ws.get("win_rope", S * rows * dr * 2)[:S * rows * dr * 2].view(torch.int16).view(S * rows, dr))
    zero_logits = torch.zeros(rows, 1, dtype=raw.dtype, device=dev)
    zero_bias = torch.zeros(1, dn + dr, dtype=torch.float32, device=dev)
    for b, P in enumerate(p["prefixes"]):
        csa_compress(raw[b], P - W, zero_logits, zero_bias, 1, 1, P - W, rows, win, out_row0=b * rows,
                     scalar_logits=True, stream=stream)
    return win
