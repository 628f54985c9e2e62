"""Seeded synthetic inputs for the CSA + HCA hybrid-attention path.

This module is shared by the tests (GPU library and CPU oracle sides) and
the benchmark. It only draws random numbers and casts them into the storage
formats with torch's own dtype conversions; none of the method's arithmetic
(compression, scoring, selection, attention, or the FP8 scale rule of
compressed entries) lives here.

Recipe (per tensor, fp32 normal draws from a torch.Generator seeded with the
given seed, in the order the builders below draw them):
  * raw KV rows, attention queries, indexer queries and keys: N(0, 1)
  * compression logits: N(0, 0.5)   (std 0.5; N(0, 1) in the tiny fp32 case)
  * position bias: N(0, 0.1)        (N(0, 1) in the tiny fp32 case)
  * indexer head weights: N(0, 1) / 8
  * precompressed split-layout entries: N(0, 1) values; each entry gets a
    power-of-two scale 2**e with e uniform in {-1, 0, 1}; the 448 FP8 dims
    hold E4M3(value / scale) via torch's float8_e4m3fn cast, the 64 RoPE
    dims hold bf16(value) via torch's bfloat16 cast
  * MXFP4 indexer rows: for each 32-element block an E8M0 scale 2**X with X
    uniform in {-2, -1, 0}; each element is the E2M1 grid point nearest to
    an N(0, 2^2) draw (saturating at +-6)

Torch's CPU and CUDA generators produce different streams for the same seed;
each is deterministic. Small cases are drawn on the CPU and uploaded; the
large benchmark case is drawn on the GPU and copied back where the oracle
needs it.
"""

from dataclasses import dataclass, field
from typing import Dict, List

import torch

E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def generator(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(g, shape, std=1.0):
    return torch.randn(shape, generator=g, device=g.device, dtype=torch.float32) * std


def bf16_bits(x):
    """fp32 tensor -> bf16 bit patterns stored as int16."""
    return x.to(torch.bfloat16).view(torch.int16)


def e4m3_codes(x):
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def split_entries(g, n, d_nope, d_rope):
    """Precompressed entries in the split layout (FP8 + scale, BF16 RoPE)."""
    v = normal(g, (n, d_nope + d_rope))
    e = torch.randint(-1, 2, (n,), generator=g, device=g.device)
    scale = torch.pow(2.0, e.to(torch.float32))
    return {"nope": e4m3_codes(v[:, :d_nope] / scale[:, None]).contiguous(),
            "scale": scale.contiguous(),
            "rope": bf16_bits(v[:, d_nope:]).contiguous()}


def mxfp4_rows(g, n, d, block=32):
    """MXFP4 rows: packed uint8 [n, d/2] (element 2i in the low nibble) and
    E8M0 scales uint8 [n, d/block]."""
    u = normal(g, (n, d), std=2.0)
    X = torch.randint(-2, 1, (n, d // block), generator=g, device=g.device)
    grid = torch.tensor(E2M1_GRID, device=g.device)
    mids = (grid[1:] + grid[:-1]) * 0.5
    code = torch.bucketize(u.abs(), mids).to(torch.uint8)          # nearest grid point
    nib = code | ((u < 0).to(torch.uint8) << 3)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).contiguous()
    scales = (X + 127).to(torch.uint8).contiguous()
    return packed, scales


# ---------------------------------------------------------------------------
# Workload builders. Each returns a Case: named tensors on `device` plus the
# integer parameters of the workload.


@dataclass
class Case:
    params: Dict[str, object]
    t: Dict[str, torch.Tensor] = field(default_factory=dict)


def tiny_fp32(seed=1001, device="cpu", L=4096, n_queries=16, heads=16, d_nope=128, d_rope=64,
              m=4, w=8, topk=64, n_idx_heads=4, d_idx=64, m_prime=128, W=128):
    """Tiny CSA+HCA decode, fp32: one sequence, full pipeline from raw KV."""
    g = generator(seed, device)
    D = d_nope + d_rope
    c = Case(dict(L=L, nq=n_queries, heads=heads, d_nope=d_nope, d_rope=d_rope, D=D, m=m, w=w,
                  topk=topk, n_idx_heads=n_idx_heads, d_idx=d_idx, m_prime=m_prime, W=W))
    c.t["raw"] = normal(g, (L, D))
    c.t["logits_csa"] = normal(g, (L, D))
    c.t["logits_hca"] = normal(g, (L, D))
    c.t["bias_csa"] = normal(g, (w, D))
    c.t["bias_hca"] = normal(g, (m_prime, D))
    c.t["q"] = normal(g, (n_queries, heads, D))
    c.t["q_idx"] = normal(g, (n_queries, n_idx_heads, d_idx))
    c.t["w_idx"] = normal(g, (n_queries, n_idx_heads))
    c.t["k_idx"] = normal(g, (L // m, d_idx))
    c.t["q_pos"] = torch.arange(L - n_queries, L, device=device, dtype=torch.int64)
    c.t["q_seq"] = torch.zeros(n_queries, dtype=torch.int32, device=device)
    return c


def decode_bf16(seed=1002, device="cpu", B=8, L=131072, heads=64, d_nope=448, d_rope=64,
                m=4, w=8, topk=512, n_idx_heads=4, d_idx=64, m_prime=128, W=128):
    """Decode, bf16: B sequences of L raw tokens, one query each at t = L-1;
    caches are compressed from the raw KV by the path."""
    g = generator(seed, device)
    D = d_nope + d_rope
    c = Case(dict(B=B, L=L, nq=B, heads=heads, d_nope=d_nope, d_rope=d_rope, D=D, m=m, w=w,
                  topk=topk, n_idx_heads=n_idx_heads, d_idx=d_idx, m_prime=m_prime, W=W))
    c.t["raw"] = bf16_bits(normal(g, (B * L, D)))
    c.t["logits_csa"] = bf16_bits(normal(g, (B * L, D), 0.5))
    c.t["logits_hca"] = bf16_bits(normal(g, (B * L, D), 0.5))
    c.t["bias_csa"] = normal(g, (w, D), 0.1)
    c.t["bias_hca"] = normal(g, (m_prime, D), 0.1)
    c.t["q"] = bf16_bits(normal(g, (B, heads, D)))
    c.t["q_idx"] = bf16_bits(normal(g, (B, n_idx_heads, d_idx)))
    c.t["w_idx"] = normal(g, (B, n_idx_heads), 0.125)
    c.t["k_idx"] = bf16_bits(normal(g, (B * (L // m), d_idx)))
    c.t["q_pos"] = torch.full((B,), L - 1, dtype=torch.int64, device=device)
    c.t["q_seq"] = torch.arange(B, dtype=torch.int32, device=device)
    return c


def decode_1m(seed=1003, device="cpu", B=4, L=1 << 20, heads=64, d_nope=448, d_rope=64,
              m=4, topk=1024, n_idx_heads=4, d_idx=64, m_prime=128, W=128, csa_store=None):
    """Decode at long context with precompressed caches: split-layout CSA and
    HCA stores, MXFP4 indexer keys, and for each of the two layers a raw
    window of the last W tokens in the split layout. `csa_store` lets several
    draws share one CSA store (it is only gathered from)."""
    g = generator(seed, device)
    D = d_nope + d_rope
    n_c, n_h = L // m, L // m_prime
    c = Case(dict(B=B, L=L, nq=B, heads=heads, d_nope=d_nope, d_rope=d_rope, D=D, m=m,
                  topk=topk, n_idx_heads=n_idx_heads, d_idx=d_idx, m_prime=m_prime, W=W))
    c.t["q_csa"] = bf16_bits(normal(g, (B, heads, D)))
    c.t["q_hca"] = bf16_bits(normal(g, (B, heads, D)))
    qp, qs = mxfp4_rows(g, B * n_idx_heads, d_idx)
    c.t["q_idx"] = qp.view(B, n_idx_heads, d_idx // 2)
    c.t["q_idx_scale"] = qs.view(B, n_idx_heads, d_idx // 32)
    c.t["w_idx"] = normal(g, (B, n_idx_heads), 0.125)
    kp, ks = mxfp4_rows(g, B * n_c, d_idx)
    c.t["k_idx"], c.t["k_idx_scale"] = kp, ks
    for name, n in (("hca", B * n_h), ("win_csa", B * W), ("win_hca", B * W)):
        for k, v in split_entries(g, n, d_nope, d_rope).items():
            c.t[f"{name}_{k}"] = v
    if csa_store is None:
        csa_store = split_entries(g, B * n_c, d_nope, d_rope)
    for k, v in csa_store.items():
        c.t[f"csa_{k}"] = v
    c.t["q_pos"] = torch.full((B,), L - 1, dtype=torch.int64, device=device)
    c.t["q_seq"] = torch.arange(B, dtype=torch.int32, device=device)
    return c


def decode_bf16_caches(seed=1012, device="cpu", B=8, L=131072, heads=64, d_nope=448, d_rope=64, m=4, topk=512,
                       n_idx_heads=4, d_idx=64, m_prime=128, W=128, csa_store=None):
    """Decode over bf16 stores with the caches generated already compressed (for timing the
    decode step at the bf16 configuration without compressing B * L raw tokens first): bf16
    CSA and HCA entries [n, D] and window rows [B * W, D] N(0, 1), bf16 indexer keys and
    queries N(0, 1), head weights N(0, 1)/8. `csa_store` lets draws share one CSA store."""
    g = generator(seed, device)
    D = d_nope + d_rope
    n_c, n_h = L // m, L // m_prime
    c = Case(dict(B=B, L=L, nq=B, heads=heads, d_nope=d_nope, d_rope=d_rope, D=D, m=m,
                  topk=topk, n_idx_heads=n_idx_heads, d_idx=d_idx, m_prime=m_prime, W=W))
    c.t["q"] = bf16_bits(normal(g, (B, heads, D)))
    c.t["q_idx"] = bf16_bits(normal(g, (B, n_idx_heads, d_idx)))
    c.t["w_idx"] = normal(g, (B, n_idx_heads), 0.125)
    c.t["k_idx"] = bf16_bits(normal(g, (B * n_c, d_idx)))
    c.t["hca_data"] = bf16_bits(normal(g, (B * n_h, D)))
    c.t["win_data"] = bf16_bits(normal(g, (B * W, D)))
    c.t["csa_data"] = csa_store if csa_store is not None else bf16_bits(normal(g, (B * n_c, D)))
    c.t["q_pos"] = torch.full((B,), L - 1, dtype=torch.int64, device=device)
    c.t["q_seq"] = torch.arange(B, dtype=torch.int32, device=device)
    return c


def compression(seed=1004, device="cpu", L=1 << 20, d_nope=448, d_rope=64, m=4, w=8, m_prime=128):
    """Compression throughput: one sequence of L raw bf16 tokens."""
    g = generator(seed, device)
    D = d_nope + d_rope
    c = Case(dict(L=L, d_nope=d_nope, d_rope=d_rope, D=D, m=m, w=w, m_prime=m_prime))
    c.t["raw"] = bf16_bits(normal(g, (L, D)))
    c.t["logits_csa"] = bf16_bits(normal(g, (L, D), 0.5))
    c.t["logits_hca"] = bf16_bits(normal(g, (L, D), 0.5))
    c.t["bias_csa"] = normal(g, (w, D), 0.1)
    c.t["bias_hca"] = normal(g, (m_prime, D), 0.1)
    return c


def indexer_keys(seed=1014, device="cpu", L=1 << 20, d_idx=64, w=8):
    """Raw indexer keys of one long sequence for their compression: bf16 keys and
    per-channel logits [L, d_idx], position bias [w, d_idx]."""
    g = generator(seed, device)
    c = Case(dict(L=L, d_idx=d_idx, w=w))
    c.t["k"] = bf16_bits(normal(g, (L, d_idx)))
    c.t["z"] = bf16_bits(normal(g, (L, d_idx), 0.5))
    c.t["bias"] = normal(g, (w, d_idx), 0.1)
    return c


def decode_tokens(seed=1015, device="cpu", B=4, D=512, d_idx=64, m=4, w=8, m_prime=128):
    """One decode step's new tokens (bf16 raw KV, both compression logits, raw indexer
    key and its logits, [B, .]) and the compressors' position biases."""
    g = generator(seed, device)
    c = Case(dict(B=B, D=D, d_idx=d_idx, m=m, w=w, m_prime=m_prime))
    c.t["x"] = bf16_bits(normal(g, (B, D)))
    c.t["z_csa"] = bf16_bits(normal(g, (B, D), 0.5))
    c.t["z_hca"] = bf16_bits(normal(g, (B, D), 0.5))
    c.t["k_idx"] = bf16_bits(normal(g, (B, d_idx)))
    c.t["z_idx"] = bf16_bits(normal(g, (B, d_idx), 0.5))
    c.t["bias_csa"] = normal(g, (w, D), 0.1)
    c.t["bias_hca"] = normal(g, (m_prime, D), 0.1)
    c.t["bias_idx"] = normal(g, (w, d_idx), 0.1)
    return c


def chunked_prefill(seed=1005, device="cpu", prefixes=(32768, 131072, 262144), chunk=8192,
                    heads=64, d_nope=448, d_rope=64, m=4, w=8, topk=1024, n_idx_heads=4,
                    d_idx=64, m_prime=128, W=128):
    """Chunked prefill: per sequence a precompressed prefix (CSA/HCA split
    stores, MXFP4 indexer keys for prefix and chunk entries) and `chunk` new
    causal query tokens whose raw bf16 KV (plus the last W prefix rows) form
    the window store and the compression input."""
    g = generator(seed, device)
    D = d_nope + d_rope
    S = len(prefixes)
    for P in prefixes:
        assert P % m_prime == 0 and chunk % m_prime == 0 and P >= W
    c = Case(dict(S=S, prefixes=list(prefixes), chunk=chunk, nq=S * chunk, heads=heads,
                  d_nope=d_nope, d_rope=d_rope, D=D, m=m, w=w, topk=topk,
                  n_idx_heads=n_idx_heads, d_idx=d_idx, m_prime=m_prime, W=W))
    n_csa = [(P + chunk) // m for P in prefixes]
    n_hca = [(P + chunk) // m_prime for P in prefixes]
    rows_win = W + chunk
    csa_parts, hca_parts = [], []
    for b, P in enumerate(prefixes):
        csa_parts.append(split_entries(g, n_csa[b], d_nope, d_rope))
        hca_parts.append(split_entries(g, n_hca[b], d_nope, d_rope))
    for name, parts in (("csa", csa_parts), ("hca", hca_parts)):
        for k in ("nope", "scale", "rope"):
            c.t[f"{name}_{k}"] = torch.cat([p[k] for p in parts]).contiguous()
    c.params["csa_row_begin"] = [sum(n_csa[:b]) for b in range(S)]
    c.params["hca_row_begin"] = [sum(n_hca[:b]) for b in range(S)]
    kp, ks = mxfp4_rows(g, sum(n_csa), d_idx)
    c.t["k_idx"], c.t["k_idx_scale"] = kp, ks
    c.t["raw"] = bf16_bits(normal(g, (S * rows_win, D)))
    c.t["logits_csa"] = bf16_bits(normal(g, (S * rows_win, D), 0.5))
    c.t["logits_hca"] = bf16_bits(normal(g, (S * rows_win, D), 0.5))
    c.t["bias_csa"] = normal(g, (w, D), 0.1)
    c.t["bias_hca"] = normal(g, (m_prime, D), 0.1)
    c.params["win_row_begin"] = [b * rows_win for b in range(S)]
    c.params["win_pos0"] = [P - W for P in prefixes]
    nq = S * chunk
    c.t["q"] = bf16_bits(normal(g, (nq, heads, D)))
    qp, qs = mxfp4_rows(g, nq * n_idx_heads, d_idx)
    c.t["q_idx"] = qp.view(nq, n_idx_heads, d_idx // 2)
    c.t["q_idx_scale"] = qs.view(nq, n_idx_heads, d_idx // 32)
    c.t["w_idx"] = normal(g, (nq, n_idx_heads), 0.125)
    c.t["q_pos"] = torch.cat([torch.arange(P, P + chunk, dtype=torch.int64, device=device)
                              for P in prefixes])
    c.t["q_seq"] = torch.cat([torch.full((chunk,), b, dtype=torch.int32, device=device)
                              for b in range(S)])
    return c
