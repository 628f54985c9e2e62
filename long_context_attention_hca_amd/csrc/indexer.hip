// Lightning indexer for gfx950: scores of the compressed entries and an exact top-k.
//
// Method: hyper.ai paper page for arXiv 2606.19348 ("DeepSeek-V4"), section 方法
// (Method), CSA paragraph (a lightning indexer selects the top-k compressed KV
// entries) and efficiency paragraph (FP4 indexer). Score of entry j for a query
// with indexer heads h: s = sum_h w_h * relu(<q_h, k_j>); entry j is visible at
// position t iff j < floor((t+1)/m); ties go to the lower j.
//
// Design.
//  * MXFP4 scoring is a skinny contraction (H <= 8 query rows against n_vis keys
//    of 64 E2M1 values). It runs on v_mfma_scale_f32_32x32x64_f8f6f4 with the
//    keys as the N dimension: lane l holds key (l % 32), MX block (l / 32), so a
//    lane's operand is exactly one 16-byte block plus its E8M0 scale byte and a
//    wave's operand load is one contiguous 1 KiB span of the key array. In decode
//    the kernel is HBM-bound (34 bytes per key against 512 useful flops), so the
//    unused query rows of the 32-row tile cost nothing that matters.
//  * Each per-head dot product of MXFP4 values is exact in float32; the score is
//    folded in head order with separately rounded multiplies and adds
//    (score_term / score_add, no fused multiply-add), which makes it bit-exact and the
//    top-k unique.
//  * Selection is on the 64-bit key (order-preserving score bits << 32 | ~j), which
//    is unique per entry. Every score block (1024 entries) keeps its keys in LDS and
//    emits, into a region of the workspace that only it writes, the keys at or above
//    a threshold thr_b: the top 11-bit bin holding its L-th largest key when that
//    bin is small (L is about twice the block's expected share of the top-k, at
//    least 16), else exactly its L largest keys, found by two more histogram passes
//    over the lower key bits with equal scores broken by index. No atomics leave the
//    block. One block per query then gathers the candidates into LDS and finds the
//    k-th largest candidate key T with 11-bit radix passes that start below the bits
//    all candidates share. A block whose thr_b exceeds T may hold unemitted keys in
//    [T, thr_b); such blocks are rescanned from their stored keys and the selection
//    is repeated once, after which every key >= the new T is a candidate, so the
//    result is exact for any input (ties included). The k indices are emitted in
//    ascending order by bucketing them per score block and ranking each inside its
//    bucket.
#include "common.h"
#include "internal.h"
#include "topk_select.h"

namespace hca {
namespace {

// The score fold: each head's term w_h * relu(r_h) and each partial sum rounded to float32 on
// its own, in head order. hipcc contracts a multiply and an add into one fused multiply-add
// unless told not to, which would round once where the fold rounds twice; these two helpers
// switch contraction off, so that every scorer produces the same bits.
__device__ __forceinline__ float score_term(float w, float r) {
#pragma clang fp contract(off)
  // relu of a finite dot product as one integer max on its bits (every negative float and -0
  // is a negative int32); fmaxf would first quiet a signalling NaN with a second instruction
  return w * __int_as_float(max(__float_as_int(r), 0));
}
__device__ __forceinline__ float score_add(float s, float t) {
#pragma clang fp contract(off)
  return s + t;
}

struct BlockLds {
  uint32_t hist[kHistBins];
  uint32_t key[kBlockKeys];
  uint32_t part[256];
  uint32_t tmp[8];
  CrossLds cx;
  uint64_t thr;
};

__device__ __forceinline__ void block_crossing(BlockLds& lds, uint32_t rem, int* d, uint32_t* above) {
  crossing2048<256>(lds.hist, lds.part, rem, lds.cx, d, above);
}


// Candidate emission of one score block (all 256 threads; lds.key / lds.hist complete).
// Thread tid owns block positions 4 tid .. 4 tid + 3.
__device__ void emit_candidates(const IndexArgs& a, int qi, int64_t jb, int64_t nv, BlockLds& lds) {
  const int tid = threadIdx.x;
  const int nvalid = (int)min<int64_t>(kBlockKeys, nv - jb);
  const uint32_t L = block_quota(a.k, nv);
  const uint4 kv = reinterpret_cast<const uint4*>(lds.key)[tid];
  const uint32_t kk[4] = {kv.x, kv.y, kv.z, kv.w};
  const int t0 = 4 * tid;
  uint64_t thr = 0;  // emit keys >= thr
  if ((uint32_t)nvalid > L) {
    int d;
    uint32_t above;
    block_crossing(lds, L, &d, &above);
    uint32_t rem = L - above;
    if (above + lds.hist[d] <= 2 * L) {
      thr = (uint64_t)d << 53;  // the whole bin
    } else {
      // exactly the L largest keys: refine on key bits 20..10, then 9..0, then break ties by index
      uint32_t pre = (uint32_t)d;
      __syncthreads();
      for (int i = tid; i < kHistBins; i += 256) lds.hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t0 + i < nvalid && (kk[i] >> 21) == pre) atomicAdd(&lds.hist[(kk[i] >> 10) & 2047u], 1u);
      __syncthreads();
      block_crossing(lds, rem, &d, &above);
      rem -= above;
      pre = (pre << 11) | (uint32_t)d;
      if (lds.hist[d] == rem) {
        thr = (uint64_t)pre << 42;
      } else {
        __syncthreads();
        for (int i = tid; i < kHistBins; i += 256) lds.hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + i < nvalid && (kk[i] >> 10) == pre) atomicAdd(&lds.hist[kk[i] & 1023u], 1u);
        __syncthreads();
        block_crossing(lds, rem, &d, &above);
        rem -= above;
        const uint32_t v = (pre << 10) | (uint32_t)d;
        // rem of the keys equal to v are taken, the lowest positions first
        uint32_t nt = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) nt += (t0 + i < nvalid && kk[i] == v);
        uint32_t tot;
        uint32_t r = block_exclusive_scan<256>(nt, lds.tmp, &tot);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (t0 + i < nvalid && kk[i] == v) {
            if (r == rem - 1) lds.thr = ((uint64_t)v << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(jb + t0 + i));
            ++r;
          }
        }
        __syncthreads();
        thr = lds.thr;
      }
    }
  }
  uint64_t k64[4];
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    k64[i] = ((uint64_t)kk[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(jb + t0 + i));
    n += (t0 + i < nvalid && k64[i] >= thr);
  }
  uint32_t tot;
  uint32_t off = block_exclusive_scan<256>(n, lds.tmp, &tot);
  const int64_t slot = (int64_t)qi * a.nblk + blockIdx.x;
  const uint32_t R = region_slots(L);
  uint64_t* dst = a.cand + (int64_t)qi * a.nblk * kBlockKeys + (int64_t)blockIdx.x * R;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (t0 + i < nvalid && k64[i] >= thr) dst[off++] = k64[i];
  for (uint32_t i = tot + tid; i < R; i += 256) dst[i] = 0;
  uint32_t* sk = a.scores + (int64_t)qi * a.nblk * kBlockKeys + jb;
  if (t0 + 3 < nvalid) {
    *reinterpret_cast<uint4*>(sk + t0) = kv;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (t0 + i < nvalid) sk[t0 + i] = kk[i];
  }
  if (tid == 0) a.blk_thr[slot] = thr;
}

// MXFP4 scores of query qi for the keys of score block blockIdx.x (all 256 threads).
__device__ __forceinline__ void score_mxfp4_one(const IndexArgs& a, int qi, BlockLds& lds) {
  int64_t rb;
  const int64_t nv = visible_keys(a, qi, &rb);
  if (nv <= a.k) return;  // every visible entry is selected; no scores needed
  const int64_t jb = (int64_t)blockIdx.x * kBlockKeys;
  if (jb >= nv) return;
  for (int i = threadIdx.x; i < kHistBins; i += 256) lds.hist[i] = 0;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 31, blk = lane >> 5;
  const uint8_t* qb = static_cast<const uint8_t*>(a.q);
  const uint8_t* kb = static_cast<const uint8_t*>(a.keys);
  i32x8 A = {0, 0, 0, 0, 0, 0, 0, 0};
  int sa = 127;
  if (row < a.H) {
    const int64_t qr = (int64_t)qi * a.H + row;
    const uint4 v = *reinterpret_cast<const uint4*>(qb + qr * 32 + blk * 16);
    A[0] = (int)v.x; A[1] = (int)v.y; A[2] = (int)v.z; A[3] = (int)v.w;
    sa = a.q_scale[qr * 2 + blk];
  }
  float w[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) w[h] = h < a.H ? a.w[(int64_t)qi * a.H + h] : 0.f;

  constexpr int U = 8;
  i32x8 B[U];
  int sb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = jb + (int64_t)(wave * U + u) * 32 + row;
    const int64_t jc = rb + (j < nv ? j : nv - 1);
    const uint4 v = *reinterpret_cast<const uint4*>(kb + jc * 32 + blk * 16);
    B[u] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    sb[u] = a.key_scale[jc * 2 + blk];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const f32x16 zero = {};
    const f32x16 acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B[u], zero, 4, 4, 0, sa, 0, sb[u]);
    // C layout: lane l holds rows 8*(i/4) + 4*(l/32) + i%4 of column l%32, so rows 0..3
    // (heads 0..3) sit in acc[0..3] of lanes 0..31 and rows 4..7 in acc[0..3] of lanes 32..63.
    float r[8];
    r[0] = acc[0]; r[1] = acc[1]; r[2] = acc[2]; r[3] = acc[3];
    if (a.H > 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) r[4 + i] = __shfl(acc[i], (lane & 31) + 32, 64);
    }
    const int pos = (wave * U + u) * 32 + row;
    if (lane < 32 && jb + pos < nv) {
      float s = score_term(w[0], r[0]);
#pragma unroll
      for (int h = 1; h < 8; ++h)
        if (h < a.H) s = score_add(s, score_term(w[h], r[h]));
      const uint32_t key = float_key(s);
      lds.key[pos] = key;
      atomicAdd(&lds.hist[key >> 21], 1u);
    }
  }
  __syncthreads();
  emit_candidates(a, qi, jb, nv, lds);
}

// bf16 keys on v_mfma_f32_32x32x16_bf16, laid out as the MXFP4 scorer: the A rows are the
// query's heads (rows H..31 zero), the 32 columns 32 keys, K 16 dims per step (lane l: dims
// 8 (l / 32) .. + 7 of the step), 4 steps for 64 dims, so a lane loads 16 bytes of one key row
// per step and the accumulators hold the same heads as the MXFP4 scorer's. The dot products
// are float32 sums of exact bf16 products in the MFMA's order (not the oracle's); bf16 scores
// are compared with the oracle within its error bound, so only the fold is shared.
// grid = (nblk, nq), 256 threads, 1024 keys per block.
__global__ __launch_bounds__(256) void score_bf16_kernel(IndexArgs a) {
  __shared__ BlockLds lds;
  const int qi = blockIdx.y;
  int64_t rb;
  const int64_t nv = visible_keys(a, qi, &rb);
  if (nv <= a.k) return;  // every visible entry is selected; no scores needed
  const int64_t jb = (int64_t)blockIdx.x * kBlockKeys;
  if (jb >= nv) return;
  for (int i = threadIdx.x; i < kHistBins; i += 256) lds.hist[i] = 0;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 31, blk = lane >> 5;
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* kp = static_cast<const uint16_t*>(a.keys);
  bf16x8 A[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < a.H) v = *reinterpret_cast<const uint4*>(qp + ((int64_t)qi * a.H + row) * 64 + 16 * st + 8 * blk);
    A[st] = __builtin_bit_cast(bf16x8, v);
  }
  float w[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) w[h] = h < a.H ? a.w[(int64_t)qi * a.H + h] : 0.f;
  __syncthreads();
  // 8 groups of 32 keys per wave, loaded 4 groups at a time (16 registers a group)
  constexpr int U = 8, UH = 4;
#pragma unroll
  for (int u0 = 0; u0 < U; u0 += UH) {
    bf16x8 Bk[UH][4];
#pragma unroll
    for (int u = 0; u < UH; ++u) {
      const int64_t j = jb + (int64_t)(wave * U + u0 + u) * 32 + row;
      const int64_t jc = rb + (j < nv ? j : nv - 1);
#pragma unroll
      for (int st = 0; st < 4; ++st)
        Bk[u][st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kp + jc * 64 + 16 * st + 8 * blk));
    }
#pragma unroll
    for (int u = 0; u < UH; ++u) {
      f32x16 acc = {};
#pragma unroll
      for (int st = 0; st < 4; ++st) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[st], Bk[u][st], acc, 0, 0, 0);
      // heads 0..3 in acc[0..3] of lanes 0..31, heads 4..7 in acc[0..3] of lanes 32..63
      float r[8];
      r[0] = acc[0]; r[1] = acc[1]; r[2] = acc[2]; r[3] = acc[3];
      if (a.H > 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[4 + i] = __shfl(acc[i], (lane & 31) + 32, 64);
      }
      const int pos = (wave * U + u0 + u) * 32 + row;
      if (lane < 32 && jb + pos < nv) {
        float sc = score_term(w[0], r[0]);
#pragma unroll
        for (int h = 1; h < 8; ++h)
          if (h < a.H) sc = score_add(sc, score_term(w[h], r[h]));
        const uint32_t key = float_key(sc);
        lds.key[pos] = key;
        atomicAdd(&lds.hist[key >> 21], 1u);
      }
    }
  }
  __syncthreads();
  emit_candidates(a, qi, jb, nv, lds);
}

// MXFP4 scores via the scaled MFMA. grid = (nblk, nq), 256 threads, 1024 keys per block.
__global__ __launch_bounds__(256) void score_mxfp4_kernel(IndexArgs a) {
  __shared__ BlockLds lds;
  score_mxfp4_one(a, blockIdx.y, lds);
}

// Many queries with 4 indexer heads (prefill): grid = (nblk, ceil(nq / 4)); a block scores the
// keys of score block blockIdx.x for the 4 consecutive queries 4 blockIdx.y .. +3. When their
// visible keys start at the same row (one sequence, one document), the keys are loaded once
// and one MFMA per 32 keys scores all of them: its A rows are the 16 (query, head) pairs
// 4 q + h. Lanes 0-31 then hold queries 0 and 2 of their key column (accumulators 0-3 and
// 4-7), lanes 32-63 queries 1 and 3. Each query keeps its own LDS keys and histogram and emits
// its candidates as score_mxfp4_one does; every score is the same float32 value, folded in
// the same order. Otherwise the block scores its queries one after another.
constexpr int kScoreQ = 4;

__global__ __launch_bounds__(256) void score_mxfp4_q4_kernel(IndexArgs a) {
  __shared__ BlockLds lds[kScoreQ];
  const int q0 = (int)blockIdx.y * kScoreQ;
  const int nqb = min(kScoreQ, a.nq - q0);
  int64_t rb[kScoreQ], nv[kScoreQ];
  bool same = true;
#pragma unroll
  for (int i = 0; i < kScoreQ; ++i) {
    nv[i] = 0;
    rb[i] = 0;
    if (i < nqb) nv[i] = visible_keys(a, q0 + i, &rb[i]);
    if (i > 0 && i < nqb) same = same && rb[i] == rb[0];
  }
  if (!same) {
    for (int i = 0; i < nqb; ++i) {
      score_mxfp4_one(a, q0 + i, lds[0]);
      __syncthreads();
    }
    return;
  }
  const int64_t jb = (int64_t)blockIdx.x * kBlockKeys;
  bool act[kScoreQ];
  bool any = false;
  int64_t nvmax = 0;
#pragma unroll
  for (int i = 0; i < kScoreQ; ++i) {
    act[i] = i < nqb && nv[i] > a.k && jb < nv[i];
    any = any || act[i];
    if (act[i]) nvmax = max(nvmax, nv[i]);
  }
  if (!any) return;
#pragma unroll
  for (int i = 0; i < kScoreQ; ++i)
    for (int j = threadIdx.x; j < kHistBins; j += 256) lds[i].hist[j] = 0;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 31, blk = lane >> 5;
  const uint8_t* qb = static_cast<const uint8_t*>(a.q);
  const uint8_t* kb = static_cast<const uint8_t*>(a.keys);
  i32x8 A = {0, 0, 0, 0, 0, 0, 0, 0};
  int sa = 127;
  if ((row >> 2) < nqb) {  // row 4 q + h: query q0 + q, head h
    const int64_t qr = (int64_t)(q0 + (row >> 2)) * 4 + (row & 3);
    const uint4 v = *reinterpret_cast<const uint4*>(qb + qr * 32 + blk * 16);
    A[0] = (int)v.x; A[1] = (int)v.y; A[2] = (int)v.z; A[3] = (int)v.w;
    sa = a.q_scale[qr * 2 + blk];
  }
  // this lane's two queries: 0 and 2 (lanes 0-31) or 1 and 3 (lanes 32-63)
  const int qa = blk, qc = blk + 2;
  float wa[4], wc[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    wa[h] = qa < nqb ? a.w[(int64_t)(q0 + qa) * 4 + h] : 0.f;
    wc[h] = qc < nqb ? a.w[(int64_t)(q0 + qc) * 4 + h] : 0.f;
  }
  const bool act_a = blk == 0 ? act[0] : act[1], act_c = blk == 0 ? act[2] : act[3];
  const int64_t nv_a = blk == 0 ? nv[0] : nv[1], nv_c = blk == 0 ? nv[2] : nv[3];

  constexpr int U = 8;
  i32x8 B[U];
  int sb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = jb + (int64_t)(wave * U + u) * 32 + row;
    const int64_t jc = rb[0] + (j < nvmax ? j : nvmax - 1);
    const uint4 v = *reinterpret_cast<const uint4*>(kb + jc * 32 + blk * 16);
    B[u] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    sb[u] = a.key_scale[jc * 2 + blk];
  }
  __syncthreads();
  BlockLds& la = lds[qa];
  BlockLds& lc = lds[qc];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const f32x16 zero = {};
    const f32x16 acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B[u], zero, 4, 4, 0, sa, 0, sb[u]);
    const int pos = (wave * U + u) * 32 + row;
    if (act_a && jb + pos < nv_a) {
      float s = score_term(wa[0], acc[0]);
#pragma unroll
      for (int h = 1; h < 4; ++h) s = score_add(s, score_term(wa[h], acc[h]));
      const uint32_t key = float_key(s);
      la.key[pos] = key;
      atomicAdd(&la.hist[key >> 21], 1u);
    }
    if (act_c && jb + pos < nv_c) {
      float s = score_term(wc[0], acc[4]);
#pragma unroll
      for (int h = 1; h < 4; ++h) s = score_add(s, score_term(wc[h], acc[4 + h]));
      const uint32_t key = float_key(s);
      lc.key[pos] = key;
      atomicAdd(&lc.hist[key >> 21], 1u);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kScoreQ; ++i)
    if (act[i]) emit_candidates(a, q0 + i, jb, nv[i], lds[i]);
}

// ---------------------------------------------------------------------------------------
// Streaming top-k for calls with many queries (prefill), MXFP4 keys, 4 indexer heads, k <= 1536.
// Block = 8 consecutive queries (the 32 MFMA rows are their (query, head) pairs), 8 waves. The
// block streams its queries' keys in tiles of 512 (wave w scores keys 64w .. 64w + 63 of a tile
// with two v_mfma_scale_f32_32x32x64_f8f6f4, the next tile's keys loaded meanwhile) and keeps,
// per query, the keys above a floor in an LDS buffer of 2048 64-bit keys (score key << 32 | ~j),
// in ascending j: every tile's candidates are placed in key order by a scan of the waves' counts.
// When a buffer could overflow on the next tile, wave q cuts query q's buffer to exactly its k
// largest keys (radix select on 8-bit digits below the bits that all its keys share, stable
// compaction) and raises the floor to the lower edge of the last digit range kept, which bounds
// the final k-th largest key from below; keys at or under the floor are never appended. At the
// end each buffer is cut to k and written out in order. Scores are the same float32 fold as
// score_mxfp4_one (bit-exact), so the result equals the oracle's stable sort. Queries whose
// visible keys start at different rows (other sequences or documents) are streamed in separate
// passes over their own rows. The counts of a tile are double-buffered, so a tile needs one
// barrier (two more when a buffer is cut).
constexpr int kSQ = 8;           // queries per block (one wave each for cuts and output)
constexpr int kSThreads = 512;   // 8 waves
constexpr int kSWaves = kSThreads / 64;
constexpr int kSTile = 512;      // keys per tile
constexpr int kSCap = 2048;      // buffered keys per query
constexpr int kStreamMaxK = kSCap - kSTile;

struct StreamLds {
  uint64_t buf[kSQ][kSCap];
  uint32_t hist[kSQ][256];             // radix-select counters, one set per cutting wave
  uint64_t floor_key[kSQ];
  uint32_t wcnt[2][kSQ][kSWaves];      // candidates of a tile per query and wave (by tile parity)
  int64_t nv[kSQ];                     // visible keys per query
};


// Orders this wave's LDS accesses before and after it (the LDS serves a wave's operations in
// order; the wait and the memory clobber keep the compiler from moving accesses across).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// OR over the wave (DPP row shifts and broadcasts as in wave_incl_scan_add; lane 63 holds it).
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Sum over each aligned group of 8 lanes, returned to all 8 (DPP: swap neighbours, swap pairs,
// then mirror the halves of the group).
__device__ __forceinline__ uint32_t group8_sum(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, false);   // quad_perm 1,0,3,2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xf, 0xf, false);   // quad_perm 2,3,0,1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xf, 0xf, false);  // row_half_mirror
  return x;
}

// One wave: cuts query q's buffer of n > K >= 1 keys to its K largest keys, keeping their order,
// and raises the query's floor. The keys are held in registers (lane l: slots 64 u + l); the
// first digit starts at the highest bit in which they differ (the bits above it are the same in
// every key and would put all of them into one counter). Once the digit range holding the K-th
// largest key has at most 64 keys, they are ranked directly and the floor becomes that key.
__device__ void stream_cut(StreamLds& s, int q, uint32_t n, uint32_t K) {
  const int lane = threadIdx.x & 63;
  uint64_t* buf = s.buf[q];
  uint32_t* hist = s.hist[q];
  constexpr int kPer = kSCap / 64;
  uint64_t v[kPer];
  uint64_t any1 = 0, all1 = ~0ull;  // OR and AND of the keys
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    v[u] = buf[64 * u + lane];
    if (64u * u + lane >= n) v[u] = 0;  // no key is 0 (its low word ~j is never zero)
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    any1 |= v[u];
    all1 &= v[u] != 0 ? v[u] : ~0ull;
  }
  any1 = ((uint64_t)wave_or_u32((uint32_t)(any1 >> 32)) << 32) | wave_or_u32((uint32_t)any1);
  all1 = ((uint64_t)~wave_or_u32(~(uint32_t)(all1 >> 32)) << 32) | ~wave_or_u32(~(uint32_t)all1);
  // the highest bit in which the keys differ (n >= 2 distinct keys)
  const int top = 63 - __builtin_clzll(any1 ^ all1);
  int shift = max(top - 7, 0);
  uint64_t mask = top == 63 ? 0ull : ~((2ull << top) - 1ull);
  uint64_t prefix = all1 & mask;
  uint32_t rem = K;
  for (int pass = 0; pass < 9; ++pass) {
    reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
    wave_lds_sync();
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (v[u] != 0 && (v[u] & mask) == prefix) atomicAdd(&hist[(uint32_t)(v[u] >> shift) & 255u], 1u);
    wave_lds_sync();
    // the digit d where the count from the top reaches rem (lane l holds bins 4l .. 4l + 3)
    const uint4 h = reinterpret_cast<const uint4*>(hist)[lane];
    const uint32_t own = h.x + h.y + h.z + h.w;
    const uint32_t pre = wave_incl_scan_add(own);
    const uint32_t above_lane = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63) - pre;  // lanes > lane
    const bool mine = above_lane < rem && above_lane + own >= rem;
    uint32_t acc = above_lane;
    int d = 4 * lane;
    if (mine) {
      const uint32_t hv[4] = {h.x, h.y, h.z, h.w};
      for (int b = 3; b >= 0; --b) {
        if (acc + hv[b] >= rem) { d = 4 * lane + b; break; }
        acc += hv[b];
      }
    }
    const int src = __builtin_ctzll(__ballot(mine));
    d = __builtin_amdgcn_readlane(d, src);
    const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)acc, src);
    const uint32_t in_bin = hist[d];
    wave_lds_sync();  // the counters are cleared by the next pass
    rem -= above;
    prefix |= (uint64_t)d << shift;
    mask |= (uint64_t)255 << shift;
    // every key of this digit range is kept; with all 64 bits fixed the range holds one key
    if (in_bin == rem || shift == 0) break;
    if (in_bin <= 64) {
      // few keys in the range: gather them (into the counters' space) and take the rem-th
      // largest directly, lane l ranking gathered key l against all of them
      uint64_t* g = reinterpret_cast<uint64_t*>(hist);
      uint32_t pos = 0;
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const bool in = (v[u] != 0) & ((v[u] & mask) == prefix);
        const uint64_t bal = __ballot(in);
        if (in) g[pos + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull))] = v[u];
        pos += (uint32_t)__popcll(bal);
      }
      wave_lds_sync();
      const uint64_t c = lane < (int)in_bin ? g[lane] : 0ull;
      const uint32_t c_hi = (uint32_t)(c >> 32), c_lo = (uint32_t)c;
      uint32_t rank = 0;  // gathered keys above this lane's
      for (uint32_t m2 = 0; m2 < in_bin; ++m2) {
        const uint64_t x = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)c_hi, (int)m2) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)c_lo, (int)m2);
        rank += x > c ? 1u : 0u;
      }
      const uint64_t hit = __ballot(lane < (int)in_bin && rank == rem - 1);
      const int src2 = __builtin_ctzll(hit);
      const uint64_t T = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(c >> 32), src2) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)c, src2);
      wave_lds_sync();  // the gathered keys are read before the counters are used again
      // the K kept keys are exactly those at or above T, the K-th largest
      prefix = T;
      mask = ~0ull;
      break;
    }
    shift = max(shift - 8, 0);
  }
  // keep the keys whose masked bits are at least the prefix (exactly K), in slot order
  uint32_t base = 0;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const bool keep = (v[u] != 0) & ((v[u] & mask) >= prefix);
    const uint64_t bal = __ballot(keep);
    if (keep) buf[base + (uint32_t)__popcll(bal & below)] = v[u];
    base += (uint32_t)__popcll(bal);
  }
  if (lane == 0 && prefix > s.floor_key[q]) s.floor_key[q] = prefix;
  wave_lds_sync();
}

__global__ __launch_bounds__(kSThreads) void index_stream_kernel(IndexArgs a) {
  __shared__ StreamLds s;
  // the last queries first: in causal prefill they see the most keys, so the longest blocks
  // start early and the short ones fill the tail
  const int q0 = (int)(gridDim.x - 1 - blockIdx.x) * kSQ;
  const int nqb = min(kSQ, a.nq - q0);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane & 31, blk = lane >> 5;
  int64_t rb[kSQ], nv[kSQ], j0[kSQ];
#pragma unroll
  for (int i = 0; i < kSQ; ++i) {
    rb[i] = -1;
    nv[i] = 0;
    j0[i] = 0;
    if (i < nqb) nv[i] = visible_keys(a, q0 + i, &rb[i], &j0[i]);
  }
  const int K = a.k;
  // queries with at most k visible entries return all of them in order, padded with -1
  uint32_t todo = 0;
#pragma unroll
  for (int i = 0; i < kSQ; ++i) {
    if (i >= nqb) continue;
    if (nv[i] <= K) {
      int32_t* out = a.out + (int64_t)(q0 + i) * K;
      for (int j = tid; j < K; j += kSThreads) out[j] = j < nv[i] ? (int32_t)(j + j0[i]) : -1;
    } else {
      todo |= 1u << i;
    }
  }
  if (!todo) return;
  if (tid == 0) {
#pragma unroll
    for (int i = 0; i < kSQ; ++i) s.nv[i] = nv[i];
  }

  // A operand: row 4 q + h is query q0 + q, indexer head h (zero for queries past the batch)
  const uint8_t* qb = static_cast<const uint8_t*>(a.q);
  const uint8_t* kb = static_cast<const uint8_t*>(a.keys);
  i32x8 A = {0, 0, 0, 0, 0, 0, 0, 0};
  int sa = 127;
  if ((row >> 2) < nqb) {
    const int64_t qr = (int64_t)(q0 + (row >> 2)) * 4 + (row & 3);
    const uint4 v = *reinterpret_cast<const uint4*>(qb + qr * 32 + blk * 16);
    A[0] = (int)v.x; A[1] = (int)v.y; A[2] = (int)v.z; A[3] = (int)v.w;
    sa = a.q_scale[qr * 2 + blk];
  }
  // accumulators 4 i + h of this lane hold query 2 i + blk, head h, of its key column
  float wq[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 4; ++h) wq[i][h] = (2 * i + blk) < nqb ? a.w[(int64_t)(q0 + 2 * i + blk) * 4 + h] : 0.f;

  int32_t jo_wave = 0;  // entry index of visible key 0 of query q0 + wave
#pragma unroll
  for (int i = 0; i < kSQ; ++i)
    if (i == wave) jo_wave = (int32_t)j0[i];
  // lane l of the count scan: query l / 8, wave l % 8
  const int cq = lane >> 3, cw = lane & 7;

  while (todo) {
    // this pass: the pending queries whose visible keys start at the lowest pending query's row
    int64_t R = 0;
#pragma unroll
    for (int i = kSQ - 1; i >= 0; --i)
      if ((todo >> i) & 1) R = rb[i];
    uint32_t set = 0;
    int64_t nvmax = 0, nvmin = INT64_MAX;
#pragma unroll
    for (int i = 0; i < kSQ; ++i)
      if (((todo >> i) & 1) && rb[i] == R) {
        set |= 1u << i;
        nvmax = max(nvmax, nv[i]);
        nvmin = min(nvmin, nv[i]);
      }
    todo &= ~set;
    if (tid < kSQ) s.floor_key[tid] = 0;  // below every key (the low word ~j is never zero)
    // buffered keys of query q, held by lanes 8 q .. 8 q + 7 of every wave
    uint32_t cnt = 0;
    __syncthreads();
    // the lane's 4 queries: visible counts and floors; the lanes of each pair of queries that
    // belong to the pass
    int64_t nvl[4];
    uint64_t fl[4], inmask[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nvl[i] = s.nv[2 * i + blk];
      fl[i] = 0;
      inmask[i] = (((set >> (2 * i)) & 1) ? 0xFFFFFFFFull : 0ull) | (((set >> (2 * i + 1)) & 1) ? ~0xFFFFFFFFull : 0ull);
    }

    const int n_tiles = (int)((nvmax + kSTile - 1) / kSTile);
    i32x8 B[2], Bn[2];
    int sb[2], sbn[2];
    auto load_b = [&](int t, i32x8(&Bx)[2], int(&sx)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t j = (int64_t)t * kSTile + 64 * wave + 32 * u + row;
        const int64_t jr = R + (j < nvmax ? j : nvmax - 1);
        const uint4 v = *reinterpret_cast<const uint4*>(kb + jr * 32 + blk * 16);
        Bx[u] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        sx[u] = a.key_scale[jr * 2 + blk];
      }
    };
    load_b(0, B, sb);
    // wait for the first tile here: the loop's own waits then cover only the prefetched tile
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    for (int t = 0; t < n_tiles; ++t) {
      if (t + 1 < n_tiles) load_b(t + 1, Bn, sbn);
      // keys j = 512 t + 64 wave + 32 u + row for the lane's 4 queries
      const bool full = (int64_t)(t + 1) * kSTile <= nvmin;  // every key of the tile visible to all
      uint64_t key[2][4];
      uint64_t bal[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f32x16 zero = {};
        const f32x16 acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B[u], zero, 4, 4, 0, sa, 0, sb[u]);
        const int64_t j = (int64_t)t * kSTile + 64 * wave + 32 * u + row;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sc = score_term(wq[i][0], acc[4 * i]);
#pragma unroll
          for (int h = 1; h < 4; ++h) sc = score_add(sc, score_term(wq[i][h], acc[4 * i + h]));
          key[u][i] = ((uint64_t)float_key(sc) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
          uint64_t m = __ballot(key[u][i] > fl[i]) & inmask[i];
          if (!full) m &= __ballot(j < nvl[i]);
          bal[u][i] = m;
        }
      }
      // per wave and query: the tile's candidates counted (u, then lane, is ascending j)
      uint32_t (*wc)[kSWaves] = s.wcnt[t & 1];
      if (lane < kSQ) {
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const uint64_t m = bal[u][i];
            const uint32_t c0 = (uint32_t)__popcll(m & 0xFFFFFFFFull), c1 = (uint32_t)__popcll(m >> 32);
            c += lane == 2 * i ? c0 : (lane == 2 * i + 1 ? c1 : 0u);
          }
        wc[lane][wave] = c;
      }
      __syncthreads();
      // lane 8 q + w holds wave w's count for query q: per query, the tile's total and the
      // count of the waves before this one
      const uint32_t cc = wc[cq][cw];
      const uint32_t bef = cnt + group8_sum(cw < wave ? cc : 0u);  // slot of this wave's first
      const uint32_t below = (1u << row) - 1u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if ((bal[0][i] | bal[1][i]) == 0) continue;  // no candidate of these two queries in this wave
        const int qq = 2 * i + blk;
        const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)bef, 16 * i);
        const uint32_t b1 = (uint32_t)__builtin_amdgcn_readlane((int)bef, 16 * i + 8);
        const uint32_t base = blk ? b1 : b0;
        const uint32_t m0 = (uint32_t)(blk ? (bal[0][i] >> 32) : bal[0][i]);
        const uint32_t m1 = (uint32_t)(blk ? (bal[1][i] >> 32) : bal[1][i]);
        if ((m0 >> row) & 1u) s.buf[qq][base + (uint32_t)__popc(m0 & below)] = key[0][i];
        if ((m1 >> row) & 1u) s.buf[qq][base + (uint32_t)__popc(m0) + (uint32_t)__popc(m1 & below)] = key[1][i];
      }
      cnt += group8_sum(cc);
      if (__ballot(cw == 0 && cnt > (uint32_t)(kSCap - kSTile))) {
        // a buffer could overflow on the next tile: every buffer holding more than k keys is cut
        // now, so that the cuts of the block's queries fall on the same tiles
        __syncthreads();  // every placement of the tile is in the buffers
        const uint32_t nw = (uint32_t)__builtin_amdgcn_readlane((int)cnt, 8 * wave);
        if (nw > (uint32_t)K) stream_cut(s, wave, nw, (uint32_t)K);
        cnt = min(cnt, (uint32_t)K);
        __syncthreads();  // the floors are raised and the buffers compacted
#pragma unroll
        for (int i = 0; i < 4; ++i) fl[i] = s.floor_key[2 * i + blk];
      }
      B[0] = Bn[0];
      B[1] = Bn[1];
      sb[0] = sbn[0];
      sb[1] = sbn[1];
    }
    __syncthreads();  // every placement of the last tile is in the buffers
    // wave q: the k largest keys of query q, in ascending j
    if ((set >> wave) & 1u) {
      const uint32_t nw = (uint32_t)__builtin_amdgcn_readlane((int)cnt, 8 * wave);
      if (nw > (uint32_t)K) stream_cut(s, wave, nw, (uint32_t)K);
      int32_t* out = a.out + (int64_t)(q0 + wave) * K;
      for (int i = lane; i < K; i += 64) out[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)s.buf[wave][i]) + jo_wave;
    }
    __syncthreads();
  }
}

// Scores on the vector ALUs (4 keys per thread), launched for fp32 keys (bf16 keys take
// score_bf16_kernel). grid = (nblk, nq).
template <typename T>
__global__ __launch_bounds__(256) void score_valu_kernel(IndexArgs a) {
  __shared__ BlockLds lds;
  __shared__ float qs[8 * 64];
  const int qi = blockIdx.y;
  int64_t rb;
  const int64_t nv = visible_keys(a, qi, &rb);
  if (nv <= a.k) return;
  const int64_t jb = (int64_t)blockIdx.x * kBlockKeys;
  if (jb >= nv) return;
  for (int i = threadIdx.x; i < kHistBins; i += 256) lds.hist[i] = 0;
  const T* q = static_cast<const T*>(a.q) + (int64_t)qi * a.H * 64;
  for (int i = threadIdx.x; i < a.H * 64; i += 256) {
    if (sizeof(T) == 4) qs[i] = reinterpret_cast<const float*>(q)[i];
    else qs[i] = bf16_to_f32(reinterpret_cast<const uint16_t*>(q)[i]);
  }
  float w[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) w[h] = h < a.H ? a.w[(int64_t)qi * a.H + h] : 0.f;
  __syncthreads();
  for (int i = 0; i < kBlockKeys / 256; ++i) {
    const int t = threadIdx.x + 256 * i;
    const int64_t j = jb + t;
    if (j >= nv) continue;
    const T* kp = static_cast<const T*>(a.keys) + (rb + j) * 64;
    float kv[64];
    if (sizeof(T) == 4) {
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float4 v = reinterpret_cast<const float4*>(kp)[c];
        kv[4 * c] = v.x; kv[4 * c + 1] = v.y; kv[4 * c + 2] = v.z; kv[4 * c + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 v = reinterpret_cast<const uint4*>(kp)[c];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv[8 * c + 2 * e] = __uint_as_float(u[e] << 16);
          kv[8 * c + 2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
        }
      }
    }
    float s = 0.f;
    for (int h = 0; h < a.H; ++h) {
      float r = 0.f;
#pragma unroll
      for (int d = 0; d < 64; ++d) r = fmaf(qs[h * 64 + d], kv[d], r);
      const float p = score_term(w[h], r);
      s = h == 0 ? p : score_add(s, p);
    }
    const uint32_t key = float_key(s);
    lds.key[t] = key;
    atomicAdd(&lds.hist[key >> 21], 1u);
  }
  __syncthreads();
  emit_candidates(a, qi, jb, nv, lds);
}

// ---------------------------------------------------------------------------------------
// Finalisation: one block of kFinThreads threads per query (topk_select.h).
__global__ __launch_bounds__(kFinThreads) void finalize_kernel(IndexArgs a) {
  __shared__ FinLds f;
  __shared__ OutLds ol;
  finalize_block(a, blockIdx.x, f, ol);
}

}  // namespace

size_t index_ws_layout(int64_t nq, int64_t max_visible, void* ws, IndexArgs* a) {
  const int64_t nblk = std::max<int64_t>(1, (max_visible + kBlockKeys - 1) / kBlockKeys);
  uintptr_t p = (reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255);
  const uintptr_t p0 = reinterpret_cast<uintptr_t>(ws);
  auto take = [&](size_t bytes) {
    const uintptr_t q = p;
    p = (p + bytes + 255) & ~uintptr_t(255);
    return reinterpret_cast<void*>(q);
  };
  void* scores = take((size_t)nq * nblk * kBlockKeys * 4);
  void* cand = take((size_t)nq * nblk * kBlockKeys * 8);
  void* ovf = take((size_t)nq * (nblk * kBlockKeys + kMaxTopK) * 8);
  void* thr = take((size_t)nq * nblk * 8);
  if (a) {
    a->nblk = (int)nblk;
    a->scores = static_cast<uint32_t*>(scores);
    a->cand = static_cast<uint64_t*>(cand);
    a->ovf = static_cast<uint64_t*>(ovf);
    a->blk_thr = static_cast<uint64_t*>(thr);
  }
  return (size_t)(p - p0) + 256;
}

hipError_t index_init() {
  return hipSuccess;
}

// The streaming kernel serves many-query MXFP4 calls with 4 indexer heads; it needs no
// workspace and writes the output itself (the scores phase of the split calls runs it, the
// select phase then has nothing left to do).
static_assert(kStreamMaxK == kStreamMaxTopK, "the streaming indexer's k bound");
bool index_streams(const IndexArgs& a) { return index_stream_path(a.dtype, a.H, a.nq, a.k); }

hipError_t launch_index_topk(const IndexArgs& a, bool scores, bool select, hipStream_t s) {
  if (index_streams(a)) {
    if (scores)
      hipLaunchKernelGGL(index_stream_kernel, dim3((unsigned)((a.nq + kSQ - 1) / kSQ)), dim3(kSThreads), 0, s, a);
    return hipGetLastError();
  }
  if (scores && a.max_visible > a.k) {
    const dim3 g((unsigned)a.nblk, (unsigned)a.nq);
    if (a.dtype == HCA_MXFP4 && a.H == 4 && a.nq >= 256) {
      const dim3 g4((unsigned)a.nblk, (unsigned)((a.nq + kScoreQ - 1) / kScoreQ));
      hipLaunchKernelGGL(score_mxfp4_q4_kernel, g4, dim3(256), 0, s, a);
    } else if (a.dtype == HCA_MXFP4) hipLaunchKernelGGL(score_mxfp4_kernel, g, dim3(256), 0, s, a);
    else if (a.dtype == HCA_F32) hipLaunchKernelGGL(score_valu_kernel<float>, g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(score_bf16_kernel, g, dim3(256), 0, s, a);
  }
  if (select) hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)a.nq), dim3(kFinThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hca
