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

constexpr int kBlockKeys = 1024;        // entries per score block
constexpr int kFinThreads = 512;        // finalize block
constexpr int kCandCap = 8192;          // candidates finalize holds in registers
constexpr int kMaxBlk = 2048;           // score blocks per query (max_visible <= 2^21)
constexpr int kBpt = kMaxBlk / kFinThreads;  // score blocks per finalize thread

// The visible entries of query qi are the rows *row0 + j, j < the returned count, which are
// entries *j0 + j of its sequence: with a document mask the entries before j_lo (their window
// starts before the document) are cut off the front, so the kernels work on the shifted range
// and add *j0 to the indices they output.
__device__ __forceinline__ int64_t visible_keys(const IndexArgs& a, int qi, int64_t* row0, int64_t* j0 = nullptr) {
  const int b = a.q_seq[qi];
  const int64_t t = a.q_pos[qi];
  const int64_t lo = a.q_lo ? a.q_lo[qi] : 0;
  const int64_t j_lo = lo > 0 ? (lo + a.cw - 1) / a.m : 0;  // ceil((lo + cw - m) / m)
  const int64_t rb = a.k_row_begin[b] + j_lo;
  int64_t nv = t >= 0 ? (t + 1) / a.m : 0;
  nv = min(nv, a.max_visible) - j_lo;
  nv = min(nv, a.k_rows - rb);
  if (rb < 0 || nv < 0) nv = 0;
  *row0 = rb;
  if (j0) *j0 = j_lo;
  return nv;
}

// ---------------------------------------------------------------------------------------
// Block-wide helpers (blockDim.x = NT, a multiple of 64).

// Exclusive prefix sum of v over the block (thread order); *total gets the block sum.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds_tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan_add(v);
  if (lane == 63) lds_tmp[wave] = x;
  __syncthreads();
  uint32_t wbase = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t t = lds_tmp[w];
    wbase += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return wbase + x - v;
}

// Over counters c[0..256*PER) in LDS: the largest index d with sum_{i >= d} c[i] >= rem, and
// above = sum_{i > d} c[i]. Wave 0 must call it; one lane writes the result to *d_out /
// *above_out (LDS). Requires sum c >= rem >= 1.
template <int PER>
__device__ __forceinline__ void find_crossing(const uint32_t* c, uint32_t rem, int* d_out, uint32_t* above_out) {
  const int lane = threadIdx.x & 63;
  constexpr int G = 4 * PER;  // counters per lane
  uint32_t v[G];
  uint32_t own = 0;
  const uint4* c4 = reinterpret_cast<const uint4*>(c);
#pragma unroll
  for (int i = 0; i < G / 4; ++i) {
    const uint4 q = c4[(G / 4) * lane + i];
    v[4 * i] = q.x;
    v[4 * i + 1] = q.y;
    v[4 * i + 2] = q.z;
    v[4 * i + 3] = q.w;
    own += q.x + q.y + q.z + q.w;
  }
  const uint32_t pre = wave_incl_scan_add(own);
  const uint32_t nxt = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63) - pre;  // sum over lanes > lane
  const uint32_t suf = nxt + own;                                                 // sum over lanes >= lane
  if (suf >= rem && nxt < rem) {
    uint32_t acc = nxt;
    int d = G * lane;
#pragma unroll
    for (int i = G - 1; i >= 0; --i) {
      if (acc + v[i] >= rem) { d = G * lane + i; break; }
      acc += v[i];
    }
    *d_out = d;
    *above_out = acc;
  }
}

struct CrossLds {
  int dc, d;
  uint32_t ac, above;
};

// Over 2048 counters h in LDS with NT threads: *d = the largest bin with
// sum_{i >= d} h[i] >= rem and *above = sum_{i > d} h[i]. Requires sum >= rem >= 1; part is
// NT words of LDS. Reads are 16-byte vectors so that the threads hit distinct LDS banks.
// Ends with the block synchronised.
template <int NT>
__device__ __forceinline__ void crossing2048(const uint32_t* h, uint32_t* part, uint32_t rem, CrossLds& x, int* d,
                                             uint32_t* above) {
  constexpr int B = kHistBins / NT;  // bins per thread
  const int tid = threadIdx.x;
  const uint4* h4 = reinterpret_cast<const uint4*>(h);
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < B / 4; ++i) {
    const uint4 q = h4[(B / 4) * tid + i];
    s += q.x + q.y + q.z + q.w;
  }
  part[tid] = s;
  __syncthreads();
  if (tid < 64) find_crossing<NT / 256>(part, rem, &x.dc, &x.ac);
  __syncthreads();
  if (tid == x.dc) {
    uint32_t acc = x.ac;
    int b = B * tid + B - 1;
    for (; b > B * tid; --b) {
      if (acc + h[b] >= rem) break;
      acc += h[b];
    }
    x.d = b;
    x.above = acc;
  }
  __syncthreads();
  *d = x.d;
  *above = x.above;
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

// Candidates of a block: L = max(16, ceil(2 k 1024 / n_vis)), about twice the block's share of
// the top-k when the top-k is spread evenly over the blocks.
__device__ __forceinline__ uint32_t block_quota(int k, int64_t nv) {
  return (uint32_t)max<int64_t>(16, (2 * (int64_t)k * kBlockKeys + nv - 1) / nv);
}
// Candidate slots per block: a block emits at most 2L keys (and at most its 1024 entries).
__device__ __forceinline__ uint32_t region_slots(uint32_t L) { return min(2 * L, (uint32_t)kBlockKeys); }

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

// Wave-wide minimum and maximum of 64-bit keys.
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off, 64), hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o < v ? o : v;
  }
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off, 64), hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

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
// Finalisation: one block of kFinThreads threads per query.

constexpr int kListCap = kHistBins / 2;         // keys of one bin ranked exactly (the histogram's LDS)
constexpr int kPer = kCandCap / kFinThreads;    // candidates per thread, held in registers

struct FinLds {
  uint32_t h[kHistBins];  // histogram; keys of the crossing bin (as u64); flagged blocks; output
  uint64_t sel[kMaxTopK];  // keys of the selected entries
  uint64_t sel_sink[64];   // per-lane targets of writes that select nothing (branch-free code)
  uint64_t list_sink[64];
  uint32_t part[kFinThreads];
  uint32_t tmp[32];
  CrossLds cx;
  uint64_t kmin, kmax, T;
  uint32_t smin, smax, nsel, nflag, novf;
};

// The candidates of one query: ns slots of the score blocks (0 = empty) and novf rescanned keys.
struct CandSet {
  const uint64_t* slots;
  uint32_t ns;
  const uint64_t* ovf;
  uint32_t novf;
};

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int32_t key_entry(uint64_t key) { return (int32_t)(0xFFFFFFFFu - (uint32_t)key); }

// The score whose float_key is k (the top half of a candidate key).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// f.kmin / f.kmax <- the smallest and largest of the per-thread extremes lo / hi.
__device__ __forceinline__ void block_min_max(uint64_t lo, uint64_t hi, FinLds& f) {
  lo = wave_min_u64(lo);
  hi = wave_max_u64(hi);
  if (threadIdx.x == 0) {
    f.kmin = ~0ull;
    f.kmax = 0;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    atomicMin(reinterpret_cast<unsigned long long*>(&f.kmin), (unsigned long long)lo);
    atomicMax(reinterpret_cast<unsigned long long*>(&f.kmax), (unsigned long long)hi);
  }
  __syncthreads();
}

// Monotone map of a candidate key to one of 2048 equal-width bins of the score range between
// the score keys k0 < k1.
struct ScoreBins {
  float s0, inv;
  __device__ __forceinline__ ScoreBins(uint32_t k0, uint32_t k1) {
    s0 = key_score(k0);
    inv = 2047.0f / (key_score(k1) - s0);
  }
  __device__ __forceinline__ int operator()(uint64_t key) const {
    return (int)fminf(fmaxf(__fmul_rn(__fsub_rn(key_score((uint32_t)(key >> 32)), s0), inv), 0.f), 2047.f);
  }
};

// Appends x to list[] (counter *n) with one LDS atomic per wave; p says whether this lane appends.
template <class Tv>
__device__ __forceinline__ void wave_append(bool p, Tv x, Tv* list, uint32_t* n, uint32_t cap) {
  const uint64_t m = __ballot(p);
  if (m == 0) return;
  const int lane = threadIdx.x & 63, leader = __ffsll((long long)m) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(n, (uint32_t)__popcll(m));
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
  const uint32_t slot = base + lanes_below(m);
  if (p && slot < cap) list[slot] = x;
}

// Selection with the candidates in registers (v[i], 0 = empty; at least K non-empty, unique).
// Returns T, the K-th largest key (exactly K keys are >= T); with kSel it also writes those K
// keys to f.sel (unordered). First pass: a histogram over 2048 equal-width bins of the
// candidates' score range; the keys of the bin holding the K-th key are then ranked exactly
// among themselves (gathered by per-wave appends when only T is wanted; with kSel every
// selected key is placed by a block scan or by its rank). Equal scores throughout, or a
// crossing bin with more than kListCap keys (heavy ties), are resolved by 11-bit radix passes
// below the bits all candidates share.
template <bool kSel>
__device__ __forceinline__ uint64_t select_regs(const uint64_t (&v)[kPer], uint32_t K, FinLds& f) {
  const int tid = threadIdx.x;
  // Elementwise steps below are written without branches (selects, sink addresses): in this
  // one-pass kernel every taken branch is a likely instruction-cache miss.
  const int lane = tid & 63;
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint32_t k = (uint32_t)(v[i] >> 32);  // 0 for an empty slot
    lo = min(lo, v[i] ? k : 0xFFFFFFFFu);
    hi = max(hi, k);
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (tid == 0) {
    f.smin = 0xFFFFFFFFu;
    f.smax = 0;
  }
  for (int i = tid; i < kHistBins; i += kFinThreads) f.h[i] = 0;
  __syncthreads();
  if ((tid & 63) == 0) {
    atomicMin(&f.smin, lo);
    atomicMax(&f.smax, hi);
  }
  __syncthreads();
  if (f.smin != f.smax) {
    const ScoreBins bin(f.smin, f.smax);
    int bn[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = bin(v[i]);
      bn[i] = v[i] ? b : -1;
      atomicAdd(v[i] ? &f.h[b] : &f.part[tid], 1u);  // part[] is rewritten by the crossing search
    }
    __syncthreads();
    int d;
    uint32_t above;
    crossing2048<kFinThreads>(f.h, f.part, K, f.cx, &d, &above);
    const uint32_t rem = K - above, cd = f.h[d];
    if (tid == 0) f.nsel = 0;
    __syncthreads();
    if (cd <= (uint32_t)kListCap && !kSel) {
      // the crossing bin's keys, in any order (one LDS atomic per wave and slot)
      uint64_t* list = reinterpret_cast<uint64_t*>(f.h);
#pragma unroll
      for (int i = 0; i < kPer; ++i) wave_append<uint64_t>(bn[i] == d, v[i], list, &f.nsel, (uint32_t)kListCap);
      __syncthreads();
      for (uint32_t i = tid; i < cd; i += kFinThreads) {
        const uint64_t x = list[i];
        uint32_t g = 0;
        for (uint32_t j = 0; j < cd; ++j) g += list[j] > x;
        if (g == rem - 1) f.T = x;
      }
      __syncthreads();
      return f.T;
    }
    if (cd <= (uint32_t)kListCap) {
      uint64_t* list = reinterpret_cast<uint64_t*>(f.h);
      uint32_t na = 0, nl = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        na += bn[i] > d;
        nl += bn[i] == d;
      }
      uint32_t tot;
      const uint32_t off = block_exclusive_scan<kFinThreads>(na | (nl << 16), f.tmp, &tot);
      uint32_t oa = off & 0xFFFFu, ol = off >> 16;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const bool a = bn[i] > d, l = bn[i] == d;
        if (kSel) *(a ? &f.sel[min(oa, K - 1)] : &f.sel_sink[lane]) = v[i];
        *(l ? &list[min(ol, (uint32_t)kListCap - 1)] : &f.list_sink[lane]) = v[i];
        oa += a;
        ol += l;
      }
      __syncthreads();
      // rank within the bin: a key with g larger keys is selected iff g < rem
      for (uint32_t i = tid; i < cd; i += kFinThreads) {
        const uint64_t x = list[i];
        uint32_t g = 0;
        for (uint32_t j = 0; j < cd; ++j) g += list[j] > x;
        if (kSel && g < rem) f.sel[above + g] = x;
        if (g == rem - 1) f.T = x;
      }
      __syncthreads();
      return f.T;
    }
  }
  // radix passes (heavy ties, or a single candidate)
  uint64_t klo = ~0ull, khi = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (v[i]) klo = v[i] < klo ? v[i] : klo;
    khi = v[i] > khi ? v[i] : khi;
  }
  block_min_max(klo, khi, f);
  const uint64_t kmin = f.kmin, kmax = f.kmax;
  uint64_t T = kmin;
  if (kmin != kmax) {
    int lb = 64 - __clzll((long long)(kmin ^ kmax));  // bits >= lb are common to all candidates
    uint64_t prefix = lb >= 64 ? 0ull : (kmax >> lb) << lb;
    uint32_t rem = K;
    while (true) {
      const int hb = lb, width = min(11, lb);
      lb -= width;
      for (int i = tid; i < kHistBins; i += kFinThreads) f.h[i] = 0;
      __syncthreads();
      const uint64_t want = hb >= 64 ? 0ull : prefix >> hb;
      const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const bool m = v[i] && (hb >= 64 || (v[i] >> hb) == want);
        atomicAdd(m ? &f.h[(uint32_t)(v[i] >> lb) & dmask] : &f.part[tid], 1u);
      }
      __syncthreads();
      int d;
      uint32_t above;
      crossing2048<kFinThreads>(f.h, f.part, rem, f.cx, &d, &above);
      rem -= above;
      prefix |= (uint64_t)d << lb;
      const bool done = f.h[d] == rem || lb == 0;
      __syncthreads();
      if (done) break;
    }
    T = prefix;
  }
  if (!kSel) return T;
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) n += v[i] >= T;  // T > 0, so empty slots never count
  uint32_t tot;
  uint32_t o = block_exclusive_scan<kFinThreads>(n, f.tmp, &tot);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const bool s = v[i] >= T;
    *(s ? &f.sel[min(o, K - 1)] : &f.sel_sink[tid & 63]) = v[i];
    o += s;
  }
  __syncthreads();
  return T;
}

// Calls fn(key) for every candidate held in global memory (empty slots skipped).
template <class F>
__device__ __forceinline__ void for_each_global(const CandSet& cs, F fn) {
  for (uint32_t i = threadIdx.x; i < cs.ns; i += kFinThreads) {
    const uint64_t key = cs.slots[i];
    if (key) fn(key);
  }
  for (uint32_t i = threadIdx.x; i < cs.novf; i += kFinThreads) fn(cs.ovf[i]);
}

// Selection over more candidates than the registers hold: the same steps as select_regs, with
// every pass reading the candidates from global memory and LDS atomics for the appends.
__device__ uint64_t select_global(const CandSet& cs, uint32_t K, FinLds& f) {
  const int tid = threadIdx.x;
  uint64_t lo = ~0ull, hi = 0;
  for_each_global(cs, [&](uint64_t x) {
    lo = x < lo ? x : lo;
    hi = x > hi ? x : hi;
  });
  block_min_max(lo, hi, f);
  const uint64_t kmin = f.kmin, kmax = f.kmax;
  if (tid == 0) f.nsel = 0;
  uint64_t T = kmin;
  if (kmin != kmax) {
    int lb = 64 - __clzll((long long)(kmin ^ kmax));
    uint64_t prefix = lb >= 64 ? 0ull : (kmax >> lb) << lb;
    uint32_t rem = K;
    while (true) {
      const int hb = lb, width = min(11, lb);
      lb -= width;
      for (int i = tid; i < kHistBins; i += kFinThreads) f.h[i] = 0;
      __syncthreads();
      const uint64_t want = hb >= 64 ? 0ull : prefix >> hb;
      const uint32_t dmask = (1u << width) - 1u;
      for_each_global(cs, [&](uint64_t key) {
        if (hb >= 64 || (key >> hb) == want) atomicAdd(&f.h[(uint32_t)(key >> lb) & dmask], 1u);
      });
      __syncthreads();
      int d;
      uint32_t above;
      crossing2048<kFinThreads>(f.h, f.part, rem, f.cx, &d, &above);
      rem -= above;
      prefix |= (uint64_t)d << lb;
      const bool done = f.h[d] == rem || lb == 0;
      __syncthreads();
      if (done) break;
    }
    T = prefix;
  }
  __syncthreads();
  for_each_global(cs, [&](uint64_t key) { wave_append<uint64_t>(key >= T, key, f.sel, &f.nsel, K); });
  __syncthreads();
  return T;
}

// Candidates tid + kFinThreads * i of cs into registers (0 past the end). Unconditional loads
// from clamped slots stay in flight together.
__device__ __forceinline__ void load_candidates(const CandSet& cs, uint64_t (&v)[kPer]) {
  const int tid = threadIdx.x;
  const uint32_t n = cs.ns + cs.novf;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint32_t s = min((uint32_t)(tid + kFinThreads * i), n - 1);
    v[i] = *(s < cs.ns ? cs.slots + s : cs.ovf + (s - cs.ns));
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (tid + kFinThreads * i >= (int)n) v[i] = 0;
}

// Score blocks whose unemitted keys (all below the block's threshold) may reach T; their
// numbers go to f.h. Returns how many.
__device__ __forceinline__ uint32_t flag_blocks(const uint64_t (&tq)[kBpt], uint64_t T, FinLds& f) {
  const int tid = threadIdx.x;
  if (tid == 0) f.nflag = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kBpt; ++i)
    if (tq[i] > T) f.h[atomicAdd(&f.nflag, 1u)] = (uint32_t)(kBpt * tid + i);
  __syncthreads();
  return f.nflag;
}

// Output of the K keys >= T when they are all among the emitted candidates. The candidate slots
// are in ascending entry order (score blocks in order, each block's keys ascending, empty slots
// 0 < T), so compacting the selected slots in slot order gives the ascending answer. Slot
// tid + kFinThreads * i is position (i, wave, lane) in row-major order: per-wave ballots give
// the lane offsets, a scan of the kPer x 8 wave counts the rest.
__device__ __forceinline__ void ordered_output(const uint64_t (&v)[kPer], uint64_t T, int K, int32_t* out, int32_t j0,
                                               FinLds& f) {
  static_assert(kPer * (kFinThreads / 64) == 128, "two counts per lane of one wave");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* cnt = f.h;  // [kPer][8] wave counts, then their exclusive prefix
  uint32_t mb[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint64_t bal = __ballot(v[i] >= T);
    mb[i] = lanes_below(bal);
    if (lane == 0) cnt[i * 8 + wave] = (uint32_t)__popcll(bal);
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t c0 = cnt[2 * lane], c1 = cnt[2 * lane + 1];
    const uint32_t incl = wave_incl_scan_add(c0 + c1);
    cnt[2 * lane] = incl - c0 - c1;
    cnt[2 * lane + 1] = incl - c1;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (v[i] >= T) out[min(cnt[i * 8 + wave] + mb[i], (uint32_t)K - 1)] = key_entry(v[i]) + j0;
}

// Output LDS: per-block counts (then their prefix), per-block cursors, entries bucketed by block.
struct OutLds {
  uint32_t pre[kMaxBlk + 1];
  uint32_t cur[kMaxBlk];
  int32_t bucket[kMaxTopK];
};

__global__ __launch_bounds__(kFinThreads) void finalize_kernel(IndexArgs a) {
  __shared__ FinLds f;
  __shared__ OutLds ol;
  const int qi = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.k;
  const int64_t q_blk = (int64_t)qi * a.nblk;
  const uint64_t* thr = a.blk_thr + q_blk;
  const uint64_t* slots = a.cand + q_blk * kBlockKeys;
  // The candidate slots and block thresholds lie in this query's workspace region, so their
  // loads go out first (clamped to the region) and are masked once the visible count is known.
  uint64_t v[kPer], tq[kBpt];
  {
    const uint32_t region = (uint32_t)a.nblk * kBlockKeys;
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = slots[min((uint32_t)(tid + kFinThreads * i), region - 1)];
#pragma unroll
    for (int i = 0; i < kBpt; ++i) tq[i] = thr[min(kBpt * tid + i, a.nblk - 1)];
  }
  int64_t rb, j0;
  const int64_t nv = visible_keys(a, qi, &rb, &j0);
  const int32_t jo = (int32_t)j0;  // entry index of visible key 0
  int32_t* out = a.out + (int64_t)qi * K;
  if (nv <= K) {  // every visible entry is selected, ascending; pad with -1
    for (int j = tid; j < K; j += kFinThreads) out[j] = j < nv ? j + jo : -1;
    return;
  }
  const int nb = (int)((nv + kBlockKeys - 1) / kBlockKeys);
  const uint32_t* sk = a.scores + q_blk * kBlockKeys;
  const int64_t ovf_cap = (int64_t)a.nblk * kBlockKeys + kMaxTopK;  // >= k + n_vis
  uint64_t* ovf = a.ovf + (int64_t)qi * ovf_cap;
  CandSet cs;
  cs.slots = slots;
  cs.ns = (uint32_t)nb * region_slots(block_quota(K, nv));
  cs.ovf = ovf;
  cs.novf = 0;
  // thresholds of blocks kBpt * tid + i
#pragma unroll
  for (int i = 0; i < kBpt; ++i)
    if (kBpt * tid + i >= nb) tq[i] = 0ull;
  if (tid == 0) f.novf = 0;
  // round 1 over the emitted candidates
  uint64_t T;
  uint32_t nflag;
  if (cs.ns <= (uint32_t)kCandCap) {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if ((uint32_t)(tid + kFinThreads * i) >= cs.ns) v[i] = 0;
    T = select_regs<false>(v, (uint32_t)K, f);
    nflag = flag_blocks(tq, T, f);
    if (nflag == 0) {
      ordered_output(v, T, K, out, jo, f);
      return;
    }
    // the round-1 winners (the K keys >= T) seed the overflow list of round 2
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) c += v[i] >= T;
    uint32_t tot;
    uint32_t o = block_exclusive_scan<kFinThreads>(c, f.tmp, &tot);
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (v[i] >= T) ovf[min(o++, (uint32_t)K - 1)] = v[i];
  } else {
    T = select_global(cs, (uint32_t)K, f);
    nflag = flag_blocks(tq, T, f);
    if (nflag > 0)
      for (int i = tid; i < K; i += kFinThreads) ovf[i] = f.sel[i];
  }
  if (nflag > 0) {
    // round 2 selects among the round-1 winners (every candidate >= T) and the unemitted keys
    // >= T of the flagged blocks (one wave per block), all gathered in the overflow list:
    // together they hold every key >= T, hence the whole top-k
    if (tid == 0) f.novf = (uint32_t)K;
    __syncthreads();
    // one wave per flagged block; the next block's keys are loaded before this block's are
    // appended, so each block's load time overlaps the previous block's appends
    constexpr int kR = kBlockKeys / 64;
    uint32_t fi = wave;
    int b = fi < nflag ? (int)f.h[fi] : 0;
    uint32_t kv[kR];
    uint64_t tb = thr[b];
#pragma unroll
    for (int r = 0; r < kR; ++r) kv[r] = sk[min<int64_t>((int64_t)b * kBlockKeys + lane + 64 * r, nv - 1)];
    while (fi < nflag) {
      const uint32_t fn = fi + kFinThreads / 64;
      const int bn = fn < nflag ? (int)f.h[fn] : b;
      uint32_t kn[kR];
      const uint64_t tbn = thr[bn];
#pragma unroll
      for (int r = 0; r < kR; ++r) kn[r] = sk[min<int64_t>((int64_t)bn * kBlockKeys + lane + 64 * r, nv - 1)];
      const int64_t jb = (int64_t)b * kBlockKeys;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int64_t j = jb + lane + 64 * r;
        const uint64_t k64 = ((uint64_t)kv[r] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
        wave_append<uint64_t>(j < nv && k64 < tb && k64 >= T, k64, ovf, &f.novf, (uint32_t)ovf_cap);
      }
      fi = fn;
      b = bn;
      tb = tbn;
#pragma unroll
      for (int r = 0; r < kR; ++r) kv[r] = kn[r];
    }
    __threadfence_block();
    __syncthreads();
    cs.ns = 0;
    cs.novf = f.novf;
    __syncthreads();
    if (cs.novf <= (uint32_t)kCandCap) {
      uint64_t v[kPer];
      load_candidates(cs, v);
      T = select_regs<true>(v, (uint32_t)K, f);
    } else {
      T = select_global(cs, (uint32_t)K, f);
    }
  }
  // ascending order: bucket the K entries by score block, then rank each within its bucket
  const uint64_t* sel = f.sel;
  for (int b = tid; b < nb; b += kFinThreads) ol.pre[b] = 0;
  __syncthreads();
  const uint32_t last = (uint32_t)nb - 1;
  for (int i = tid; i < K; i += kFinThreads) atomicAdd(&ol.pre[min((uint32_t)key_entry(sel[i]) >> 10, last)], 1u);
  __syncthreads();
  {
    uint32_t c[kBpt], sum = 0;
#pragma unroll
    for (int i = 0; i < kBpt; ++i) {
      const int b = kBpt * tid + i;
      c[i] = b < nb ? ol.pre[b] : 0u;
      sum += c[i];
    }
    uint32_t tot;
    uint32_t off = block_exclusive_scan<kFinThreads>(sum, f.tmp, &tot);
#pragma unroll
    for (int i = 0; i < kBpt; ++i) {
      const int b = kBpt * tid + i;
      if (b <= nb) ol.pre[b] = off;  // b == nb receives the total K
      if (b < nb) ol.cur[b] = off;
      off += c[i];
    }
    if (tid == 0) ol.pre[nb] = tot;
  }
  __syncthreads();
  for (int i = tid; i < K; i += kFinThreads) {
    const int32_t j = key_entry(sel[i]);
    ol.bucket[min(atomicAdd(&ol.cur[min((uint32_t)j >> 10, last)], 1u), (uint32_t)K - 1)] = j;
  }
  __syncthreads();
  int32_t* sorted = reinterpret_cast<int32_t*>(f.h);
  for (int i = tid; i < K; i += kFinThreads) {
    const int32_t j = ol.bucket[i];
    const uint32_t b = min((uint32_t)j >> 10, last);
    const uint32_t s0 = ol.pre[b], s1 = ol.pre[b + 1];
    uint32_t r = 0;
    for (uint32_t s = s0; s < s1; ++s) r += ol.bucket[s] < j;
    sorted[min(s0 + r, (uint32_t)K - 1)] = j;
  }
  __syncthreads();
  for (int i = tid; i < K; i += kFinThreads) out[i] = sorted[i] + jo;
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
