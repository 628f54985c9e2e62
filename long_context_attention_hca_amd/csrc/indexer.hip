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
//    (__fmul_rn / __fadd_rn), which makes it bit-exact and the top-k unique.
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
//    ascending order through an LDS bitmap over the visible entries.
#include "common.h"
#include "internal.h"

namespace hca {
namespace {

constexpr int kBlockKeys = 1024;        // entries per score block
constexpr int kFinThreads = 1024;       // finalize block
constexpr int64_t kBitmapBits = 1 << 19;
constexpr int kCandCap = 16384;         // candidates held in LDS by finalize (128 KB)
constexpr int kMaxBlk = 2048;           // score blocks per query (max_visible <= 2^21)

__device__ __forceinline__ int64_t visible_keys(const IndexArgs& a, int qi, int64_t* row0) {
  const int b = a.q_seq[qi];
  const int64_t t = a.q_pos[qi];
  const int64_t rb = a.k_row_begin[b];
  int64_t nv = t >= 0 ? (t + 1) / a.m : 0;
  nv = min(nv, a.max_visible);
  nv = min(nv, a.k_rows - rb);
  if (rb < 0 || nv < 0) nv = 0;
  *row0 = rb;
  return nv;
}

// ---------------------------------------------------------------------------------------
// Block-wide helpers (blockDim.x = NT, a multiple of 64).

// Exclusive prefix sum of v over the block (thread order); *total gets the block sum.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds_tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(x, off, 64);
    if (lane >= off) x += t;
  }
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
#pragma unroll
  for (int i = 0; i < G; ++i) {
    v[i] = c[G * lane + i];
    own += v[i];
  }
  uint32_t suf = own;  // inclusive suffix sum over lanes lane..63
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_down(suf, off, 64);
    if (lane + off < 64) suf += t;
  }
  uint32_t nxt = __shfl_down(suf, 1, 64);
  if (lane == 63) nxt = 0;
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

struct BlockLds {
  uint32_t hist[kHistBins];
  uint32_t key[kBlockKeys];
  uint32_t part[256];
  uint32_t tmp[8];
  int d, bin;
  uint32_t above, above_bin;
  uint64_t thr;
};

// Over the 2048 counters lds.hist (256 threads): the largest bin d with sum_{i >= d} >= rem
// and above = sum_{i > d}. Requires sum >= rem >= 1. Ends with the block synchronised.
__device__ __forceinline__ void block_crossing(BlockLds& lds, uint32_t rem, int* d, uint32_t* above) {
  const int tid = threadIdx.x;
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) sum += lds.hist[8 * tid + i];
  lds.part[tid] = sum;
  __syncthreads();
  if (tid < 64) find_crossing<1>(lds.part, rem, &lds.d, &lds.above);
  __syncthreads();
  if (tid == lds.d) {
    uint32_t acc = lds.above;
    int b = 8 * tid + 7;
    for (; b > 8 * tid; --b) {
      if (acc + lds.hist[b] >= rem) break;
      acc += lds.hist[b];
    }
    lds.bin = b;
    lds.above_bin = acc;
  }
  __syncthreads();
  *d = lds.bin;
  *above = lds.above_bin;
}

// Candidates of a block: L = max(16, ceil(2 k 1024 / n_vis)), about twice the block's share of
// the top-k when the top-k is spread evenly over the blocks.
__device__ __forceinline__ uint32_t block_quota(int k, int64_t nv) {
  return (uint32_t)max<int64_t>(16, (2 * (int64_t)k * kBlockKeys + nv - 1) / nv);
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
  uint64_t* dst = a.cand + slot * kBlockKeys;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (t0 + i < nvalid && k64[i] >= thr) dst[off++] = k64[i];
  uint32_t* sk = a.scores + (int64_t)qi * a.nblk * kBlockKeys + jb;
  if (t0 + 3 < nvalid) {
    *reinterpret_cast<uint4*>(sk + t0) = kv;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (t0 + i < nvalid) sk[t0 + i] = kk[i];
  }
  if (tid == 0) {
    a.blk_cnt[slot] = tot;
    a.blk_thr[slot] = thr;
  }
}

// MXFP4 scores via the scaled MFMA. grid = (nblk, nq), 256 threads, 1024 keys per block.
__global__ __launch_bounds__(256) void score_mxfp4_kernel(IndexArgs a) {
  __shared__ BlockLds lds;
  const int qi = blockIdx.y;
  int64_t rb;
  const int64_t nv = visible_keys(a, qi, &rb);
  if (nv <= a.k) return;  // every visible entry is selected; no scores needed
  const int64_t jb = (int64_t)blockIdx.x * kBlockKeys;
  if (jb >= nv) return;
  for (int i = threadIdx.x; i < kHistBins; i += 256) lds.hist[i] = 0;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
      float s = __fmul_rn(w[0], fmaxf(r[0], 0.f));
#pragma unroll
      for (int h = 1; h < 8; ++h)
        if (h < a.H) s = __fadd_rn(s, __fmul_rn(w[h], fmaxf(r[h], 0.f)));
      const uint32_t key = float_key(s);
      lds.key[pos] = key;
      atomicAdd(&lds.hist[key >> 21], 1u);
    }
  }
  __syncthreads();
  emit_candidates(a, qi, jb, nv, lds);
}

// fp32 / bf16 scores on the vector ALUs (4 keys per thread). grid = (nblk, nq).
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
      const float p = __fmul_rn(w[h], fmaxf(r, 0.f));
      s = h == 0 ? p : __fadd_rn(s, p);
    }
    const uint32_t key = float_key(s);
    lds.key[t] = key;
    atomicAdd(&lds.hist[key >> 21], 1u);
  }
  __syncthreads();
  emit_candidates(a, qi, jb, nv, lds);
}

// ---------------------------------------------------------------------------------------
// Finalisation: one block of 1024 threads per query.

struct FinLds {
  uint32_t h[kHistBins];        // radix histogram; list of flagged blocks
  int32_t sel[kMaxTopK];        // the selected entries
  uint32_t pre[kMaxBlk + 1];    // exclusive prefix of the per-block candidate counts
  uint32_t tmp[32];
  uint64_t kmin, kmax;
  int d;
  uint32_t above, nsel, nflag;
};

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Calls f(key) once for every candidate: from LDS (lk[0..nc)) or from the per-block regions.
template <bool kLds, class F>
__device__ __forceinline__ void for_each_cand(const uint64_t* lk, uint32_t nc, const uint64_t* cq, const FinLds& f,
                                              int nb, F fn) {
  if (kLds) {
    for (uint32_t i = threadIdx.x; i < nc; i += kFinThreads) fn(lk[i]);
  } else {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int b = wave; b < nb; b += kFinThreads / 64) {
      const uint32_t c = f.pre[b + 1] - f.pre[b];
      for (uint32_t i = lane; i < c; i += 64) fn(cq[(int64_t)b * kBlockKeys + i]);
    }
  }
}

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

// Per-block counts -> f.pre, then (if they fit) the candidates into lk; f.kmin / f.kmax get
// the smallest and largest candidate key. Returns the candidate count.
__device__ uint32_t gather_candidates(const uint32_t* cnt, const uint64_t* cq, int nb, uint64_t* lk, FinLds& f) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t c0 = 2 * tid < nb ? cnt[2 * tid] : 0u, c1 = 2 * tid + 1 < nb ? cnt[2 * tid + 1] : 0u;
  uint32_t nc;
  const uint32_t off = block_exclusive_scan<kFinThreads>(c0 + c1, f.tmp, &nc);
  f.pre[2 * tid] = off;
  f.pre[2 * tid + 1] = off + c0;
  if (tid == 0) {
    f.pre[nb] = nc;
    f.kmin = ~0ull;
    f.kmax = 0;
  }
  __syncthreads();
  uint64_t lo = ~0ull, hi = 0;
  if (nc <= (uint32_t)kCandCap) {
    constexpr int kBatch = 8, kStride = kFinThreads / 64;
    for (int b0 = wave; b0 < nb; b0 += kStride * kBatch) {
      uint64_t v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int b = b0 + kStride * u;
        const uint32_t c = b < nb ? f.pre[b + 1] - f.pre[b] : 0u;
        v[u] = (uint32_t)lane < c ? cq[(int64_t)b * kBlockKeys + lane] : 0ull;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int b = b0 + kStride * u;
        const uint32_t c = b < nb ? f.pre[b + 1] - f.pre[b] : 0u;
        for (uint32_t i = lane; i < c; i += 64) {
          const uint64_t x = i == (uint32_t)lane ? v[u] : cq[(int64_t)b * kBlockKeys + i];
          lk[f.pre[b] + i] = x;
          lo = x < lo ? x : lo;
          hi = x > hi ? x : hi;
        }
      }
    }
  } else {
    for_each_cand<false>(lk, nc, cq, f, nb, [&](uint64_t x) {
      lo = x < lo ? x : lo;
      hi = x > hi ? x : hi;
    });
  }
  lo = wave_min_u64(lo);
  hi = wave_max_u64(hi);
  if (lane == 0) {
    atomicMin(reinterpret_cast<unsigned long long*>(&f.kmin), (unsigned long long)lo);
    atomicMax(reinterpret_cast<unsigned long long*>(&f.kmax), (unsigned long long)hi);
  }
  __syncthreads();
  return nc;
}

// The K-th largest of the nc >= K unique candidate keys: returns T such that exactly K
// candidates are >= T. Radix passes of 11 bits start below the bits every candidate shares
// and stop once the bin holding the K-th key is taken whole.
template <bool kLds>
__device__ uint64_t select_kth(const uint64_t* lk, uint32_t nc, const uint64_t* cq, FinLds& f, int nb, uint32_t K) {
  const int tid = threadIdx.x;
  const uint64_t kmin = f.kmin, kmax = f.kmax;
  if (kmin == kmax) return kmin;
  int lo = 64 - __clzll((long long)(kmin ^ kmax));  // bits >= lo are common to all candidates
  uint64_t prefix = lo >= 64 ? 0ull : (kmax >> lo) << lo;
  uint32_t rem = K;
  while (true) {
    const int hi = lo, width = min(11, lo);
    lo -= width;
    for (int i = tid; i < kHistBins; i += kFinThreads) f.h[i] = 0;
    __syncthreads();
    const uint64_t want = hi >= 64 ? 0ull : prefix >> hi;
    const uint32_t dmask = (1u << width) - 1u;
    for_each_cand<kLds>(lk, nc, cq, f, nb, [&](uint64_t key) {
      if (hi >= 64 || (key >> hi) == want) atomicAdd(&f.h[(uint32_t)(key >> lo) & dmask], 1u);
    });
    __syncthreads();
    if (tid < 64) find_crossing<8>(f.h, rem, &f.d, &f.above);
    __syncthreads();
    const int d = f.d;
    rem -= f.above;
    prefix |= (uint64_t)d << lo;
    const bool done = f.h[d] == rem || lo == 0;
    __syncthreads();
    if (done) return prefix;
  }
}

__host__ __device__ __forceinline__ int64_t bitmap_words(int64_t nv) { return (nv + 31) >> 5; }

__global__ __launch_bounds__(kFinThreads) void finalize_kernel(IndexArgs a) {
  extern __shared__ uint64_t lk[];  // kCandCap candidate keys, later the output bitmap
  __shared__ FinLds f;
  const int qi = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.k;
  int64_t rb;
  const int64_t nv = visible_keys(a, qi, &rb);
  int32_t* out = a.out + (int64_t)qi * K;
  if (nv <= K) {  // every visible entry is selected, ascending; pad with -1
    for (int j = tid; j < K; j += kFinThreads) out[j] = j < nv ? j : -1;
    return;
  }
  const int nb = (int)((nv + kBlockKeys - 1) / kBlockKeys);
  const int64_t q_blk = (int64_t)qi * a.nblk;
  uint32_t* cnt = a.blk_cnt + q_blk;
  const uint64_t* thr = a.blk_thr + q_blk;
  uint64_t* cq = a.cand + q_blk * kBlockKeys;
  const uint32_t* sk = a.scores + q_blk * kBlockKeys;
  uint32_t nc = gather_candidates(cnt, cq, nb, lk, f);
  bool in_lds = nc <= (uint32_t)kCandCap;
  uint64_t T = in_lds ? select_kth<true>(lk, nc, cq, f, nb, (uint32_t)K) : select_kth<false>(lk, nc, cq, f, nb, (uint32_t)K);
  // blocks whose unemitted keys (all below their threshold) may reach T
  if (tid == 0) f.nflag = 0;
  __syncthreads();
  for (int b = tid; b < nb; b += kFinThreads)
    if (thr[b] > T) f.h[atomicAdd(&f.nflag, 1u)] = (uint32_t)b;
  __syncthreads();
  const uint32_t nflag = f.nflag;
  if (nflag > 0) {
    // append their unemitted keys >= T to their own regions, one wave per block
    for (uint32_t fi = wave; fi < nflag; fi += kFinThreads / 64) {
      const int b = (int)f.h[fi];
      const int64_t jb = (int64_t)b * kBlockKeys;
      const uint64_t tb = thr[b];
      uint32_t c = cnt[b];
      uint32_t kv[kBlockKeys / 64];
#pragma unroll
      for (int r = 0; r < kBlockKeys / 64; ++r) {
        const int64_t j = jb + lane + 64 * r;
        kv[r] = j < nv ? sk[j] : 0u;
      }
#pragma unroll
      for (int r = 0; r < kBlockKeys / 64; ++r) {
        const int64_t j = jb + lane + 64 * r;
        const uint64_t k64 = ((uint64_t)kv[r] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
        const bool p = j < nv && k64 < tb && k64 >= T;
        const uint64_t m = __ballot(p);
        if (p) cq[jb + c + lanes_below(m)] = k64;
        c += (uint32_t)__popcll(m);
      }
      if (lane == 0) cnt[b] = c;
    }
    __threadfence_block();
    __syncthreads();
    nc = gather_candidates(cnt, cq, nb, lk, f);
    in_lds = nc <= (uint32_t)kCandCap;
    T = in_lds ? select_kth<true>(lk, nc, cq, f, nb, (uint32_t)K) : select_kth<false>(lk, nc, cq, f, nb, (uint32_t)K);
  }
  // the K selected entries: candidate keys >= T (one LDS atomic per wave and pass)
  if (tid == 0) f.nsel = 0;
  __syncthreads();
  auto collect = [&](uint64_t key) {
    const bool p = key >= T;
    const uint64_t m = __ballot(p);
    if (m == 0) return;
    const int leader = __ffsll((long long)m) - 1;
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(&f.nsel, (uint32_t)__popcll(m));
    base = __shfl(base, leader, 64);
    const uint32_t slot = base + lanes_below(m);
    if (p && slot < (uint32_t)K) f.sel[slot] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
  };
  if (in_lds) for_each_cand<true>(lk, nc, cq, f, nb, collect);
  else for_each_cand<false>(lk, nc, cq, f, nb, collect);
  __syncthreads();
  int32_t* sel = f.sel;
  if (nv <= kBitmapBits) {
    // ascending order through a bitmap over the visible entries (reusing the candidate LDS)
    uint32_t* bm = reinterpret_cast<uint32_t*>(lk);
    const int64_t nw = bitmap_words(nv);
    for (int64_t i = tid; i < nw; i += kFinThreads) bm[i] = 0;
    __syncthreads();
    for (int i = tid; i < K; i += kFinThreads) atomicOr(&bm[sel[i] >> 5], 1u << (sel[i] & 31));
    __syncthreads();
    const int64_t per = (nw + kFinThreads - 1) / kFinThreads;
    const int64_t w0 = tid * per, w1 = min<int64_t>(nw, w0 + per);
    uint32_t pc = 0;
    for (int64_t w = w0; w < w1; ++w) pc += __popc(bm[w]);
    uint32_t tot;
    uint32_t pos = block_exclusive_scan<kFinThreads>(pc, f.tmp, &tot);
    for (int64_t w = w0; w < w1; ++w) {
      uint32_t bits = bm[w];
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        if (pos < (uint32_t)K) out[pos] = (int32_t)(w * 32 + b);
        ++pos;
      }
    }
    return;
  }
  // very long sequences: bitonic sort of the K indices in LDS
  int N = 1;
  while (N < K) N <<= 1;
  for (int i = K + tid; i < N; i += kFinThreads) sel[i] = 0x7FFFFFFF;
  __syncthreads();
  for (int k2 = 2; k2 <= N; k2 <<= 1) {
    for (int jj = k2 >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < N; i += kFinThreads) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const int32_t x = sel[i], y = sel[ixj];
          const bool asc = (i & k2) == 0;
          if ((x > y) == asc) { sel[i] = y; sel[ixj] = x; }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < K; i += kFinThreads) out[i] = sel[i];
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
  void* cnt = take((size_t)nq * nblk * 4);
  void* thr = take((size_t)nq * nblk * 8);
  if (a) {
    a->nblk = (int)nblk;
    a->scores = static_cast<uint32_t*>(scores);
    a->cand = static_cast<uint64_t*>(cand);
    a->blk_cnt = static_cast<uint32_t*>(cnt);
    a->blk_thr = static_cast<uint64_t*>(thr);
  }
  return (size_t)(p - p0) + 256;
}

hipError_t index_init() {
  return hipFuncSetAttribute((const void*)finalize_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             kCandCap * 8);
}

hipError_t launch_index_topk(const IndexArgs& a, hipStream_t s) {
  if (a.max_visible > a.k) {
    const dim3 g((unsigned)a.nblk, (unsigned)a.nq);
    if (a.dtype == HCA_MXFP4) hipLaunchKernelGGL(score_mxfp4_kernel, g, dim3(256), 0, s, a);
    else if (a.dtype == HCA_F32) hipLaunchKernelGGL(score_valu_kernel<float>, g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(score_valu_kernel<uint16_t>, g, dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)a.nq), dim3(kFinThreads), (size_t)kCandCap * 8, s, a);
  return hipGetLastError();
}

}  // namespace hca
