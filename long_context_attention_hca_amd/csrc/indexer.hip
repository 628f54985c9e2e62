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
//    is unique per entry. Every score block (1024 entries) keeps its keys in LDS,
//    histograms their top 11 bits there, and emits as candidates the entries at or
//    above the bin holding its L-th largest key (L about twice the block's expected
//    share of the top-k, at least 32), recording that bin. One block per query then
//    selects the k-th largest candidate key T by 8-bit radix passes in LDS. Entries
//    a block did not emit all lie below its recorded bin, so if no recorded bin is
//    above T's bin the candidates contain the whole top-k; otherwise the blocks in
//    question are rescanned from their stored keys and the selection is repeated,
//    which keeps the result exact for any input (ties included). The k indices are
//    emitted in ascending order through an LDS bitmap over the visible entries.
#include "common.h"
#include "internal.h"

namespace hca {
namespace {

constexpr int kBlockKeys = 1024;        // entries per score block
constexpr int kFinThreads = 1024;       // finalize block
constexpr int64_t kBitmapBits = 1 << 19;
constexpr int kCandCap = 16384;         // candidates held in LDS by finalize (128 KB)

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

// Zeroes n words (the per-query counters).
__global__ __launch_bounds__(256) void clear_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
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
  uint32_t above, base;
};

// Candidate emission of one score block (all 256 threads; lds.key / lds.hist complete).
__device__ void emit_candidates(const IndexArgs& a, int qi, int64_t jb, int64_t nv, BlockLds& lds) {
  const int tid = threadIdx.x;
  const int nvalid = (int)min<int64_t>(kBlockKeys, nv - jb);
  const int64_t L = max<int64_t>(32, (2 * (int64_t)a.k * kBlockKeys + nv - 1) / nv);
  uint32_t tb = 0;
  if (nvalid > L) {
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += lds.hist[8 * tid + i];
    lds.part[tid] = sum;
    __syncthreads();
    if (tid < 64) find_crossing<1>(lds.part, (uint32_t)L, &lds.d, &lds.above);
    __syncthreads();
    if (tid == lds.d) {
      uint32_t acc = lds.above;
      int b = 8 * tid + 7;
      for (; b > 8 * tid; --b) {
        if (acc + lds.hist[b] >= (uint32_t)L) break;
        acc += lds.hist[b];
      }
      lds.bin = b;
    }
    __syncthreads();
    tb = (uint32_t)lds.bin;
  }
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < kBlockKeys / 256; ++i) {
    const int t = tid + 256 * i;
    n += (t < nvalid && (lds.key[t] >> 21) >= tb);
  }
  uint32_t tot;
  uint32_t off = block_exclusive_scan<256>(n, lds.tmp, &tot);
  if (tid == 0) lds.base = atomicAdd(&a.counters[(int64_t)qi * 4], tot);
  __syncthreads();
  off += lds.base;
  uint32_t* ck = a.cand_key + (int64_t)qi * a.max_visible;
  int32_t* ci = a.cand_idx + (int64_t)qi * a.max_visible;
  uint32_t* sk = a.scores + (int64_t)qi * a.max_visible;
#pragma unroll
  for (int i = 0; i < kBlockKeys / 256; ++i) {
    const int t = tid + 256 * i;
    if (t < nvalid) {
      const uint32_t key = lds.key[t];
      sk[jb + t] = key;
      if ((key >> 21) >= tb) {
        ck[off] = key;
        ci[off] = (int32_t)(jb + t);
        ++off;
      }
    }
  }
  if (tid == 0) a.blk_bin[(int64_t)qi * a.nblk + blockIdx.x] = (int32_t)tb;
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

// The K-th largest of nc unique 64-bit keys (from LDS, or rebuilt from the global candidate
// arrays), by 8-bit radix passes with early exit: returns T such that exactly K keys are >= T.
template <bool kLds>
__device__ uint64_t select_kth(const uint64_t* lk, const uint32_t* gk, const int32_t* gi, uint32_t nc, uint32_t K,
                               uint32_t* h, int* s_d, uint32_t* s_above) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;
  uint32_t rem = K;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    if (tid < 256) h[tid] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < nc; i += kFinThreads) {
      const uint64_t key = kLds ? lk[i] : (((uint64_t)gk[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)gi[i]));
      const bool match = pass == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8));
      if (match) atomicAdd(&h[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) find_crossing<1>(h, rem, s_d, s_above);
    __syncthreads();
    const int d = *s_d;
    rem -= *s_above;
    prefix |= (uint64_t)d << shift;
    const bool done = h[d] == rem;
    __syncthreads();
    if (done) break;
  }
  return prefix;
}

__host__ __device__ __forceinline__ int64_t bitmap_words(int64_t nv) { return (nv + 31) >> 5; }

__global__ __launch_bounds__(kFinThreads) void finalize_kernel(IndexArgs a) {
  extern __shared__ uint64_t lk[];  // kCandCap candidate keys, later the output bitmap
  __shared__ uint32_t h[256];
  __shared__ uint32_t tmp[32];
  __shared__ int32_t sel[kMaxTopK];
  __shared__ int s_d;
  __shared__ uint32_t s_above, s_slot, s_flag;
  const int qi = blockIdx.x, tid = threadIdx.x;
  const int K = a.k;
  int64_t rb;
  const int64_t nv = visible_keys(a, qi, &rb);
  int32_t* out = a.out + (int64_t)qi * K;
  if (nv <= K) {  // every visible entry is selected, ascending; pad with -1
    for (int j = tid; j < K; j += kFinThreads) out[j] = j < nv ? j : -1;
    return;
  }
  uint32_t* cnt = a.counters + (int64_t)qi * 4;
  uint32_t* gk = a.cand_key + (int64_t)qi * a.max_visible;
  int32_t* gi = a.cand_idx + (int64_t)qi * a.max_visible;
  const uint32_t* sk = a.scores + (int64_t)qi * a.max_visible;
  const int32_t* bb = a.blk_bin + (int64_t)qi * a.nblk;
  const int nblk = (int)((nv + kBlockKeys - 1) / kBlockKeys);
  uint32_t nc = cnt[0];
  uint64_t T = 0;
  bool in_lds = false;
  for (int round = 0; round < 2; ++round) {
    in_lds = nc <= (uint32_t)kCandCap;
    if (in_lds) {
      for (uint32_t i = tid; i < nc; i += kFinThreads)
        lk[i] = ((uint64_t)gk[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)gi[i]);
      __syncthreads();
      T = select_kth<true>(lk, gk, gi, nc, (uint32_t)K, h, &s_d, &s_above);
    } else {
      T = select_kth<false>(lk, gk, gi, nc, (uint32_t)K, h, &s_d, &s_above);
    }
    if (round == 1) break;
    // would any block's unemitted entries (all below its recorded bin) reach T?
    const int32_t tbin = (int32_t)(T >> 53);
    if (tid == 0) s_flag = 0;
    __syncthreads();
    for (int b = tid; b < nblk; b += kFinThreads)
      if (bb[b] > tbin) s_flag = 1;
    __syncthreads();
    if (!s_flag) break;
    // rescan those blocks: append their unemitted entries whose key is >= T
    for (int b = 0; b < nblk; ++b) {
      const int32_t tb = bb[b];
      if (tb <= tbin) continue;
      for (int t = tid; t < kBlockKeys; t += kFinThreads) {
        const int64_t j = (int64_t)b * kBlockKeys + t;
        if (j >= nv) continue;
        const uint32_t k32 = sk[j];
        if ((int32_t)(k32 >> 21) >= tb) continue;  // already a candidate
        const uint64_t k64 = ((uint64_t)k32 << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
        if (k64 >= T) {
          const uint32_t slot = atomicAdd(&cnt[0], 1u);
          gk[slot] = k32;
          gi[slot] = (int32_t)j;
        }
      }
    }
    __threadfence();
    __syncthreads();
    nc = atomicAdd(&cnt[0], 0u);
    __syncthreads();
  }
  // the K selected entries: keys >= T
  if (tid == 0) s_slot = 0;
  __syncthreads();
  for (uint32_t i = tid; i < nc; i += kFinThreads) {
    const uint64_t key = in_lds ? lk[i] : (((uint64_t)gk[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)gi[i]));
    if (key >= T) sel[atomicAdd(&s_slot, 1u)] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
  }
  __syncthreads();
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
    uint32_t pos = block_exclusive_scan<kFinThreads>(pc, tmp, &tot);
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
  const int64_t mv = (max_visible + 63) / 64 * 64;
  const int64_t nblk = (max_visible + kBlockKeys - 1) / kBlockKeys;
  uintptr_t p = (reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255);
  const uintptr_t p0 = reinterpret_cast<uintptr_t>(ws);
  auto take = [&](size_t bytes) {
    const uintptr_t q = p;
    p = (p + bytes + 255) & ~uintptr_t(255);
    return reinterpret_cast<void*>(q);
  };
  void* scores = take((size_t)nq * mv * 4);
  void* ckey = take((size_t)nq * mv * 4);
  void* cidx = take((size_t)nq * mv * 4);
  void* bins = take((size_t)nq * (nblk > 0 ? nblk : 1) * 4);
  void* counters = take((size_t)nq * 4 * 4);
  if (a) {
    a->nblk = (int)nblk;
    a->scores = static_cast<uint32_t*>(scores);
    a->cand_key = static_cast<uint32_t*>(ckey);
    a->cand_idx = static_cast<int32_t*>(cidx);
    a->blk_bin = static_cast<int32_t*>(bins);
    a->counters = static_cast<uint32_t*>(counters);
  }
  return (size_t)(p - p0) + 256;
}

hipError_t index_init() {
  return hipFuncSetAttribute((const void*)finalize_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             kCandCap * 8);
}

hipError_t launch_index_topk(const IndexArgs& a, hipStream_t s) {
  const int64_t nclr = 4 * (int64_t)a.nq;
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)((nclr + 255) / 256)), dim3(256), 0, s, a.counters, nclr);
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
