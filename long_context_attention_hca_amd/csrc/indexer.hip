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
//  * Top-k is a radix select on 64-bit keys (order-preserving score bits << 32 |
//    ~j). The score kernel also builds, per query, a histogram of the top 11 key
//    bits (LDS per block, then global atomics). The select kernel finds the
//    threshold bin from that histogram, streams the scores once, emits every
//    entry above the bin directly and collects the bin's entries as candidates;
//    the last block of each query (device-scope counter) resolves the candidates
//    by 8-bit radix passes and sorts the k indices ascending.
#include "common.h"
#include "internal.h"

namespace hca {
namespace {

constexpr int kScoreBlockKeys = 1024;  // MXFP4 score kernel: 4 waves x 8 tiles x 32 keys
constexpr int kSelBlock = 4096;        // scores per select block

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

// Zeroes n words (the histograms and counters, laid out back to back in the workspace).
__global__ __launch_bounds__(256) void clear_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

__device__ __forceinline__ void flush_hist(uint32_t* lhist, uint32_t* ghist) {
  __syncthreads();
  for (int i = threadIdx.x; i < kHistBins; i += 256) {
    const uint32_t c = lhist[i];
    if (c) atomicAdd(&ghist[i], c);
  }
}

// MXFP4 scores via the scaled MFMA. grid = (ceil(max_visible / 1024), nq).
__global__ __launch_bounds__(256) void score_mxfp4_kernel(IndexArgs a) {
  __shared__ uint32_t lhist[kHistBins];
  const int qi = blockIdx.y;
  int64_t rb;
  const int64_t nv = visible_keys(a, qi, &rb);
  if (nv <= a.k) return;  // every visible entry is selected; no scores needed
  const int64_t jb = (int64_t)blockIdx.x * kScoreBlockKeys;
  if (jb >= nv) return;
  for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0;

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
  __syncthreads();

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
  float* scores = a.scores + (int64_t)qi * a.max_visible;
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
    const int64_t j = jb + (int64_t)(wave * U + u) * 32 + row;
    if (lane < 32 && j < nv) {
      float s = __fmul_rn(w[0], fmaxf(r[0], 0.f));
#pragma unroll
      for (int h = 1; h < 8; ++h)
        if (h < a.H) s = __fadd_rn(s, __fmul_rn(w[h], fmaxf(r[h], 0.f)));
      scores[j] = s;
      atomicAdd(&lhist[float_key(s) >> 21], 1u);
    }
  }
  flush_hist(lhist, a.hist + (int64_t)qi * kHistBins);
}

// fp32 / bf16 scores on the vector ALUs (one key per thread). grid = (ceil(max_visible/256), nq).
template <typename T>
__global__ __launch_bounds__(256) void score_valu_kernel(IndexArgs a) {
  __shared__ uint32_t lhist[kHistBins];
  __shared__ float qs[8 * 64];
  const int qi = blockIdx.y;
  int64_t rb;
  const int64_t nv = visible_keys(a, qi, &rb);
  if (nv <= a.k) return;
  const int64_t jb = (int64_t)blockIdx.x * 256;
  if (jb >= nv) return;
  for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0;
  const T* q = static_cast<const T*>(a.q) + (int64_t)qi * a.H * 64;
  for (int i = threadIdx.x; i < a.H * 64; i += 256) {
    if (sizeof(T) == 4) qs[i] = reinterpret_cast<const float*>(q)[i];
    else qs[i] = bf16_to_f32(reinterpret_cast<const uint16_t*>(q)[i]);
  }
  float w[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) w[h] = h < a.H ? a.w[(int64_t)qi * a.H + h] : 0.f;
  __syncthreads();
  const int64_t j = jb + threadIdx.x;
  if (j < nv) {
    const T* kp = static_cast<const T*>(a.keys) + (rb + j) * 64;
    float kv[64];
    if (sizeof(T) == 4) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float4 v = reinterpret_cast<const float4*>(kp)[i];
        kv[4 * i] = v.x; kv[4 * i + 1] = v.y; kv[4 * i + 2] = v.z; kv[4 * i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 v = reinterpret_cast<const uint4*>(kp)[i];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          kv[8 * i + 2 * c] = __uint_as_float(u[c] << 16);
          kv[8 * i + 2 * c + 1] = __uint_as_float(u[c] & 0xFFFF0000u);
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
    a.scores[(int64_t)qi * a.max_visible + j] = s;
    atomicAdd(&lhist[float_key(s) >> 21], 1u);
  }
  flush_hist(lhist, a.hist + (int64_t)qi * kHistBins);
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

// Over counters c[0..n) in LDS (n = 256 * per, per in {1, 4, 8}): the largest index d with
// sum_{i >= d} c[i] >= rem, and above = sum_{i > d} c[i]. Wave 0 must call it; the result is
// written to *d_out / *above_out (LDS) by one lane. Requires sum c >= rem >= 1.
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

// ---------------------------------------------------------------------------------------
// Classification: each block takes 4096 scores of one query, finds the threshold bin b* of the
// top-11-bit histogram (the bin holding the k-th largest), appends every entry above b* to the
// selected list and every entry in b* to the candidate lists, and histograms the candidates'
// next 11 key bits. grid = (ceil(max(max_visible, k) / 4096), nq), 256 threads.
__global__ __launch_bounds__(256) void classify_kernel(IndexArgs a) {
  __shared__ uint32_t sh[kHistBins];
  __shared__ uint32_t part[256];
  __shared__ uint32_t tmp[8];
  __shared__ int s_d, s_bin;
  __shared__ uint32_t s_above, s_above2, s_base[2];
  const int qi = blockIdx.y, tid = threadIdx.x;
  const int K = a.k;
  int64_t rb;
  const int64_t nv = visible_keys(a, qi, &rb);
  int32_t* out = a.out + (int64_t)qi * K;
  const int64_t j0 = (int64_t)blockIdx.x * kSelBlock;

  if (nv <= K) {  // all visible entries selected, ascending; pad with -1
    for (int64_t j = j0 + tid; j < min<int64_t>(j0 + kSelBlock, K); j += 256) out[j] = j < nv ? (int32_t)j : -1;
    return;
  }
  if (j0 >= nv) return;

  const uint32_t* gh = a.hist + (int64_t)qi * kHistBins;
  uint32_t loc = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h = gh[tid * 8 + i];
    sh[tid * 8 + i] = h;
    loc += h;
  }
  part[tid] = loc;
  // this block's scores, 16 per thread
  const float* sc = a.scores + (int64_t)qi * a.max_visible;
  uint32_t key[kSelBlock / 256];
#pragma unroll
  for (int it = 0; it < kSelBlock / 256; ++it) {
    const int64_t j = j0 + it * 256 + tid;
    key[it] = j < nv ? float_key(sc[j]) : 0u;
  }
  __syncthreads();
  if (tid < 64) find_crossing<1>(part, (uint32_t)K, &s_d, &s_above);
  __syncthreads();
  if (tid == s_d) {
    uint32_t acc = s_above;
    int b = 8 * tid + 7;
    for (; b > 8 * tid; --b) {
      if (acc + sh[b] >= (uint32_t)K) break;
      acc += sh[b];
    }
    s_bin = b;
  }
  __syncthreads();
  const uint32_t bstar = (uint32_t)s_bin;
  uint32_t nhi = 0, neq = 0;
#pragma unroll
  for (int it = 0; it < kSelBlock / 256; ++it) {
    const int64_t j = j0 + it * 256 + tid;
    const uint32_t bin = key[it] >> 21;
    nhi += (j < nv && bin > bstar);
    neq += (j < nv && bin == bstar);
  }
  uint32_t thi, teq;
  uint32_t ohi = block_exclusive_scan<256>(nhi, tmp, &thi);
  uint32_t oeq = block_exclusive_scan<256>(neq, tmp + 4, &teq);
  uint32_t* cnt = a.counters + (int64_t)qi * 4;
  if (tid == 0) {
    s_base[0] = thi ? atomicAdd(&cnt[0], thi) : 0u;
    s_base[1] = teq ? atomicAdd(&cnt[1], teq) : 0u;
  }
  for (int i = tid; i < kHistBins; i += 256) sh[i] = 0;
  __syncthreads();
  int32_t* sel = a.sel + (int64_t)qi * kMaxTopK;
  uint32_t* ck = a.cand_key + (int64_t)qi * a.max_visible;
  int32_t* ci = a.cand_idx + (int64_t)qi * a.max_visible;
  ohi += s_base[0];
  oeq += s_base[1];
#pragma unroll
  for (int it = 0; it < kSelBlock / 256; ++it) {
    const int64_t j = j0 + it * 256 + tid;
    const uint32_t bin = key[it] >> 21;
    if (j < nv && bin > bstar) sel[ohi++] = (int32_t)j;
    if (j < nv && bin == bstar) {
      ck[oeq] = key[it];
      ci[oeq] = (int32_t)j;
      ++oeq;
      atomicAdd(&sh[(key[it] >> 10) & 2047u], 1u);
    }
  }
  if (teq) flush_hist(sh, a.hist2 + (int64_t)qi * kHistBins);
}

// Finalisation, one block of 1024 threads per query. With T the 32-bit key of the k-th largest
// score (found from the second-level histogram and a third-level one over the candidates), the
// selection is: every entry above T, plus the r lowest-index entries whose key equals T. The
// selection is assembled in an LDS bitmap over the visible entries and compacted in ascending
// order. Beyond kBitmapBits visible entries a 64-bit radix select and a bitonic sort are used.
constexpr int kFinThreads = 1024;
constexpr int64_t kBitmapBits = 1 << 19;

__host__ __device__ __forceinline__ int64_t bitmap_words(int64_t nv) { return (nv + 31) >> 5; }

__global__ __launch_bounds__(kFinThreads) void finalize_kernel(IndexArgs a) {
  extern __shared__ uint32_t dyn[];
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t part[256];
  __shared__ uint32_t tmp[32];
  __shared__ int s_d, s_b;
  __shared__ uint32_t s_above, s_acc, s_cut_word, s_cut_bit;
  const int qi = blockIdx.x, tid = threadIdx.x;
  const int K = a.k;
  int64_t rb;
  const int64_t nv = visible_keys(a, qi, &rb);
  if (nv <= K) return;
  int32_t* out = a.out + (int64_t)qi * K;
  const uint32_t* cnt = a.counters + (int64_t)qi * 4;
  const uint32_t above = cnt[0], nc = cnt[1];
  const int32_t* sel = a.sel + (int64_t)qi * kMaxTopK;
  const uint32_t* ck = a.cand_key + (int64_t)qi * a.max_visible;
  const int32_t* ci = a.cand_idx + (int64_t)qi * a.max_visible;
  const uint32_t rem = (uint32_t)K - above;  // >= 1

  if (nv <= kBitmapBits) {
    // level 2: next 11 bits of the candidates
    const uint32_t* g2 = a.hist2 + (int64_t)qi * kHistBins;
    for (int i = tid; i < kHistBins; i += kFinThreads) h[i] = g2[i];
    __syncthreads();
    if (tid < 256) {
      uint32_t sum = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += h[8 * tid + i];
      part[tid] = sum;
    }
    __syncthreads();
    if (tid < 64) find_crossing<1>(part, rem, &s_d, &s_above);
    __syncthreads();
    if (tid == s_d) {
      uint32_t acc = s_above;
      int b = 8 * tid + 7;
      for (; b > 8 * tid; --b) {
        if (acc + h[b] >= rem) break;
        acc += h[b];
      }
      s_b = b;
      s_acc = acc;
    }
    __syncthreads();
    const uint32_t b2 = (uint32_t)s_b, rem2 = rem - s_acc;
    __syncthreads();
    // level 3: the last 10 bits of the candidates in (b*, b2)
    h[tid] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < nc; i += kFinThreads) {
      const uint32_t k32 = ck[i];
      if (((k32 >> 10) & 2047u) == b2) atomicAdd(&h[k32 & 1023u], 1u);
    }
    __syncthreads();
    if (tid < 64) find_crossing<4>(h, rem2, &s_d, &s_above);
    __syncthreads();
    const uint32_t b3 = (uint32_t)s_d, r = rem2 - s_above;  // r >= 1 entries with key == T
    const uint32_t T = nc ? ((ck[0] >> 21) << 21) | (b2 << 10) | b3 : 0u;
    // bitmaps: A = selection, B = entries whose key equals T
    const int64_t nw = bitmap_words(nv);
    uint32_t* A = dyn;
    uint32_t* Bm = dyn + nw;
    for (int64_t i = tid; i < 2 * nw; i += kFinThreads) dyn[i] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < above; i += kFinThreads) {
      const int32_t j = sel[i];
      atomicOr(&A[j >> 5], 1u << (j & 31));
    }
    for (uint32_t i = tid; i < nc; i += kFinThreads) {
      const uint32_t k32 = ck[i];
      const int32_t j = ci[i];
      if (k32 > T) atomicOr(&A[j >> 5], 1u << (j & 31));
      else if (k32 == T) atomicOr(&Bm[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    // the r lowest set bits of B join A: find the word holding the r-th set bit
    const int64_t per = (nw + kFinThreads - 1) / kFinThreads;
    const int64_t w0 = tid * per, w1 = min<int64_t>(nw, w0 + per);
    uint32_t pc = 0;
    for (int64_t w = w0; w < w1; ++w) pc += __popc(Bm[w]);
    uint32_t tot;
    uint32_t before = block_exclusive_scan<kFinThreads>(pc, tmp, &tot);
    if (before < r && before + pc >= r) {
      uint32_t acc = before;
      for (int64_t w = w0; w < w1; ++w) {
        const uint32_t c = __popc(Bm[w]);
        if (acc + c >= r) {
          // the (r - acc)-th set bit of this word
          uint32_t bits = Bm[w], need = r - acc;
          int bit = 0;
          for (int b = 0; b < 32; ++b) {
            if ((bits >> b) & 1u) {
              if (--need == 0) { bit = b; break; }
            }
          }
          s_cut_word = (uint32_t)w;
          s_cut_bit = (uint32_t)bit;
          break;
        }
        acc += c;
      }
    }
    __syncthreads();
    const uint32_t cw = s_cut_word, cb = s_cut_bit;
    for (int64_t w = w0; w < w1; ++w) {
      uint32_t bits = Bm[w];
      if ((uint32_t)w > cw) bits = 0;
      else if ((uint32_t)w == cw) bits &= (cb == 31) ? 0xFFFFFFFFu : ((2u << cb) - 1u);
      A[w] |= bits;
    }
    __syncthreads();
    // compaction in ascending order
    pc = 0;
    for (int64_t w = w0; w < w1; ++w) pc += __popc(A[w]);
    uint32_t pos = block_exclusive_scan<kFinThreads>(pc, tmp, &tot);
    for (int64_t w = w0; w < w1; ++w) {
      uint32_t bits = A[w];
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        if (pos < (uint32_t)K) out[pos] = (int32_t)(w * 32 + b);
        ++pos;
      }
    }
    return;
  }

  // Fallback for very long sequences: 64-bit keys (score key << 32 | ~j) of the candidates,
  // 8-bit radix passes over L2, then a bitonic sort of the k indices.
  uint64_t prefix = 0, thr = 0;
  uint32_t rr = rem;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    if (tid < 256) h[tid] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < nc; i += kFinThreads) {
      const uint64_t key = ((uint64_t)ck[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)ci[i]);
      const bool match = pass == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8));
      if (match) atomicAdd(&h[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) find_crossing<1>(h, rr, &s_d, &s_above);
    __syncthreads();
    const int d = s_d;
    rr -= s_above;
    prefix |= (uint64_t)d << shift;
    const bool done = h[d] == rr;
    __syncthreads();
    if (done) { thr = prefix; break; }
  }
  int32_t* buf = reinterpret_cast<int32_t*>(h);
  if (tid == 0) s_acc = 0;
  __syncthreads();
  for (uint32_t i = tid; i < above; i += kFinThreads) buf[i] = sel[i];
  for (uint32_t i = tid; i < nc; i += kFinThreads) {
    const uint64_t key = ((uint64_t)ck[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)ci[i]);
    if (key >= thr) buf[above + atomicAdd(&s_acc, 1u)] = ci[i];
  }
  __syncthreads();
  int N = 1;
  while (N < K) N <<= 1;
  for (int i = K + tid; i < N; i += kFinThreads) buf[i] = 0x7FFFFFFF;
  __syncthreads();
  for (int k2 = 2; k2 <= N; k2 <<= 1) {
    for (int jj = k2 >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < N; i += kFinThreads) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const int32_t x = buf[i], y = buf[ixj];
          const bool asc = (i & k2) == 0;
          if ((x > y) == asc) { buf[i] = y; buf[ixj] = x; }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < K; i += kFinThreads) out[i] = buf[i];
}

}  // namespace

size_t index_ws_layout(int64_t nq, int64_t max_visible, void* ws, IndexArgs* a) {
  const int64_t mv = (max_visible + 63) / 64 * 64;
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
  void* sel = take((size_t)nq * kMaxTopK * 4);
  void* hist = take((size_t)nq * kHistBins * 4);
  void* hist2 = take((size_t)nq * kHistBins * 4);
  void* counters = take((size_t)nq * 4 * 4);
  if (a) {
    a->scores = static_cast<float*>(scores);
    a->cand_key = static_cast<uint32_t*>(ckey);
    a->cand_idx = static_cast<int32_t*>(cidx);
    a->sel = static_cast<int32_t*>(sel);
    a->hist = static_cast<uint32_t*>(hist);
    a->hist2 = static_cast<uint32_t*>(hist2);
    a->counters = static_cast<uint32_t*>(counters);
  }
  return (size_t)(p - p0) + 256;
}

hipError_t index_init() {
  return hipFuncSetAttribute((const void*)finalize_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)(2 * bitmap_words(kBitmapBits) * 4));
}

hipError_t launch_index_topk(const IndexArgs& a, hipStream_t s) {
  // clear both histograms and the counters (laid out back to back by index_ws_layout)
  const int64_t nclr = (a.counters + 4 * (int64_t)a.nq) - a.hist;
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)((nclr + 255) / 256)), dim3(256), 0, s, a.hist, nclr);
  if (a.max_visible > a.k) {
    if (a.dtype == HCA_MXFP4) {
      const dim3 g((unsigned)((a.max_visible + kScoreBlockKeys - 1) / kScoreBlockKeys), (unsigned)a.nq);
      hipLaunchKernelGGL(score_mxfp4_kernel, g, dim3(256), 0, s, a);
    } else if (a.dtype == HCA_F32) {
      const dim3 g((unsigned)((a.max_visible + 255) / 256), (unsigned)a.nq);
      hipLaunchKernelGGL(score_valu_kernel<float>, g, dim3(256), 0, s, a);
    } else {
      const dim3 g((unsigned)((a.max_visible + 255) / 256), (unsigned)a.nq);
      hipLaunchKernelGGL(score_valu_kernel<uint16_t>, g, dim3(256), 0, s, a);
    }
  }
  const int64_t span = a.max_visible > a.k ? a.max_visible : a.k;
  const dim3 g((unsigned)((span + kSelBlock - 1) / kSelBlock), (unsigned)a.nq);
  hipLaunchKernelGGL(classify_kernel, g, dim3(256), 0, s, a);
  if (a.max_visible > a.k) {
    const int64_t mvb = a.max_visible < kBitmapBits ? a.max_visible : kBitmapBits;
    const size_t lds = (size_t)(2 * bitmap_words(mvb) * 4);
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)a.nq), dim3(kFinThreads), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace hca
