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

__global__ __launch_bounds__(256) void clear_kernel(uint32_t* hist, uint32_t* counters, int nq) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nh = (int64_t)nq * kHistBins;
  if (i < nh) hist[i] = 0;
  else if (i < nh + 4 * nq) counters[i - nh] = 0;
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

// Wave-aggregated append: returns this lane's slot (only meaningful where pred is true).
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0) return 0;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((long long)mask) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
  base = __shfl(base, leader, 64);
  return base + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
}

// grid = (ceil(max(max_visible, k) / 4096), nq).
__global__ __launch_bounds__(256) void select_kernel(IndexArgs a) {
  __shared__ uint32_t sh[kHistBins];
  __shared__ uint32_t part[256];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  __shared__ int s_last;
  __shared__ uint32_t s_slot;
  __shared__ uint64_t s_prefix;
  __shared__ uint32_t s_rem;
  __shared__ int s_done;
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

  // 1. threshold bin: the largest bin b with sum_{b' >= b} hist[b'] >= K
  const uint32_t* gh = a.hist + (int64_t)qi * kHistBins;
  uint32_t loc = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sh[tid * 8 + i] = gh[tid * 8 + i];
    loc += sh[tid * 8 + i];
  }
  part[tid] = loc;
  __syncthreads();
  if (tid == 0) {
    uint32_t acc = 0;
    int t = 255;
    for (; t >= 0; --t) {
      if (acc + part[t] >= (uint32_t)K) break;
      acc += part[t];
    }
    int b = t * 8 + 7;
    for (; b >= t * 8; --b) {
      if (acc + sh[b] >= (uint32_t)K) break;
      acc += sh[b];
    }
    s_bin = b;
    s_above = acc;
  }
  __syncthreads();
  const uint32_t bstar = (uint32_t)s_bin, above = s_above;

  // 2. classify this block's scores
  uint32_t* cnt = a.counters + (int64_t)qi * 4;  // [0] selected, [1] candidates, [2] done blocks
  const float* sc = a.scores + (int64_t)qi * a.max_visible;
  uint64_t* cand = a.cand + (int64_t)qi * a.max_visible;
  for (int it = 0; it < kSelBlock / 256; ++it) {
    const int64_t j = j0 + it * 256 + tid;
    const bool valid = j < nv;
    const uint32_t key = valid ? float_key(sc[j]) : 0u;
    const uint32_t bin = key >> 21;
    const bool hi = valid && bin > bstar;
    const bool eq = valid && bin == bstar;
    const uint32_t s1 = wave_append(hi, &cnt[0]);
    if (hi) out[s1] = (int32_t)j;
    const uint32_t s2 = wave_append(eq, &cnt[1]);
    if (eq) cand[s2] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t nblk = (uint32_t)((nv + kSelBlock - 1) / kSelBlock);
    s_last = atomicAdd(&cnt[2], 1u) == nblk - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // 3. last block: radix-select the remaining `need` among the candidates (unique 64-bit keys)
  const uint32_t need = (uint32_t)K - above;
  const uint32_t nc = atomicAdd(&cnt[1], 0u);
  const volatile uint64_t* vc = cand;
  if (tid == 0) { s_prefix = 0; s_rem = need; s_done = 0; }
  __syncthreads();
  uint64_t thr = 0;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int i = tid; i < 256; i += 256) sh[i] = 0;
    __syncthreads();
    const uint64_t prefix = s_prefix;
    for (uint32_t i = tid; i < nc; i += 256) {
      const uint64_t key = vc[i];
      const bool match = pass == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8));
      if (match) atomicAdd(&sh[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t acc = 0, rem = s_rem;
      int d = 255;
      for (; d > 0; --d) {
        if (acc + sh[d] >= rem) break;
        acc += sh[d];
      }
      rem -= acc;
      s_prefix = prefix | ((uint64_t)d << shift);
      s_rem = rem;
      s_done = sh[d] == rem;
    }
    __syncthreads();
    if (s_done) { thr = s_prefix; break; }
  }
  if (tid == 0) s_slot = 0;
  __syncthreads();
  for (uint32_t i = tid; i < nc; i += 256) {
    const uint64_t key = vc[i];
    if (key >= thr) {
      const uint32_t slot = atomicAdd(&s_slot, 1u);
      out[above + slot] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
    }
  }
  __threadfence_block();
  __syncthreads();

  // 4. sort the k selected indices ascending (bitonic in LDS, padded with INT_MAX)
  int N = 1;
  while (N < K) N <<= 1;
  int32_t* buf = reinterpret_cast<int32_t*>(sh);
  volatile int32_t* vout = out;
  for (int i = tid; i < N; i += 256) buf[i] = i < K ? vout[i] : 0x7FFFFFFF;
  __syncthreads();
  for (int k2 = 2; k2 <= N; k2 <<= 1) {
    for (int jj = k2 >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < N; i += 256) {
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
  for (int i = tid; i < K; i += 256) out[i] = buf[i];
}

}  // namespace

size_t index_ws_per_query(int64_t max_visible) {
  const int64_t mv = (max_visible + 63) / 64 * 64;
  return (size_t)(mv * 4 + mv * 8 + (int64_t)kHistBins * 4 + 16);
}

hipError_t launch_index_topk(const IndexArgs& a, hipStream_t s) {
  const int64_t nclear = (int64_t)a.nq * (kHistBins + 4);
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)((nclear + 255) / 256)), dim3(256), 0, s, a.hist, a.counters, a.nq);
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
  hipLaunchKernelGGL(select_kernel, g, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hca
