// CSA sparse and HCA dense MQA core attention with the sliding-window branch, gfx950.
//
// Method: hyper.ai paper page for arXiv 2606.19348 ("DeepSeek-V4"), section 方法
// (Method). CSA paragraph: MQA with shared keys and values over the top-k
// compressed entries; HCA paragraph: dense attention over all heavily compressed
// entries, both with a supplementary sliding-window branch. Per query and head,
// one softmax runs over the union of the compressed entries and the raw window
// tokens (the log-sum-exp merge of the two branches), with K = V = the stored
// row; scores are scale * <q_h, e>.
//
// Each query's entry list is: compressed part (CSA: idx[q, r], r < k, skipping
// -1; HCA: entries 0 .. n_vis-1), then window positions t-n_w+1 .. t. The list is
// cut into n_split ranges (split-K); each block writes a normalised partial
// (o, lse) that a combine kernel merges, or the final output when n_split == 1.
//
// MFMA kernel (bf16 queries; bf16 or split FP8/bf16 stores; D = 512):
//  * block = (query, group of 16 heads, split); its 4 waves take the split's
//    32-entry chunks round-robin and keep independent online-softmax states that
//    are merged through LDS at the end. The 4 head-group blocks of one range are
//    adjacent after the XCD remap, so their entry reads share one XCD's L2.
//  * a wave stages its chunk in LDS as bf16 rows (FP8 codes times the entry's
//    power-of-two scale via v_cvt_scalef32_pk_bf16_fp8, exact), rows padded by
//    16 bytes so the operand reads below are bank-conflict free.
//  * scores S^T = K Q^T with v_mfma_f32_16x16x32_bf16: entries are the M
//    dimension and the 16 heads the N dimension, so each lane's accumulators all
//    belong to one head and the online softmax needs only two cross-lane maxima.
//  * O^T = V^T P^T: P^T is taken straight from the score accumulators (the
//    contraction order of the 32 entries is permuted identically on both
//    operands), and V^T tiles come from ds_read_b64_tr_b16 transpose reads of the
//    row-major chunk.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "internal.h"
#include "topk_select.h"

namespace hca {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct QueryCtx {
  int64_t t, n_c, n_w, cache_rb, win_rb, win_p0;
};

// With a document mask (lo > 0) the window starts at lo at the earliest and HCA skips the
// entries j < ceil(lo / m') whose window starts before lo: the cache rows then begin j_lo
// rows later (CSA's selected entries come from the indexer, which applies the mask).
__device__ __forceinline__ QueryCtx query_ctx(const AttnArgs& a, int qi) {
  QueryCtx c;
  const int b = a.q_seq[qi];
  c.t = a.q_pos[qi];
  const int64_t lo = a.q_lo ? max<int64_t>(a.q_lo[qi], 0) : 0;
  int64_t j_lo = 0;
  if (a.idx) {
    c.n_c = a.k;
  } else {
    int64_t nv = c.t >= 0 ? (c.t + 1) / a.m_prime : 0;
    if (lo > 0) j_lo = (lo + a.m_prime - 1) / a.m_prime;  // no division on the common path
    c.n_c = max<int64_t>(min(nv, a.max_visible) - j_lo, 0);
  }
  c.n_w = c.t >= 0 ? max<int64_t>(min<int64_t>(a.W, c.t + 1 - lo), 0) : 0;  // positions max(lo, t-W+1) .. t
  c.cache_rb = a.cache_row_begin[b] + j_lo;
  c.win_rb = a.win_row_begin[b];
  c.win_p0 = a.win_pos0[b];
  return c;
}

// Row of list position r, or -1 (padding / outside the stores). *win set for window rows.
__device__ __forceinline__ int64_t list_row(const AttnArgs& a, const QueryCtx& c, int qi, int64_t r, bool* win) {
  if (r < c.n_c) {
    *win = false;
    int64_t j = r;
    if (a.idx) {
      j = a.idx[(int64_t)qi * a.k + r];
      if (j < 0) return -1;
    }
    const int64_t row = c.cache_rb + j;
    return (row >= 0 && row < a.cache.n_rows) ? row : -1;
  }
  *win = true;
  if (r >= c.n_c + c.n_w) return -1;
  const int64_t p = c.t - c.n_w + 1 + (r - c.n_c);
  const int64_t row = c.win_rb + (p - c.win_p0);
  return (row >= 0 && row < a.win.n_rows) ? row : -1;
}

// ---------------------------------------------------------------------------------------
// float32 path (vector ALUs): block = (query, split), 256 threads, 16-entry chunks in LDS.
constexpr int kValuChunk = 16;

__device__ __forceinline__ float load_f32(const StoreView& v, int64_t row, int d) {
  return static_cast<const float*>(v.data)[row * v.row_stride + d];
}

__global__ __launch_bounds__(256) void attn_valu_kernel(AttnArgs a) {
  extern __shared__ float smem_f[];
  const int H = a.H, D = a.D;
  float* qs = smem_f;                       // [H*D]
  float* ent = qs + H * D;                  // [16][D]
  float* pr = ent + kValuChunk * D;         // [H][16]
  float* mrun = pr + H * kValuChunk;        // [H]
  float* lrun = mrun + H;                   // [H]
  float* corr = lrun + H;                   // [H]
  __shared__ int valid[kValuChunk];
  const int qi = blockIdx.y, s = blockIdx.x, tid = threadIdx.x;
  const QueryCtx c = query_ctx(a, qi);
  const int64_t N = c.n_c + c.n_w;
  const int64_t lo = (int64_t)s * a.per_split, hi = min<int64_t>(N, lo + a.per_split);
  const float* q = static_cast<const float*>(a.q) + (int64_t)qi * H * D;
  for (int i = tid; i < H * D; i += 256) qs[i] = q[i];
  for (int h = tid; h < H; h += 256) { mrun[h] = -INFINITY; lrun[h] = 0.f; }
  constexpr int kMaxOut = 32;  // H*D <= 8192
  float O[kMaxOut];
#pragma unroll
  for (int i = 0; i < kMaxOut; ++i) O[i] = 0.f;
  const float sc = a.scale;
  __syncthreads();
  for (int64_t base = lo; base < hi; base += kValuChunk) {
    if (tid < kValuChunk) {
      bool w;
      const int64_t r = base + tid;
      valid[tid] = r < hi ? (int)(list_row(a, c, qi, r, &w) >= 0) : 0;
    }
    for (int i = tid; i < kValuChunk * D; i += 256) {
      const int e = i / D, d = i % D;
      bool w;
      const int64_t r = base + e;
      const int64_t row = r < hi ? list_row(a, c, qi, r, &w) : -1;
      ent[i] = row >= 0 ? load_f32(w ? a.win : a.cache, row, d) : 0.f;
    }
    __syncthreads();
    for (int i = tid; i < H * kValuChunk; i += 256) {
      const int h = i / kValuChunk, e = i % kValuChunk;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(qs[h * D + d], ent[e * D + d], acc);
      pr[i] = valid[e] ? acc * sc : -INFINITY;
    }
    __syncthreads();
    for (int h = tid; h < H; h += 256) {
      float mx = -INFINITY;
      for (int e = 0; e < kValuChunk; ++e) mx = fmaxf(mx, pr[h * kValuChunk + e]);
      const float mo = mrun[h], mn = fmaxf(mo, mx);
      const float cr = mn == -INFINITY ? 1.f : expf(mo - mn);
      float sum = 0.f;
      for (int e = 0; e < kValuChunk; ++e) {
        const float p = mn == -INFINITY ? 0.f : expf(pr[h * kValuChunk + e] - mn);
        pr[h * kValuChunk + e] = p;
        sum += p;
      }
      lrun[h] = lrun[h] * cr + sum;
      mrun[h] = mn;
      corr[h] = cr;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxOut; ++k) {
      const int i = tid + 256 * k;
      if (i < H * D) {
        const int h = i / D, d = i % D;
        float acc = O[k] * corr[h];
        for (int e = 0; e < kValuChunk; ++e) acc = fmaf(pr[h * kValuChunk + e], ent[e * D + d], acc);
        O[k] = acc;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < kMaxOut; ++k) {
    const int i = tid + 256 * k;
    if (i < H * D) {
      const int h = i / D, d = i % D;
      const float l = lrun[h];
      const float o = l > 0.f ? O[k] / l : 0.f;
      if (a.n_split == 1) {
        static_cast<float*>(a.o)[(int64_t)qi * H * D + i] = o;
        if (d == 0) a.lse[(int64_t)qi * H + h] = l > 0.f ? mrun[h] + logf(l) : -INFINITY;
      } else {
        const int64_t pi = ((int64_t)qi * a.n_split + s) * H + h;
        a.part_o[pi * D + d] = o;
        if (d == 0) a.part_lse[pi] = l > 0.f ? mrun[h] + logf(l) : -INFINITY;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// MFMA path.
constexpr int kD = 512;
constexpr int kChunk = 32;
constexpr int kRowB = kD * 2 + 16;           // padded bf16 row in LDS
constexpr int kWaveLds = kChunk * kRowB;      // 33,280 bytes per wave
constexpr int kMfmaLds = 4 * kWaveLds;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 8 consecutive dims [8*seg, 8*seg+8) of a stored row as 8 bf16 (16 bytes).
__device__ __forceinline__ uint4 load_seg8(const StoreView& v, int64_t row, int seg) {
  const int d0 = seg * 8;
  if (v.layout == HCA_LAYOUT_BF16) {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(v.data) + row * v.row_stride + d0);
  }
  if (d0 < v.d_nope) {
    const uint2 b = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(v.data) + row * v.row_stride + d0);
    const float sc = v.scale[row];
    const bf16x2 r0 = fp8x2_to_bf16x2(b.x, sc, false), r1 = fp8x2_to_bf16x2(b.x, sc, true);
    const bf16x2 r2 = fp8x2_to_bf16x2(b.y, sc, false), r3 = fp8x2_to_bf16x2(b.y, sc, true);
    uint4 o;
    o.x = __builtin_bit_cast(uint32_t, r0); o.y = __builtin_bit_cast(uint32_t, r1);
    o.z = __builtin_bit_cast(uint32_t, r2); o.w = __builtin_bit_cast(uint32_t, r3);
    return o;
  }
  return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(v.rope) + row * v.rope_stride + (d0 - v.d_nope));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Work item id < total of an attn_mfma grid: (query, split, 16-head group); smem is the
// block's kMfmaLds bytes of dynamic LDS.
__device__ __forceinline__ void attn_mfma_block(const AttnArgs& a, int n_hg, int id, uint8_t* smem) {
  const int hg = id % n_hg;
  const int rest = id / n_hg;
  const int s = rest % a.n_split;
  const int qi = rest / a.n_split;
  const int H = a.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int head = hg * 16 + c;
  uint8_t* lds = smem + wave * kWaveLds;

  const QueryCtx ctx = query_ctx(a, qi);
  const int64_t N = ctx.n_c + ctx.n_w;
  const int64_t lo = (int64_t)s * a.per_split;
  const int64_t hi = min<int64_t>(N, lo + a.per_split);

  // Q^T operand (B of S^T = K Q^T): lane holds Q[head][32ks + 8g .. +8).
  bf16x8 qv[kD / 32];
  const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)qi * H + head) * kD + 8 * g;
#pragma unroll
  for (int ks = 0; ks < kD / 32; ++ks)
    qv[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 32 * ks));

  f32x4 O[kD / 16];
#pragma unroll
  for (int i = 0; i < kD / 16; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  // both stores bf16 rows of 512 dims: rows go to LDS unconverted, by DMA
  const bool dense_bf16 = a.cache.layout == HCA_LAYOUT_BF16 && a.win.layout == HCA_LAYOUT_BF16;

  for (int64_t base = lo + (int64_t)wave * kChunk; base < hi; base += 4 * kChunk) {
    // rows of the chunk: lane e < 32 resolves list position base + e once; the wave then
    // stages the 32 rows as bf16 (lane = 16-byte segment of dims 8*lane .. +8), 8 rows in flight
    int64_t myrow = -1;
    bool mywin = false;
    if (lane < kChunk) {
      const int64_t r = base + lane;
      myrow = r < hi ? list_row(a, ctx, qi, r, &mywin) : -1;
    }
    const uint64_t vmask = __ballot(lane < kChunk && myrow >= 0);
    const uint64_t wmask = __ballot(lane < kChunk && mywin);
    const int row_lo = (int)(uint32_t)myrow, row_hi = (int)((uint64_t)myrow >> 32);
    if (dense_bf16) {
      // bf16 rows are 64 lanes x 16 bytes: one LDS DMA per valid row, all 32 requested before
      // one wait. The waits are explicit: hipcc does not order reads of this dynamically sized
      // LDS after the DMAs into it. The previous chunk's reads of these rows are done first.
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        uint8_t* dst = lds + e * kRowB;
        if ((vmask >> e) & 1) {
          const int64_t row = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(row_hi, e) << 32) |
                                        (uint64_t)(uint32_t)__builtin_amdgcn_readlane(row_lo, e));
          const StoreView& v = ((wmask >> e) & 1) ? a.win : a.cache;
          const uint16_t* src = static_cast<const uint16_t*>(v.data) + row * v.row_stride + 8 * lane;
          __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        } else {
          *reinterpret_cast<uint4*>(dst + lane * 16) = make_uint4(0, 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the rows have landed
    } else {
#pragma unroll
      for (int e0 = 0; e0 < kChunk; e0 += 8) {
        uint4 val[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = e0 + u;
          const int64_t row = (int64_t)(((uint64_t)(uint32_t)__shfl(row_hi, e, 64) << 32) |
                                        (uint64_t)(uint32_t)__shfl(row_lo, e, 64));
          val[u] = make_uint4(0, 0, 0, 0);
          if ((vmask >> e) & 1) val[u] = load_seg8(((wmask >> e) & 1) ? a.win : a.cache, row, lane);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) *reinterpret_cast<uint4*>(lds + (e0 + u) * kRowB + lane * 16) = val[u];
      }
    }
    // validity of the 8 entries this lane scores: 16mt + 4g + i
    bool vld[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) vld[mt][i] = (vmask >> (16 * mt + 4 * g + i)) & 1;
    wave_lds_sync();

    // S^T = K Q^T
    f32x4 st[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* rowp = lds + (16 * mt + c) * kRowB + 16 * g;
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks) {
        const bf16x8 kv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rowp + 64 * ks));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv[ks], acc, 0, 0, 0);
      }
      st[mt] = acc;
    }
    // online softmax (log2 domain); lanes c, c+16, c+32, c+48 share head c
    float sv[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[4 * mt + i] = vld[mt][i] ? st[mt][i] * sl2 : -INFINITY;
        cmax = fmaxf(cmax, sv[4 * mt + i]);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float m_new = fmaxf(m_run, cmax);
    const bool none = m_new == -INFINITY;
    const float corr = none ? 1.f : exp2f(m_run - m_new);
    float p[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = none ? 0.f : exp2f(sv[i] - m_new);
      psum += p[i];
    }
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < kD / 16; ++dt) O[dt] *= corr;
    // P^T operand: contraction order [4g..4g+3, 16+4g..16+4g+3]
    const uint4 pu = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pu);
    // O^T += V^T P^T; V^T via transpose reads: lane (4r + qd) of group g reads
    // row 4g + r (and 16 + 4g + r), dims 16dt + 4qd .. +4.
    const int rsel = c >> 2, qd = c & 3;
    const uint8_t* v0 = lds + (4 * g + rsel) * kRowB + 8 * qd;
    const uint8_t* v1 = v0 + 16 * kRowB;
#pragma unroll
    for (int dt = 0; dt < kD / 16; ++dt) {
      const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + 32 * dt));
      const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v1 + 32 * dt));
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 av = __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7);
      O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pb, O[dt], 0, 0, 0);
    }
    wave_lds_sync();
  }

  // per-head totals over the 4 lane groups
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  // merge the 4 waves through LDS: region of wave w = [m(16) | l(16) | O 16 x 512 fp32]
  float* wm = reinterpret_cast<float*>(lds);
  float* wl = wm + 16;
  float* wo = wl + 16;
  if (g == 0) { wm[c] = m_run; wl[c] = l_run; }
#pragma unroll
  for (int dt = 0; dt < kD / 16; ++dt)
    *reinterpret_cast<f32x4*>(wo + c * kD + 16 * dt + 4 * g) = O[dt];
  __syncthreads();

  // thread -> head hc = tid / 16, dims 4 * (tid % 16) + 64 * k
  const int hc = tid >> 4, dl = (tid & 15) * 4;
  float mw[4], fw[4];
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = reinterpret_cast<const float*>(smem + w * kWaveLds)[hc];
    M = fmaxf(M, mw[w]);
  }
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    fw[w] = mw[w] == -INFINITY ? 0.f : exp2f(mw[w] - M);
    L += fw[w] * reinterpret_cast<const float*>(smem + w * kWaveLds)[16 + hc];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const float lse = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  const int hd = hg * 16 + hc;
#pragma unroll
  for (int k = 0; k < kD / 64; ++k) {
    const int d = dl + 64 * k;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x4 ow = *reinterpret_cast<const f32x4*>(
          reinterpret_cast<const float*>(smem + w * kWaveLds) + 32 + hc * kD + d);
      acc += ow * fw[w];
    }
    acc *= inv;
    if (a.n_split == 1) {
      const int64_t oi = ((int64_t)qi * H + hd) * kD + d;
      if (a.o_dtype == HCA_BF16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + oi) =
            make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + oi) = acc;
      }
    } else {
      const int64_t pi = ((int64_t)qi * a.n_split + s) * H + hd;
      *reinterpret_cast<f32x4*>(a.part_o + pi * kD + d) = acc;
    }
  }
  if ((tid & 15) == 0) {
    if (a.n_split == 1) a.lse[(int64_t)qi * H + hd] = lse;
    else a.part_lse[((int64_t)qi * a.n_split + s) * H + hd] = lse;
  }
}

__global__ __launch_bounds__(256, 1) void attn_mfma_kernel(AttnArgs a, int n_hg, int total) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  if (id >= total) return;
  attn_mfma_block(a, n_hg, id, smem);
}

// The indexer's top-k selection and an HCA attention call on bf16 stores in one grid, as
// select_attn_fp8_kernel for the FP8 stores: blocks b < n_sel (a multiple of 8) select query b
// of `sel` (b < sel.nq) with the selection's 256-thread variant, the others are the attention
// call's blocks b - n_sel; the selection's LDS lies in the attention's dynamic LDS.
constexpr int kSelOutOff = 32768;  // OutLds of the selection after its FinLdsT<256>
static_assert(sizeof(FinLdsT<256>) <= kSelOutOff && kSelOutOff + sizeof(OutLds) <= kMfmaLds,
              "selection LDS inside the bf16 attention's LDS");
__global__ __launch_bounds__(256, 1) void select_attn_mfma_kernel(IndexArgs sel, int n_sel, AttnArgs a, int n_hg,
                                                                  int total) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int b = blockIdx.x;
  if (b >= n_sel) {
    const int id = xcd_remap(b - n_sel, (int)gridDim.x - n_sel);
    if (id < total) attn_mfma_block(a, n_hg, id, smem);
    return;
  }
  if (b < sel.nq)
    finalize_block(sel, b, *reinterpret_cast<FinLdsT<256>*>(smem), *reinterpret_cast<OutLds*>(smem + kSelOutOff));
}

// ---------------------------------------------------------------------------------------
// MFMA path for split stores (FP8 E4M3 non-RoPE dims + power-of-two scale + bf16 RoPE dims,
// 448 + 64), cache and window alike. block = (query, group of 16 heads, split), 8 waves:
//  * the split's list is walked in chunks of 128 entries staged in LDS as FP8 rows (double
//    buffered); wave w stages and scores entries 16w .. 16w+15 of every chunk, one
//    global_load_lds per row (36 lanes x 16 bytes: 448 FP8 bytes, then 128 RoPE bytes);
//  * S^T = K Q^T runs on v_mfma_scale_f32_16x16x128_f8f6f4 with the FP8 rows as stored: the
//    bf16 query is split into an FP8 high part and an FP8 residual, each with power-of-two
//    scales per 32 dims, so hi + lo carries the query to about 2^-8 relative; the entry's
//    scale multiplies the FP8 part of the score and the RoPE dims use
//    v_mfma_f32_16x16x32_bf16;
//  * the online softmax keeps one reference maximum per head for the whole block (the
//    waves' chunk maxima meet in LDS), and P goes to LDS in bf16, with and without the entry
//    scales;
//  * O^T += V^T P^T is split by output dims: wave w owns dims 64w .. 64w+63 over all 128
//    entries of the chunk (waves 0-6 the FP8 dims, read with ds_read_b64_tr_b8 and converted
//    to bf16; wave 7 the RoPE dims, read with ds_read_b64_tr_b16), so O is never merged
//    across waves.
constexpr int kNope = 448;
constexpr int kRope = 64;
constexpr int kRowF8 = 592;                 // 448 FP8 + 128 RoPE + 16 pad: conflict-free row reads
constexpr int kCh = 128;                    // entries per chunk
constexpr int kBufF8 = kCh * kRowF8;        // 75,776 bytes
constexpr int kPRow = kCh + 8;              // bf16 per P row (padded)
constexpr int kPBytes = 16 * kPRow * 2;     // 4,352 bytes
constexpr int kF8Lds = 2 * kBufF8 + 2 * kPBytes + 2 * 8 * 16 * 4;  // 161,280 bytes
static_assert(kF8Lds <= 160 * 1024, "LDS");

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;

__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = fp8x2_to_bf16x2(lo, 1.0f, false), b = fp8x2_to_bf16x2(lo, 1.0f, true);
  const bf16x2 c = fp8x2_to_bf16x2(hi, 1.0f, false), d = fp8x2_to_bf16x2(hi, 1.0f, true);
  uint4 u;
  u.x = __builtin_bit_cast(uint32_t, a); u.y = __builtin_bit_cast(uint32_t, b);
  u.z = __builtin_bit_cast(uint32_t, c); u.w = __builtin_bit_cast(uint32_t, d);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t x, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Row sources of one wave's R (16, or 8 in the wide kernel) entries of a chunk (list positions
// base + e, e < R).
struct WaveRows {
  uint64_t src;    // lane e < R: FP8-row address of entry e; lane R + e: its RoPE-row address
                   // minus 448, so that LDS row byte o >= 448 comes from src + o
  float esc;       // lane e < R: entry scale (its load is left in flight)
  uint32_t vmask;  // valid entries
};

// Zero: the entry scale that lanes without a row read in the wide kernel's wave_rows.
__device__ float g_zero_scale;

// The top-k slot value of list position base + (lane & 15) (CSA), loaded one chunk before its
// rows are computed so that no wait on it sits behind row loads in flight. Positions past the
// top-k list are clamped to a valid slot; their value is not used.
template <bool kSparse, int R = 16>
__device__ __forceinline__ int32_t prefetch_slot(const AttnArgs& a, int qi, int64_t base, int lane) {
  if (!kSparse) return 0;
  const int64_t r = min<int64_t>(base + (lane & (R - 1)), (int64_t)a.k - 1);
  return a.idx[(int64_t)qi * a.k + r];
}

// The rows of positions base .. base + R - 1 from their prefetched slot values (no dependent
// loads; the entry-scale load is issued and left in flight). Store fields are selected one by
// one so that they stay in scalar registers.
template <bool kSparse, int R = 16>
__device__ __forceinline__ WaveRows wave_rows(const AttnArgs& a, const QueryCtx& ctx, int64_t base, int64_t hi,
                                              int32_t slot, int lane) {
  WaveRows w;
  const int e = lane & (R - 1);
  const int64_t r = base + e;
  const bool win = r >= ctx.n_c;
  int64_t row = -1;
  if (lane < 2 * R && r < hi) {
    if (!win) {
      const int64_t j = kSparse ? (int64_t)slot : r;
      const int64_t cr = ctx.cache_rb + j;
      row = (j >= 0 && cr >= 0 && cr < a.cache.n_rows) ? cr : -1;
    } else if (r < ctx.n_c + ctx.n_w) {
      const int64_t pos = ctx.t - ctx.n_w + 1 + (r - ctx.n_c);
      const int64_t wr = ctx.win_rb + (pos - ctx.win_p0);
      row = (wr >= 0 && wr < a.win.n_rows) ? wr : -1;
    }
  }
  const uint64_t data = win ? reinterpret_cast<uint64_t>(a.win.data) : reinterpret_cast<uint64_t>(a.cache.data);
  const uint64_t rope = win ? reinterpret_cast<uint64_t>(a.win.rope) : reinterpret_cast<uint64_t>(a.cache.rope);
  const int64_t rs = win ? a.win.row_stride : a.cache.row_stride;
  const int64_t ps = win ? a.win.rope_stride : a.cache.rope_stride;
  const float* scale = win ? a.win.scale : a.cache.scale;
  w.src = lane < R ? data + (uint64_t)(row * rs) : rope + (uint64_t)(row * ps * 2) - kNope;
  if constexpr (R == 8) {
    // one unconditional load (lanes without a row read g_zero_scale): the wide kernel counts
    // the loads it issues after its DMAs
    w.esc = *((lane < R && row >= 0) ? scale + row : &g_zero_scale);
  } else {
    w.esc = (lane < R && row >= 0) ? scale[row] : 0.f;
  }
  w.vmask = (uint32_t)__ballot(lane < R && row >= 0);
  return w;
}

// Invalid rows of a wave's 16 are zeroed so that their (masked) P = 0 never meets a NaN; this
// precedes the row loads into the same buffer.
template <int R = 16>
__device__ __forceinline__ void zero_invalid_rows(const WaveRows& w, uint8_t* dst, int lane) {
  uint32_t inval = ~w.vmask & ((1u << R) - 1u);
  while (inval) {
    const int e = __builtin_ctz(inval);
    inval &= inval - 1;
    if (lane < kRowF8 / 16) *reinterpret_cast<uint4*>(dst + e * kRowF8 + 16 * lane) = make_uint4(0, 0, 0, 0);
  }
}

// A wave's 16 rows fill 16 * 592 = 9,472 LDS bytes, loaded by 10 lane-linear DMAs of up to
// 1 KiB (16 bytes a lane); DMAs I0 .. I0 + kN - 1 here (8 rows: 5 DMAs). The cost of a DMA is
// per instruction, not per byte, so full 64-lane DMAs beat one 36-lane DMA per row. Lanes that
// fall on a row's 16 padding bytes, past the R rows, or on an invalid row stay idle.
template <int I0, int kN, int R = 16>
__device__ __forceinline__ void stage_rows(const WaveRows& w, uint8_t* dst, int lane) {
#pragma unroll
  for (int i = I0; i < I0 + kN; ++i) {
    const int b = 1024 * i + 16 * lane;  // LDS byte within the wave's rows
    const int e = b / kRowF8, o = b - e * kRowF8;
    const int sl = o < kNope ? e : R + e;
    const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)w.src, sl, 64);
    const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(w.src >> 32), sl, 64);
    const uint64_t src = (((uint64_t)hi << 32) | lo) + (uint64_t)o;
    if (e < R && o < kNope + 2 * kRope && ((w.vmask >> (e & (R - 1))) & 1))
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                       (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, 0, 0);
  }
}

// Dense calls (HCA): a wave's R rows from list position p0 are consecutive cache rows, all
// valid, when they end before the split and the cache part of the list and lie inside the
// store (a uniform test; away from the window and the store's end this holds for every chunk).
// Their DMA sources then follow from the store's bases, the row and the lane's byte offset,
// with no shuffle of per-row addresses, and their row sources are just the entry scales.
template <int R>
__device__ __forceinline__ bool dense_run(const AttnArgs& a, const QueryCtx& ctx, int64_t p0, int64_t hi,
                                          int64_t* row0) {
  const int64_t r0 = ctx.cache_rb + p0;
  *row0 = r0;
  return p0 + R <= min(hi, ctx.n_c) && r0 >= 0 && r0 + R <= a.cache.n_rows;
}

// stage_rows<I0, kN, R> for a dense run starting at cache row row0 (all R rows valid).
template <int I0, int kN, int R>
__device__ __forceinline__ void stage_dense(const AttnArgs& a, int64_t row0, uint8_t* dst, int lane_in) {
  // the lane-only offsets come from an opaque copy of the lane index, so that they are
  // recomputed at each call instead of being kept live (and spilled) across the chunk loop
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  // the run's first row is the same in every lane: its part bases are scalar
  const int64_t r0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(row0 >> 32)) << 32) |
                               (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)row0));
  const int64_t rs = a.cache.row_stride, rps = 2 * a.cache.rope_stride;
  const uint64_t fp8 = reinterpret_cast<uint64_t>(a.cache.data) + (uint64_t)(r0 * rs);
  const uint64_t rope = reinterpret_cast<uint64_t>(a.cache.rope) + (uint64_t)(r0 * rps) - kNope;
  // a lane's byte offset from its part's base (rows e < R of the run) fits in 32 bits: the
  // strides are bounded on the host, so only the base is 64-bit
  const uint32_t rs32 = (uint32_t)rs, rps32 = (uint32_t)rps;
#pragma unroll
  for (int i = I0; i < I0 + kN; ++i) {
    const int b = 1024 * i + 16 * lane;  // LDS byte within the wave's rows
    const int e = b / kRowF8, o = b - e * kRowF8;
    const bool nope = o < kNope;
    const uint32_t off = (uint32_t)e * (nope ? rs32 : rps32) + (uint32_t)o;
    const uint64_t src = (nope ? fp8 : rope) + (uint64_t)off;
    if (e < R && o < kNope + 2 * kRope)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                       (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, 0, 0);
  }
}

// wave_rows<false, R> for a dense run starting at cache row row0: src is unused (stage_dense
// computes the sources), the scales of the R entries are requested and left in flight. Every
// lane loads (lane e + R i holds entry e's scale; only lanes below R are read), so the load is
// one unconditional instruction.
template <int R>
__device__ __forceinline__ WaveRows dense_rows(const AttnArgs& a, int64_t row0, int lane) {
  WaveRows w;
  w.src = 0;
  w.esc = a.cache.scale[row0 + (lane & (R - 1))];
  w.vmask = (1u << R) - 1u;
  return w;
}

// Workgroup barrier that waits for this wave's LDS accesses only: row loads into the other
// chunk buffer stay in flight across it. The signal fences stop the compiler from moving LDS
// accesses over the barrier.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left alone
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

struct F8Query {
  i32x8 qh[4], ql[4];  // FP8 hi / lo parts of the 448 non-RoPE dims, per K step
  bf16x8 qr[2];        // RoPE dims
  uint32_t sh, sl;     // per K step scale byte (E8M0) of the hi / lo parts
};

struct F8State {
  f32x4 O[4];
  float m_run, l_part;
  WaveRows cur, nxt;  // rows of this chunk (staged) and of the next one (known)
  int32_t slot2;      // prefetched slot values of the chunk after next
};

// One 128-entry chunk in buf, whose rows this wave has requested: wait for all of them, request
// the next chunk's rows into nbuf (spread over this chunk's phases), then scores, softmax and
// PV. The chunk buffers are distinct LDS objects, so the compiler knows that reads of buf need
// not wait for the loads into nbuf.
template <bool kSparse>
__device__ __forceinline__ void f8_chunk(const AttnArgs& a, const QueryCtx& ctx, int qi, int64_t base, int64_t hi,
                                         const uint8_t* buf, uint8_t* nbuf, const F8Query& q, F8State& st,
                                         uint16_t* pbs, uint16_t* pb, float* wmax, float sl2, int wave, int lane) {
  const int g = lane >> 4, c = lane & 15;
  __builtin_amdgcn_s_waitcnt(0);  // this chunk's rows staged by this wave; next rows' loads done
  __syncthreads();                // all rows of the chunk; the other buffer is free
  const bool more = base + kCh < hi;
  const WaveRows cur = st.cur, nxt = st.nxt;
  uint8_t* ndst = nbuf + 16 * wave * kRowF8;
  if (more) {
    zero_invalid_rows(nxt, ndst, lane);
    stage_rows<0, 3>(nxt, ndst, lane);
  }
  // rows of the chunk after next from their prefetched slots; slots one further ahead
  const int64_t b2 = base + 2 * kCh + 16 * wave;
  st.cur = nxt;
  st.nxt = wave_rows<kSparse>(a, ctx, b2, hi, st.slot2, lane);
  st.slot2 = prefetch_slot<kSparse>(a, qi, b2 + kCh, lane);

  // scores of this wave's 16 entries (lane: entries 4g + i, head c)
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, sr = s0;
  {
    const uint8_t* rowp = buf + (16 * wave + c) * kRowF8 + 16 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(rowp + 128 * ks);
      uint4 x1 = make_uint4(0, 0, 0, 0);  // dims 448.. (K step 3, bytes 16-31) are RoPE bytes: zero
      if (ks < 3) x1 = *reinterpret_cast<const uint4*>(rowp + 128 * ks + 64);
      const i32x8 A = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      s0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, q.qh[ks], s0, 0, 0, 0, 127, 0,
                                                             (int)((q.sh >> (8 * ks)) & 255u));
      s1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, q.ql[ks], s1, 0, 0, 0, 127, 0,
                                                             (int)((q.sl >> (8 * ks)) & 255u));
    }
    const uint8_t* ropep = buf + (16 * wave + c) * kRowF8 + kNope + 16 * g;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 kv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ropep + 64 * ks));
      sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, q.qr[ks], sr, 0, 0, 0);
    }
  }
  if (more) stage_rows<3, 3>(nxt, ndst, lane);
  float sv[4], escl[4];
  float cmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * g + i;
    escl[i] = __shfl(cur.esc, e, 64);
    const float st_ = fmaf(escl[i], s0[i] + s1[i], sr[i]);
    sv[i] = ((cur.vmask >> e) & 1) ? st_ * sl2 : -INFINITY;
    cmax = fmaxf(cmax, sv[i]);
  }
  cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
  if (g == 0) wmax[16 * wave + c] = cmax;
  // lazy rescaling: the reference max moves only when a score exceeds it by more than 2^8
  // (log2 units), so p <= 256 and O is rescaled rarely instead of every chunk. P is written
  // against the current reference before the block's maxima are known (one barrier publishes
  // both); when some head's block maximum does move the reference, every wave sees it in the
  // same maxima, rewrites its P with the new reference and waits once more.
  const int pe = c * kPRow + 16 * wave + 4 * g;
  auto put_p = [&](float m_ref, float* p) {
    const bool none = m_ref == -INFINITY;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = none ? 0.f : exp2f(sv[i] - m_ref);
      psum += p[i];
    }
    *reinterpret_cast<uint2*>(pbs + pe) =
        make_uint2(pack_bf16x2(p[0] * escl[0], p[1] * escl[1]), pack_bf16x2(p[2] * escl[2], p[3] * escl[3]));
    *reinterpret_cast<uint2*>(pb + pe) = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
    return psum;
  };
  float p[4];
  float psum = put_p(st.m_run, p);
  if (more) stage_rows<6, 2>(nxt, ndst, lane);
  lds_barrier();
#pragma unroll
  for (int w = 0; w < 8; ++w) cmax = fmaxf(cmax, wmax[16 * w + c]);
  const bool grow = cmax > st.m_run + 8.f;
  if (__ballot(grow)) {  // the same in every wave of the block
    const float m_ref = grow ? cmax : st.m_run;
    const float corr = grow ? exp2f(st.m_run - cmax) : 1.f;
    psum = put_p(m_ref, p);
    st.l_part = st.l_part * corr + psum;
    st.m_run = m_ref;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.O[dt] *= corr;
    lds_barrier();
  } else {
    st.l_part = st.l_part * 1.f + psum;
  }
  // O^T (this wave's 64 dims x 16 heads) += V^T P^T over the chunk's 128 entries
  if (wave < 7) {
    const int r = c >> 1, hsel = c & 1;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 B = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(pbs + c * kPRow + 32 * kk + 8 * g));
      const uint8_t* vp = buf + (32 * kk + 8 * g + r) * kRowF8 + 64 * wave + 8 * hsel;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const i32x2_t t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vp + 16 * dt));
        st.O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8((uint32_t)t[0], (uint32_t)t[1]), B,
                                                           st.O[dt], 0, 0, 0);
      }
    }
  } else {
    const int rs = c >> 2, qd = c & 3;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 B = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(pb + c * kPRow + 32 * kk + 8 * g));
      const uint8_t* v0 = buf + (32 * kk + 8 * g + rs) * kRowF8 + kNope + 8 * qd;
      const uint8_t* v1 = v0 + 4 * kRowF8;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + 32 * dt));
        const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v1 + 32 * dt));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 av = __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7);
        st.O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), B, st.O[dt], 0, 0, 0);
      }
    }
  }
  if (more) stage_rows<8, 2>(nxt, ndst, lane);
}

// The LDS of one attn_fp8 block: two chunk buffers as separate LDS objects (see f8_chunk), then
// the P tiles and maxima. A kernel declares them and hands them to attn_fp8_block.
#define ATTN_FP8_LDS                                                                             \
  __shared__ __attribute__((aligned(16))) uint8_t buf0[kBufF8];                                  \
  __shared__ __attribute__((aligned(16))) uint8_t buf1[kBufF8];                                  \
  __shared__ __attribute__((aligned(16))) uint16_t pbs[16 * kPRow]; /* [16][kPRow] P x scale */  \
  __shared__ __attribute__((aligned(16))) uint16_t pb[16 * kPRow];  /* [16][kPRow] P */          \
  __shared__ float wmax[8 * 16], wsum[8 * 16];

// Work item id < total of an attn_fp8 grid: (query, split, 16-head group).
// kSparse: CSA (entries listed by idx, a.idx set) or HCA (dense, a.idx null).
template <bool kSparse>
__device__ __forceinline__ void attn_fp8_block(const AttnArgs& a, int n_hg, int id, uint8_t (&buf0)[kBufF8],
                                               uint8_t (&buf1)[kBufF8], uint16_t (&pbs)[16 * kPRow],
                                               uint16_t (&pb)[16 * kPRow], float (&wmax)[8 * 16],
                                               float (&wsum)[8 * 16]) {
  const int hg = id % n_hg;
  const int rest = id / n_hg;
  const int s = rest % a.n_split;
  const int qi = rest / a.n_split;
  const int H = a.H;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int head = hg * 16 + c;

  // query: FP8 hi/lo parts of the 448 non-RoPE dims. Operand layout of the 16x16x128 FP8
  // MFMA: in K step ks, lane (g, c) holds dims 128ks + 16g .. +16 in bytes 0-15 and dims
  // 128ks + 64 + 16g .. +16 in bytes 16-31; the 32-dim scale block b of the step is the pair
  // of half rows (g = 0/1 low halves: b = 0, high halves: b = 2; g = 2/3: b = 1 and 3), and
  // lane group g supplies block g's scale. Waves 0-3 build K step ks = wave for all lanes in
  // the second chunk buffer (unused until the first chunk is staged); every wave then loads
  // all four steps.
  const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)qi * H + head) * kD;
  uint8_t* qbuf = buf1;  // [4 ks][64 lanes][32 hi + 32 lo bytes], then [4][64] scale words
  uint32_t* qsc = reinterpret_cast<uint32_t*>(qbuf + 4 * 64 * 64);
  uint4 qraw[4];
  if (wave < 4) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int d0 = 128 * wave + 64 * half + 16 * g;
#pragma unroll
      for (int v = 0; v < 2; ++v)
        qraw[2 * half + v] = d0 < kNope ? *reinterpret_cast<const uint4*>(qp + d0 + 8 * v) : make_uint4(0, 0, 0, 0);
    }
  }
  bf16x8 qr[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    qr[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + kNope + 32 * ks + 8 * g));

  const int64_t lo = (int64_t)s * a.per_split;
  const int64_t b0 = lo + 16 * wave;
  const int32_t s0 = prefetch_slot<kSparse>(a, qi, b0, lane), s1 = prefetch_slot<kSparse>(a, qi, b0 + kCh, lane);
  // Top-k slots of the first three chunks (CSA) need only the query and the split; the
  // sequence-offset loads follow. The query is prepared while both are in flight, and the first
  // chunk's rows are requested once they are known.
  F8State st;
  st.slot2 = prefetch_slot<kSparse>(a, qi, b0 + 2 * kCh, lane);
  const QueryCtx ctx = query_ctx(a, qi);

  if (wave < 4) {
    float x[32];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t w4[4] = {qraw[v].x, qraw[v].y, qraw[v].z, qraw[v].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[8 * v + 2 * k] = __uint_as_float(w4[k] << 16);
        x[8 * v + 2 * k + 1] = __uint_as_float(w4[k] & 0xFFFF0000u);
      }
    }
    float am[2] = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 32; ++j) am[j >> 4] = fmaxf(am[j >> 4], fabsf(x[j]));
    int eb[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const float m = fmaxf(am[half], __shfl_xor(am[half], 16, 64));  // the other half row of the block
      int E = 0;
      if (m > 0.f) (void)frexpf(m, &E);  // m < 2^E: scaled values stay below 256
      eb[half] = m > 0.f ? min(max(E - 8, -120), 120) : 0;
    }
    uint32_t hw[8], lw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = eb[j >> 2];
      const float inv_hi = __builtin_ldexpf(1.f, -e), inv_lo = __builtin_ldexpf(1.f, 4 - e);
      const float sc_hi = __builtin_ldexpf(1.f, e);
      const float* xj = x + 4 * j;
      int h2 = __builtin_amdgcn_cvt_pk_fp8_f32(xj[0] * inv_hi, xj[1] * inv_hi, 0, false);
      h2 = __builtin_amdgcn_cvt_pk_fp8_f32(xj[2] * inv_hi, xj[3] * inv_hi, h2, true);
      const float r0 = xj[0] - __builtin_amdgcn_cvt_f32_fp8(h2, 0) * sc_hi;
      const float r1 = xj[1] - __builtin_amdgcn_cvt_f32_fp8(h2, 1) * sc_hi;
      const float r2 = xj[2] - __builtin_amdgcn_cvt_f32_fp8(h2, 2) * sc_hi;
      const float r3 = xj[3] - __builtin_amdgcn_cvt_f32_fp8(h2, 3) * sc_hi;
      int l2 = __builtin_amdgcn_cvt_pk_fp8_f32(r0 * inv_lo, r1 * inv_lo, 0, false);
      l2 = __builtin_amdgcn_cvt_pk_fp8_f32(r2 * inv_lo, r3 * inv_lo, l2, true);
      hw[j] = (uint32_t)h2;
      lw[j] = (uint32_t)l2;
    }
    uint4* dst = reinterpret_cast<uint4*>(qbuf + (64 * wave + lane) * 64);
    dst[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    dst[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
    dst[2] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    dst[3] = make_uint4(lw[4], lw[5], lw[6], lw[7]);
    // block g's exponent: g0 its low half, g1 the low half of g2 (block 1), g2 the high half of
    // g0 (block 2), g3 its high half (block 3)
    const int from_lo2 = __shfl(eb[0], 32 + c, 64), from_hi0 = __shfl(eb[1], c, 64);
    const int eop = g == 0 ? eb[0] : g == 1 ? from_lo2 : g == 2 ? from_hi0 : eb[1];
    qsc[64 * wave + lane] = (uint32_t)(eop + 127) | ((uint32_t)(eop - 4 + 127) << 8);
  }
  const int64_t N = ctx.n_c + ctx.n_w;
  const int64_t hi = min<int64_t>(N, lo + a.per_split);
  st.cur = wave_rows<kSparse>(a, ctx, b0, hi, s0, lane);
  st.nxt = wave_rows<kSparse>(a, ctx, b0 + kCh, hi, s1, lane);
  if (lo < hi) {
    uint8_t* dst = buf0 + 16 * wave * kRowF8;
    zero_invalid_rows(st.cur, dst, lane);
    stage_rows<0, 10>(st.cur, dst, lane);
  }
  lds_barrier();
  F8Query q;
  q.sh = q.sl = 0;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint4* src = reinterpret_cast<const uint4*>(qbuf + (64 * ks + lane) * 64);
    const uint4 h0 = src[0], h1 = src[1], l0 = src[2], l1 = src[3];
    q.qh[ks] = i32x8{(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w, (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
    q.ql[ks] = i32x8{(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w, (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
    const uint32_t sw = qsc[64 * ks + lane];
    q.sh |= (sw & 255u) << (8 * ks);
    q.sl |= ((sw >> 8) & 255u) << (8 * ks);
  }
  q.qr[0] = qr[0];
  q.qr[1] = qr[1];

#pragma unroll
  for (int i = 0; i < 4; ++i) st.O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_part = 0.f;
  const float sl2 = a.scale * kLog2e;
  // unrolled by two so that each call names its chunk buffers statically
  for (int64_t base = lo; base < hi; base += 2 * kCh) {
    f8_chunk<kSparse>(a, ctx, qi, base, hi, buf0, buf1, q, st, pbs, pb, wmax, sl2, wave, lane);
    if (base + kCh >= hi) break;
    f8_chunk<kSparse>(a, ctx, qi, base + kCh, hi, buf1, buf0, q, st, pbs, pb, wmax, sl2, wave, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);

  // the softmax denominator: this lane's entries, then over the lane groups and the waves
  st.l_part += __shfl_xor(st.l_part, 16, 64);
  st.l_part += __shfl_xor(st.l_part, 32, 64);
  if (g == 0) wsum[16 * wave + c] = st.l_part;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) L += wsum[16 * w + c];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const float lse = L > 0.f ? (st.m_run + log2f(L)) * kLn2 : -INFINITY;
  // the output row is recomputed here from an opaque copy of the head index: otherwise the
  // compiler keeps the prologue's 64-bit query-row products live across the chunk loop
  int head_o = head;
  asm volatile("" : "+v"(head_o));
  const int64_t hrow = (int64_t)qi * H + head_o;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int d = 64 * wave + 16 * dt + 4 * g;
    const f32x4 acc = st.O[dt] * inv;
    if (a.n_split == 1) {
      if (a.o_dtype == HCA_BF16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + hrow * kD + d) =
            make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + hrow * kD + d) = acc;
      }
    } else {
      const int64_t pi = ((int64_t)qi * a.n_split + s) * H + head_o;
      *reinterpret_cast<f32x4*>(a.part_o + pi * kD + d) = acc;
    }
  }
  if (wave == 0 && g == 0) {
    if (a.n_split == 1) a.lse[hrow] = lse;
    else a.part_lse[((int64_t)qi * a.n_split + s) * H + head_o] = lse;
  }
}

template <bool kSparse>
__global__ __launch_bounds__(512, 1) void attn_fp8_kernel(AttnArgs a, int n_hg, int total) {
  ATTN_FP8_LDS
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  if (id >= total) return;
  attn_fp8_block<kSparse>(a, n_hg, id, buf0, buf1, pbs, pb, wmax, wsum);
}

// The indexer's top-k selection and an HCA attention call in one grid, for callers whose
// selection and attention are independent (the selection feeds a later CSA call): blocks
// b < n_sel (a multiple of 8) select query b of `sel` (b < sel.nq), the others are the
// attention call's blocks b - n_sel, so their XCD placement is the attention kernel's own.
// The selection takes one block of the 8 that share an XCD slot and its LDS aliases the chunk
// buffers. One launch instead of two on separate streams, whose cross-stream waits cost more
// than the selection itself.
static_assert(kFinThreads == 512, "the selection runs in 512-thread attention blocks");
static_assert(sizeof(FinLds) <= kBufF8 && sizeof(OutLds) <= kBufF8, "selection LDS inside the chunk buffers");
__global__ __launch_bounds__(512, 1) void select_attn_fp8_kernel(IndexArgs sel, int n_sel, AttnArgs a, int n_hg,
                                                                 int total) {
  ATTN_FP8_LDS
  const int b = blockIdx.x;
  if (b >= n_sel) {
    const int id = xcd_remap(b - n_sel, (int)gridDim.x - n_sel);
    if (id < total) attn_fp8_block<false>(a, n_hg, id, buf0, buf1, pbs, pb, wmax, wsum);
    return;
  }
  if (b < sel.nq) finalize_block(sel, b, *reinterpret_cast<FinLds*>(buf0), *reinterpret_cast<OutLds*>(buf1));
}

// ---------------------------------------------------------------------------------------
// Row-owning FP8 kernel for calls with many queries (prefill). block = (query, split), 4 waves
// (one per SIMD) for H = 64; wave w owns heads 16w .. 16w+15 over every entry of the split and
// all 512 dims, so one staged chunk serves all 64 heads (the kernel above stages it once per
// group of 16 heads, in four blocks).
//  * staging through registers: wave w brings entries 32w .. 32w+31 of the next chunk (18,944
//    LDS bytes) with 19 lane-linear 16-byte loads issued a chunk ahead, and writes them to LDS
//    at the end of the current chunk; invalid rows are written as zeros;
//  * S^T = K Q^T as above (scaled FP8 MFMA for the 448 dims, bf16 MFMA for RoPE) over the
//    chunk's 8 tiles of 16 entries. Tile 2kk + u row r holds entry 32kk + 8(r/4) + 4u + r%4, so
//    a lane's accumulators of tiles 2kk and 2kk + 1 are entries 32kk + 8g .. 32kk + 8g + 7 of
//    its head: the B operand of the PV MFMA over that 32-entry step, without going through LDS;
//  * the online softmax is per head inside the wave (two cross-lane maxima), lazy rescale;
//  * O^T (512 dims x 16 heads: 28 FP8-dim tiles and 4 RoPE tiles) += V^T P^T, V^T from the
//    same transpose reads as above.
constexpr int kRowsWaves = 4;
constexpr int kRowsEnt = kCh / kRowsWaves;                     // 32 entries staged per wave
constexpr int kRowsBytes = kRowsEnt * kRowF8;                  // 18,944 bytes
constexpr int kRowsLoads = (kRowsBytes + 1023) / 1024;         // 19 loads of 16 bytes a lane

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct RowsSrc {
  uint64_t src;    // lane e < 32: FP8-row address of entry e; lane 32 + e: RoPE-row address - 448
  float esc;       // lane e < 32: entry scale (load left in flight)
  uint32_t vmask;  // valid entries
};


// Slot value of list position base + (lane & 31) (CSA); positions past the top-k list are
// clamped to a valid slot whose value is not used.
template <bool kSparse>
__device__ __forceinline__ int32_t rows_slot(const AttnArgs& a, int qi, int64_t base, int lane) {
  if (!kSparse) return 0;
  const int64_t r = min<int64_t>(base + (lane & 31), (int64_t)a.k - 1);
  return a.idx[(int64_t)qi * a.k + r];
}

template <bool kSparse>
__device__ __forceinline__ RowsSrc rows_src(const AttnArgs& a, const QueryCtx& ctx, int64_t base, int64_t hi,
                                            int32_t slot, int lane) {
  RowsSrc w;
  const int64_t r = base + (lane & 31);
  const bool win = r >= ctx.n_c;
  int64_t row = -1;
  if (r < hi) {
    if (!win) {
      const int64_t j = kSparse ? (int64_t)slot : r;
      const int64_t cr = ctx.cache_rb + j;
      row = (j >= 0 && cr >= 0 && cr < a.cache.n_rows) ? cr : -1;
    } else if (r < ctx.n_c + ctx.n_w) {
      const int64_t pos = ctx.t - ctx.n_w + 1 + (r - ctx.n_c);
      const int64_t wr = ctx.win_rb + (pos - ctx.win_p0);
      row = (wr >= 0 && wr < a.win.n_rows) ? wr : -1;
    }
  }
  const uint64_t data = win ? reinterpret_cast<uint64_t>(a.win.data) : reinterpret_cast<uint64_t>(a.cache.data);
  const uint64_t rope = win ? reinterpret_cast<uint64_t>(a.win.rope) : reinterpret_cast<uint64_t>(a.cache.rope);
  const int64_t rs = win ? a.win.row_stride : a.cache.row_stride;
  const int64_t ps = win ? a.win.rope_stride : a.cache.rope_stride;
  const float* scale = win ? a.win.scale : a.cache.scale;
  const int64_t rr = row >= 0 ? row : 0;  // invalid entries are never loaded
  w.src = lane < 32 ? data + (uint64_t)(rr * rs) : rope + (uint64_t)(rr * ps * 2) - kNope;
  w.esc = (lane < 32 && row >= 0) ? scale[row] : 0.f;
  w.vmask = (uint32_t)__ballot(lane < 32 && row >= 0);
  return w;
}

// Loads I0 .. I0 + kN - 1 of a wave's 32 rows: LDS byte b = 1024 i + 16 lane of the wave's
// region is entry b / 592, byte b % 592 (FP8 bytes, then RoPE bytes, then 16 pad bytes). Lanes on
// padding, past the 32 rows or on an invalid row load nothing and hold zeros.
// The per-lane offsets depend on the lane only; they are derived from an opaque copy of the lane
// index so that the compiler recomputes them at each call instead of keeping all of them live
// across the chunk loop.
template <int I0, int kN>
__device__ __forceinline__ void rows_load(const RowsSrc& w, uint4 (&v)[kN], int lane) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int j = 0; j < kN; ++j) {
    const int b = 1024 * (I0 + j) + 16 * ln;
    const int e = b / kRowF8, o = b - e * kRowF8;
    const int sl = (o < kNope ? e : 32 + e) & 63;
    const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)w.src, sl, 64);
    const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(w.src >> 32), sl, 64);
    const uint64_t src = (((uint64_t)hi << 32) | lo) + (uint64_t)o;
    uint4 x = make_uint4(0, 0, 0, 0);
    // a global (not generic) load: a flat load would also count against the LDS wait counter,
    // so every LDS wait of the chunk would wait for these loads too
    if (e < kRowsEnt && o < kNope + 2 * kRope && ((w.vmask >> (e & 31)) & 1))
      x = __builtin_bit_cast(uint4, *reinterpret_cast<const __attribute__((address_space(1))) u32x4_t*>(src));
    v[j] = x;
  }
}

template <int I0, int kN>
__device__ __forceinline__ void rows_store(const uint4 (&v)[kN], uint8_t* dst, int lane) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int j = 0; j < kN; ++j) {
    const int b = 1024 * (I0 + j) + 16 * ln;
    if (b < kRowsBytes) *reinterpret_cast<uint4*>(dst + b) = v[j];
  }
}

constexpr int kRowsHalfA = 10, kRowsHalfB = kRowsLoads - kRowsHalfA;

struct RowsState {
  f32x4 O[32];
  float m_run, l_part;
};

// Scores and softmax of one chunk in buf (scales sc, validity masks vm): O^T is rescaled if the
// reference maximum moved, and the PV B operands of the four 32-entry steps are returned packed:
// P times the entry scale (bs, for the FP8 dims) and P (br, for the RoPE dims).
__device__ __forceinline__ void rows_scores(const uint8_t* buf, const float* sc, const uint32_t* vm, const F8Query& q,
                                            RowsState& st, float sl2, int lane, uint4 (&bs)[4], uint4 (&br)[4]) {
  asm volatile("" : "+v"(lane));  // lane-only addresses are recomputed per chunk, not kept live
  const int g = lane >> 4, c = lane & 15;
  const uint4 vmk = *reinterpret_cast<const uint4*>(vm);
  const uint32_t vmw[4] = {vmk.x, vmk.y, vmk.z, vmk.w};
  float sv[8][4];
  float cmax = -INFINITY;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int kk = t >> 1, u = t & 1;
    const int ent = 32 * kk + 8 * (c >> 2) + 4 * u + (c & 3);  // entry of A row c
    const uint8_t* rowp = buf + ent * kRowF8 + 16 * g;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, sr = s0;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(rowp + 128 * ks);
      uint4 x1 = make_uint4(0, 0, 0, 0);
      if (ks < 3) x1 = *reinterpret_cast<const uint4*>(rowp + 128 * ks + 64);
      const i32x8 A = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      s0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, q.qh[ks], s0, 0, 0, 0, 127, 0,
                                                             (int)((q.sh >> (8 * ks)) & 255u));
      s1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, q.ql[ks], s1, 0, 0, 0, 127, 0,
                                                             (int)((q.sl >> (8 * ks)) & 255u));
    }
    const uint8_t* ropep = buf + ent * kRowF8 + kNope + 16 * g;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 kv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ropep + 64 * ks));
      sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, q.qr[ks], sr, 0, 0, 0);
    }
    // lane (g, c): entries 32kk + 8g + 4u + i of head c
    const int e0 = 32 * kk + 8 * g + 4 * u;
    const float4 e4 = *reinterpret_cast<const float4*>(sc + e0);
    const float esc[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + i;
      const float v = fmaf(esc[i], s0[i] + s1[i], sr[i]);
      sv[t][i] = ((vmw[e >> 5] >> (e & 31)) & 1) ? v * sl2 : -INFINITY;
      cmax = fmaxf(cmax, sv[t][i]);
    }
    __builtin_amdgcn_sched_barrier(0);  // one tile's operands live at a time
  }
  cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
  // lazy rescaling: the reference max moves only when a score exceeds it by more than 2^8
  const bool grow = cmax > st.m_run + 8.f;
  const float m_ref = grow ? cmax : st.m_run;
  const bool none = m_ref == -INFINITY;
  const float corr = grow ? exp2f(st.m_run - cmax) : 1.f;
  float psum = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[t][i] = none ? 0.f : exp2f(sv[t][i] - m_ref);
      psum += sv[t][i];
    }
  st.l_part = st.l_part * corr + psum;
  st.m_run = m_ref;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const float* p0 = sv[2 * kk];
    const float* p1 = sv[2 * kk + 1];
    const float4 x0 = *reinterpret_cast<const float4*>(sc + 32 * kk + 8 * g);
    const float4 x1 = *reinterpret_cast<const float4*>(sc + 32 * kk + 8 * g + 4);
    bs[kk].x = pack_bf16x2(p0[0] * x0.x, p0[1] * x0.y); bs[kk].y = pack_bf16x2(p0[2] * x0.z, p0[3] * x0.w);
    bs[kk].z = pack_bf16x2(p1[0] * x1.x, p1[1] * x1.y); bs[kk].w = pack_bf16x2(p1[2] * x1.z, p1[3] * x1.w);
    br[kk].x = pack_bf16x2(p0[0], p0[1]); br[kk].y = pack_bf16x2(p0[2], p0[3]);
    br[kk].z = pack_bf16x2(p1[0], p1[1]); br[kk].w = pack_bf16x2(p1[2], p1[3]);
  }
  if (__ballot(grow)) {
#pragma unroll
    for (int d = 0; d < 32; ++d) st.O[d] *= corr;
  }
  __builtin_amdgcn_sched_barrier(0);
}

// O^T += V^T P^T over the chunk's four 32-entry steps.
__device__ __forceinline__ void rows_pv(const uint8_t* buf, const uint4 (&bs)[4], const uint4 (&br)[4], RowsState& st,
                                        int lane) {
  asm volatile("" : "+v"(lane));
  const int g = lane >> 4, c = lane & 15;
  const int r = c >> 1, hsel = c & 1, rs = c >> 2, qd = c & 3;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const bf16x8 Bs = __builtin_bit_cast(bf16x8, bs[kk]), Br = __builtin_bit_cast(bf16x8, br[kk]);
    const uint8_t* vp = buf + (32 * kk + 8 * g + r) * kRowF8 + 8 * hsel;
#pragma unroll
    for (int d = 0; d < 28; ++d) {
      const i32x2_t tv = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vp + 16 * d));
      st.O[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8((uint32_t)tv[0], (uint32_t)tv[1]), Bs,
                                                         st.O[d], 0, 0, 0);
      if ((d & 7) == 7) __builtin_amdgcn_sched_barrier(0);  // eight tiles' reads in flight at most
    }
    const uint8_t* v0 = buf + (32 * kk + 8 * g + rs) * kRowF8 + kNope + 8 * qd;
    const uint8_t* v1 = v0 + 4 * kRowF8;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + 32 * d));
      const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v1 + 32 * d));
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 av = __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7);
      st.O[28 + d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), Br, st.O[28 + d], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The FP8 hi / lo query operands of the wave's 16 heads (lane (g, c): head 16 wave + c), built
// in registers: K step ks takes dims 128ks + 16g .. +16 (bytes 0-15) and 128ks + 64 + 16g .. +16
// (bytes 16-31), each 32-dim block with a power-of-two scale, laid out as the kernel above does
// through LDS.
__device__ __forceinline__ F8Query rows_query(const uint16_t* qp, int lane) {
  const int g = lane >> 4, c = lane & 15;
  F8Query q;
  q.sh = q.sl = 0;
  uint4 qraw[4][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int d0 = 128 * ks + 64 * half + 16 * g;
#pragma unroll
      for (int v = 0; v < 2; ++v)
        qraw[ks][2 * half + v] = d0 < kNope ? *reinterpret_cast<const uint4*>(qp + d0 + 8 * v) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    q.qr[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + kNope + 32 * ks + 8 * g));
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float x[32];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t w4[4] = {qraw[ks][v].x, qraw[ks][v].y, qraw[ks][v].z, qraw[ks][v].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[8 * v + 2 * k] = __uint_as_float(w4[k] << 16);
        x[8 * v + 2 * k + 1] = __uint_as_float(w4[k] & 0xFFFF0000u);
      }
    }
    float am[2] = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 32; ++j) am[j >> 4] = fmaxf(am[j >> 4], fabsf(x[j]));
    int eb[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const float m = fmaxf(am[half], __shfl_xor(am[half], 16, 64));  // the other half row of the block
      int E = 0;
      if (m > 0.f) (void)frexpf(m, &E);
      eb[half] = m > 0.f ? min(max(E - 8, -120), 120) : 0;
    }
    uint32_t hw[8], lw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = eb[j >> 2];
      const float inv_hi = __builtin_ldexpf(1.f, -e), inv_lo = __builtin_ldexpf(1.f, 4 - e);
      const float sc_hi = __builtin_ldexpf(1.f, e);
      const float* xj = x + 4 * j;
      int h2 = __builtin_amdgcn_cvt_pk_fp8_f32(xj[0] * inv_hi, xj[1] * inv_hi, 0, false);
      h2 = __builtin_amdgcn_cvt_pk_fp8_f32(xj[2] * inv_hi, xj[3] * inv_hi, h2, true);
      const float r0 = xj[0] - __builtin_amdgcn_cvt_f32_fp8(h2, 0) * sc_hi;
      const float r1 = xj[1] - __builtin_amdgcn_cvt_f32_fp8(h2, 1) * sc_hi;
      const float r2 = xj[2] - __builtin_amdgcn_cvt_f32_fp8(h2, 2) * sc_hi;
      const float r3 = xj[3] - __builtin_amdgcn_cvt_f32_fp8(h2, 3) * sc_hi;
      int l2 = __builtin_amdgcn_cvt_pk_fp8_f32(r0 * inv_lo, r1 * inv_lo, 0, false);
      l2 = __builtin_amdgcn_cvt_pk_fp8_f32(r2 * inv_lo, r3 * inv_lo, l2, true);
      hw[j] = (uint32_t)h2;
      lw[j] = (uint32_t)l2;
    }
    q.qh[ks] = i32x8{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3], (int)hw[4], (int)hw[5], (int)hw[6], (int)hw[7]};
    q.ql[ks] = i32x8{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3], (int)lw[4], (int)lw[5], (int)lw[6], (int)lw[7]};
    // block g's exponent: g0 its low half, g1 the low half of g2 (block 1), g2 the high half of
    // g0 (block 2), g3 its high half (block 3)
    const int from_lo2 = __shfl(eb[0], 32 + c, 64), from_hi0 = __shfl(eb[1], c, 64);
    const int eop = g == 0 ? eb[0] : g == 1 ? from_lo2 : g == 2 ? from_hi0 : eb[1];
    q.sh |= (uint32_t)(eop + 127) << (8 * ks);
    q.sl |= (uint32_t)(eop - 4 + 127) << (8 * ks);
  }
  return q;
}

template <bool kSparse>
__global__ __launch_bounds__(256, 1) void attn_rows_kernel(AttnArgs a, int total) {
  __shared__ __attribute__((aligned(16))) uint8_t buf0[kBufF8];
  __shared__ __attribute__((aligned(16))) uint8_t buf1[kBufF8];
  __shared__ __attribute__((aligned(16))) float sc0[kCh];
  __shared__ __attribute__((aligned(16))) float sc1[kCh];
  __shared__ __attribute__((aligned(16))) uint32_t vm0[kRowsWaves];
  __shared__ __attribute__((aligned(16))) uint32_t vm1[kRowsWaves];
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  if (id >= total) return;
  const int s = id % a.n_split;
  const int qi = id / a.n_split;
  const int H = a.H;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int head = 16 * wave + c;

  const int64_t lo = (int64_t)s * a.per_split;
  const int64_t b0 = lo + kRowsEnt * wave;
  const int32_t s0 = rows_slot<kSparse>(a, qi, b0, lane), s1 = rows_slot<kSparse>(a, qi, b0 + kCh, lane);
  int32_t slot2 = rows_slot<kSparse>(a, qi, b0 + 2 * kCh, lane);
  const QueryCtx ctx = query_ctx(a, qi);
  const int64_t N = ctx.n_c + ctx.n_w;
  const int64_t hi = min<int64_t>(N, lo + a.per_split);
  const RowsSrc cur = rows_src<kSparse>(a, ctx, b0, hi, s0, lane);
  RowsSrc nxt = rows_src<kSparse>(a, ctx, b0 + kCh, hi, s1, lane);
  // the first chunk's rows are requested before the query is quantized, which hides their latency
  uint4 va0[kRowsHalfA], vb0[kRowsHalfB];
  rows_load<0, kRowsHalfA>(cur, va0, lane);
  rows_load<kRowsHalfA, kRowsHalfB>(cur, vb0, lane);
  const F8Query q = rows_query(static_cast<const uint16_t*>(a.q) + ((int64_t)qi * H + head) * kD, lane);
  rows_store<0, kRowsHalfA>(va0, buf0 + kRowsBytes * wave, lane);
  rows_store<kRowsHalfA, kRowsHalfB>(vb0, buf0 + kRowsBytes * wave, lane);
  if (lane < 32) sc0[kRowsEnt * wave + lane] = cur.esc;
  if (lane == 0) vm0[wave] = cur.vmask;
  __syncthreads();

  RowsState st;
#pragma unroll
  for (int d = 0; d < 32; ++d) st.O[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_part = 0.f;
  const float sl2 = a.scale * kLog2e;
  // one chunk in buf; the next chunk's rows go to the other buffer in two halves (loaded at the
  // start and written after the softmax, loaded then and written after PV), so that at most
  // half of them sit in registers; one LDS barrier then publishes them and frees buf
  auto chunk = [&](int64_t base, const uint8_t* buf, const float* sc, const uint32_t* vm, uint8_t* nbuf, float* nsc,
                   uint32_t* nvm) {
    const bool more = base + kCh < hi;
    uint8_t* ndst = nbuf + kRowsBytes * wave;
    uint4 va[kRowsHalfA], vb[kRowsHalfB];
    if (more) rows_load<0, kRowsHalfA>(nxt, va, lane);
    uint4 bs[4], br[4];
    rows_scores(buf, sc, vm, q, st, sl2, lane, bs, br);
    if (more) {
      rows_store<0, kRowsHalfA>(va, ndst, lane);
      rows_load<kRowsHalfA, kRowsHalfB>(nxt, vb, lane);
    }
    rows_pv(buf, bs, br, st, lane);
    if (more) {
      rows_store<kRowsHalfA, kRowsHalfB>(vb, ndst, lane);
      if (lane < 32) nsc[kRowsEnt * wave + lane] = nxt.esc;
      if (lane == 0) nvm[wave] = nxt.vmask;
      const int64_t b2 = base + 2 * kCh + kRowsEnt * wave;
      nxt = rows_src<kSparse>(a, ctx, b2, hi, slot2, lane);
      slot2 = rows_slot<kSparse>(a, qi, b2 + kCh, lane);
    }
    // LDS only: the scale and slot loads just issued stay in flight across the barrier
    lds_barrier();
  };
  // unrolled by two so that each call names its buffers statically
  for (int64_t base = lo; base < hi; base += 2 * kCh) {
    chunk(base, buf0, sc0, vm0, buf1, sc1, vm1);
    if (base + kCh >= hi) break;
    chunk(base + kCh, buf1, sc1, vm1, buf0, sc0, vm0);
  }

  // the softmax denominator of head c: this lane's entries, then over the lane groups
  float L = st.l_part;
  L += __shfl_xor(L, 16, 64);
  L += __shfl_xor(L, 32, 64);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const float lse = L > 0.f ? (st.m_run + log2f(L)) * kLn2 : -INFINITY;
  int head_o = head;
  asm volatile("" : "+v"(head_o));
  const int64_t hrow = (int64_t)qi * H + head_o;
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    const int dd = 16 * d + 4 * g;  // FP8 dims for d < 28, then RoPE dims 448 + 16 (d - 28) + 4 g
    const f32x4 acc = st.O[d] * inv;
    if (a.n_split == 1) {
      if (a.o_dtype == HCA_BF16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + hrow * kD + dd) =
            make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + hrow * kD + dd) = acc;
      }
    } else {
      const int64_t pi = ((int64_t)qi * a.n_split + s) * H + head_o;
      *reinterpret_cast<f32x4*>(a.part_o + pi * kD + dd) = acc;
    }
  }
  if (g == 0) {
    if (a.n_split == 1) a.lse[hrow] = lse;
    else a.part_lse[((int64_t)qi * a.n_split + s) * H + head_o] = lse;
  }
}

// ---------------------------------------------------------------------------------------
// Wide FP8 kernel: one block serves 64 heads (a group of 64 of the query's heads), so every
// staged row is used by all 64 heads (attn_fp8_kernel stages each row once per group of 16
// heads, in four blocks). block = (query, 64-head group, split), 8 waves: wave w computes for
// heads 16 (w & 3) .. +15 of the group and works on half h = w >> 2 of each chunk; the two waves
// of a head group share a SIMD.
//  * chunks of 64 entries, double buffered in LDS. Every wave stages a share: wave w requests
//    entries 8 w .. 8 w + 7 of the next chunk with 5 lane-linear 1 KiB global_load_lds DMAs
//    before its scores; its rows for the chunk after next (with their scale loads) are found
//    after PV, where no DMAs are queued. The scales and validity of every entry go through LDS
//    once a chunk's rows have landed;
//  * S^T = K Q^T for entries 32h .. 32h + 31 (two tiles of 16) and the wave's 16 heads, on the
//    scaled FP8 MFMA with the query split into two FP8 parts, RoPE dims on bf16 MFMA, as in
//    attn_fp8_kernel;
//  * the two waves of a head group share one reference maximum per head (their chunk maxima meet
//    in LDS, lazy rescale) and write P for their 32 entries to LDS, with and without the entry
//    scales;
//  * O^T += V^T P^T over all 64 entries of the chunk, split by output dims and heads: wave w owns
//    dims 128 (w & 3) .. + 127 (FP8 dims 0 .. 447, then the 64 RoPE dims) of heads 32 (w >> 2)
//    .. + 31 (8 x 2 tiles of 16 dims x 16 heads), so each V^T tile is read (ds_read_b64_tr_b8 /
//    tr_b16) and converted to bf16 by two waves of the block and feeds 2 MFMAs in each. The head
//    groups' rescale factors reach the dim owners through LDS with P.
constexpr int kWCh = 64;                  // entries per chunk
constexpr int kWBuf = kWCh * kRowF8;      // 37,888 bytes
constexpr int kWPRow = kWCh + 8;          // bf16 per P row (padded)

struct WideLds {
  float esc[kWCh];      // entry scales of the chunk being computed
  float esc2[kWCh];     // the scale times scale * log2(e) for a valid entry, 0 otherwise
  float bias[kWCh];     // 0 for a valid entry, -inf otherwise
  float wmax[8][16], wsum[8][16];
  float corr[16][4];    // [c][hg]: the chunk's rescale factor of head 16 hg + c
  uint64_t grow[8];     // [wave]: lanes (heads) whose chunk maximum moves the reference
};

struct WideState {
  f32x4 O[16];
  float m_run, l_part;
  WaveRows cur, nxt;  // this wave's 8 rows of this chunk (staged) and of the next one (known)
  int32_t slot2;      // slot values of the chunk after next
};

// Per-lane constants of a wave's 5 row DMAs (8 rows of 592 LDS bytes from LDS byte 1024 i +
// 16 lane), the same for every wave and chunk, so they are computed once per block:
//  * dense[i][lane]: bit 31 set for a byte of the FP8 part, bit 30 for a lane inside the 8 rows;
//    low bits the byte offset from the part's base at the run's first row (e * stride + o);
//  * listed[i][lane]: bits 16.. the lane holding the row's source address (e, or 8 + e for the
//    RoPE part), bit 15 for a lane inside the 8 rows, bits 0..9 the row byte o.
// A lane on a row's 16 padding bytes reads the row's last 16 RoPE bytes again (they land in the
// padding, which nothing reads), so only the lanes past the 8 rows stay idle.
struct WideDmaTab {
  uint32_t dense[5][64];
  uint32_t listed[5][64];
};

__device__ __forceinline__ void wide_dma_table(const AttnArgs& a, WideDmaTab& t, int tid) {
  if (tid < 5 * 64) {
    const int i = tid >> 6, ln = tid & 63;
    const int b = 1024 * i + 16 * ln;
    const int e = b / kRowF8, o = min(b - e * kRowF8, kNope + 2 * kRope - 16);
    const bool nope = o < kNope, in = e < 8;
    const uint32_t stride = nope ? (uint32_t)a.cache.row_stride : (uint32_t)(2 * a.cache.rope_stride);
    const uint32_t off = in ? (uint32_t)e * stride + (uint32_t)o : 0u;
    t.dense[i][ln] = off | (nope ? 0x80000000u : 0u) | (in ? 0x40000000u : 0u);
    t.listed[i][ln] = ((uint32_t)(nope ? e : 8 + e) << 16) | (in ? 0x8000u : 0u) | (uint32_t)o;
  }
}

// stage_dense<0, 5, 8> from the table: the part bases are scalar, each lane adds its offset.
__device__ __forceinline__ void wide_stage_dense(const AttnArgs& a, int64_t row0, const WideDmaTab& t, uint8_t* dst,
                                                 int lane) {
  const int64_t r0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(row0 >> 32)) << 32) |
                               (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)row0));
  const uint64_t fp8 = reinterpret_cast<uint64_t>(a.cache.data) + (uint64_t)(r0 * a.cache.row_stride);
  const uint64_t rope = reinterpret_cast<uint64_t>(a.cache.rope) + (uint64_t)(r0 * 2 * a.cache.rope_stride) - kNope;
  uint32_t v[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) v[i] = t.dense[i][lane];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint64_t src = ((int32_t)v[i] < 0 ? fp8 : rope) + (uint64_t)(v[i] & 0x3FFFFFFFu);
    if (i < 4 || (v[i] & 0x40000000u))
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                       (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, 0, 0);
  }
}

// stage_rows<0, 5, 8> from the table (rows listed by address in w.src; invalid rows skipped).
__device__ __forceinline__ void wide_stage_rows(const WaveRows& w, const WideDmaTab& t, uint8_t* dst, int lane) {
  uint32_t v[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) v[i] = t.listed[i][lane];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int sl = (int)(v[i] >> 16);
    const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)w.src, sl, 64);
    const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(w.src >> 32), sl, 64);
    const uint64_t src = (((uint64_t)hi << 32) | lo) + (uint64_t)(v[i] & 0x3FFu);
    if ((v[i] & 0x8000u) && ((w.vmask >> (sl & 7)) & 1))
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                       (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, 0, 0);
  }
}

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// One chunk in buf whose rows the waves requested a chunk earlier: publish the chunk's scales
// and validity, wait for every wave's rows, request the next chunk's rows into nbuf, then
// scores, softmax, P to LDS and PV. The chunk buffers are distinct LDS objects, so reads of buf
// need not wait for the DMAs into nbuf.
template <bool kSparse>
__device__ __forceinline__ void wide_chunk(const AttnArgs& a, const QueryCtx& ctx, int qi, int64_t base, int64_t hi,
                                           const uint8_t* buf, uint8_t* nbuf, const F8Query& q, WideState& st,
                                           uint16_t* ps, uint16_t* pp, WideLds& wl, const WideDmaTab& dt, float sl2,
                                           int wave, int lane) {
  const int g = lane >> 4, c = lane & 15;
  const int hg = wave & 3, hf = wave >> 2;
  // this wave's rows of the chunk and the scales of its entries have landed: the memory
  // instructions issued after its DMAs are the previous chunk's last ones, one scale load and,
  // for listed rows, one slot load (each a single unconditional instruction), which may stay
  // in flight
  __builtin_amdgcn_s_waitcnt(kSparse ? 0x0F72 : 0x0F71);  // vmcnt(2) / vmcnt(1)
  if (lane < 8) {
    const bool ok = (st.cur.vmask >> lane) & 1u;
    wl.esc[8 * wave + lane] = st.cur.esc;
    wl.esc2[8 * wave + lane] = ok ? st.cur.esc * sl2 : 0.f;
    wl.bias[8 * wave + lane] = ok ? 0.f : -INFINITY;
  }
  lds_barrier();  // every wave's rows; the other buffer is free
  const bool more = base + kWCh < hi;
  if (more) {
    // lane-only DMA offsets are derived from an opaque copy of the lane index, so that they are
    // recomputed here instead of being kept live (and spilled) across the chunk loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    uint8_t* ndst = nbuf + 8 * wave * kRowF8;
    int64_t row0;
    if (!kSparse && dense_run<8>(a, ctx, base + kWCh + 8 * wave, hi, &row0)) {
      wide_stage_dense(a, row0, dt, ndst, ln);
    } else {
      zero_invalid_rows<8>(st.nxt, ndst, ln);
      wide_stage_rows(st.nxt, dt, ndst, ln);
    }
  }

  // scores of entries 32 hf + 16 u + 4 g + i (i < 4), head c of the wave's group
  float sv[2][4];
  float cmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e0 = 32 * hf + 16 * u;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, sr = s0;
    const uint8_t* rowp = buf + (e0 + c) * kRowF8 + 16 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(rowp + 128 * ks);
      uint4 x1 = make_uint4(0, 0, 0, 0);  // dims 448.. (K step 3, bytes 16-31) are RoPE bytes: zero
      if (ks < 3) x1 = *reinterpret_cast<const uint4*>(rowp + 128 * ks + 64);
      const i32x8 A = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      s0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, q.qh[ks], s0, 0, 0, 0, 127, 0,
                                                             (int)((q.sh >> (8 * ks)) & 255u));
      s1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, q.ql[ks], s1, 0, 0, 0, 127, 0,
                                                             (int)((q.sl >> (8 * ks)) & 255u));
    }
    const uint8_t* ropep = buf + (e0 + c) * kRowF8 + kNope + 16 * g;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 kv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ropep + 64 * ks));
      sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, q.qr[ks], sr, 0, 0, 0);
    }
    // scale * log2(e) * (entry scale * FP8 part + RoPE part); an invalid entry (zero row, zero
    // scale) scores -inf through its bias
    const float4 e4 = *reinterpret_cast<const float4*>(wl.esc2 + e0 + 4 * g);
    const float4 b4 = *reinterpret_cast<const float4*>(wl.bias + e0 + 4 * g);
    const float esc[4] = {e4.x, e4.y, e4.z, e4.w}, bias[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[u][i] = fmaf(esc[i], s0[i] + s1[i], fmaf(sr[i], sl2, bias[i]));
      cmax = fmaxf(cmax, sv[u][i]);
    }
  }
  cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
  if (g == 0) wl.wmax[wave][c] = cmax;
  // lazy rescaling (both waves of the group see the same maxima, so they agree on the reference).
  // P is written against the current reference before the group's maxima are known, and each
  // wave publishes which of its heads would move the reference (a group's maximum exceeds it
  // by more than 2^8 exactly when one of its two halves does); one barrier publishes both. If
  // any head of the block moves its reference, every wave sees it in the same flags and the
  // block rewrites P, publishes the rescale factors and waits once more.
  const int prow = (16 * hg + c) * kWPRow;
  auto put_p = [&](float m_ref) {
    const bool none = m_ref == -INFINITY;
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e0 = 32 * hf + 16 * u + 4 * g;
      const float4 e4 = *reinterpret_cast<const float4*>(wl.esc + e0);
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = none ? 0.f : __builtin_amdgcn_exp2f(sv[u][i] - m_ref);
        psum += p[i];
      }
      *reinterpret_cast<uint2*>(ps + prow + e0) = make_uint2(pk_bf16(p[0] * e4.x, p[1] * e4.y), pk_bf16(p[2] * e4.z, p[3] * e4.w));
      *reinterpret_cast<uint2*>(pp + prow + e0) = make_uint2(pk_bf16(p[0], p[1]), pk_bf16(p[2], p[3]));
    }
    return psum;
  };
  float psum = put_p(st.m_run);
  const uint64_t mine = __ballot(cmax > st.m_run + 8.f);
  if (lane == 0) wl.grow[wave] = mine;
  lds_barrier();
  uint64_t any = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) any |= wl.grow[w];
  const bool rescale = any != 0;  // the same in every wave of the block
  if (rescale) {
    cmax = fmaxf(wl.wmax[hg][c], wl.wmax[hg + 4][c]);
    const bool grow = cmax > st.m_run + 8.f;
    const float m_ref = grow ? cmax : st.m_run;
    const float corr = grow ? __builtin_amdgcn_exp2f(st.m_run - cmax) : 1.f;
    psum = put_p(m_ref);
    st.l_part = st.l_part * corr + psum;
    st.m_run = m_ref;
    if (hf == 0 && g == 0) wl.corr[c][hg] = corr;
    lds_barrier();
  } else {
    st.l_part = st.l_part * 1.f + psum;
  }
  // O^T (8 x 2 tiles of 16 dims x 16 heads: this wave's 128 dims of 32 heads) += V^T P^T over
  // the chunk's 64 entries; first the rescale of the heads whose reference maximum grew
  const int dq = wave & 3, hh = wave >> 2;
  if (rescale) {
    const float2 cr = *reinterpret_cast<const float2*>(&wl.corr[c][2 * hh]);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      st.O[dt] *= cr.x;
      st.O[8 + dt] *= cr.y;
    }
  }
  const int r = c >> 1, hsel = c & 1;
  const int nf = dq < 3 ? 8 : 4;  // FP8 dim tiles of this wave; the last quarter ends with RoPE
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    bf16x8 Bh[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
      Bh[ht] = __builtin_bit_cast(bf16x8,
                                  *reinterpret_cast<const uint4*>(ps + (32 * hh + 16 * ht + c) * kWPRow + 32 * kk + 8 * g));
    const uint8_t* vp = buf + (32 * kk + 8 * g + r) * kRowF8 + 128 * dq + 8 * hsel;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      if (dt < nf) {
        const i32x2_t t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vp + 16 * dt));
        const bf16x8 av = fp8x8_to_bf16x8((uint32_t)t[0], (uint32_t)t[1]);
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
          st.O[8 * ht + dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, Bh[ht], st.O[8 * ht + dt], 0, 0, 0);
      }
    }
    if (dq == 3) {
      // RoPE dims: bf16 rows, P without the entry scales
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
        Bh[ht] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(pp + (32 * hh + 16 * ht + c) * kWPRow + 32 * kk + 8 * g));
      const int rs = c >> 2, qd = c & 3;
      const uint8_t* v0 = buf + (32 * kk + 8 * g + rs) * kRowF8 + kNope + 8 * qd;
      const uint8_t* v1 = v0 + 4 * kRowF8;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + 32 * dt));
        const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v1 + 32 * dt));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
          st.O[8 * ht + 4 + dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, Bh[ht], st.O[8 * ht + 4 + dt], 0, 0, 0);
      }
    }
  }
  {
    // rows of the chunk after next from their prefetched slots; slots one further ahead
    const int64_t b2 = base + 2 * kWCh + 8 * wave;
    st.cur = st.nxt;
    int64_t row0;
    if (!kSparse && dense_run<8>(a, ctx, b2, hi, &row0)) st.nxt = dense_rows<8>(a, row0, lane);
    else st.nxt = wave_rows<kSparse, 8>(a, ctx, b2, hi, st.slot2, lane);
    st.slot2 = prefetch_slot<kSparse, 8>(a, qi, b2 + kWCh, lane);
  }
}

template <bool kSparse>
__global__ __launch_bounds__(512, 1) void attn_wide_kernel(AttnArgs a, int n_hg, int total) {
  __shared__ __attribute__((aligned(16))) uint8_t buf0[kWBuf];
  __shared__ __attribute__((aligned(16))) uint8_t buf1[kWBuf];
  __shared__ __attribute__((aligned(16))) uint16_t ps[64 * kWPRow];  // [64 heads][entries] P x entry scale
  __shared__ __attribute__((aligned(16))) uint16_t pp[64 * kWPRow];  // [64 heads][entries] P
  __shared__ __attribute__((aligned(16))) WideLds wl;
  __shared__ WideDmaTab dt;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  if (id >= total) return;
  wide_dma_table(a, dt, threadIdx.x);
  const int s = id % a.n_split;
  const int rest = id / a.n_split;
  const int hg64 = rest % n_hg;
  const int qi = rest / n_hg;
  const int H = a.H;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int hg = wave & 3, hf = wave >> 2;
  const int head = 64 * hg64 + 16 * hg + c;

  const int64_t lo = (int64_t)s * a.per_split;
  const QueryCtx ctx = query_ctx(a, qi);
  const int64_t N = ctx.n_c + ctx.n_w;
  const int64_t hi = min<int64_t>(N, lo + a.per_split);
  WideState st;
  {
    const int64_t b0 = lo + 8 * wave;
    const int32_t s0 = prefetch_slot<kSparse, 8>(a, qi, b0, lane);
    const int32_t s1 = prefetch_slot<kSparse, 8>(a, qi, b0 + kWCh, lane);
    st.slot2 = prefetch_slot<kSparse, 8>(a, qi, b0 + 2 * kWCh, lane);
    st.cur = wave_rows<kSparse, 8>(a, ctx, b0, hi, s0, lane);
    st.nxt = wave_rows<kSparse, 8>(a, ctx, b0 + kWCh, hi, s1, lane);
    lds_barrier();  // the DMA table
    if (lo < hi) {
      uint8_t* dst = buf0 + 8 * wave * kRowF8;
      zero_invalid_rows<8>(st.cur, dst, lane);
      wide_stage_rows(st.cur, dt, dst, lane);
    }
  }
  // the first chunk's rows are in flight while the query is split into its FP8 parts
  const F8Query q = rows_query(static_cast<const uint16_t*>(a.q) + ((int64_t)qi * H + head) * kD, lane);
#pragma unroll
  for (int j = 0; j < 16; ++j) st.O[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_part = 0.f;
  const float sl2 = a.scale * kLog2e;
  // the query's loads and the first chunk's rows have landed (the first chunk waits for its rows
  // anyway); without this wait hipcc may wait for every load before the chunks' RoPE scores
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // unrolled by two so that each call names its chunk buffers statically
  for (int64_t base = lo; base < hi; base += 2 * kWCh) {
    wide_chunk<kSparse>(a, ctx, qi, base, hi, buf0, buf1, q, st, ps, pp, wl, dt, sl2, wave, lane);
    if (base + kWCh >= hi) break;
    wide_chunk<kSparse>(a, ctx, qi, base + kWCh, hi, buf1, buf0, q, st, ps, pp, wl, dt, sl2, wave, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);

  // the softmax denominator of head c: this lane's entries, the lane groups, then the two halves
  float L = st.l_part;
  L += __shfl_xor(L, 16, 64);
  L += __shfl_xor(L, 32, 64);
  if (g == 0) wl.wsum[wave][c] = L;
  __syncthreads();
  L = wl.wsum[hg][c] + wl.wsum[hg + 4][c];
  const float lse = L > 0.f ? (st.m_run + log2f(L)) * kLn2 : -INFINITY;
  if (hf == 0 && g == 0) {
    const int64_t hrow = (int64_t)qi * H + head;
    if (a.n_split == 1) a.lse[hrow] = lse;
    else a.part_lse[((int64_t)qi * a.n_split + s) * H + head] = lse;
  }
  // this wave's output: dims 128 (wave & 3) + 16 dt + 4 g of head 64 hg64 + 32 (wave >> 2) + 16 ht + c
  // (the RoPE dims follow the FP8 dims 384 .. 447, so the dims stay contiguous)
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int hl = 32 * (wave >> 2) + 16 * ht;  // head tile within the 64
    const float Lh = wl.wsum[hl >> 4][c] + wl.wsum[(hl >> 4) + 4][c];
    const float inv = Lh > 0.f ? 1.f / Lh : 0.f;
    int head_o = 64 * hg64 + hl + c;
    asm volatile("" : "+v"(head_o));
    const int64_t hrow = (int64_t)qi * H + head_o;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 128 * (wave & 3) + 16 * dt + 4 * g;
      const f32x4 acc = st.O[8 * ht + dt] * inv;
      if (a.n_split == 1) {
        if (a.o_dtype == HCA_BF16) {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + hrow * kD + d) =
              make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + hrow * kD + d) = acc;
        }
      } else {
        const int64_t pi = ((int64_t)qi * a.n_split + s) * H + head_o;
        *reinterpret_cast<f32x4*>(a.part_o + pi * kD + d) = acc;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Log-sum-exp merge of the split partials of one (query, head) over the dims held by a lane
// (V = f32x4 for 4 dims at po + d, float for one). The lse values and partial outputs of kG
// splits are loaded at once (positions past S clamp to the last split and get weight 0), so a
// merge of up to kG splits is one memory round trip. Returns the merged sum and, through *M and
// *L, the max and the scaled denominator.
template <typename V>
__device__ __forceinline__ V merge_splits(const float* pl, const float* po, int S, int H, int64_t sstride, float* M,
                                          float* L) {
  constexpr int kG = 16;
  V acc = V{};
  float m = -INFINITY, l_sum = 0.f;
  for (int s0 = 0; s0 < S; s0 += kG) {
    float l[kG];
    V v[kG];
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      const int s = min(s0 + i, S - 1);
      l[i] = pl[(int64_t)s * H];
      v[i] = *reinterpret_cast<const V*>(po + s * sstride);
    }
    float gm = m;
#pragma unroll
    for (int i = 0; i < kG; ++i)
      if (s0 + i < S) gm = fmaxf(gm, l[i]);
    if (gm == -INFINITY) continue;  // nothing visible so far
    const float corr = expf(m - gm);  // 0 while m is -inf
    acc *= corr;
    l_sum *= corr;
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      const float w = (s0 + i < S && l[i] != -INFINITY) ? expf(l[i] - gm) : 0.f;
      acc += w * v[i];
      l_sum += w;
    }
    m = gm;
  }
  *M = m;
  *L = l_sum;
  return acc;
}

// Merge of the split partials. grid = (H, nq), 128 threads; a thread takes 4 dims (a vector
// pass over D & ~3 dims, then single dims).
__device__ __forceinline__ void combine_one(const MergeArgs& a, int h, int qi) {
  const int tid = threadIdx.x;
  const int S = a.n_split, H = a.H, D = a.D;
  const float* pl = a.part_lse + (int64_t)qi * S * H + h;
  const float* po = a.part_o + ((int64_t)qi * S * H + h) * D;
  const int64_t sstride = (int64_t)H * D, orow = ((int64_t)qi * H + h) * D;
  const int D4 = D & ~3;
  float M = -INFINITY, L = 0.f;
  for (int d = tid * 4; d < D4; d += 512) {
    f32x4 acc = merge_splits<f32x4>(pl, po + d, S, H, sstride, &M, &L);
    acc *= L > 0.f ? 1.f / L : 0.f;
    if (a.o_dtype == HCA_BF16) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + orow + d) =
          make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + orow + d) = acc;
    }
  }
  for (int d = D4 + tid; d < D; d += 128) {
    float acc = merge_splits<float>(pl, po + d, S, H, sstride, &M, &L);
    acc *= L > 0.f ? 1.f / L : 0.f;
    if (a.o_dtype == HCA_BF16) static_cast<uint16_t*>(a.o)[orow + d] = (uint16_t)(pack_bf16x2(acc, 0.f) & 0xFFFFu);
    else static_cast<float*>(a.o)[orow + d] = acc;
  }
  // thread 0 merged dim 0 (vector or single pass), so it holds the (dim-independent) M and L
  if (tid == 0) a.lse[(int64_t)qi * H + h] = L > 0.f ? M + logf(L) : -INFINITY;
}

__device__ __forceinline__ MergeArgs merge_args(const AttnArgs& a) {
  MergeArgs m;
  m.part_o = a.part_o;
  m.part_lse = a.part_lse;
  m.o = a.o;
  m.lse = a.lse;
  m.nq = a.nq;
  m.H = a.H;
  m.D = a.D;
  m.n_split = a.n_split;
  m.o_dtype = a.o_dtype;
  return m;
}

__global__ __launch_bounds__(128) void combine_kernel(AttnArgs a) {
  combine_one(merge_args(a), blockIdx.x, blockIdx.y);
}

// Deferred merge of up to two calls: grid = (max heads, nq_a + nq_b); rows y < nq_a are call a's.
__global__ __launch_bounds__(128) void merge2_kernel(MergeArgs a, MergeArgs b) {
  const int y = blockIdx.y;
  const bool first = y < a.nq;
  const MergeArgs& m = first ? a : b;
  const int qi = first ? y : y - a.nq;
  if ((int)blockIdx.x >= m.H) return;
  combine_one(m, blockIdx.x, qi);
}

}  // namespace

// Both stores split with 448 FP8 + 64 bf16 dims, rows addressable with 32-bit indices.
bool attn_fp8_supported(const StoreView& c, const StoreView& w) {
  // row strides below 2^26 bytes keep the byte offsets within a wave's rows in 32 bits
  auto ok = [](const StoreView& v) {
    return v.layout == HCA_LAYOUT_SPLIT && v.d_nope == kNope && v.d_rope == kRope && v.n_rows < (1ll << 31) &&
           v.row_stride < (1ll << 26) && v.rope_stride < (1ll << 25);
  };
  return ok(c) && ok(w);
}

bool attn_mfma_supported(int q_dtype, int o_dtype, const StoreView& c, const StoreView& w, int H, int D) {
  auto ok_store = [](const StoreView& v) {
    if (v.layout == HCA_LAYOUT_BF16) return true;
    return v.layout == HCA_LAYOUT_SPLIT && v.d_nope % 8 == 0 && v.d_rope % 8 == 0;
  };
  return q_dtype == HCA_BF16 && (o_dtype == HCA_BF16 || o_dtype == HCA_F32) && D == kD && H % 16 == 0 &&
         ok_store(c) && ok_store(w);
}

void attn_split_policy(int nq, int H, int D, int64_t max_entries, bool mfma, int* n_split, int* per_split) {
  (void)D;
  const int n_hg = mfma ? H / 16 : 1;
  const int64_t align = mfma ? 4 * kChunk : kValuChunk;
  const int64_t target = mfma ? 256 : 512;  // MFMA kernels run one block per CU
  int64_t want = (target + (int64_t)nq * n_hg - 1) / ((int64_t)nq * n_hg);
  const int64_t max_split = std::max<int64_t>(1, (max_entries + align - 1) / align);
  want = std::max<int64_t>(1, std::min(want, max_split));
  int64_t per = (max_entries + want - 1) / want;
  per = std::max<int64_t>(align, (per + align - 1) / align * align);
  const int64_t ns = std::max<int64_t>(1, (max_entries + per - 1) / per);
  *n_split = (int)ns;
  *per_split = (int)per;
}

// The wide kernel: blocks of 64 heads and chunks of 64 entries; about 256 blocks in all (one per
// CU), each split a whole number of chunks.
void attn_split_policy_wide(int nq, int H, int64_t max_entries, int* n_split, int* per_split) {
  const int64_t blocks_per_split = (int64_t)nq * std::max(1, H / 64);
  const int64_t want = std::max<int64_t>(1, (256 + blocks_per_split - 1) / blocks_per_split);
  const int64_t chunks = std::max<int64_t>(1, (max_entries + kWCh - 1) / kWCh);
  const int64_t per = ((chunks + want - 1) / want) * kWCh;
  *per_split = (int)per;
  *n_split = (int)std::max<int64_t>(1, (max_entries + per - 1) / per);
}

// Taken for calls with many queries (prefill); decode keeps attn_fp8_kernel, whose 16-head blocks
// write a quarter of the split-K partials.
bool attn_wide_supported(int q_dtype, const StoreView& c, const StoreView& w, int H, int nq) {
  return q_dtype == HCA_BF16 && H % 64 == 0 && nq >= 64 && attn_fp8_supported(c, w);
}

// The row-owning kernel serves all 64 heads of a query per block. It is chosen when there are
// enough (query, split) blocks to fill the chip on their own (many queries, as in prefill);
// with few queries the per-head-group kernel's four blocks per split range fill it better.
bool attn_rows_eligible(const AttnArgs& a) {
  return a.H == 16 * kRowsWaves && (int64_t)a.nq * a.n_split >= 256;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s, bool combine, const IndexArgs* sel) {
  const bool mfma = a.q_dtype == HCA_BF16;
  const bool fp8 = mfma && attn_fp8_supported(a.cache, a.win);
  const bool wide = attn_wide_supported(a.q_dtype, a.cache, a.win, a.H, a.nq);
  // a selection to run with this call shares the grid of the dense attn_fp8 or attn_mfma kernel;
  // beside any other kernel it is launched first on the same stream
  const bool dense_sel = sel && sel->nq > 0 && !wide && !a.idx;
  const bool fused = dense_sel && fp8 && !attn_rows_eligible(a);
  const bool fused_bf16 = dense_sel && !fp8 && mfma;
  if (sel && !fused && !fused_bf16) {
    const hipError_t e = launch_index_topk(*sel, false, true, s);
    if (e != hipSuccess) return e;
  }
  if (wide) {
    const int n_hg = a.H / 64;
    const int total = a.nq * a.n_split * n_hg;
    const int grid = (total + 7) / 8 * 8;
    if (a.idx) hipLaunchKernelGGL(attn_wide_kernel<true>, dim3(grid), dim3(512), 0, s, a, n_hg, total);
    else hipLaunchKernelGGL(attn_wide_kernel<false>, dim3(grid), dim3(512), 0, s, a, n_hg, total);
  } else if (fp8 && attn_rows_eligible(a)) {
    const int total = a.nq * a.n_split;
    const int grid = (total + 7) / 8 * 8;
    if (a.idx) hipLaunchKernelGGL(attn_rows_kernel<true>, dim3(grid), dim3(64 * kRowsWaves), 0, s, a, total);
    else hipLaunchKernelGGL(attn_rows_kernel<false>, dim3(grid), dim3(64 * kRowsWaves), 0, s, a, total);
  } else if (fp8) {
    const int n_hg = a.H / 16;
    const int total = a.nq * a.n_split * n_hg;
    const int grid = (total + 7) / 8 * 8;
    if (fused) {
      const int n_sel = (sel->nq + 7) / 8 * 8;
      hipLaunchKernelGGL(select_attn_fp8_kernel, dim3(n_sel + grid), dim3(512), 0, s, *sel, n_sel, a, n_hg, total);
    } else if (a.idx) {
      hipLaunchKernelGGL(attn_fp8_kernel<true>, dim3(grid), dim3(512), 0, s, a, n_hg, total);
    } else {
      hipLaunchKernelGGL(attn_fp8_kernel<false>, dim3(grid), dim3(512), 0, s, a, n_hg, total);
    }
  } else if (mfma) {
    const int n_hg = a.H / 16;
    const int total = a.nq * a.n_split * n_hg;
    const int grid = (total + 7) / 8 * 8;
    if (fused_bf16) {
      const int n_sel = (sel->nq + 7) / 8 * 8;
      hipLaunchKernelGGL(select_attn_mfma_kernel, dim3(n_sel + grid), dim3(256), kMfmaLds, s, *sel, n_sel, a, n_hg,
                         total);
    } else {
      hipLaunchKernelGGL(attn_mfma_kernel, dim3(grid), dim3(256), kMfmaLds, s, a, n_hg, total);
    }
  } else {
    static_assert(kValuChunk == 16, "attn_valu_lds_bytes assumes 16-entry chunks");
    hipLaunchKernelGGL(attn_valu_kernel, dim3(a.n_split, a.nq), dim3(256), attn_valu_lds_bytes(a.H, a.D), s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.n_split > 1 && combine) {
    hipLaunchKernelGGL(combine_kernel, dim3(a.H, a.nq), dim3(128), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_merge(const MergeArgs& a, const MergeArgs* b, hipStream_t s) {
  // a call that was not split wrote its output itself: it takes no rows of the merge grid
  MergeArgs ma = a, mb{};
  if (ma.n_split <= 1) ma.nq = 0;
  if (b) {
    mb = *b;
    if (mb.n_split <= 1) mb.nq = 0;
  }
  const int rows = ma.nq + mb.nq;
  if (rows == 0) return hipSuccess;
  const int heads = std::max(ma.nq > 0 ? ma.H : 0, mb.nq > 0 ? mb.H : 0);
  hipLaunchKernelGGL(merge2_kernel, dim3(heads, rows), dim3(128), 0, s, ma, mb);
  return hipGetLastError();
}

// Scratch of hca_dense_mqa_attn_noalloc (its split-K partials): a file-scope device array, one
// copy per GPU the library runs on, held until the process ends. Host code never uses the
// array's name as an address (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, once per device with that device current, and is
// what the kernels receive.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t attention_init() {
  hipError_t e = hipFuncSetAttribute((const void*)attn_mfma_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kMfmaLds);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)select_attn_mfma_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kMfmaLds);
  if (e != hipSuccess) return e;
  // the float32 kernel's LDS grows with H * D (66,752 bytes at 16 heads of 512)
  return hipFuncSetAttribute((const void*)attn_valu_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)kAttnValuMaxLds);
}

}  // namespace hca
