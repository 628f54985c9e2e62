// CSA / HCA KV compression for gfx950.
//
// Method: hyper.ai paper page for arXiv 2606.19348 ("DeepSeek-V4"), section 方法
// (Method), CSA paragraph (every m tokens -> one entry, learnable compression
// weights and a position bias) and HCA paragraph (every m' tokens, no overlap).
// Entry j covers raw positions [j*m - (w-m), j*m + m) (>= 0); per channel c the
// entry is the softmax over window positions p of z[t,c] + bias[p,c], used as
// weights on x[t,c].
//
// Design: HBM-bound streaming reduction. One wavefront owns one entry; each lane
// owns VEC consecutive channels (16 bytes of a raw row), so every row load of a
// wave is one fully coalesced 64 x 16 B transaction. Window positions are taken
// in blocks of 8 rows held in registers (8 independent 16-byte loads in flight
// per lane) with an online softmax across blocks, so HCA's 128-row windows need
// one exp per element plus one per block. The output encoding (float32, bf16,
// or FP8 E4M3 + per-entry power-of-two scale + bf16 RoPE dims) is fused into
// the store; the FP8 scale needs one wave-wide max. MXFP4 outputs (the indexer keys) take one
// max per 32-channel block across the lanes that hold it.
//
// Decode: decode_append_kernel runs one sequence per block and one wave per task (CSA entry,
// HCA entry, indexer key, window row, ring write). The entry tasks call the same per-entry
// reduction as compress_kernel, reading the raw ring and the step's own token through a
// row-source functor, so an entry emitted at decode time equals the bulk one bit for bit.
#include "common.h"
#include "internal.h"

namespace hca {
namespace {

template <typename T>
struct Raw;
template <>
struct Raw<float> {
  static constexpr int VEC = 4;
  __device__ static void load(const float* p, float* v) {
    float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
  __device__ static float scalar(const float* p) { return *p; }
  // value v (compile-time) of a 16-byte packet
  __device__ static float get(uint4 x, int v) {
    const uint32_t w = v == 0 ? x.x : v == 1 ? x.y : v == 2 ? x.z : x.w;
    return __uint_as_float(w);
  }
};
template <>
struct Raw<uint16_t> {
  static constexpr int VEC = 8;
  __device__ static void load(const uint16_t* p, float* v) {
    uint4 x = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static float scalar(const uint16_t* p) { return bf16_to_f32(*p); }
  // value v (compile-time) of a 16-byte packet
  __device__ static float get(uint4 x, int v) {
    const uint32_t w = (v >> 1) == 0 ? x.x : (v >> 1) == 1 ? x.y : (v >> 1) == 2 ? x.z : x.w;
    return __uint_as_float((v & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
};

// Smallest e >= -126 with amax <= 448 * 2^e (0 for amax == 0); 448 = 1.75 * 2^8.
__device__ __forceinline__ int fp8_scale_exp(float amax) {
  if (amax == 0.f) return 0;
  const uint32_t u = __float_as_uint(amax);
  const uint32_t ef = (u >> 23) & 0xFFu;
  if (ef == 0) return -126;
  const int e = (int)ef - 127 - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -126 ? -126 : e;
}

// Writes entry row orow from y: lane's channels (g * 64 + lane) * VEC + v, g < G. Float32 and
// bf16 rows are RNE; the split layout takes the smallest power-of-two scale with amax <= 448 *
// scale (one wave max), E4M3 codes (RNE, saturating) for the first d_nope dims and bf16 for the
// rest.
template <int VEC, int G, int LAYOUT>
__device__ __forceinline__ void store_entry(const CompressArgs& a, int64_t orow, const float (&y)[G][VEC], int lane) {
  constexpr int GMAX = G;
  if (LAYOUT == HCA_LAYOUT_F32) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      const int c0 = (g * 64 + lane) * VEC;
      if (c0 >= a.D) continue;
      float* op = static_cast<float*>(a.out) + orow * a.out_stride + c0;
#pragma unroll
      for (int v = 0; v < VEC; v += 4)
        *reinterpret_cast<float4*>(op + v) = make_float4(y[g][v], y[g][v + 1], y[g][v + 2], y[g][v + 3]);
    }
  } else if (LAYOUT == HCA_LAYOUT_BF16) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      const int c0 = (g * 64 + lane) * VEC;
      if (c0 >= a.D) continue;
      uint16_t* op = static_cast<uint16_t*>(a.out) + orow * a.out_stride + c0;
      if (VEC == 8) {
        *reinterpret_cast<uint4*>(op) = make_uint4(pack_bf16x2(y[g][0], y[g][1]), pack_bf16x2(y[g][2], y[g][3]),
                                                   pack_bf16x2(y[g][4], y[g][5]), pack_bf16x2(y[g][6], y[g][7]));
      } else {
        *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16x2(y[g][0], y[g][1]), pack_bf16x2(y[g][2], y[g][3]));
      }
    }
  } else if (LAYOUT == HCA_LAYOUT_MXFP4) {
    // blocks of 32 channels = LPB consecutive lanes: shared exponent floor(log2 amax) - 2
    // (>= -127; -127 for a zero block), E2M1 codes of y * 2^-e, nearest with ties to the even
    // code (the thresholds below: strict at ties that fall to the lower, even code), saturating
    // at 6; zero magnitudes are +0. Two codes per byte, channel 2i in the low nibble of byte i.
    constexpr int LPB = 32 / VEC;
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      const int c0 = (g * 64 + lane) * VEC;
      float amax = 0.f;
      if (c0 < a.D) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) amax = fmaxf(amax, fabsf(y[g][v]));
      }
#pragma unroll
      for (int off = 1; off < LPB; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
      if (c0 >= a.D) continue;
      const uint32_t ef = (__float_as_uint(amax) >> 23) & 0xFFu;
      const int ex = ef == 0 ? -127 : max((int)ef - 129, -127);
      const float inv = __builtin_ldexpf(1.0f, -ex);
      uint32_t word = 0;
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const float q = y[g][v] * inv;  // exact: a power-of-two scaling within range
        const float m = fabsf(q);
        uint32_t code = (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) +
                        (uint32_t)(m >= 1.75f) + (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) + (uint32_t)(m > 5.0f);
        if (code != 0 && (__float_as_uint(q) >> 31)) code |= 8u;
        word |= code << (4 * v);
      }
      uint8_t* op = static_cast<uint8_t*>(a.out) + orow * a.out_stride + c0 / 2;
      if (VEC == 8) *reinterpret_cast<uint32_t*>(op) = word;
      else *reinterpret_cast<uint16_t*>(op) = (uint16_t)word;
      if ((lane & (LPB - 1)) == 0)
        static_cast<uint8_t*>(a.out_rope)[orow * a.out_rope_stride + c0 / 32] = (uint8_t)(ex + 127);
    }
  } else {  // split: FP8 E4M3 non-RoPE dims with a per-entry power-of-two scale, bf16 RoPE dims
    float amax = 0.f;
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      const int c0 = (g * 64 + lane) * VEC;
      if (c0 < a.d_nope) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) amax = fmaxf(amax, fabsf(y[g][v]));
      }
    }
    amax = wave_max(amax);
    const int ex = fp8_scale_exp(amax);
    if (lane == 0) a.out_scale[orow] = ldexpf(1.0f, ex);
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      const int c0 = (g * 64 + lane) * VEC;
      if (c0 >= a.D) continue;
      if (c0 < a.d_nope) {
        float v[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) v[i] = fminf(fmaxf(ldexpf(y[g][i], -ex), -448.f), 448.f);
        uint8_t* op = static_cast<uint8_t*>(a.out) + orow * a.out_stride + c0;
        uint32_t w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w0, true);
        if (VEC == 8) {
          uint32_t w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
          w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], w1, true);
          *reinterpret_cast<uint2*>(op) = make_uint2(w0, w1);
        } else {
          *reinterpret_cast<uint32_t*>(op) = w0;
        }
      } else {
        uint16_t* op = static_cast<uint16_t*>(a.out_rope) + orow * a.out_rope_stride + (c0 - a.d_nope);
        if (VEC == 8) {
          *reinterpret_cast<uint4*>(op) = make_uint4(pack_bf16x2(y[g][0], y[g][1]), pack_bf16x2(y[g][2], y[g][3]),
                                                     pack_bf16x2(y[g][4], y[g][5]), pack_bf16x2(y[g][6], y[g][7]));
        } else {
          *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16x2(y[g][0], y[g][1]), pack_bf16x2(y[g][2], y[g][3]));
        }
      }
    }
  }
}

// Raw and logit rows of a contiguous input: position p is row p - first_pos.
template <typename T>
struct LinearRows {
  const T* raw;
  const T* lg;
  int64_t raw_stride, lg_stride, first_pos;
  __device__ const T* x(int64_t p) const { return raw + (p - first_pos) * raw_stride; }
  __device__ const T* z(int64_t p) const { return lg + (p - first_pos) * lg_stride; }
};

constexpr int kGMax = 2;  // column groups of 64*VEC channels: D <= 1024 (bf16) / 512 (f32)

constexpr int kPB = 8;  // window positions per register block of the online softmax

// Folds window positions pb .. pb + nb - 1 (nb <= kPB) of the entry whose window starts at
// absolute position `start` into the lane's running softmax state (max M, sum S, weighted sum A)
// of channels c0 .. c0 + VEC - 1.
template <typename T, bool SCALAR, class Rows>
__device__ __forceinline__ void fold_block(const CompressArgs& a, const Rows& rows, int64_t start, int pb, int nb,
                                           int c0, float (&M)[Raw<T>::VEC], float (&S)[Raw<T>::VEC],
                                           float (&A)[Raw<T>::VEC]) {
  constexpr int VEC = Raw<T>::VEC;
  float xv[kPB][VEC], zv[kPB][VEC];
#pragma unroll
  for (int i = 0; i < kPB; ++i) {
    if (i < nb) {
      const int64_t pos = start + pb + i;
      Raw<T>::load(rows.x(pos) + c0, xv[i]);
      if (SCALAR) {
        const float zz = Raw<T>::scalar(rows.z(pos));
#pragma unroll
        for (int v = 0; v < VEC; ++v) zv[i][v] = zz;
      } else {
        Raw<T>::load(rows.z(pos) + c0, zv[i]);
      }
      const float* bp = a.bias + (int64_t)(pb + i) * a.D + c0;
#pragma unroll
      for (int v = 0; v < VEC; v += 4) {
        float4 bb = *reinterpret_cast<const float4*>(bp + v);
        zv[i][v] += bb.x; zv[i][v + 1] += bb.y; zv[i][v + 2] += bb.z; zv[i][v + 3] += bb.w;
      }
    }
  }
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    float bm = zv[0][v];
#pragma unroll
    for (int i = 1; i < kPB; ++i)
      if (i < nb) bm = fmaxf(bm, zv[i][v]);
    const float mn = fmaxf(M[v], bm);
    const float corr = __expf(M[v] - mn);  // 0 on the first block (M = -inf)
    float s = S[v] * corr, acc = A[v] * corr;
#pragma unroll
    for (int i = 0; i < kPB; ++i) {
      if (i < nb) {
        const float pe = __expf(zv[i][v] - mn);
        s += pe;
        acc = fmaf(pe, xv[i][v], acc);
      }
    }
    M[v] = mn; S[v] = s; A[v] = acc;
  }
}

// Entry j into y (lane's channels (g * 64 + lane) * VEC + v): per channel the softmax over the
// window's positions of logit + bias, weighting the raw values. Window positions are taken in
// blocks of kPB rows held in registers, with an online softmax across blocks.
template <typename T, bool SCALAR, class Rows>
__device__ __forceinline__ void compress_entry(const CompressArgs& a, const Rows& rows, int64_t j,
                                               float (&y)[kGMax][Raw<T>::VEC], int lane) {
  constexpr int VEC = Raw<T>::VEC;
  const int64_t start = j * a.m - (a.w - a.m);  // absolute position of window position 0
  const int p0 = start < 0 ? (int)(-start) : 0;
#pragma unroll
  for (int g = 0; g < kGMax; ++g) {
    const int c0 = (g * 64 + lane) * VEC;
#pragma unroll
    for (int v = 0; v < VEC; ++v) y[g][v] = 0.f;
    if (c0 >= a.D) continue;
    float M[VEC], S[VEC], A[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) { M[v] = -INFINITY; S[v] = 0.f; A[v] = 0.f; }
    for (int pb = p0; pb < a.w; pb += kPB) fold_block<T, SCALAR>(a, rows, start, pb, min(kPB, a.w - pb), c0, M, S, A);
#pragma unroll
    for (int v = 0; v < VEC; ++v) y[g][v] = A[v] / S[v];
  }
}

template <typename T, int LAYOUT, bool SCALAR>
__global__ __launch_bounds__(256) void compress_kernel(CompressArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= a.n_entries) return;
  const LinearRows<T> rows{static_cast<const T*>(a.raw), static_cast<const T*>(a.logits), a.raw_stride,
                           a.logit_row_stride, a.first_pos};
  float y[kGMax][Raw<T>::VEC];
  compress_entry<T, SCALAR>(a, rows, a.first_entry + e, y, lane);
  store_entry<Raw<T>::VEC, kGMax, LAYOUT>(a, a.out_row0 + e, y, lane);
}

// CSA-shaped windows (w = 2m = 8) with D <= 64 VEC: one wave takes kRun consecutive entries
// and slides the window, so each raw and logit row is loaded once per wave instead of once per
// entry that covers it, and the position bias once per run instead of once per entry. The
// window's rows stay in registers in the input format; the next entry's four rows are
// requested before the current entry is reduced. Per entry the reduction is the same
// expression in the same order as compress_kernel's (positions before 0 weigh 0).
// Narrow rows (D <= 64 VEC / NR, e.g. the 64-dim indexer keys) run NR runs side by side in a
// wave, 64 / NR lanes each, so that every row load still spans the whole wave; this needs a
// layout whose store reduces within a row's lanes only (not the split layout's wave-wide max).
template <typename T, int LAYOUT, bool SCALAR, int NR>
__global__ __launch_bounds__(256) void compress_slide_kernel(CompressArgs a) {
  constexpr int VEC = Raw<T>::VEC;
  constexpr int W = 8, M = 4, kRun = 16, LPR = 64 / NR;
  static_assert(NR == 1 || LAYOUT != HCA_LAYOUT_SPLIT, "the split store reduces across the wave");
  const int lane = (threadIdx.x & 63) % LPR, sub = (threadIdx.x & 63) / LPR;
  const int64_t e0 = (((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * NR + sub) * kRun;
  if (e0 >= a.n_entries) return;
  const int ne = (int)min<int64_t>(kRun, a.n_entries - e0);
  const int c0 = lane * VEC;
  const int cc = c0 < a.D ? c0 : 0;  // lanes past D load channel 0 and store nothing
  const T* raw = static_cast<const T*>(a.raw);
  const T* lg = static_cast<const T*>(a.logits);
  float bias[W][VEC];
#pragma unroll
  for (int p = 0; p < W; ++p) {
    const float* bp = a.bias + (int64_t)p * a.D + cc;
#pragma unroll
    for (int v = 0; v < VEC; v += 4) {
      const float4 bb = *reinterpret_cast<const float4*>(bp + v);
      bias[p][v] = bb.x; bias[p][v + 1] = bb.y; bias[p][v + 2] = bb.z; bias[p][v + 3] = bb.w;
    }
  }
  // rows of positions pos0 .. pos0 + M - 1 (positions below 0 read row 0 of the input; masked)
  auto load_rows = [&](int64_t pos0, uint4 (&x)[M], uint4 (&z)[M], float (&zs)[M]) {
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int64_t r = max<int64_t>(pos0 + i - a.first_pos, 0);
      x[i] = *reinterpret_cast<const uint4*>(raw + r * a.raw_stride + cc);
      if (SCALAR) zs[i] = Raw<T>::scalar(lg + r * a.logit_row_stride);
      else z[i] = *reinterpret_cast<const uint4*>(lg + r * a.logit_row_stride + cc);
    }
  };
  const int64_t j0 = a.first_entry + e0;
  uint4 xr[W], zr[W], nx[M], nz[M];
  float zsr[W], nzs[M];
  {
    uint4 px[M], pz[M];
    float pzs[M];
    load_rows(j0 * M - (W - M), px, pz, pzs);  // the first window's first half
#pragma unroll
    for (int i = 0; i < M; ++i) { xr[M + i] = px[i]; zr[M + i] = pz[i]; zsr[M + i] = pzs[i]; }
  }
  load_rows(j0 * M, nx, nz, nzs);
  for (int k = 0; k < ne; ++k) {
    const int64_t j = j0 + k, start = j * M - (W - M);
#pragma unroll
    for (int i = 0; i < M; ++i) {
      xr[i] = xr[M + i]; zr[i] = zr[M + i]; zsr[i] = zsr[M + i];
      xr[M + i] = nx[i]; zr[M + i] = nz[i]; zsr[M + i] = nzs[i];
    }
    if (k + 1 < ne) load_rows((j + 1) * M, nx, nz, nzs);
    float y[1][VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      float zv[W];
#pragma unroll
      for (int p = 0; p < W; ++p) {
        const float zz = SCALAR ? zsr[p] : Raw<T>::get(zr[p], v);
        zv[p] = start + p >= 0 ? zz + bias[p][v] : -INFINITY;
      }
      float mn = zv[0];
#pragma unroll
      for (int p = 1; p < W; ++p) mn = fmaxf(mn, zv[p]);
      float s = 0.f, acc = 0.f;
#pragma unroll
      for (int p = 0; p < W; ++p) {
        const float pe = __expf(zv[p] - mn);
        s += pe;
        acc = fmaf(pe, Raw<T>::get(xr[p], v), acc);
      }
      y[0][v] = acc / s;
    }
    store_entry<VEC, 1, LAYOUT>(a, a.out_row0 + e0 + k, y, lane);
  }
}

template <typename T, int LAYOUT, int NR>
hipError_t launch_slide(const CompressArgs& a, hipStream_t s) {
  const int64_t per_block = 4 * NR * 16;  // 4 waves x NR runs x 16 entries
  const dim3 grid((unsigned)((a.n_entries + per_block - 1) / per_block)), block(256);
  if (a.logit_col_stride == 0)
    hipLaunchKernelGGL((compress_slide_kernel<T, LAYOUT, true, NR>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((compress_slide_kernel<T, LAYOUT, false, NR>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <typename T, int LAYOUT>
hipError_t launch_t(const CompressArgs& a, hipStream_t s) {
  constexpr int VEC = Raw<T>::VEC;
  if (a.m == 4 && a.w == 8 && a.D <= 64 * VEC) {
    if (LAYOUT != HCA_LAYOUT_SPLIT && a.D <= 8 * VEC) return launch_slide<T, LAYOUT, (LAYOUT != HCA_LAYOUT_SPLIT ? 8 : 1)>(a, s);
    if (LAYOUT != HCA_LAYOUT_SPLIT && a.D <= 16 * VEC) return launch_slide<T, LAYOUT, (LAYOUT != HCA_LAYOUT_SPLIT ? 4 : 1)>(a, s);
    return launch_slide<T, LAYOUT, 1>(a, s);
  }
  const dim3 grid((unsigned)((a.n_entries + 3) / 4)), block(256);
  if (a.logit_col_stride == 0)
    hipLaunchKernelGGL((compress_kernel<T, LAYOUT, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((compress_kernel<T, LAYOUT, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_layout(const CompressArgs& a, hipStream_t s) {
  switch (a.out_layout) {
    case HCA_LAYOUT_F32: return launch_t<T, HCA_LAYOUT_F32>(a, s);
    case HCA_LAYOUT_BF16: return launch_t<T, HCA_LAYOUT_BF16>(a, s);
    case HCA_LAYOUT_MXFP4: return launch_t<T, HCA_LAYOUT_MXFP4>(a, s);
    default: return launch_t<T, HCA_LAYOUT_SPLIT>(a, s);
  }
}

// Rows of one sequence at a decode step: the token at position t from the step's inputs, older
// positions t - R < p < t from the raw ring, row p mod R = tr - d (+ R when d > tr) for
// d = t - p and tr = t mod R.
struct RingRows {
  const uint16_t* ring_x;
  const uint16_t* ring_z;
  const uint16_t* in_x;
  const uint16_t* in_z;
  int64_t t;
  int tr, R, stride;
  __device__ int row(int64_t p) const {
    const int d = (int)(t - p);
    return tr - d + (d > tr ? R : 0);
  }
  __device__ const uint16_t* x(int64_t p) const { return p == t ? in_x : ring_x + (size_t)row(p) * stride; }
  __device__ const uint16_t* z(int64_t p) const { return p == t ? in_z : ring_z + (size_t)row(p) * stride; }
};

// store_entry for a layout known at run time (uniform across the wave).
template <int VEC, int G>
__device__ __forceinline__ void store_any(const CompressArgs& a, int layout, int64_t orow, const float (&y)[G][VEC],
                                          int lane) {
  switch (layout) {
    case HCA_LAYOUT_F32: store_entry<VEC, G, HCA_LAYOUT_F32>(a, orow, y, lane); break;
    case HCA_LAYOUT_BF16: store_entry<VEC, G, HCA_LAYOUT_BF16>(a, orow, y, lane); break;
    case HCA_LAYOUT_MXFP4: store_entry<VEC, G, HCA_LAYOUT_MXFP4>(a, orow, y, lane); break;
    default: store_entry<VEC, G, HCA_LAYOUT_SPLIT>(a, orow, y, lane); break;
  }
}

// Output fields of a store view for store_entry.
__device__ __forceinline__ void set_out(CompressArgs& c, const StoreView& v, int D) {
  c.D = D;
  c.d_nope = v.d_nope;
  c.out_layout = v.layout;
  c.out = const_cast<void*>(v.data);
  c.out_stride = v.row_stride;
  c.out_scale = const_cast<float*>(v.scale);
  c.out_rope = const_cast<void*>(v.rope);
  c.out_rope_stride = v.rope_stride;
}

// One block per sequence, wave k runs task k: 0 CSA entry, 1 HCA entry, 2 indexer key,
// 3 window rows, 4 ring row. The entry tasks read positions t - w + 1 .. t - 1 (t - m' + 1 ..)
// from the ring, none of which is the ring row that task 4 overwrites (R >= w, m').
// HCA: the entry's window starts at j m' >= 0, and compress_entry folds it in blocks of kPB
// positions; each block is folded here at the step that completes it, into the sequence's
// running state (M, S, A per channel, float32 [B, 3, D]), and the last block gives the entry,
// so the arithmetic is compress_entry's, step for step, at one block's latency per step.
__global__ __launch_bounds__(320) void decode_append_kernel(DecodeArgs a) {
  constexpr int VEC = 8;
  const int b = blockIdx.x;
  const int task = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t t = a.pos[b];
  if (t < 0) return;
  const int D = a.D, di = a.d_idx;
  const int tr = (int)(t % a.R);
  const uint16_t* xin = a.x + (int64_t)b * D;
  const size_t ring_row = (size_t)b * a.R + (size_t)tr;
  if (task == 0 || task == 2) {
    const bool idx = task == 2;
    if (idx && di == 0) return;
    if ((t + 1) % a.m != 0) return;
    const int64_t j = (t + 1) / a.m - 1;
    const StoreView& st = idx ? a.idx : a.csa;
    const int64_t orow = (idx ? a.idx_rb : a.csa_rb)[b] + j;
    if (orow < 0 || orow >= st.n_rows) return;
    const int width = idx ? di : D;
    CompressArgs c;
    c.m = a.m;
    c.w = a.w;
    c.bias = idx ? a.bias_idx : a.bias_csa;
    set_out(c, st, width);
    const RingRows rows{idx ? a.ring_ki + (size_t)b * a.R * di : a.ring_x + (size_t)b * a.R * D,
                        (idx ? a.ring_zi : a.ring_zc) + (size_t)b * a.R * width,
                        idx ? a.ki + (int64_t)b * di : xin,
                        (idx ? a.zi : a.zc) + (int64_t)b * width, t, tr, a.R, width};
    float y[kGMax][VEC];
    compress_entry<uint16_t, false>(c, rows, j, y, lane);
    store_any<VEC, kGMax>(c, st.layout, orow, y, lane);
  } else if (task == 1) {
    const int mp = a.m_prime;
    const int q = (int)((t + 1) % mp), seen = q == 0 ? mp : q;  // positions of the entry so far
    if (q % kPB != 0 && q != 0) return;                          // no block completes here
    const int pb = (seen - 1) / kPB * kPB, nb = seen - pb;
    const int64_t j = (t + 1 - seen) / mp, start = j * mp;
    CompressArgs c;
    c.m = mp;
    c.w = mp;
    c.bias = a.bias_hca;
    set_out(c, a.hca, D);
    const RingRows rows{a.ring_x + (size_t)b * a.R * D, a.ring_zh + (size_t)b * a.R * D, xin,
                        a.zh + (int64_t)b * D, t, tr, a.R, D};
    float* state = a.hca_state + (size_t)b * 3 * D;
    float y[kGMax][VEC];
#pragma unroll
    for (int g = 0; g < kGMax; ++g) {
      const int c0 = (g * 64 + lane) * VEC;
#pragma unroll
      for (int v = 0; v < VEC; ++v) y[g][v] = 0.f;
      if (c0 >= D) continue;
      float M[VEC], S[VEC], A[VEC];
      if (pb == 0) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) { M[v] = -INFINITY; S[v] = 0.f; A[v] = 0.f; }
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) { M[v] = state[c0 + v]; S[v] = state[D + c0 + v]; A[v] = state[2 * D + c0 + v]; }
      }
      fold_block<uint16_t, false>(c, rows, start, pb, nb, c0, M, S, A);
      if (q != 0) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) { state[c0 + v] = M[v]; state[D + c0 + v] = S[v]; state[2 * D + c0 + v] = A[v]; }
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) y[g][v] = A[v] / S[v];
      }
    }
    if (q != 0) return;
    const int64_t orow = a.hca_rb[b] + j;
    if (orow >= 0 && orow < a.hca.n_rows) store_any<VEC, kGMax>(c, a.hca.layout, orow, y, lane);
  } else if (task == 3) {
    // the token into both window rows of its position; the window's base position
    CompressArgs c;
    set_out(c, a.win, D);
    float y[kGMax][VEC];
#pragma unroll
    for (int g = 0; g < kGMax; ++g) {
      const int c0 = (g * 64 + lane) * VEC;
      if (c0 < D) Raw<uint16_t>::load(xin + c0, y[g]);
      else
#pragma unroll
        for (int v = 0; v < VEC; ++v) y[g][v] = 0.f;
    }
    const int64_t r0 = a.win_rb[b] + t % a.W;
    if (r0 >= 0 && r0 < a.win.n_rows) store_any<VEC, kGMax>(c, a.win.layout, r0, y, lane);
    if (r0 + a.W >= 0 && r0 + a.W < a.win.n_rows) store_any<VEC, kGMax>(c, a.win.layout, r0 + a.W, y, lane);
    if (lane == 0) a.win_pos0[b] = (int64_t)a.W * (max<int64_t>(0, t - a.W + 1) / a.W);
  } else {
    // ring row of position t: raw KV, both logit rows, the indexer-key pair
    auto copy = [&](uint16_t* dst, const uint16_t* src, int n) {
      for (int c0 = lane * VEC; c0 < n; c0 += 64 * VEC)
        *reinterpret_cast<uint4*>(dst + c0) = *reinterpret_cast<const uint4*>(src + c0);
    };
    copy(a.ring_x + ring_row * D, xin, D);
    copy(a.ring_zc + ring_row * D, a.zc + (int64_t)b * D, D);
    copy(a.ring_zh + ring_row * D, a.zh + (int64_t)b * D, D);
    if (di > 0) {
      copy(a.ring_ki + ring_row * di, a.ki + (int64_t)b * di, di);
      copy(a.ring_zi + ring_row * di, a.zi + (int64_t)b * di, di);
    }
  }
}

}  // namespace

hipError_t launch_decode_append(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(decode_append_kernel, dim3((unsigned)a.B), dim3(320), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  if (a.n_entries <= 0) return hipSuccess;
  return a.raw_dtype == HCA_F32 ? launch_layout<float>(a, s) : launch_layout<uint16_t>(a, s);
}

}  // namespace hca
