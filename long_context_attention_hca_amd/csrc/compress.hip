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
// the store; the FP8 scale needs one wave-wide max.
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

template <typename T, int LAYOUT, bool SCALAR>
__global__ __launch_bounds__(256) void compress_kernel(CompressArgs a) {
  constexpr int VEC = Raw<T>::VEC;
  constexpr int GMAX = 2;  // column groups of 64*VEC channels: D <= 1024 (bf16) / 512 (f32)
  constexpr int PB = 8;    // window positions per register block
  const int lane = threadIdx.x & 63;
  const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= a.n_entries) return;
  const int64_t j = a.first_entry + e;
  const int64_t start = j * a.m - (a.w - a.m);  // absolute position of window position 0
  const int p0 = start < 0 ? (int)(-start) : 0;
  const T* raw = static_cast<const T*>(a.raw);
  const T* lg = static_cast<const T*>(a.logits);

  float y[GMAX][VEC];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    const int c0 = (g * 64 + lane) * VEC;
#pragma unroll
    for (int v = 0; v < VEC; ++v) y[g][v] = 0.f;
    if (c0 >= a.D) continue;
    float M[VEC], S[VEC], A[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) { M[v] = -INFINITY; S[v] = 0.f; A[v] = 0.f; }
    for (int pb = p0; pb < a.w; pb += PB) {
      const int nb = min(PB, a.w - pb);
      float xv[PB][VEC], zv[PB][VEC];
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        if (i < nb) {
          const int64_t r = start + pb + i - a.first_pos;
          Raw<T>::load(raw + r * a.raw_stride + c0, xv[i]);
          if (SCALAR) {
            const float zz = Raw<T>::scalar(lg + r * a.logit_row_stride);
#pragma unroll
            for (int v = 0; v < VEC; ++v) zv[i][v] = zz;
          } else {
            Raw<T>::load(lg + r * a.logit_row_stride + c0, zv[i]);
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
        for (int i = 1; i < PB; ++i)
          if (i < nb) bm = fmaxf(bm, zv[i][v]);
        const float mn = fmaxf(M[v], bm);
        const float corr = __expf(M[v] - mn);  // 0 on the first block (M = -inf)
        float s = S[v] * corr, acc = A[v] * corr;
#pragma unroll
        for (int i = 0; i < PB; ++i) {
          if (i < nb) {
            const float pe = __expf(zv[i][v] - mn);
            s += pe;
            acc = fmaf(pe, xv[i][v], acc);
          }
        }
        M[v] = mn; S[v] = s; A[v] = acc;
      }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) y[g][v] = A[v] / S[v];
  }

  store_entry<VEC, GMAX, LAYOUT>(a, a.out_row0 + e, y, lane);
}

// CSA-shaped windows (w = 2m = 8) with D <= 64 VEC: one wave takes kRun consecutive entries
// and slides the window, so each raw and logit row is loaded once per wave instead of once per
// entry that covers it, and the position bias once per run instead of once per entry. The
// window's rows stay in registers in the input format; the next entry's four rows are
// requested before the current entry is reduced. Per entry the reduction is the same
// expression in the same order as compress_kernel's (positions before 0 weigh 0).
template <typename T, int LAYOUT, bool SCALAR>
__global__ __launch_bounds__(256) void compress_slide_kernel(CompressArgs a) {
  constexpr int VEC = Raw<T>::VEC;
  constexpr int W = 8, M = 4, kRun = 16;
  const int lane = threadIdx.x & 63;
  const int64_t e0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kRun;
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

template <typename T, int LAYOUT>
hipError_t launch_t(const CompressArgs& a, hipStream_t s) {
  if (a.m == 4 && a.w == 8 && a.D <= 64 * Raw<T>::VEC) {
    const dim3 grid((unsigned)((a.n_entries + 63) / 64)), block(256);  // 4 waves x 16 entries
    if (a.logit_col_stride == 0)
      hipLaunchKernelGGL((compress_slide_kernel<T, LAYOUT, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((compress_slide_kernel<T, LAYOUT, false>), grid, block, 0, s, a);
    return hipGetLastError();
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
    default: return launch_t<T, HCA_LAYOUT_SPLIT>(a, s);
  }
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  if (a.n_entries <= 0) return hipSuccess;
  return a.raw_dtype == HCA_F32 ? launch_layout<float>(a, s) : launch_layout<uint16_t>(a, s);
}

}  // namespace hca
