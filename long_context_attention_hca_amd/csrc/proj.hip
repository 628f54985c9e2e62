// Grouped output projection for gfx950 (the step after core attention).
//
// Method: hyper.ai paper page for arXiv 2606.19348 ("DeepSeek-V4"), section 方法 (Method),
// CSA paragraph: core attention is followed by a grouped output projection to manage the
// computational cost. The heads are split into G groups; group g's concatenated head outputs
// (K = (h/G) D values per query) are multiplied by the group's own weight [N, K]:
//   y[r, g N + c] = sum_k x[r, g K + k] * w[g, c, k].
//
// Design: bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation, the weights as the B
// operand (a lane loads 8 consecutive k of one output feature: 16 bytes of a weight row) and
// the queries as the A operand (8 consecutive k of one row). A wave owns 64 rows x 16 CT
// output features; the K range of a tile is split over the KS waves of a block, whose partial
// tiles are summed in LDS in wave order (deterministic). Decode (a handful of rows) is bound
// by streaming the weights from HBM: CT = 1 and KS up to 8 put enough waves and loads in
// flight; many rows take CT = 4, which reuses each loaded fragment across 4 x 4 MFMAs.
#include "common.h"
#include "internal.h"

namespace hca {
namespace {

constexpr int kRT = 4;  // 16-row tiles per wave

template <int KS, int CT, int U>
__global__ __launch_bounds__(64 * KS) void proj_kernel(ProjArgs a) {
  __shared__ f32x4 red[KS > 1 ? KS - 1 : 1][kRT * CT][64];
  const int lane = threadIdx.x & 63, ks = threadIdx.x >> 6;
  const int q = lane >> 4, c = lane & 15;
  const int g = blockIdx.y;
  const int col0 = blockIdx.x * 16 * CT;
  const int64_t row0 = (int64_t)blockIdx.z * 16 * kRT;
  const int Kw = a.Kg / KS, kb = ks * Kw;
  const uint16_t* wp[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) wp[ct] = a.w + ((int64_t)g * a.Ng + col0 + 16 * ct + c) * a.Kg + kb + 8 * q;
  const uint16_t* xp[kRT];
  bool rv[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int64_t r = row0 + 16 * rt + c;
    rv[rt] = r < a.n;
    xp[rt] = a.x + (rv[rt] ? r : 0) * a.ldx + (int64_t)g * a.Kg + kb + 8 * q;
  }
  f32x4 acc[kRT][CT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](int k) {
    uint4 bw[CT], ax[kRT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) bw[ct] = *reinterpret_cast<const uint4*>(wp[ct] + k);
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
      ax[rt] = rv[rt] ? *reinterpret_cast<const uint4*>(xp[rt] + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ax[rt]),
                                                              __builtin_bit_cast(bf16x8, bw[ct]), acc[rt][ct], 0, 0, 0);
  };
  int k = 0;
  for (; k + 32 * U <= Kw; k += 32 * U) {
    // U steps' loads are issued together (independent), then their MFMAs
    uint4 bw[U][CT], ax[U][kRT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) bw[u][ct] = *reinterpret_cast<const uint4*>(wp[ct] + k + 32 * u);
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        ax[u][rt] = rv[rt] ? *reinterpret_cast<const uint4*>(xp[rt] + k + 32 * u) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ax[u][rt]),
                                                                __builtin_bit_cast(bf16x8, bw[u][ct]), acc[rt][ct], 0, 0,
                                                                0);
  }
  for (; k < Kw; k += 32) step(k);

  // partial tiles of waves 1.. to LDS; wave 0 adds them in wave order and writes y
  if (KS > 1) {
    if (ks > 0) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) red[ks - 1][rt * CT + ct][lane] = acc[rt][ct];
    }
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int w = 0; w < KS - 1; ++w)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[rt][ct] += red[w][rt * CT + ct][lane];
  }
  // lane (q, c) of tile (rt, ct) holds rows 16 rt + 4 q + i of feature col0 + 16 ct + c
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = row0 + 16 * rt + 4 * q + i;
      if (r >= a.n) continue;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int64_t o = r * a.ldy + (int64_t)g * a.Ng + col0 + 16 * ct + c;
        if (a.y_dtype == HCA_F32) static_cast<float*>(a.y)[o] = acc[rt][ct][i];
        else static_cast<uint16_t*>(a.y)[o] = (uint16_t)(pack_bf16x2(acc[rt][ct][i], 0.f) & 0xFFFFu);
      }
    }
  }
}

template <int KS, int CT, int U>
hipError_t launch_ks(const ProjArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.Ng / (16 * CT)), (unsigned)a.G, (unsigned)((a.n + 63) / 64));
  hipLaunchKernelGGL((proj_kernel<KS, CT, U>), grid, dim3(64 * KS), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int proj_split(const ProjArgs& a, int* ct) {
  *ct = (a.n >= 256 && a.Ng % 64 == 0) ? 4 : 1;
  const int64_t blocks = (int64_t)(a.Ng / (16 * *ct)) * a.G * ((a.n + 63) / 64);
  int ks = 1;
  while (ks < 8 && blocks * ks < 2048 && a.Kg % (32 * ks * 2) == 0) ks *= 2;
  return ks;
}

hipError_t launch_proj(const ProjArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  int ct;
  const int ks = proj_split(a, &ct);
  if (ct == 4) return launch_ks<1, 4, 2>(a, s);
  switch (ks) {
    case 8: return launch_ks<8, 1, 4>(a, s);
    case 4: return launch_ks<4, 1, 4>(a, s);
    case 2: return launch_ks<2, 1, 4>(a, s);
    default: return launch_ks<1, 1, 4>(a, s);
  }
}

}  // namespace hca
