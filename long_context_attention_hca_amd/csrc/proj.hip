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
// flight; many rows take 128 x 128 LDS-tiled blocks (proj_tiled_kernel), or CT = 4 (each
// loaded fragment reused across 4 x 4 MFMAs) where the features are not a multiple of 128.
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

// Many rows: 128 x 128 output tiles per block of 4 waves (wave (wr, wc) owns rows 64 wr.. and
// features 64 wc.., 4 x 4 MFMA tiles), K in steps of 32 staged through LDS (double-buffered):
// each thread brings 16 bytes of the x tile and 16 of the weight tile per step, the next
// step's while the current one is multiplied. LDS rows are padded to 80 bytes so that the
// 16-byte fragment reads of 16 consecutive rows hit distinct banks.
constexpr int kTM = 128, kTN = 128, kTK = 32, kLRow = kTK * 2 + 16;  // LDS row: 64 + 16 pad bytes

__global__ __launch_bounds__(256, 2) void proj_tiled_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t la[2][kTM * kLRow];
  __shared__ __attribute__((aligned(16))) uint8_t lb[2][kTN * kLRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, c = lane & 15;
  const int wr = wave >> 1, wc = wave & 1;
  const int g = blockIdx.z;
  const int64_t row0 = (int64_t)blockIdx.y * kTM;
  const int col0 = blockIdx.x * kTN;
  // loader: thread tid brings row (tid >> 2) and row (tid >> 2) + 64 of each tile, 16 bytes at
  // k offset 8 (tid & 3)... as 2 rows x 16 bytes for x and 2 for the weights
  const int lr = tid >> 2, lk = 8 * (tid & 3);
  const uint16_t* xs[2];
  bool xv[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t r = row0 + lr + 64 * h;
    xv[h] = r < a.n;
    xs[h] = a.x + (xv[h] ? r : 0) * a.ldx + (int64_t)g * a.Kg + lk;
  }
  const uint16_t* ws[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) ws[h] = a.w + ((int64_t)g * a.Ng + col0 + lr + 64 * h) * a.Kg + lk;
  // the global loads of step kt + 3 are issued at step kt, into one of three register sets
  // rotated by unrolling (named sets, not an indexed array, so that they stay in registers)
  struct Tile { uint4 x[2], w[2]; };
  Tile s0, s1, s2;
  auto load = [&](Tile& d, int k) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      d.x[h] = xv[h] ? *reinterpret_cast<const uint4*>(xs[h] + k) : make_uint4(0, 0, 0, 0);
      d.w[h] = *reinterpret_cast<const uint4*>(ws[h] + k);
    }
  };
  auto store = [&](const Tile& d, int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<uint4*>(&la[buf][(lr + 64 * h) * kLRow + 2 * lk]) = d.x[h];
      *reinterpret_cast<uint4*>(&lb[buf][(lr + 64 * h) * kLRow + 2 * lk]) = d.w[h];
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nk = a.Kg / kTK;
  load(s0, 0);
  if (nk > 1) load(s1, kTK);
  if (nk > 2) load(s2, 2 * kTK);
  store(s0, 0);
  __syncthreads();
  // step kt multiplies LDS buffer kt & 1, writes step kt + 1's tile (set `next`) to the other
  // buffer and refills set `mine` (step kt's tile, already in LDS) with step kt + 3's
  auto step = [&](int kt, Tile& mine, const Tile& next) {
    const int cur = kt & 1;
    bf16x8 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&la[cur][(64 * wr + 16 * i + c) * kLRow + 16 * q]));
      fb[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&lb[cur][(64 * wc + 16 * i + c) * kLRow + 16 * q]));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    if (kt + 1 < nk) store(next, cur ^ 1);
    if (kt + 3 < nk) load(mine, (kt + 3) * kTK);
    __syncthreads();
  };
  int kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
    step(kt, s0, s1);
    step(kt + 1, s1, s2);
    step(kt + 2, s2, s0);
  }
  if (kt < nk) step(kt, s0, s1);  // at most two steps remain
  if (kt + 1 < nk) step(kt + 1, s1, s2);
  // lane (q, c) of tile (i, j): rows 64 wr + 16 i + 4 q + e, feature 64 wc + 16 j + c
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t r = row0 + 64 * wr + 16 * i + 4 * q + e;
      if (r >= a.n) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t o = r * a.ldy + (int64_t)g * a.Ng + col0 + 64 * wc + 16 * j + c;
        if (a.y_dtype == HCA_F32) static_cast<float*>(a.y)[o] = acc[i][j][e];
        else static_cast<uint16_t*>(a.y)[o] = (uint16_t)(pack_bf16x2(acc[i][j][e], 0.f) & 0xFFFFu);
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
  if (a.n >= 256 && a.Ng % kTN == 0) {
    const dim3 grid((unsigned)(a.Ng / kTN), (unsigned)((a.n + kTM - 1) / kTM), (unsigned)a.G);
    hipLaunchKernelGGL(proj_tiled_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
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
