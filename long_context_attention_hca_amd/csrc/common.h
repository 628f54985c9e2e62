// Device helpers shared by the gfx950 kernels of the hybrid-attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hca.h"

namespace hca {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Two E4M3 codes (bytes 0 and 1 of `w`, or 2 and 3 if hi) -> 2 bf16 values times `scale`.
// gfx950's v_cvt_scalef32_pk_bf16_fp8; exact for power-of-two scales.
__device__ __forceinline__ bf16x2 fp8x2_to_bf16x2(uint32_t w, float scale, bool hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, true)
            : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, false);
}

// Order-preserving map of a float32 to uint32 (larger float -> larger key); -0 maps as +0.
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);  // negative: ~u; otherwise u | sign bit
}

// Wave64 inclusive prefix sum in lane order: DPP row shifts by 1, 2, 4, 8 within each row of
// 16 lanes (lanes without a source add 0), then row broadcasts of lanes 15 and 31.
__device__ __forceinline__ uint32_t wave_incl_scan_add(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);
  return x;
}

// Wave64 maximum / minimum of unsigned values (the same DPP pattern; the result is read from
// lane 63 and returned to every lane).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return ~wave_max_u32(~x);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// XCD-aware block remap: hardware dispatches consecutive block ids round-robin over the 8
// XCDs; remapping makes logically adjacent work items (which share data through L2) land on
// the same XCD. `n` must be a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int n) { return (bid & 7) * (n >> 3) + (bid >> 3); }

}  // namespace hca
