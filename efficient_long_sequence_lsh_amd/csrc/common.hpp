// Internal helpers shared by the gfx950 kernels and the host launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlsh {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kWave = 64;

// bfloat16 <-> float on raw 16-bit patterns.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats -> packed bf16 pair (lo in bits 0..15) with gfx950's conversion
// instruction (v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN).
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Lane id within the 64-wide wavefront.
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Shuffle helpers (ds_bpermute based) for 32-bit values.
__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, kWave); }
__device__ __forceinline__ uint32_t shfl_xor_u(uint32_t v, int mask) {
  return static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), mask, kWave));
}
__device__ __forceinline__ double shfl_xor_d(double v, int mask) { return __shfl_xor(v, mask, kWave); }

__host__ __device__ constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// gfx950 transposing LDS read (ds_read_b64_tr_b16): within each group of 16
// lanes, lane 4k+q names 4 consecutive b16 (row k, columns 4q..4q+3 of a 4x16
// block) and lane i receives column i, i.e. the 4 rows' values at column i.
typedef short lds_s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  lds_s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(u32x2, r);
}

}  // namespace rlsh
