// Device-side helpers shared by the layer's HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef int i32x8_t __attribute__((ext_vector_type(8)));  // operand of the scaled (MX) MFMA

constexpr int kWave = 64;

// fp32 -> bf16 bits, round to nearest even (gfx950's v_cvt_pk_bf16_f32; a NaN stays a NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// The E8M0 scale byte as an fp32 multiplier 2^(s-127): exponent field s for 1..254,
// the fp32 subnormal 2^-127 for s = 0, NaN for s = 255.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  uint32_t bits = s << 23;
  bits = (s == 0u) ? 0x00400000u : bits;
  bits = (s == 255u) ? 0x7fc00000u : bits;
  return __uint_as_float(bits);
}

// Eight MXFP4 elements (one dword of codes: byte j = elements 2j (low nibble), 2j+1 (high))
// -> eight bf16 in element order, each multiplied by `scale`. Uses gfx950's scaled FP4
// convert, one instruction per byte; E2M1 times a power of two is exact in bf16.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16x8(uint32_t codes, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  u32x4_t u;
  u[0] = __builtin_bit_cast(uint32_t, p0);
  u[1] = __builtin_bit_cast(uint32_t, p1);
  u[2] = __builtin_bit_cast(uint32_t, p2);
  u[3] = __builtin_bit_cast(uint32_t, p3);
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Clamped gated SwiGLU with the +1 on the linear branch, for one (gate, linear) pair.
__device__ __forceinline__ float swiglu_unit(float g, float l, float limit, float alpha) {
  g = __builtin_amdgcn_fmed3f(g, -limit, limit);  // clamp to [-limit, limit] in one instruction
  l = __builtin_amdgcn_fmed3f(l, -limit, limit);
  // sigma(alpha g) = 1 / (1 + 2^(-alpha g log2 e)) on the hardware's base-2 exponential and
  // reciprocal (about 1 ulp each: far inside the bf16 rounding that follows)
  const float e = __builtin_amdgcn_exp2f(-alpha * 1.44269504088896341f * g);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * (l + 1.0f);
}

// Wave-wide helpers.
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Inclusive prefix sum over the wave's 64 lanes by DPP moves (register speed): shifts by 1,
// 2, 4, 8 within each row of 16 (lanes shifted in from outside the row add 0), then lane 15
// of rows 0 / 2 into rows 1 / 3 and lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
#define MOE_DPP_ADD(CTRL, ROWS, BOUND) v += __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, BOUND)
  MOE_DPP_ADD(0x111, 0xF, true);   // row_shr:1
  MOE_DPP_ADD(0x112, 0xF, true);   // row_shr:2
  MOE_DPP_ADD(0x114, 0xF, true);   // row_shr:4
  MOE_DPP_ADD(0x118, 0xF, true);   // row_shr:8
  MOE_DPP_ADD(0x142, 0xA, false);  // row_bcast15 into rows 1 and 3
  MOE_DPP_ADD(0x143, 0xC, false);  // row_bcast31 into rows 2 and 3
#undef MOE_DPP_ADD
  return v;
}

// Minimum over the wave's 64 lanes (the same DPP pattern as wave_max_f32), read from lane 63.
__device__ __forceinline__ int wave_min_i32(int x) {
#define MOE_DPP_MIN(CTRL, ROWS) x = min(x, __builtin_amdgcn_update_dpp(x, x, CTRL, ROWS, 0xF, false))
  MOE_DPP_MIN(0xB1, 0xF);   // quad_perm [1, 0, 3, 2]
  MOE_DPP_MIN(0x4E, 0xF);   // quad_perm [2, 3, 0, 1]
  MOE_DPP_MIN(0x141, 0xF);  // row_half_mirror
  MOE_DPP_MIN(0x140, 0xF);  // row_mirror
  MOE_DPP_MIN(0x142, 0xA);  // row_bcast15 into rows 1 and 3
  MOE_DPP_MIN(0x143, 0xC);  // row_bcast31 into rows 2 and 3
#undef MOE_DPP_MIN
  return __builtin_amdgcn_readlane(x, 63);
}

// Value of lane `l` (wave-uniform) for every lane.
__device__ __forceinline__ int wave_read(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// Maximum over the wave's 64 lanes, for every lane. DPP moves (register speed, no LDS round
// trip): swap neighbours, swap pairs, mirror within 8 and within 16 lanes (every row of 16
// now holds its maximum), then broadcast lane 15 of a row into the next row and lane 31 into
// the upper half, so lane 63 holds the maximum of all 64.
__device__ __forceinline__ float wave_max_f32(float v) {
  int x = __float_as_int(v);
#define MOE_DPP_MAX(CTRL, ROWS) \
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, CTRL, ROWS, 0xF, false))))
  MOE_DPP_MAX(0xB1, 0xF);   // quad_perm [1, 0, 3, 2]
  MOE_DPP_MAX(0x4E, 0xF);   // quad_perm [2, 3, 0, 1]
  MOE_DPP_MAX(0x141, 0xF);  // row_half_mirror
  MOE_DPP_MAX(0x140, 0xF);  // row_mirror
  MOE_DPP_MAX(0x142, 0xA);  // row_bcast15 into rows 1 and 3
  MOE_DPP_MAX(0x143, 0xC);  // row_bcast31 into rows 2 and 3
#undef MOE_DPP_MAX
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}

// Sum over the wave's 64 lanes by butterfly exchanges, for every lane; the same pairing on
// every lane, so the result is the same on all of them and from run to run.
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

}  // namespace moe
