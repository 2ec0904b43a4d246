// Two-term block-scaled forms of activation rows, the operands the block-scaled expert GEMM
// reads: MXFP8 (exact for bf16 values; the gate_up input and, on one path, the down input) and
// MXFP6 (the down input on the other path; below).
//
// The expert weights are MXFP4 (OCP MX: E2M1 elements, one E8M0 scale per 32; gpt-oss
// walkthrough at pnsm.cn, sections 1 and 4), and gfx950's scaled MFMA multiplies such blocks
// by MXFP8 blocks directly. A bf16 activation has 8 significant bits and E4M3 has 4, so each
// activation is carried as two E4M3 terms, each with its own E8M0 block scale:
//     v = hi * 2^(sh - 127) + lo * 2^(sl - 127).
// Per 32-element block with largest magnitude m (biased fp32 exponent e): sh = e - 7, so
// the block's largest element scales into [128, 256) and never reaches E4M3's 448 after
// rounding; hi = RNE_E4M3(v * 2^(127 - sh)); sl = sh - 5; lo = RNE_E4M3(32 (v * 2^(127 - sh) - hi)).
// The residual of a 4-bit rounding is at most 8 at that scale, so 32 times it stays <= 256.
// For a bf16 v no more than 14 binades below the block maximum both terms are exact and
// hi + lo reproduces v exactly; smaller elements keep an error below 2^-22 of the maximum.
//
// Memory layout of a row of K elements: ceil(K / 128) records of 256 bytes (record c: elements
// 128c..128c+127 as E4M3 codes, the hi term's 128 bytes then the lo term's), and, in a
// separate array, 8 bytes per (row, record): the hi term's four block scales (blocks
// 4c..4c+3, one byte each), then the lo term's. Elements past K are zero codes.
#pragma once

#include "common.h"

namespace moe {

constexpr int kMxRecElems = 128;  // elements per record
constexpr int kMxRecBytes = 256;  // hi codes, then lo codes
constexpr int kMxScBytes = 8;     // hi scale bytes of the record's 4 blocks, then lo

__host__ __device__ constexpr int mx_records(int K) { return (K + kMxRecElems - 1) / kMxRecElems; }

struct MxBlockScale {
  uint32_t sh, sl;  // E8M0 bytes of the hi and lo terms
  float inv;        // 2^(127 - sh): scales an element to the hi term's units
  bool lo_ok;       // sl = sh - 5 fits a byte (else the lo term is zero)
};

// Scales of a block from its largest magnitude.
__device__ __forceinline__ MxBlockScale mx_block_scale(float maxabs) {
  const int e = (int)((__float_as_uint(maxabs) >> 23) & 0xffu);
  const int sh = e > 7 ? e - 7 : 0;
  MxBlockScale s;
  s.sh = (uint32_t)sh;
  s.lo_ok = sh >= 5;
  s.sl = s.lo_ok ? (uint32_t)(sh - 5) : 0u;
  s.inv = __uint_as_float((uint32_t)(254 - sh) << 23);
  return s;
}

// Two elements -> their hi codes (bits 0..15, element 0 in the low byte) and lo codes.
__device__ __forceinline__ void mx_split2(float v0, float v1, const MxBlockScale &s, uint32_t &hi, uint32_t &lo) {
  const float a0 = v0 * s.inv, a1 = v1 * s.inv;
  const uint32_t h = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false) & 0xffffu;
  float r0 = (a0 - __builtin_amdgcn_cvt_f32_fp8((int)h, 0)) * 32.0f;
  float r1 = (a1 - __builtin_amdgcn_cvt_f32_fp8((int)h, 1)) * 32.0f;
  r0 = s.lo_ok ? r0 : 0.0f;
  r1 = s.lo_ok ? r1 : 0.0f;
  hi = h;
  lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false) & 0xffffu;
}

// One lane's share of a row's records: elements 8j..8j+7 of record c (lane j = 0..15 of a
// 16-lane group; a lane quad is one 32-element block). Every lane of the quad must call it
// (the block maximum moves between them by two DPP quad swaps); c >= nrec stores nothing.
__device__ __forceinline__ void mx_store_piece(const float (&f)[8], int c, int j, int nrec, uint8_t *__restrict__ drow,
                                               uint8_t *__restrict__ srow) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  int mi = __float_as_int(m);
  mi = __float_as_int(fmaxf(__int_as_float(mi), __int_as_float(__builtin_amdgcn_update_dpp(mi, mi, 0xB1, 0xF, 0xF, false))));
  mi = __float_as_int(fmaxf(__int_as_float(mi), __int_as_float(__builtin_amdgcn_update_dpp(mi, mi, 0x4E, 0xF, 0xF, false))));
  const MxBlockScale s = mx_block_scale(__int_as_float(mi));
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) mx_split2(f[2 * i], f[2 * i + 1], s, h[i], l[i]);
  if (c < nrec) {
    uint8_t *d = drow + c * kMxRecBytes + 8 * j;
    *reinterpret_cast<uint2 *>(d) = uint2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    *reinterpret_cast<uint2 *>(d + 128) = uint2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
    if ((j & 3) == 0) {
      srow[c * kMxScBytes + j / 4] = (uint8_t)s.sh;
      srow[c * kMxScBytes + 4 + j / 4] = (uint8_t)s.sl;
    }
  }
}


// ---------------------------------------------------------------------------------------------
// Two-term MXFP6 (E2M3) form: the cheaper operand of the block-scaled GEMM (the FP6 x FP4 scaled
// MFMA issues faster than FP8 x FP4). E2M3 holds sign, 2 exponent bits (bias 1) and 3 mantissa
// bits: 0, 1/8 .. 7/8, 1 .. 7.5 (OCP MX v1.0). Per 32-element block with largest magnitude m
// (biased fp32 exponent e):
//     sh = e - 1 (0 if e <= 1): m scales into [2, 4), so its rounding never passes 4.0;
//     a  = v * 2^(127 - sh);   hi = RNE_E2M3(a);   r = a - hi  (|r| <= 1/8, exact in fp32);
//     sl = sh - 5 (0 if sh < 5): lo = RNE_E2M3(r * 2^(sh - sl))  (|lo| <= 4);
//     v ~ hi * 2^(sh - 127) + lo * 2^(sl - 127),   |error| <= 2^-9 m.
// Every element within 2^3 of its block maximum is reproduced exactly (a bf16 value there has
// at most 3 bits below the hi term's quantum, and the lo term holds them); smaller ones keep
// an error below 2^-9 of the block maximum.
//
// Memory layout of a row of K elements: ceil(K / 128) records of 192 bytes, plus 8 scale bytes
// per (row, record) in a separate array (the hi term's four block scales, then the lo term's,
// as in the MXFP8 form). A block of one term is 32 six-bit codes, a 192-bit stream (element j
// in bits 6j .. 6j + 5: the order of the scaled MFMA's FP6 operand, in which lane group g holds
// elements 32g .. 32g + 31 of a 64-element half): dwords 0-3 and dwords 4-5. In a record:
//     bytes   0 .. 127: 16-byte units (t, b) at 16 (4t + b): dwords 0-3 of block b of term t;
//     bytes 128 .. 191: 16-byte units (t, g) at 128 + 16 (2t + g): dwords 4-5 of block g of
//                       term t, then of block 2 + g (the pieces one lane needs for halves 0, 1).
// So every operand read is a 16-byte and an 8-byte LDS read at their natural alignment.
constexpr int kMx6RecBytes = 192;
constexpr int kMx6BPart = 128;  // byte offset of the dwords-4-5 part in a record

__host__ __device__ constexpr int mx6_a_off(int t, int b) { return 16 * (4 * t + b); }
__host__ __device__ constexpr int mx6_b_off(int t, int b) { return kMx6BPart + 16 * (2 * t + (b & 1)) + 8 * (b >> 1); }

typedef float f32x16v_t __attribute__((ext_vector_type(16)));
typedef float f32x32v_t __attribute__((ext_vector_type(32)));
typedef int i32x6_t __attribute__((ext_vector_type(6)));

// One block (v[0..31], element order, bf16-exact fp32 values) -> the two terms' codes (6 dwords
// each, element j at bits 6j) and their E8M0 scale bytes. gfx950's 32-value converts
// (RNE with saturation; the interleaving pair takes even elements from its first source and
// odd ones from its second) see only values that are exact or inside E2M3's range.
__device__ __forceinline__ void mx6_split_block(const float (&v)[32], uint32_t (&hi)[6], uint32_t (&lo)[6],
                                                uint32_t &sh_out, uint32_t &sl_out) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
  const int e = (int)((__float_as_uint(m) >> 23) & 0xffu);
  const int sh = e > 1 ? e - 1 : 0;
  const int sl = sh > 5 ? sh - 5 : 0;
  const float inv = __uint_as_float((uint32_t)(254 - sh) << 23);     // 2^(127 - sh)
  const float up = __uint_as_float((uint32_t)(127 + sh - sl) << 23);  // 2^(sh - sl)
  f32x16v_t a0, a1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    a0[i] = v[2 * i] * inv;
    a1[i] = v[2 * i + 1] * inv;
  }
  const i32x6_t h = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a0, a1, 1.0f);
  const f32x32v_t hv = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(h, 1.0f);  // element order
  f32x16v_t r0, r1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    r0[i] = (a0[i] - hv[2 * i]) * up;
    r1[i] = (a1[i] - hv[2 * i + 1]) * up;
  }
  const i32x6_t l = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(r0, r1, 1.0f);
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    hi[i] = (uint32_t)h[i];
    lo[i] = (uint32_t)l[i];
  }
  sh_out = (uint32_t)sh;
  sl_out = (uint32_t)sl;
}

// Store one block's two terms into record `rec` (block b of the record).
__device__ __forceinline__ void mx6_store_block(uint8_t *__restrict__ rec, int b, const uint32_t (&hi)[6],
                                                const uint32_t (&lo)[6]) {
  *reinterpret_cast<u32x4_t *>(rec + mx6_a_off(0, b)) = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
  *reinterpret_cast<uint2 *>(rec + mx6_b_off(0, b)) = uint2{hi[4], hi[5]};
  *reinterpret_cast<u32x4_t *>(rec + mx6_a_off(1, b)) = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
  *reinterpret_cast<uint2 *>(rec + mx6_b_off(1, b)) = uint2{lo[4], lo[5]};
}

}  // namespace moe
