// Two-term MXFP8 form of activation rows, the operand the block-scaled expert GEMM reads.
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

}  // namespace moe
