// RMSNorm of the layer input, the step before the MoE layer in each decoder block (review of
// the from-scratch gpt-oss-20B at pomoai.com, section 3.2: the row divided by its root mean
// square, times a per-feature scale, no mean subtraction; gpt-oss walkthrough at pnsm.cn,
// section 2.3: RMSNorm, no bias):
//     xn[t][h] = bf16( x[t][h] / sqrt(mean_h x[t][h]^2 + eps) * scale[h] ),
// rounded to nearest-even bf16 once, since the layer's input is bf16. The block-scaled
// expert GEMM reads its activations as two-term MXFP8 records (mx_act.h); this kernel writes
// those records of the normalised row too, from the same bf16-rounded values, so on that path
// the normalisation replaces the gather that would otherwise make them.
#include "common.h"
#include "kernels.h"
#include "mx_act.h"

namespace moe {

// One wave per token, four tokens per workgroup. Lane l takes the 8-element pieces
// p = l + 64 i of the row, which is also the record layout of the gather (piece p is elements
// 8j..8j+7 of record c = p / 16, j = p % 16; 16 lanes per record, 4 records per pass). Pass 1:
// each lane sums the squares of its pieces in fp32, then the wave adds the lanes' sums
// (butterfly, fixed pairing). Pass 2 scales and rounds each piece and writes it (and its
// share of the records). With NP > 0 the row (at most NP pieces per lane, H <= 512 NP) stays
// in registers between the passes; NP = 0 reads it again (from cache).
template <bool MX, int NP>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t *__restrict__ x, int64_t T, int H,
                                                      const float *__restrict__ scale, float eps,
                                                      uint16_t *__restrict__ xn, uint8_t *__restrict__ rec,
                                                      uint8_t *__restrict__ rec_scales) {
  const int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;  // wave-uniform
  const int lane = threadIdx.x % kWave;
  const uint16_t *src = x + t * H;
  const u32x4_t *src4 = reinterpret_cast<const u32x4_t *>(src);
  const int npiece = H / 8;
  const int passes = (npiece + kWave - 1) / kWave;  // = ceil(records / 4)
  constexpr int kKeep = NP > 0 ? NP : 1;
  u32x4_t keep[kKeep];
  float ss = 0.0f;
  auto square_add = [&](const u32x4_t &v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = __uint_as_float(v[i] << 16), b = __uint_as_float(v[i] & 0xffff0000u);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  };
  if constexpr (NP > 0) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = lane + kWave * i;
      keep[i] = (i < passes && p < npiece) ? src4[p] : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) square_add(keep[i]);
  } else {
    for (int p = lane; p < npiece; p += kWave) square_add(src4[p]);
  }
  ss = wave_sum_f32(ss);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);  // correctly rounded sqrt and divisions

  const int nrec = mx_records(H);
  uint16_t *dst = xn + t * H;
  uint8_t *drow = MX ? rec + t * nrec * kMxRecBytes : nullptr;
  uint8_t *srow = MX ? rec_scales + t * nrec * kMxScBytes : nullptr;
  auto piece = [&](int i, const u32x4_t &v) {
    const int c = 4 * i + lane / 16, j = lane % 16;
    const int p = lane + kWave * i, e0 = 8 * p;  // H % 32 == 0: a piece is wholly inside or past H
    const bool in = p < npiece;
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    if (in) {
      s0 = *reinterpret_cast<const f32x4_t *>(scale + e0);
      s1 = *reinterpret_cast<const f32x4_t *>(scale + e0 + 4);
    }
    float f[8];
    uint32_t packed[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = __uint_as_float(v[q] << 16), b = __uint_as_float(v[q] & 0xffff0000u);
      const float sa = q < 2 ? s0[2 * q] : s1[2 * q - 4], sb = q < 2 ? s0[2 * q + 1] : s1[2 * q - 3];
      const uint16_t ha = f32_to_bf16_rne((a * r) * sa), hb = f32_to_bf16_rne((b * r) * sb);
      packed[q] = (uint32_t)ha | ((uint32_t)hb << 16);
      f[2 * q] = bf16_to_f32(ha);
      f[2 * q + 1] = bf16_to_f32(hb);
    }
    if (in) *reinterpret_cast<u32x4_t *>(dst + e0) = u32x4_t{packed[0], packed[1], packed[2], packed[3]};
    if constexpr (MX) mx_store_piece(f, c, j, nrec, drow, srow);
  };
  if constexpr (NP > 0) {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if (i < passes) piece(i, keep[i]);
  } else {
    for (int i = 0; i < passes; ++i) {
      const int p = lane + kWave * i;
      piece(i, p < npiece ? src4[p] : u32x4_t{0u, 0u, 0u, 0u});
    }
  }
}

// The row stays in registers up to this many pieces per lane (H <= 4096).
constexpr int kNormKeepPieces = 8;

hipError_t launch_rmsnorm(const uint16_t *x, int64_t T, int H, const float *scale, float eps, uint16_t *xn,
                          uint8_t *rec, uint8_t *rec_scales, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  const bool keep = H <= kNormKeepPieces * 8 * kWave;
#define MOE_LAUNCH_NORM(MX, NP) \
  hipLaunchKernelGGL((rmsnorm_kernel<MX, NP>), grid, block, 0, stream, x, T, H, scale, eps, xn, rec, rec_scales)
  if (rec != nullptr) {
    if (keep) MOE_LAUNCH_NORM(true, kNormKeepPieces);
    else MOE_LAUNCH_NORM(true, 0);
  } else {
    if (keep) MOE_LAUNCH_NORM(false, kNormKeepPieces);
    else MOE_LAUNCH_NORM(false, 0);
  }
#undef MOE_LAUNCH_NORM
  return hipGetLastError();
}

}  // namespace moe
