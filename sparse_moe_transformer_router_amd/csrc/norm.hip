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

// One wave per token, four tokens per workgroup. Pass 1: each lane sums the squares of its
// 8-element pieces in fp32, then the wave adds the lanes' sums (butterfly, fixed pairing).
// Pass 2 re-reads the row (now in cache) in the record layout of the gather: a lane takes 8
// consecutive elements, 16 lanes one 128-element record, 4 records per pass.
template <bool MX>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t *__restrict__ x, int64_t T, int H,
                                                      const float *__restrict__ scale, float eps,
                                                      uint16_t *__restrict__ xn, uint8_t *__restrict__ rec,
                                                      uint8_t *__restrict__ rec_scales) {
  const int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;  // wave-uniform
  const int lane = threadIdx.x % kWave;
  const uint16_t *src = x + t * H;
  const u32x4_t *src4 = reinterpret_cast<const u32x4_t *>(src);
  float ss = 0.0f;
  for (int p = lane; p < H / 8; p += kWave) {
    const u32x4_t v = src4[p];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = __uint_as_float(v[i] << 16), b = __uint_as_float(v[i] & 0xffff0000u);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  ss = wave_sum_f32(ss);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);  // correctly rounded sqrt and divisions

  const int nrec = mx_records(H);
  uint16_t *dst = xn + t * H;
  uint8_t *drow = MX ? rec + t * nrec * kMxRecBytes : nullptr;
  uint8_t *srow = MX ? rec_scales + t * nrec * kMxScBytes : nullptr;
  for (int c0 = 0; c0 < nrec; c0 += 4) {
    const int c = c0 + lane / 16, j = lane % 16;
    const int e0 = c * kMxRecElems + 8 * j;  // H % 32 == 0: a piece is wholly inside or past H
    const bool in = c < nrec && e0 < H;
    u32x4_t v = {0u, 0u, 0u, 0u};
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    if (in) {
      v = *reinterpret_cast<const u32x4_t *>(src + e0);
      s0 = *reinterpret_cast<const f32x4_t *>(scale + e0);
      s1 = *reinterpret_cast<const f32x4_t *>(scale + e0 + 4);
    }
    float f[8];
    uint32_t packed[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = __uint_as_float(v[i] << 16), b = __uint_as_float(v[i] & 0xffff0000u);
      const float sa = i < 2 ? s0[2 * i] : s1[2 * i - 4], sb = i < 2 ? s0[2 * i + 1] : s1[2 * i - 3];
      const uint16_t ha = f32_to_bf16_rne((a * r) * sa), hb = f32_to_bf16_rne((b * r) * sb);
      packed[i] = (uint32_t)ha | ((uint32_t)hb << 16);
      f[2 * i] = bf16_to_f32(ha);
      f[2 * i + 1] = bf16_to_f32(hb);
    }
    if (in) *reinterpret_cast<u32x4_t *>(dst + e0) = u32x4_t{packed[0], packed[1], packed[2], packed[3]};
    if constexpr (MX) mx_store_piece(f, c, j, nrec, drow, srow);
  }
}

hipError_t launch_rmsnorm(const uint16_t *x, int64_t T, int H, const float *scale, float eps, uint16_t *xn,
                          uint8_t *rec, uint8_t *rec_scales, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (rec != nullptr)
    hipLaunchKernelGGL(rmsnorm_kernel<true>, grid, block, 0, stream, x, T, H, scale, eps, xn, rec, rec_scales);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<false>, grid, block, 0, stream, x, T, H, scale, eps, xn, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace moe
