// Weighted combine: out[t] = sum_j w[t][j] * y[slot_row[t*k + j]], the routing-weighted sum
// of the picked experts' outputs (review of the from-scratch gpt-oss-20B at pomoai.com,
// section 3.4). A gather in rank order with fp32 accumulation, so no atomics and a
// deterministic result; the output is rounded to nearest-even bf16 or kept in fp32. With a
// residual (the block's input row, review section 3.3: a residual path joins the FFN's
// output and its input), it is added to the sum last, before the one rounding.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y,
                                                      const int32_t *__restrict__ slot_row,
                                                      const float *__restrict__ topk_w, int64_t T,
                                                      int k, int H, const uint16_t *__restrict__ residual,
                                                      void *__restrict__ out, int out_f32) {
  const int chunks = (H / 4 + blockDim.x - 1) / blockDim.x;
  const int64_t t = blockIdx.x / chunks;
  const int h = ((blockIdx.x % chunks) * blockDim.x + threadIdx.x) * 4;
  if (h >= H) return;
  const int64_t S = T * k;
  // all index/weight loads first, then all row loads, then the sum in rank order
  int32_t r[8];
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    r[j] = (j < k) ? slot_row[t * k + j] : -1;
    w[j] = (j < k) ? topk_w[t * k + j] : 0.f;
  }
  f32x4_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    v[j] = ((uint32_t)r[j] < (uint64_t)S) ? *reinterpret_cast<const f32x4_t *>(y + (int64_t)r[j] * H + h)
                                          : f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint2 res = {0u, 0u};
  if (residual != nullptr) res = *reinterpret_cast<const uint2 *>(residual + t * H + h);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k && (uint32_t)r[j] < (uint64_t)S) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(w[j], v[j][i], acc[i]);
    }
  }
  if (residual != nullptr) {
    acc[0] += __uint_as_float(res.x << 16);
    acc[1] += __uint_as_float(res.x & 0xffff0000u);
    acc[2] += __uint_as_float(res.y << 16);
    acc[3] += __uint_as_float(res.y & 0xffff0000u);
  }
  if (out_f32) {
    *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(out) + t * H + h) = acc;
  } else {
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    uint32_t *o = reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(out) + t * H + h);
    o[0] = lo;
    o[1] = hi;
  }
}

hipError_t launch_combine(const float *y, const int32_t *slot_row, const float *topk_w, int64_t T,
                          int k, int H, void *out, bool out_f32, hipStream_t stream, const uint16_t *residual) {
  const int threads = 256;
  const int64_t chunks = (H / 4 + threads - 1) / threads;
  dim3 grid((unsigned)(T * chunks));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(threads), 0, stream, y, slot_row, topk_w, T, k, H,
                     residual, out, out_f32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
