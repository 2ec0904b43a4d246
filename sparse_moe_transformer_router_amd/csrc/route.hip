// Router: logits = x W_r^T + b_r in fp32, then the k best experts per token and the softmax
// over their logits (review of the from-scratch gpt-oss-20B at pomoai.com, section 3.4: a
// linear projection plus top-k, outputs weighted by softmax-normalised scores; gpt-oss
// walkthrough at pnsm.cn, section 2.2: top-4 with softmax weighting of the picked experts).
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kRouteTok = 4;  // tokens per wave in the logits kernel

// One wave computes the logits of kRouteTok consecutive tokens for one expert. Lane l
// accumulates 8 consecutive features at a time; the wave then reduces its lanes.
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t *__restrict__ x, int64_t T,
                                                            int H, const float *__restrict__ w,
                                                            const float *__restrict__ b, int E,
                                                            float *__restrict__ logits) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int e = blockIdx.y * 4 + wave;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteTok;
  if (e >= E) return;
  const float *wr = w + (int64_t)e * H;
  float acc[kRouteTok];
#pragma unroll
  for (int i = 0; i < kRouteTok; ++i) acc[i] = 0.f;
  for (int h = lane * 8; h < H; h += kWave * 8) {
    const f32x4_t w0 = *reinterpret_cast<const f32x4_t *>(wr + h);
    const f32x4_t w1 = *reinterpret_cast<const f32x4_t *>(wr + h + 4);
#pragma unroll
    for (int i = 0; i < kRouteTok; ++i) {
      if (t0 + i < T) {
        const u32x4_t xv = *reinterpret_cast<const u32x4_t *>(x + (t0 + i) * H + h);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = __uint_as_float(xv[q] << 16);
          const float hi = __uint_as_float(xv[q] & 0xffff0000u);
          const float wl = (q < 2) ? w0[2 * q] : w1[2 * q - 4];
          const float wh = (q < 2) ? w0[2 * q + 1] : w1[2 * q - 3];
          acc[i] = fmaf(lo, wl, acc[i]);
          acc[i] = fmaf(hi, wh, acc[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRouteTok; ++i) {
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) acc[i] += __shfl_xor(acc[i], d, kWave);
  }
  if (lane == 0) {
    const float be = b ? b[e] : 0.f;
#pragma unroll
    for (int i = 0; i < kRouteTok; ++i)
      if (t0 + i < T) logits[(t0 + i) * E + e] = acc[i] + be;
  }
}

// One wave per token: k rounds of a wave-wide argmax (larger logit wins, equal logits go to
// the lower expert id), then softmax over the k picked logits.
__global__ __launch_bounds__(256) void router_topk_kernel(const float *__restrict__ logits, int64_t T,
                                                          int E, int k, int32_t *__restrict__ topk_idx,
                                                          float *__restrict__ topk_w) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  float v[4];
  int taken = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + i * kWave;
    v[i] = (e < E) ? logits[t * E + e] : 0.f;
    if (e >= E) taken |= 1 << i;
  }
  float sel_v[8];
  int sel_e[8];
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // lane-local best; ids ascend with i, so '>' keeps the lower id
      const int e = lane + i * kWave;
      if (!(taken & (1 << i)) && (be == 0x7fffffff || v[i] > bv)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(bv, d, kWave);
      const int oe = __shfl_xor(be, d, kWave);
      const bool other = (oe != 0x7fffffff) &&
                         (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
      if (other) {
        bv = ov;
        be = oe;
      }
    }
    sel_v[j] = bv;
    sel_e[j] = be;
    if ((be % kWave) == lane) taken |= 1 << (be / kWave);
  }
  if (lane == 0) {
    const float m = sel_v[0];
    float z[8], sum = 0.f;
    for (int j = 0; j < k; ++j) {
      z[j] = expf(sel_v[j] - m);
      sum += z[j];
    }
    const float inv = 1.0f / sum;
    for (int j = 0; j < k; ++j) {
      topk_idx[t * k + j] = sel_e[j];
      topk_w[t * k + j] = z[j] * inv;
    }
  }
}

hipError_t launch_router_logits(const uint16_t *x, int64_t T, int H, const float *w, const float *b,
                                int E, float *logits, hipStream_t stream) {
  dim3 grid((unsigned)((T + kRouteTok - 1) / kRouteTok), (unsigned)((E + 3) / 4));
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, stream, x, T, H, w, b, E, logits);
  return hipGetLastError();
}

hipError_t launch_router_topk(const float *logits, int64_t T, int E, int k, int32_t *topk_idx,
                              float *topk_w, hipStream_t stream) {
  dim3 grid((unsigned)((T + 3) / 4));
  hipLaunchKernelGGL(router_topk_kernel, grid, dim3(256), 0, stream, logits, T, E, k, topk_idx,
                     topk_w);
  return hipGetLastError();
}

}  // namespace moe
