// Router top-k pieces shared by the router's own top-k kernel and the fused top-k +
// permutation kernel, so both reach bit-identical routing: the fixed-order sum of a logit's
// split-K partials, and the wave-wide top-k with softmax over the picked logits (review of the
// from-scratch gpt-oss-20B at pomoai.com, section 3.4; gpt-oss walkthrough at pnsm.cn,
// section 2.2: top-4, softmax over the picked experts' scores).
#pragma once

#include "common.h"

namespace moe {

constexpr int kMaxSplits = 48;  // split-K pieces of a router logit

constexpr int kMaxSplitVec = kMaxSplits / 4;

// Logit (t, e) from split-major partials partial[(s * T + t) * E + e], s = 0 .. nsplit - 1
// (all loads issued before the first add), added in split order, then the bias.
__device__ __forceinline__ float router_logit_sm(const float *__restrict__ partial, int nsplit,
                                                 const float *__restrict__ bias, int64_t t, int e, int64_t T, int E) {
  const float *p = partial + t * E + e;
  const int64_t stride = T * E;
  float pv[kMaxSplits];
#pragma unroll
  for (int c = 0; c < kMaxSplits; ++c) pv[c] = (c < nsplit) ? p[c * stride] : 0.f;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxSplits; ++c)
    if (c < nsplit) s += pv[c];
  if (bias) s += bias[e];
  return s;
}

// The same from token-major partials partial[(t * E + e) * nsp + s] (contiguous, nsp a
// multiple of 4, read as 16-byte loads).
__device__ __forceinline__ float router_logit_tm(const float *__restrict__ partial, int nsplit, int nsp,
                                                 const float *__restrict__ bias, int64_t t, int e, int E) {
  const f32x4_t *p = reinterpret_cast<const f32x4_t *>(partial + (t * E + e) * nsp);
  f32x4_t pv[kMaxSplitVec];
#pragma unroll
  for (int c = 0; c < kMaxSplitVec; ++c) pv[c] = (4 * c < nsplit) ? p[c] : f32x4_t{0.f, 0.f, 0.f, 0.f};
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxSplitVec; ++c)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (4 * c + u < nsplit) s += pv[c][u];
  if (bias) s += bias[e];
  return s;
}

// k rounds of a wave-wide argmax over a token's logits (lane holds experts lane + 64 i;
// larger logit wins, equal logits go to the lower expert id): the maximum by DPP moves, then
// the lowest id holding it by ballots. Then softmax over the k picked logits; lane 0 writes
// the token's ids and weights (and, if lds_idx is given, the ids there too).
__device__ __forceinline__ void topk_softmax_wave(const float (&v)[4], int E, int k, int lane,
                                                  int32_t *__restrict__ idx_out, float *__restrict__ w_out,
                                                  int *lds_idx = nullptr) {
  int taken = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (lane + i * kWave >= E) taken |= 1 << i;
  float sel_v[8];
  int sel_e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sel_v[j] = 0.f;
    sel_e[j] = 0;
    if (j < k) {
      float lm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!(taken & (1 << i))) lm = fmaxf(lm, v[i]);
      const float m = wave_max_f32(lm);
      int be = -1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // ids ascend with i, then with the lane
        const uint64_t hit = __ballot(!(taken & (1 << i)) && v[i] == m);
        if (be < 0 && hit != 0) be = i * kWave + __ffsll((unsigned long long)hit) - 1;
      }
      sel_v[j] = m;
      sel_e[j] = be;
      if ((be % kWave) == lane) taken |= 1 << (be / kWave);
    }
  }
  if (lane == 0) {
    float z[8], sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      z[j] = (j < k) ? expf(sel_v[j] - sel_v[0]) : 0.f;
      sum += z[j];
    }
    const float inv = 1.0f / sum;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        idx_out[j] = sel_e[j];
        w_out[j] = z[j] * inv;
        if (lds_idx != nullptr) lds_idx[j] = sel_e[j];
      }
    }
  }
}

}  // namespace moe
