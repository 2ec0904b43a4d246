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

// Every load below is issued unconditionally from an in-bounds address (split pieces past
// nsplit re-read the last one, a missing bias reads the partials' first element) and the extra
// values are dropped at the add: with a load under a branch the compiler waits for every load
// in flight at that branch, and a logit's dozen loads then cost a dozen memory round trips.
// A scheduling barrier keeps the first add behind the last load, so the loads of a logit (or
// of the two logits of router_logit_tm2) make one round trip together.

// Logit (t, e) from split-major partials partial[(s * T + t) * E + e], s = 0 .. nsplit - 1,
// added in split order, then the bias.
__device__ __forceinline__ float router_logit_sm(const float *__restrict__ partial, int nsplit,
                                                 const float *__restrict__ bias, int64_t t, int e, int64_t T, int E) {
  const float *p = partial + t * E + e;
  const int64_t stride = T * E;
  const float bv = *(bias != nullptr ? bias + e : partial);
  float pv[kMaxSplits];
#pragma unroll
  for (int c = 0; c < kMaxSplits; ++c) pv[c] = p[(c < nsplit ? c : nsplit - 1) * stride];
  __builtin_amdgcn_sched_barrier(0);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxSplits; ++c)
    if (c < nsplit) s += pv[c];
  return bias != nullptr ? s + bv : s;
}

// The same from token-major partials partial[(t * E + e) * nsp + s] (contiguous, nsp a
// multiple of 4, read as 16-byte loads): the loads, then the sum.
struct TmLogitLoads {
  f32x4_t pv[kMaxSplitVec];
  float bv;
};

__device__ __forceinline__ void router_logit_tm_issue(const float *__restrict__ partial, int nsp,
                                                      const float *__restrict__ bias, int64_t t, int e, int E,
                                                      TmLogitLoads &l) {
  const f32x4_t *p = reinterpret_cast<const f32x4_t *>(partial + (t * E + e) * nsp);
  // opaque to the compiler: otherwise it computes the clamped offsets (and, below, the split
  // predicates) once for all of a wave's logits and keeps them in scalar registers, dozens of
  // them, which spill where a kernel has few to spare
  int nv = nsp / 4;
  asm volatile("" : "+s"(nv));
  l.bv = *(bias != nullptr ? bias + e : partial);
#pragma unroll
  for (int c = 0; c < kMaxSplitVec; ++c) l.pv[c] = p[c < nv ? c : nv - 1];
}

__device__ __forceinline__ float router_logit_tm_add(const TmLogitLoads &l, int nsplit,
                                                     const float *__restrict__ bias) {
  asm volatile("" : "+s"(nsplit));
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxSplitVec; ++c)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (4 * c + u < nsplit) s += l.pv[c][u];
  return bias != nullptr ? s + l.bv : s;
}

__device__ __forceinline__ float router_logit_tm(const float *__restrict__ partial, int nsplit, int nsp,
                                                 const float *__restrict__ bias, int64_t t, int e, int E) {
  TmLogitLoads l;
  router_logit_tm_issue(partial, nsp, bias, t, e, E, l);
  __builtin_amdgcn_sched_barrier(0);
  return router_logit_tm_add(l, nsplit, bias);
}

// Two token-major logits, (ta, ea) and (tb, eb), with all their loads in flight together.
__device__ __forceinline__ void router_logit_tm2(const float *__restrict__ partial, int nsplit, int nsp,
                                                 const float *__restrict__ bias, int64_t ta, int ea, int64_t tb,
                                                 int eb, int E, float &la, float &lb) {
  TmLogitLoads a, b;
  router_logit_tm_issue(partial, nsp, bias, ta, ea, E, a);
  router_logit_tm_issue(partial, nsp, bias, tb, eb, E, b);
  __builtin_amdgcn_sched_barrier(0);
  la = router_logit_tm_add(a, nsplit, bias);
  lb = router_logit_tm_add(b, nsplit, bias);
}

// A wave's logits of token t: lane holds experts lane + 64 i (i < 4; 0 past E, never picked).
// SM selects the split-major partials (router_logit_sm), else token-major (router_logit_tm).
template <bool SM>
__device__ __forceinline__ void router_logits_wave(const float *__restrict__ partial, int nsplit,
                                                   const float *__restrict__ bias, int64_t t, int64_t T, int E,
                                                   int lane, float (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = 0.f;
    if (i * kWave < E) {  // wave-uniform; lanes past E read expert E - 1
      const int e = lane + i * kWave;
      const int ec = e < E ? e : E - 1;
      const float s = SM ? router_logit_sm(partial, nsplit, bias, t, ec, T, E)
                         : router_logit_tm(partial, nsplit, (nsplit + 3) / 4 * 4, bias, t, ec, E);
      v[i] = e < E ? s : 0.f;
    }
  }
}

// K rounds of a wave-wide argmax over a token's logits (lane holds experts lane + 64 i;
// larger logit wins, equal logits go to the lower expert id): the maximum of the experts not
// yet picked by DPP moves, then the lowest id holding it by a DPP minimum over the lanes'
// candidate ids. Then softmax over the K picked logits (in pick order, relative to the
// largest). Branch-free per round; the picks and weights come out wave-uniform. A logit that
// equals no maximum (all remaining NaN) gives id -1.
template <int K>
__device__ __forceinline__ void topk_picks_wave_k(const float (&v)[4], int E, int lane, int (&sel_e)[K],
                                                  float (&wt)[K]) {
  bool tk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) tk[i] = lane + i * kWave >= E;
  float sel_v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    float lm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) lm = tk[i] ? lm : fmaxf(lm, v[i]);
    const float m = wave_max_f32(lm);
    int cid = 0x7fffffff;
#pragma unroll
    for (int i = 3; i >= 0; --i) cid = (!tk[i] && v[i] == m) ? lane + i * kWave : cid;
    const int be = wave_min_i32(cid);
#pragma unroll
    for (int i = 0; i < 4; ++i) tk[i] = tk[i] || be == lane + i * kWave;
    sel_v[j] = m;
    sel_e[j] = be == 0x7fffffff ? -1 : be;
  }
  float z[K], sum = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    z[j] = expf(sel_v[j] - sel_v[0]);
    sum += z[j];
  }
  const float inv = 1.0f / sum;
#pragma unroll
  for (int j = 0; j < K; ++j) wt[j] = z[j] * inv;
}

// The picks above, then lane j < K writes pick j's id and weight (and, if lds_idx is given,
// the id there too).
template <int K>
__device__ __forceinline__ void topk_softmax_wave_k(const float (&v)[4], int E, int lane, int32_t *__restrict__ idx_out,
                                                    float *__restrict__ w_out, int *lds_idx) {
  int sel_e[K];
  float wt[K];
  topk_picks_wave_k<K>(v, E, lane, sel_e, wt);
  int my_e = 0;
  float my_w = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    my_e = lane == j ? sel_e[j] : my_e;
    my_w = lane == j ? wt[j] : my_w;
  }
  if (lane < K) {
    idx_out[lane] = my_e;
    w_out[lane] = my_w;
    if (lds_idx != nullptr) lds_idx[lane] = my_e;
  }
}

// The same for a run-time k in 1 .. 8.
__device__ __forceinline__ void topk_softmax_wave(const float (&v)[4], int E, int k, int lane,
                                                  int32_t *__restrict__ idx_out, float *__restrict__ w_out,
                                                  int *lds_idx = nullptr) {
  switch (k) {
    case 1: topk_softmax_wave_k<1>(v, E, lane, idx_out, w_out, lds_idx); break;
    case 2: topk_softmax_wave_k<2>(v, E, lane, idx_out, w_out, lds_idx); break;
    case 3: topk_softmax_wave_k<3>(v, E, lane, idx_out, w_out, lds_idx); break;
    case 4: topk_softmax_wave_k<4>(v, E, lane, idx_out, w_out, lds_idx); break;
    case 5: topk_softmax_wave_k<5>(v, E, lane, idx_out, w_out, lds_idx); break;
    case 6: topk_softmax_wave_k<6>(v, E, lane, idx_out, w_out, lds_idx); break;
    case 7: topk_softmax_wave_k<7>(v, E, lane, idx_out, w_out, lds_idx); break;
    default: topk_softmax_wave_k<8>(v, E, lane, idx_out, w_out, lds_idx); break;
  }
}

}  // namespace moe
