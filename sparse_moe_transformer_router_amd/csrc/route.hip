// Router: logits = x W_r^T + b_r in fp32, then the k best experts per token and the softmax
// over their logits (review of the from-scratch gpt-oss-20B at pomoai.com, section 3.4: a
// linear projection plus top-k, outputs weighted by softmax-normalised scores; gpt-oss
// walkthrough at pnsm.cn, section 2.2: top-4 with softmax weighting of the picked experts).
//
// Logits on the matrix cores: x is bf16, and each fp32 router weight w is split exactly into
// three bf16 terms (hi = w with its low 16 bits cleared, mid = the same of w - hi, lo = the
// rest, which has at most 8 significant bits), so every product x * term is exact and
// v_mfma_f32_16x16x32_bf16 accumulates them in fp32. The input dimension is split across
// waves (split-K) when there are few tokens, so decode batches still spread over the chip;
// the partial sums are added in a fixed order by the top-k kernel.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

__device__ __forceinline__ void split3(const f32x4_t &a, const f32x4_t &b, bf16x8_t &hi, bf16x8_t &mid,
                                       bf16x8_t &lo) {
  u32x4_t h, m, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float w0 = (i < 2) ? a[2 * i] : b[2 * i - 4];
    const float w1 = (i < 2) ? a[2 * i + 1] : b[2 * i - 3];
    const uint32_t h0 = __float_as_uint(w0) & 0xffff0000u, h1 = __float_as_uint(w1) & 0xffff0000u;
    const float r0 = w0 - __uint_as_float(h0), r1 = w1 - __uint_as_float(h1);  // exact
    const uint32_t m0 = __float_as_uint(r0) & 0xffff0000u, m1 = __float_as_uint(r1) & 0xffff0000u;
    const float s0 = r0 - __uint_as_float(m0), s1 = r1 - __uint_as_float(m1);  // exact, <= 8 bits
    h[i] = (h0 >> 16) | h1;
    m[i] = (m0 >> 16) | m1;
    l[i] = (__float_as_uint(s0) >> 16) | (__float_as_uint(s1) & 0xffff0000u);
  }
  hi = as_bf16x8(h);
  mid = as_bf16x8(m);
  lo = as_bf16x8(l);
}

// One wave: 16 NTT tokens x 16 NET experts over the MX-block range of split blockIdx.z
// (NTT x NET 16x16 accumulators, so each weight element loaded and split serves 16 NTT tokens
// and each x element 16 NET experts). Split-major (SM, many tokens): writes
// partial[(split * T + t) * E + e], so a wave's stores are runs of consecutive experts. Else
// token-major: partial[(t * E + e) * nsp + split] (nsp = split count rounded up to 4), so the
// top-k kernel reads a logit's partials as a few 16-byte loads.
template <int NTT, int NET, bool SM>
__global__ __launch_bounds__(kWave) void router_partial_kernel(const uint16_t *__restrict__ x, int64_t T,
                                                               int H, const float *__restrict__ w, int E,
                                                               int blocks_per_split, int nsp,
                                                               float *__restrict__ partial,
                                                               int *__restrict__ counter) {
  const int lane = threadIdx.x;
  if (counter != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && lane == 0) *counter = 0;
  const int64_t t0 = (int64_t)blockIdx.x * 16 * NTT;
  const int e0 = blockIdx.y * 16 * NET;
  const int split = blockIdx.z;
  const int KB = H / 32;
  const int b0 = split * blocks_per_split;
  const int b1 = (b0 + blocks_per_split < KB) ? b0 + blocks_per_split : KB;
  const int r = lane % 16, q = lane / 16;
  const uint16_t *xp[NTT];
  bool t_ok[NTT];
#pragma unroll
  for (int i = 0; i < NTT; ++i) {
    const int64_t t = t0 + 16 * i + r;
    t_ok[i] = t < T;
    xp[i] = x + (t_ok[i] ? t : 0) * H + 8 * q;
  }
  const float *wp[NET];
  bool e_ok[NET];
#pragma unroll
  for (int j = 0; j < NET; ++j) {
    const int e = e0 + 16 * j + r;
    e_ok[j] = e < E;
    wp[j] = w + (int64_t)(e_ok[j] ? e : 0) * H + 8 * q;
  }
  f32x4_t acc[NTT][NET];
#pragma unroll
  for (int i = 0; i < NTT; ++i)
#pragma unroll
    for (int j = 0; j < NET; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  constexpr int U = (NTT * NET == 1) ? 4 : 2;  // MX blocks per round: all loads first, then the math
  for (int bb = b0; bb < b1; bb += U) {
    u32x4_t xa[U][NTT];
    f32x4_t wa[U][NET], wb[U][NET];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = bb + u;
      const bool ok = b < b1;
#pragma unroll
      for (int i = 0; i < NTT; ++i)
        xa[u][i] = (ok && t_ok[i]) ? *reinterpret_cast<const u32x4_t *>(xp[i] + 32 * b) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < NET; ++j) {
        wa[u][j] = (ok && e_ok[j]) ? *reinterpret_cast<const f32x4_t *>(wp[j] + 32 * b) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        wb[u][j] =
            (ok && e_ok[j]) ? *reinterpret_cast<const f32x4_t *>(wp[j] + 32 * b + 4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int j = 0; j < NET; ++j) {
        bf16x8_t hi, mid, lo;
        split3(wa[u][j], wb[u][j], hi, mid, lo);
#pragma unroll
        for (int i = 0; i < NTT; ++i) {
          const bf16x8_t xb = as_bf16x8(xa[u][i]);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, lo, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, mid, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, hi, acc[i][j], 0, 0, 0);
        }
      }
    }
  }
  // lane holds tokens 16 i + 4q + ii, expert 16 j + r of the tile
#pragma unroll
  for (int j = 0; j < NET; ++j) {
    const int e = e0 + 16 * j + r;
    if (!e_ok[j]) continue;
#pragma unroll
    for (int i = 0; i < NTT; ++i)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int64_t t = t0 + 16 * i + 4 * q + ii;
        if (t < T) {
          if constexpr (SM)
            partial[((int64_t)split * T + t) * E + e] = acc[i][j][ii];
          else
            partial[(t * E + e) * nsp + split] = acc[i][j][ii];
        }
      }
  }
}

// One wave per token: sum the split partials in order and add the bias, then the top k and
// their softmax.
template <bool SM>
__global__ __launch_bounds__(256) void router_topk_kernel(const float *__restrict__ partial, int nsplit,
                                                          const float *__restrict__ bias, int64_t T,
                                                          int E, int k, int32_t *__restrict__ topk_idx,
                                                          float *__restrict__ topk_w) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  float v[4];
  router_logits_wave<SM>(partial, nsplit, bias, t, T, E, lane, v);
  topk_softmax_wave(v, E, k, lane, topk_idx + t * k, topk_w + t * k);
}

// Tile shape: 64 tokens x 32 experts per wave once there are many tokens (fewer re-reads of
// the router matrix and of x), else 16 x 16.
static bool router_wide(int64_t T, int E) { return T >= 1024 && E >= 32; }

// Split count for the router's input dimension: enough waves (about 2048, eight per SIMD) to
// spread any batch over the chip, at most kMaxSplits, at least 2 MX blocks per split.
int router_splits(int64_t T, int E, int H) {
  const int tt = router_wide(T, E) ? 64 : 16, et = router_wide(T, E) ? 32 : 16;
  const int64_t tiles = ((T + tt - 1) / tt) * ((E + et - 1) / et);
  const int KB = H / 32;
  if (tiles <= 0 || KB < 2) return 1;
  int64_t s = (2048 + tiles - 1) / tiles;
  if (s > KB / 2) s = KB / 2;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  const int bps = (KB + (int)s - 1) / (int)s;
  return (KB + bps - 1) / bps;
}

size_t router_partial_floats(int64_t T, int E, int H) {
  const int ns = router_splits(T, E, H);
  return (size_t)(router_wide(T, E) ? ns : (ns + 3) / 4 * 4) * T * E;
}

hipError_t launch_router_partial(const uint16_t *x, int64_t T, int H, const float *w, int E, float *partial,
                                 hipStream_t stream, int *counter) {
  const int KB = H / 32;
  const int ns = router_splits(T, E, H);
  const int bps = (KB + ns - 1) / ns;
  if (router_wide(T, E)) {
    dim3 grid((unsigned)((T + 63) / 64), (unsigned)((E + 31) / 32), (unsigned)ns);
    hipLaunchKernelGGL((router_partial_kernel<4, 2, true>), grid, dim3(kWave), 0, stream, x, T, H, w, E, bps, ns,
                       partial, counter);
  } else {
    dim3 grid((unsigned)((T + 15) / 16), (unsigned)((E + 15) / 16), (unsigned)ns);
    hipLaunchKernelGGL((router_partial_kernel<1, 1, false>), grid, dim3(kWave), 0, stream, x, T, H, w, E, bps,
                       (ns + 3) / 4 * 4, partial, counter);
  }
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t *x, int64_t T, int H, const float *w, const float *b, int E, int k,
                         float *partial, int32_t *topk_idx, float *topk_w, hipStream_t stream) {
  const hipError_t err = launch_router_partial(x, T, H, w, E, partial, stream);
  if (err != hipSuccess) return err;
  const int ns = router_splits(T, E, H);
  if (router_wide(T, E))
    hipLaunchKernelGGL(router_topk_kernel<true>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, partial, ns, b,
                       T, E, k, topk_idx, topk_w);
  else
    hipLaunchKernelGGL(router_topk_kernel<false>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, partial, ns, b,
                       T, E, k, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe
