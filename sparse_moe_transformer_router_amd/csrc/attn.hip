// One decode step of grouped-query attention with per-head sink logits (gpt-oss walkthrough
// at pnsm.cn, section 2.1: 64 query heads share 8 key/value heads, layers alternate between a
// 128-token banded window and dense attention, and every head learns a logit that joins the
// softmax's denominator; review of the from-scratch gpt-oss-20B at pomoai.com, section 3.5;
// launch retrospective at youniszhang.com, "工程影响": head dimension 64, 2-byte cache):
//     s_j  = q_h . k_j / 8                        (query head h, its group's key head)
//     out  = sum_j e^(s_j - m) v_j / (sum_j e^(s_j - m) + e^(sink_h - m)),   m = max(s, sink_h)
// over the visible positions j: all lens[b] of them (dense) or the last `window`.
//
// Split-K ("flash decoding"): one wave per (sequence, key head, range of up to kAttnChunk
// positions) computes, for the group's query heads, the range's maximum score, its sum of
// exponentials and its unnormalised output; a second kernel merges the ranges in order and
// adds the sink. Scores and the weighted sum of values run on the matrix cores
// (v_mfma_f32_16x16x32_bf16): scores as K (16 positions x 32 dims) times Q^T (32 dims x up to
// 16 heads); the output as P (heads x 32 positions) times V (32 positions x 16 dims), with
// the weights P split exactly enough into two bf16 terms (hi + lo, relative error ~2^-17) and
// V transposed through LDS. Positions are assigned to the score instruction's rows so that
// its result lands in each lane in the order the output instruction reads P: no shuffles.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kAttnD = 64;          // head dimension
constexpr int kAttnChunk = 256;     // positions per wave
constexpr int kAttnBlock = 32;      // positions per step (two score MFMAs, eight output MFMAs)
constexpr int kAttnMaxGroup = 16;   // query heads per key head (the MFMA's N)

__device__ __forceinline__ u32x4_t load16_or_zero(const uint16_t *p, bool ok) {
  return ok ? *reinterpret_cast<const u32x4_t *>(p) : u32x4_t{0u, 0u, 0u, 0u};
}

// Two floats as RNE bf16, the first in the low half of the dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
}

// Partials: m and l [B][Hkv][nsplit][16], o [B][Hkv][nsplit][16][64] fp32 (heads past the
// group are not written).
// FINAL (one range covers every visible position): the wave adds the sink and writes the
// normalised output itself (sinks, out, out_f32), and no merge runs.
template <bool FINAL>
__global__ __launch_bounds__(kWave) void attn_decode_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
    const int32_t *__restrict__ lens, int Hq, int Hkv, int64_t L, int window, int nsplit,
    float *__restrict__ part_m, float *__restrict__ part_l, float *__restrict__ part_o,
    const float *__restrict__ sinks, void *__restrict__ out, int out_f32) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[kAttnBlock][kAttnD + 8];  // one V block, padded rows
  const int lane = threadIdx.x;
  const int split = blockIdx.x, kvh = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int G = Hq / Hkv;
  const int g = lane / 16, r = lane % 16;
  int64_t n = lens[b];
  n = n < 0 ? 0 : (n > L ? L : n);
  const int64_t lo = (window > 0 && n > window) ? n - window : 0;
  const int64_t k0 = lo + (int64_t)split * kAttnChunk;
  const int64_t k1 = (k0 + kAttnChunk < n) ? k0 + kAttnChunk : n;
  const int64_t pbase = ((b * Hkv + kvh) * nsplit + split) * kAttnMaxGroup;
  if (k0 >= k1) {  // an empty range: neutral partials (the merge gives them weight 0)
    if constexpr (FINAL) {  // no visible position: the output is 0
      for (int h = 0; h < G; ++h) {
        const int64_t oi = ((b * Hq) + (int64_t)kvh * G + h) * kAttnD + lane;
        if (out_f32)
          reinterpret_cast<float *>(out)[oi] = 0.0f;
        else
          reinterpret_cast<uint16_t *>(out)[oi] = 0;
      }
      return;
    }
    if (lane < G) {
      part_m[pbase + lane] = -INFINITY;
      part_l[pbase + lane] = 0.0f;
    }
    for (int h = 0; h < G; ++h) part_o[(pbase + h) * kAttnD + lane] = 0.0f;
    return;
  }
  // Q^T as the score instruction's B operand: lane (g, r) holds head r, dims 8g..8g+7 (and
  // 32 + those for the second half of the dimension)
  const uint16_t *qh = q + ((b * Hq) + (int64_t)kvh * G + (r < G ? r : 0)) * kAttnD;
  const bf16x8_t qb0 = as_bf16x8(load16_or_zero(qh + 8 * g, r < G));
  const bf16x8_t qb1 = as_bf16x8(load16_or_zero(qh + 32 + 8 * g, r < G));
  const uint16_t *kbase = kc + ((b * Hkv + kvh) * L) * kAttnD;
  const uint16_t *vbase = vc + ((b * Hkv + kvh) * L) * kAttnD;
  const int nblk = (int)((k1 - k0 + kAttnBlock - 1) / kAttnBlock);
  // V block j in registers: lane l holds 32 dims (4 x 16 bytes) of position l / 2 of the block;
  // positions past the range read as zeros. Block 0 is requested before the scores, block
  // j + 1 while block j is used.
  u32x4_t vr[4];
  auto vload = [&](int j) {
    const int64_t pos = k0 + kAttnBlock * j + lane / 2;
    const bool ok = pos < k1;
    const uint16_t *vp = vbase + (ok ? pos : k0) * kAttnD + 32 * (lane % 2);
#pragma unroll
    for (int c = 0; c < 4; ++c) vr[c] = load16_or_zero(vp + 8 * c, ok);
  };
  vload(0);

  // Phase 1: every score of the range. Block j, instruction a: row m = r is position
  // 8 (r / 4) + 4 a + r % 4 of the block, so result i of lane (g, r) is position 8 g + 4 a + i
  // for head r -- the A-operand order of the output instruction.
  float s[kAttnChunk / kAttnBlock][2][4];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kAttnChunk / kAttnBlock; ++j) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      if (j < nblk) {
        const int64_t pos = k0 + kAttnBlock * j + 8 * (r / 4) + 4 * a + (r % 4);
        const bool ok = pos < k1;
        const uint16_t *kp = kbase + (ok ? pos : k0) * kAttnD + 8 * g;
        const bf16x8_t ka0 = as_bf16x8(load16_or_zero(kp, ok));
        const bf16x8_t ka1 = as_bf16x8(load16_or_zero(kp + 32, ok));
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0, qb0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1, qb1, acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t pi = k0 + kAttnBlock * j + 8 * g + 4 * a + i;
          const float v = pi < k1 ? acc[i] * 0.125f : -INFINITY;  // 1 / sqrt(64), exact
          s[j][a][i] = v;
          mx = fmaxf(mx, v);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) s[j][a][i] = -INFINITY;
      }
    }
  }
  // the range's maximum per head: over the lane's own scores, then the four lanes of head r
  mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
  mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));

  // Phase 2: weights, their sum, and P V
  f32x4_t o[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) o[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.0f;
#pragma unroll
  for (int j = 0; j < kAttnChunk / kAttnBlock; ++j) {
    if (j < nblk) {  // wave-uniform
      // V block j into LDS (row = position, 64 dims), then the next block's request
#pragma unroll
      for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4_t *>(&vt[lane / 2][32 * (lane % 2) + 8 * c]) = vr[c];
      if (j + 1 < nblk) vload(j + 1);
      // the weights of lane (g, r): head r, positions 8 g .. 8 g + 7 (the output instruction's
      // A operand), as hi + lo bf16 terms
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float p0 = __expf(s[j][t / 2][2 * (t % 2)] - mx), p1 = __expf(s[j][t / 2][2 * (t % 2) + 1] - mx);
        lsum += p0 + p1;
        const uint32_t h = pack_bf16x2(p0, p1);
        ph[t] = h;
        pl[t] = pack_bf16x2(p0 - __uint_as_float(h << 16), p1 - __uint_as_float(h & 0xffff0000u));
      }
      const bf16x8_t pa_hi = as_bf16x8(u32x4_t{ph[0], ph[1], ph[2], ph[3]});
      const bf16x8_t pa_lo = as_bf16x8(u32x4_t{pl[0], pl[1], pl[2], pl[3]});
      __syncthreads();  // the block's V rows are in LDS
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // V^T as the B operand: lane (g, r) holds dim 16 c + r of positions 8 g .. 8 g + 7
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          w[t] = (uint32_t)vt[8 * g + 2 * t][16 * c + r] | ((uint32_t)vt[8 * g + 2 * t + 1][16 * c + r] << 16);
        const bf16x8_t vb = as_bf16x8(u32x4_t{w[0], w[1], w[2], w[3]});
        o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, vb, o[c], 0, 0, 0);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, vb, o[c], 0, 0, 0);
      }
      __syncthreads();  // the block's LDS reads are done before the next block overwrites it
    }
  }
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
  if constexpr (FINAL) {
    // lane r (< 16) holds head r's maximum and sum: the scale of each head's output row
    const float sk = (sinks != nullptr && r < G) ? sinks[(int64_t)kvh * G + r] : -INFINITY;
    const float M = fmaxf(mx, sk);
    const float fo = __expf(mx - M);
    const float den = lsum * fo + (sinks != nullptr ? __expf(sk - M) : 0.0f);
    const float scale_r = den > 0.0f ? fo / den : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      const float sc = __shfl(scale_r, h, kWave);
      if (h < G) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t oi = ((b * Hq) + (int64_t)kvh * G + h) * kAttnD + 16 * c + r;
          const float v = o[c][i] * sc;
          if (out_f32)
            reinterpret_cast<float *>(out)[oi] = v;
          else
            reinterpret_cast<uint16_t *>(out)[oi] = f32_to_bf16_rne(v);
        }
      }
    }
    return;
  }
  if (g == 0 && r < G) {
    part_m[pbase + r] = mx;
    part_l[pbase + r] = lsum;
  }
  // o[c][i] of lane (g, r): head 4 g + i, dim 16 c + r
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    if (h < G) {
#pragma unroll
      for (int c = 0; c < 4; ++c) part_o[(pbase + h) * kAttnD + 16 * c + r] = o[c][i];
    }
  }
}

// Merge the ranges of one (sequence, query head), add the sink, normalise. NW waves: the
// maximum and the denominator with lanes over ranges (every wave computes the maximum), the
// output with lane = dim, wave w summing ranges w, w + NW, ... in order, then the NW sums
// added in wave order. Four waves once there are many ranges (long contexts), else one.
constexpr int kMergeWideSplits = 64;

template <int NW>
__global__ __launch_bounds__(NW *kWave) void attn_decode_merge_kernel(
    const float *__restrict__ part_m, const float *__restrict__ part_l, const float *__restrict__ part_o,
    const float *__restrict__ sinks, int Hq, int Hkv, int nsplit, void *__restrict__ out, int out_f32) {
  __shared__ float red[NW][kAttnD];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int hq = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int G = Hq / Hkv;
  const int kvh = hq / G, h = hq % G;
  const int64_t base = (b * Hkv + kvh) * nsplit;
  float mloc = -INFINITY;
  for (int sp = lane; sp < nsplit; sp += kWave) mloc = fmaxf(mloc, part_m[(base + sp) * kAttnMaxGroup + h]);
  float M = wave_max_f32(mloc);
  const bool sink = sinks != nullptr;
  if (sink) M = fmaxf(M, sinks[hq]);
  // a range's weight e^(m - M), 0 for an empty range (its m is -inf and M may be too);
  // branch-free, so the loads of consecutive ranges stay in flight together
  auto weight = [&](float m, float ls) {
    const float e = __expf(m - M);
    return ls > 0.0f ? e : 0.0f;
  };
  float den = 0.0f;
  if (wave == 0) {
    float dloc = 0.0f;
    for (int sp = lane; sp < nsplit; sp += kWave) {
      const int64_t pi = (base + sp) * kAttnMaxGroup + h;
      const float ls = part_l[pi];
      dloc = fmaf(ls, weight(part_m[pi], ls), dloc);
    }
    den = wave_sum_f32(dloc);
    if (sink && M != -INFINITY) den += __expf(sinks[hq] - M);
  }
  float acc = 0.0f;
  int sp = wave;
  for (; sp + 3 * NW < nsplit; sp += 4 * NW) {  // four ranges' loads at once
    float m[4], ls[4], ov[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t pi = (base + sp + u * NW) * kAttnMaxGroup + h;
      m[u] = part_m[pi];
      ls[u] = part_l[pi];
      ov[u] = part_o[pi * kAttnD + lane];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = fmaf(ov[u], weight(m[u], ls[u]), acc);
  }
  for (; sp < nsplit; sp += NW) {
    const int64_t pi = (base + sp) * kAttnMaxGroup + h;
    const float ls = part_l[pi];
    acc = fmaf(part_o[pi * kAttnD + lane], weight(part_m[pi], ls), acc);
  }
  float tot = acc;
  if constexpr (NW > 1) {
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    tot = red[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) tot += red[w][lane];
  }
  const float v = den > 0.0f ? tot / den : 0.0f;
  const int64_t oi = ((b * Hq) + hq) * kAttnD + lane;
  if (out_f32)
    reinterpret_cast<float *>(out)[oi] = v;
  else
    reinterpret_cast<uint16_t *>(out)[oi] = f32_to_bf16_rne(v);
}

int attn_splits(int64_t L, int window) {
  const int64_t span = (window > 0 && window < L) ? window : L;
  return (int)((span + kAttnChunk - 1) / kAttnChunk);
}

size_t attn_partial_floats(int64_t B, int Hkv, int64_t L, int window) {
  const int64_t rows = B * Hkv * attn_splits(L, window) * kAttnMaxGroup;
  return (size_t)rows * (2 + kAttnD);
}

hipError_t launch_attn_decode(const uint16_t *q, const uint16_t *kc, const uint16_t *vc, const int32_t *lens,
                              const float *sinks, int64_t B, int Hq, int Hkv, int64_t L, int window, void *out,
                              bool out_f32, float *ws, hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  const int ns = attn_splits(L, window);
  const int64_t rows = B * Hkv * ns * kAttnMaxGroup;
  float *pm = ws, *pl = ws + rows, *po = ws + 2 * rows;
  const dim3 grid((unsigned)ns, (unsigned)Hkv, (unsigned)B);
  if (ns == 1) {  // one range per (sequence, key head): the wave finishes the output itself
    hipLaunchKernelGGL(attn_decode_split_kernel<true>, grid, dim3(kWave), 0, stream, q, kc, vc, lens, Hq, Hkv, L,
                       window, ns, pm, pl, po, sinks, out, out_f32 ? 1 : 0);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(attn_decode_split_kernel<false>, grid, dim3(kWave), 0, stream, q, kc, vc, lens, Hq, Hkv, L,
                     window, ns, pm, pl, po, nullptr, nullptr, 0);
  const dim3 mgrid((unsigned)Hq, (unsigned)B);
  if (ns >= kMergeWideSplits)
    hipLaunchKernelGGL(attn_decode_merge_kernel<4>, mgrid, dim3(4 * kWave), 0, stream, pm, pl, po, sinks, Hq, Hkv, ns,
                       out, out_f32 ? 1 : 0);
  else
    hipLaunchKernelGGL(attn_decode_merge_kernel<1>, mgrid, dim3(kWave), 0, stream, pm, pl, po, sinks, Hq, Hkv, ns, out,
                       out_f32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
