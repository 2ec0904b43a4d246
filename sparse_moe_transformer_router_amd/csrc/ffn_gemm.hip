// Expert FFN projections for prefill-sized batches: a grouped GEMM on the matrix cores.
//
// Each expert's slots (review of the from-scratch gpt-oss-20B at pomoai.com, section 3.4)
// are multiplied by its MXFP4 weights (gpt-oss walkthrough at pnsm.cn, sections 1 and 4),
// with the clamped SwiGLU (+1 on the linear branch) fused into the gate_up epilogue
// (walkthrough section 2.2; review section 3.3). Weights must be in the tiled layout.
//
// Workgroup tile: 192 weight rows x 128 slots of one expert (192 divides 5760 and 2880).
// Four waves in a 2 x 2 arrangement; a wave owns 96 rows (three 32-row weight tiles) x 64
// slots (two 32-slot column groups): six v_mfma_f32_32x32x16_bf16 accumulators (96 fp32 in
// AGPRs). The 32x32x16 form issues at twice the rate of 16x16x32 on gfx950. Weights are the
// cheap operand (0.53 B per element against 2 B for a bf16 activation), so the tile is wide
// in weight rows. Per 128-element chunk of the input dimension (one "stage"):
//   * the 128 slots' bf16 activations (gathered rows of x, or rows of act) go straight from
//     global memory to LDS with gfx950's global_load_lds_dwordx4 (no staging registers),
//     into a 3-deep ring of 32 KB stages; each 256-byte slot row has its 16-byte columns
//     XOR-swizzled by the row index, so a wave's 16-row reads land on distinct banks (the
//     swizzle is applied on the global side: lane l of a DMA writes LDS column l % 16);
//   * the workgroup's six weight tiles (2 KB each) and their scale tiles go to LDS the same
//     way, so no global load has a register destination (register reuse would otherwise
//     force the compiler to drain every load in flight);
//   * all of a stage's loads are issued two stages ahead (12 DMA instructions per wave),
//     spread over the eight MFMA k-steps of the chunk before. A stage is consumed after an
//     explicit s_waitcnt vmcnt(12) (the next stage's loads may stay in flight) and a bare
//     s_barrier -- no fence, which would drain the prefetches. Every DMA is issued
//     unconditionally from a clamped, in-bounds address (past the last chunk the last chunk
//     is re-loaded into the ring slot nobody reads), so the count is exact; tiles past N
//     read tile 0 and their rows are never stored;
//   * the LDS reads of the next MFMA k-step's slot operands are issued before the current
//     step's MFMAs;
//   * lane l of a weight tile holds MX block 4c + 2p + l/32 of row l%32 (p = 0, 1), split into
//     four 8-element k-steps; the B operand reads the same k-assignment from LDS.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kG2Cols = 128;            // slots per tile
constexpr int kG2Stages = 3;            // LDS ring depth
constexpr int kG2RowBytes = 256;        // one 128-element bf16 chunk of a slot
constexpr int kG2StageBytes = kG2Cols * kG2RowBytes;
constexpr int kG2RGW = 3;               // 32-row weight tiles per wave (wave owns 96 rows)
constexpr int kG2Rows = 2 * 32 * kG2RGW;  // weight rows per workgroup
constexpr int kG2Waves = 8;             // two per SIMD: 2 x 2 output quarters x 2 k-halves
constexpr int kG2GroupM = 4;            // m-tiles per group of the XCD-local tile order
constexpr int kXcds = 8;                // accelerator complex dies, one L2 each

__device__ __forceinline__ int g2_off(int row, int col16) { return row * kG2RowBytes + ((col16 ^ (row & 15)) << 4); }

__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
  // s_waitcnt immediate with vmcnt = n (split field) and expcnt / lgkmcnt left at their maxima
  return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8);
}

template <int EPI>
__global__ __launch_bounds__(kG2Waves * 64) void ffn_gemm2_kernel(const uint16_t *__restrict__ a_src, int a_by_token,
                                                        const int32_t *__restrict__ sorted_slot, int k,
                                                        const int32_t *__restrict__ offsets, int E,
                                                        const uint8_t *__restrict__ pcodes,
                                                        const uint8_t *__restrict__ pscales,
                                                        const uint16_t *__restrict__ bias, int N, int K, int ntiles_n,
                                                        void *__restrict__ out, float limit, float alpha) {
  constexpr int RGW = kG2RGW;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform: LDS targets stay scalar
  const int wk = wave >> 2;                       // which half of every chunk's k-steps
  const int wy = (wave >> 1) & 1, wx = wave & 1;  // weight-row half, slot half
  // Real m-tile count: the grid is sized for the worst case, the surplus blocks exit.
  int mt_total = 0;
  for (int eb = 0; eb < E; eb += 64) {
    const int ex = eb + lane;
    const int cnt = (ex < E) ? offsets[ex + 1] - offsets[ex] : 0;
    mt_total += __shfl(wave_inclusive_scan((cnt + kG2Cols - 1) / kG2Cols), 63, 64);
  }
  const int nb = mt_total * ntiles_n;
  if ((int)blockIdx.x >= nb) return;
  int mt, nt;
  {
    // Workgroups are dispatched round-robin over the 8 XCDs (block b to XCD b % 8), each with
    // its own L2. Give XCD x a contiguous range of the nb logical tiles, and order a range in
    // groups of kG2GroupM m-tiles x all n-tiles, n-major: the ~32 workgroups an XCD runs at a
    // time then share 4 slot tiles and 8 weight tiles.
    const int b = blockIdx.x, x = b % kXcds, loc = b / kXcds;
    const int q = nb / kXcds, rr = nb % kXcds;
    const int L = (x < rr) ? x * (q + 1) + loc : rr * (q + 1) + (x - rr) * q + loc;
    const int grp = L / (kG2GroupM * ntiles_n);
    const int gm = (mt_total - grp * kG2GroupM < kG2GroupM) ? mt_total - grp * kG2GroupM : kG2GroupM;
    const int rem = L - grp * kG2GroupM * ntiles_n;
    nt = rem / gm;
    mt = grp * kG2GroupM + rem % gm;
  }
  int e = -1, m0 = 0, rbase = 0, mcount = 0;
  {
    int carry = 0;
    for (int eb = 0; eb < E; eb += 64) {
      const int ex = eb + lane;
      const int cnt = (ex < E) ? offsets[ex + 1] - offsets[ex] : 0;
      const int tiles = (cnt + kG2Cols - 1) / kG2Cols;
      const int inc = wave_inclusive_scan(tiles);
      const int excl = inc - tiles + carry;
      const uint64_t hit = __ballot(tiles > 0 && mt >= excl && mt < excl + tiles);
      if (hit) {
        const int src = __ffsll((unsigned long long)hit) - 1;
        const int sel_excl = __shfl(excl, src, 64);
        e = eb + src;
        m0 = (mt - sel_excl) * kG2Cols;
        rbase = offsets[e];
        const int cnt_e = offsets[e + 1] - rbase;
        mcount = (cnt_e - m0 < kG2Cols) ? cnt_e - m0 : kG2Cols;
        break;
      }
      carry += __shfl(inc, 63, 64);
    }
  }
  if (e < 0) return;
  const int KB = K / 32;
  const int nchunk = (KB + 3) / 4;
  const int NG = N / 32;
  const int r32 = lane % 32, kh = lane / 32;

  // staging: wave stages slot rows 16 wave + 4 i + lane / 16 (i = 0..3), physical 16-byte
  // column lane % 16
  const uint16_t *aptr[4];
  int lcol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * wave + 4 * i + lane / 16;
    const int srow = row < mcount ? row : 0;  // padding slots re-read slot 0 (results discarded)
    const int r = rbase + m0 + srow;
    lcol[i] = ((lane % 16) ^ (row & 15)) * 8;  // logical element offset within the chunk
    aptr[i] = a_src + (a_by_token ? (int64_t)(sorted_slot[r] / k) : (int64_t)r) * K;
  }
  // One DMA of stage cc (a chunk index, always < nchunk) into ring slot `slot`; a wave issues
  // six per stage:
  //   i = 0..3: activation rows 4 i .. 4 i + 3 of this wave's 16;
  //   i = 4, 5: waves 0..5: 1 KB half i - 4 of weight tile `wave`; waves 6, 7: 256 bytes of
  //             the stage's scale block (bytes 512 (wave - 6) + 256 (i - 4) ...; the block
  //             holds 2 RGW x 128 bytes, the rest is padding).
  constexpr int kWStage = 2 * RGW * 2048;
  constexpr int kSStage = 1024;
  unsigned char *lds_w = lds + kG2Stages * kG2StageBytes;
  unsigned char *lds_s = lds_w + kG2Stages * kWStage;
  const int gt0 = nt * 2 * RGW;  // first weight tile of the workgroup
  const uint8_t *cexp = pcodes + (int64_t)e * NG * nchunk * 2048 + lane * 16;
  const uint8_t *sexp = pscales + (int64_t)e * NG * nchunk * 128;
  auto dma = [&](int i, int cc, int slot) {
    if (i < 4) {
      int kk = cc * 128 + lcol[i];
      kk = kk < K ? kk : 0;  // past K: any in-bounds element (its weight is an exact zero)
      __builtin_amdgcn_global_load_lds(aptr[i] + kk,
                                       lds + slot * kG2StageBytes + (16 * wave + 4 * i) * kG2RowBytes, 16, 0, 0);
    } else if (wave < 2 * RGW) {
      const int g = gt0 + wave;
      const int64_t t = (g < NG) ? (int64_t)g * nchunk + cc : 0;
      __builtin_amdgcn_global_load_lds(cexp + t * 2048 + (i - 4) * 1024,
                                       lds_w + slot * kWStage + wave * 2048 + (i - 4) * 1024, 16, 0, 0);
    } else {
      const int ob = 512 * (wave - 2 * RGW) + 256 * (i - 4);  // first byte of this DMA
      const int o = ob + 4 * lane;
      const int ti = o / 128;
      const int g = gt0 + ti;
      const int64_t t = (ti < 2 * RGW && g < NG) ? (int64_t)g * nchunk + cc : 0;
      __builtin_amdgcn_global_load_lds(sexp + t * 128 + (o % 128), lds_s + slot * kSStage + ob, 4, 0, 0);
    }
  };

  f32x16_t acc[RGW][2];
#pragma unroll
  for (int g = 0; g < RGW; ++g)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[g][b][i] = 0.f;

  // Every chunk issues exactly 6 DMAs per wave (past the last chunk they re-load the last
  // chunk into the ring slot nobody reads), so before chunk c the younger loads are always
  // chunk c+1's 6.
#pragma unroll
  for (int i = 0; i < 6; ++i) dma(i, 0, 0);
#pragma unroll
  for (int i = 0; i < 6; ++i) dma(i, nchunk > 1 ? 1 : 0, 1);
  const int p = wk;  // this wave's half of each chunk: MX blocks 4c + 2p + kh
  for (int c = 0; c < nchunk; ++c) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(6));
    __builtin_amdgcn_s_barrier();
    const int cn = (c + 2 < nchunk) ? c + 2 : nchunk - 1;  // chunk staged during this one
    const int sn = (c + 2) % kG2Stages;                      // its ring slot (read by nobody now)
    const int sc_ = c % kG2Stages;
    const unsigned char *abuf = lds + sc_ * kG2StageBytes;
    const unsigned char *wbuf = lds_w + sc_ * kWStage + (wy * RGW) * 2048 + p * 1024 + lane * 16;
    const unsigned char *sbuf = lds_s + sc_ * kSStage + (wy * RGW) * 128 + r32 * 4;
    u32x4_t cw[RGW];
    float sc[RGW];
#pragma unroll
    for (int g = 0; g < RGW; ++g) {
      cw[g] = *reinterpret_cast<const u32x4_t *>(wbuf + g * 2048);
      sc[g] = e8m0_to_f32((*reinterpret_cast<const uint32_t *>(sbuf + g * 128) >> (8 * (2 * p + kh))) & 0xffu);
    }
    auto bload = [&](int j, bf16x8_t *bv) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bv[b] = as_bf16x8(
            *reinterpret_cast<const u32x4_t *>(abuf + g2_off(wx * 64 + 32 * b + r32, 4 * (2 * p + kh) + j)));
    };
    bf16x8_t bcur[2], bnext[2];
    bload(0, bcur);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < 3) bload(j + 1, bnext);
      // this k-step's share of the next stage's DMAs, issued in the shadow of its MFMAs
      if (j < 2) {
        dma(2 * j, cn, sn);
        dma(2 * j + 1, cn, sn);
      } else {
        dma(j + 2, cn, sn);
      }
#pragma unroll
      for (int g = 0; g < RGW; ++g) {
        const bf16x8_t wa = fp4x8_to_bf16x8(cw[g][j], sc[g]);
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[g][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, bcur[b], acc[g][b], 0, 0, 0);
      }
      bcur[0] = bnext[0];
      bcur[1] = bnext[1];
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no DMA may still target this workgroup's LDS
  __syncthreads();                // every wave is done reading the ring

  // The two halves of each output tile: the p = 1 waves hand their sums to the p = 0 waves
  // through LDS (fixed order: p = 0 sum + p = 1 sum).
  {
    f32x4_t *red = reinterpret_cast<f32x4_t *>(lds) + (wave & 3) * (RGW * 2 * 4) * 64 + lane;
    if (wk == 1) {
#pragma unroll
      for (int g = 0; g < RGW; ++g)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            red[((g * 2 + b) * 4 + q) * 64] =
                f32x4_t{acc[g][b][4 * q], acc[g][b][4 * q + 1], acc[g][b][4 * q + 2], acc[g][b][4 * q + 3]};
    }
    __syncthreads();
    if (wk == 1) return;
#pragma unroll
    for (int g = 0; g < RGW; ++g)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t o = red[((g * 2 + b) * 4 + q) * 64];
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[g][b][4 * q + u] += o[u];
        }
  }

  // epilogue: lane holds slot column wx*64 + 32b + r32 and, per tile g, rows 8i + 4kh + jj.
  // The bias of a lane's rows is 4 consecutive bf16 per (g, i): twelve 8-byte loads, all
  // issued before any is used (clamped rows past N read row 0 and are never stored).
  const int nbase = nt * kG2Rows + wy * 32 * RGW;
  uint2 bq[RGW][4];
#pragma unroll
  for (int g = 0; g < RGW; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) bq[g][i] = uint2{0u, 0u};
  if (bias != nullptr) {
    const uint16_t *be = bias + (int64_t)e * N;
#pragma unroll
    for (int g = 0; g < RGW; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = nbase + 32 * g + 8 * i + 4 * kh;
        bq[g][i] = *reinterpret_cast<const uint2 *>(be + (n < N ? n : 0));
      }
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int col = wx * 64 + 32 * b + r32;
    if (col >= mcount) continue;
    const int64_t r = rbase + m0 + col;
#pragma unroll
    for (int g = 0; g < RGW; ++g) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = nbase + 32 * g + 8 * i + 4 * kh;
        if (n >= N) continue;
        float h[4];
        h[0] = acc[g][b][4 * i + 0] + __uint_as_float(bq[g][i].x << 16);
        h[1] = acc[g][b][4 * i + 1] + __uint_as_float(bq[g][i].x & 0xffff0000u);
        h[2] = acc[g][b][4 * i + 2] + __uint_as_float(bq[g][i].y << 16);
        h[3] = acc[g][b][4 * i + 3] + __uint_as_float(bq[g][i].y & 0xffff0000u);
        if (EPI == kEpiSwigluBf16 || EPI == kEpiActF32) {
          const int half = N / 2;
          const uint16_t a0 = f32_to_bf16_rne(swiglu_unit(h[0], h[1], limit, alpha));
          const uint16_t a1 = f32_to_bf16_rne(swiglu_unit(h[2], h[3], limit, alpha));
          if (EPI == kEpiSwigluBf16) {
            *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(out) + r * half + n / 2) =
                (uint32_t)a0 | ((uint32_t)a1 << 16);
          } else {
            *reinterpret_cast<float2 *>(reinterpret_cast<float *>(out) + r * half + n / 2) =
                float2{bf16_to_f32(a0), bf16_to_f32(a1)};
          }
        } else {
          *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(out) + r * N + n) = f32x4_t{h[0], h[1], h[2], h[3]};
        }
      }
    }
  }
}

hipError_t launch_ffn_gemm(const uint16_t *a_src, bool a_by_token, const int32_t *sorted_slot, int k,
                           const int32_t *offsets, int E, int64_t S, const MxWeight &w, int epilogue, void *out,
                           float limit, float alpha, hipStream_t stream) {
  const int64_t busy = (S < E) ? S : E;
  const int64_t mtiles = (S + kG2Cols - 1) / kG2Cols + busy;
  const int ntn = (w.N + kG2Rows - 1) / kG2Rows;
  dim3 grid((unsigned)(mtiles * ntn));
  const size_t lds = (size_t)kG2Stages * (kG2StageBytes + 2 * kG2RGW * 2048 + 1024);
#define MOE_LAUNCH_GEMM(EPI)                                                                          \
  hipLaunchKernelGGL(ffn_gemm2_kernel<EPI>, grid, dim3(kG2Waves * 64), lds, stream, a_src, a_by_token ? 1 : 0, \
                     sorted_slot, k, offsets, E, w.codes, w.scales, w.bias, w.N, w.K, ntn, out, limit, alpha)
  switch (epilogue) {
    case kEpiSwigluBf16: MOE_LAUNCH_GEMM(kEpiSwigluBf16); break;
    case kEpiPreactF32: MOE_LAUNCH_GEMM(kEpiPreactF32); break;
    case kEpiActF32: MOE_LAUNCH_GEMM(kEpiActF32); break;
    default: MOE_LAUNCH_GEMM(kEpiLinearF32); break;
  }
#undef MOE_LAUNCH_GEMM
  return hipGetLastError();
}

}  // namespace moe
