// Expert FFN projections for prefill-sized batches: a persistent grouped GEMM on the matrix
// cores.
//
// Each expert's slots (review of the from-scratch gpt-oss-20B at pomoai.com, section 3.4)
// are multiplied by its MXFP4 weights (gpt-oss walkthrough at pnsm.cn, sections 1 and 4),
// with the clamped SwiGLU (+1 on the linear branch) fused into the gate_up epilogue
// (walkthrough section 2.2; review section 3.3). Weights must be in the tiled layout; the
// activations are expert-sorted rows (x gathered by launch_gather_rows, or the act rows).
//
// Output tile: 64 RGW weight rows x 128 slots of one expert, RGW = 4 (256 rows) or 3 (192,
// which divides 5760 and 2880; chosen by the padding each leaves). Four waves in a 2 x 2
// arrangement; a wave owns 32 RGW rows (RGW 32-row weight tiles) x 64 slots (two 32-slot
// column groups): 2 RGW v_mfma_f32_32x32x16_bf16 accumulators. Weights are the cheap operand
// (0.53 B per element against 2 B for a bf16 activation), so the tile is tall in weight rows.
//
// Persistent: one workgroup per CU walks a list of tiles, and its load stream runs across
// tile boundaries, so a tile's start-up (locating its expert, first loads) and its epilogue
// hide behind the neighbouring tiles' matrix work. Per 128-element chunk of the input
// dimension (one "stage"), everything the chunk needs goes from global memory to LDS with
// gfx950's global_load_lds (no register destinations: with loads into registers in flight
// beside LDS DMA the compiler can only wait for all of them):
//   * 128 slot rows x 256 bytes of bf16 activations into a 3-deep ring; each row's 16-byte
//     columns are XOR-swizzled by the row index so a wave's 16-row reads hit distinct banks
//     (applied on the global side: lane l of a DMA writes LDS column l % 16);
//   * the 2 RGW 2 KB weight tiles, their 128-byte scale tiles and the tile's bias values.
// Each wave issues exactly 10 + RGW DMAs per stage, two stages ahead, spread over the eight
// MFMA k-steps of the chunk before; a stage is consumed after an explicit s_waitcnt vmcnt
// of that count
// and a bare s_barrier (a fence would drain the prefetches). Every DMA reads a clamped,
// in-bounds address (past the end of the list the last chunk is re-loaded into the ring
// slot nobody reads), so the count is exact. Rows past N read tile 0 and are never stored;
// slots past an m-tile's count re-read its first slot and are never stored.
//
// Tile order: workgroups are dispatched round-robin over the 8 XCDs (block b to XCD b % 8),
// each with its own L2. XCD x owns a contiguous range of the tile list, ordered in groups of
// kGGroupM m-tiles x all n-tiles (n-major), and its workgroups sweep the range together, so
// the ~32 tiles an XCD works on at a time share 4 slot tiles and 8 weight tiles.
//
// Lane l of a weight tile holds MX block 4c + 2p + l/32 of row l%32 (p = 0, 1), split into
// four 8-element k-steps; the B operand reads the same k-assignment from LDS.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kGCols = 128;       // slots per tile
constexpr int kGStages = 3;       // LDS ring depth
constexpr int kGRowBytes = 256;   // one 128-element bf16 chunk of a slot row
constexpr int kGActBytes = kGCols * kGRowBytes;
constexpr int kGSBytes = 1024;    // the tiles' scales (2 RGW x 128 bytes, padded)
constexpr int kGBBytes = 1024;    // the tile's bias (64 RGW rows x 2 bytes, padded)
constexpr int kGGroupM = 4;       // m-tiles per group of the XCD-local tile order
constexpr int kXcds = 8;
constexpr int kGMaxExperts = 256;
// RGW = 32-row weight tiles per wave: a tile is 64 RGW weight rows x 128 slots
template <int RGW>
struct GShape {
  static constexpr int kRows = 64 * RGW;
  static constexpr int kWBytes = 2 * RGW * 2048;  // codes of the 2 RGW weight tiles
  static constexpr int kStageBytes = kGActBytes + kWBytes + kGSBytes + kGBBytes;
  static constexpr int kDma = 8 + RGW + 2;        // DMAs per wave per stage
  static constexpr size_t kLds = (size_t)kGStages * kStageBytes + (kGMaxExperts + 4) * sizeof(int32_t);
};

__device__ __forceinline__ int g_off(int row, int col16) { return row * kGRowBytes + ((col16 ^ (row & 15)) << 4); }

__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
  // s_waitcnt immediate with vmcnt = n (split field) and expcnt / lgkmcnt left at their maxima
  return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8);
}

// An 8-byte LDS read that waits for its own result (inside the asm block). The compiler
// cannot see that it reads LDS the in-flight DMAs do not touch, and would otherwise wait
// for every load in flight before it.
__device__ __forceinline__ uint2 lds_read_b64_sync(const void *p) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
  uint2 v;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}

struct GTile {
  int e, nt, row0, mcount;  // expert, weight-row tile, first sorted row, slots (1..128)
};

// Tile L of the global list -> its expert and rows, from the expert offsets held in LDS.
__device__ GTile g_tile(int L, const int32_t *off, int E, int mt_total, int ntn, int lane) {
  const int grp = L / (kGGroupM * ntn);
  const int gm = (mt_total - grp * kGGroupM < kGGroupM) ? mt_total - grp * kGGroupM : kGGroupM;
  const int rem = L - grp * kGGroupM * ntn;
  const int mt = grp * kGGroupM + rem % gm;
  GTile t{0, rem / gm, 0, 1};
  int carry = 0;
  for (int eb = 0; eb < E; eb += 64) {
    const int ex = eb + lane;
    const int cnt = (ex < E) ? off[ex + 1] - off[ex] : 0;
    const int tiles = (cnt + kGCols - 1) / kGCols;
    const int inc = wave_inclusive_scan(tiles);
    const int excl = inc - tiles + carry;
    const uint64_t hit = __ballot(tiles > 0 && mt >= excl && mt < excl + tiles);
    if (hit) {
      const int src = __ffsll((unsigned long long)hit) - 1;
      const int e = eb + src;
      const int m0 = (mt - wave_read(excl, src)) * kGCols;
      const int cnt_e = off[e + 1] - off[e];
      t.e = e;
      t.row0 = off[e] + m0;
      t.mcount = (cnt_e - m0 < kGCols) ? cnt_e - m0 : kGCols;
      break;
    }
    carry += wave_read(inc, 63);
  }
  // wave-uniform by construction; say so, so the fields live in scalar registers
  t.e = __builtin_amdgcn_readfirstlane(t.e);
  t.nt = __builtin_amdgcn_readfirstlane(t.nt);
  t.row0 = __builtin_amdgcn_readfirstlane(t.row0);
  t.mcount = __builtin_amdgcn_readfirstlane(t.mcount);
  return t;
}

template <int EPI, int RGW>
__global__ __launch_bounds__(256) void ffn_gemm_kernel(const uint16_t *__restrict__ a, const int32_t *__restrict__ offsets,
                                                       int E, const uint8_t *__restrict__ pcodes,
                                                       const uint8_t *__restrict__ pscales,
                                                       const uint16_t *__restrict__ bias, int N, int K, int ntn,
                                                       void *__restrict__ out, float limit, float alpha) {
  using SH = GShape<RGW>;
  constexpr int kGRows = SH::kRows, kGWBytes = SH::kWBytes, kGStageBytes = SH::kStageBytes, kGDma = SH::kDma;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  int32_t *off = reinterpret_cast<int32_t *>(lds + kGStages * kGStageBytes);
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform: LDS targets stay scalar
  const int wy = wave >> 1, wx = wave & 1;                      // weight-row half, slot half
  const int r32 = lane % 32, kh = lane / 32;

  for (int i = tid; i <= E; i += 256) off[i] = offsets[i];
  __syncthreads();
  int mt_total = 0;  // m-tiles over all experts (the list is sized from them, not from the grid)
  for (int eb = 0; eb < E; eb += 64) {
    const int ex = eb + lane;
    const int cnt = (ex < E) ? off[ex + 1] - off[ex] : 0;
    mt_total += wave_read(wave_inclusive_scan((cnt + kGCols - 1) / kGCols), 63);
  }
  mt_total = __builtin_amdgcn_readfirstlane(mt_total);
  const int nb = mt_total * ntn;
  // nx contiguous ranges of the list, one per XCD (fewer when the grid is smaller, so every
  // range has workgroups); range x belongs to the workgroups b with b % nx == x
  const int nx = (int)gridDim.x < kXcds ? (int)gridDim.x : kXcds;
  const int x = blockIdx.x % nx, q = blockIdx.x / nx;
  const int nq = ((int)gridDim.x - x + nx - 1) / nx;  // workgroups on range x
  const int lo = (int)((int64_t)nb * x / nx), hi = (int)((int64_t)nb * (x + 1) / nx);
  const int first = lo + q;
  if (first >= hi) return;
  const int ntiles = (hi - first + nq - 1) / nq;  // this workgroup's tiles: first + nq j
  const int KB = K / 32;
  const int nchunk = (KB + 3) / 4;
  const int NG = N / 32;

  // ---- issue side: the tile and chunk whose stage is loaded next
  int ji = 0, ci = 0;
  GTile ti = g_tile(first, off, E, mt_total, ntn, lane);
  const uint16_t *aptr[8];
  int lcol[8];
  auto set_rows = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 32 * wave + 4 * i + lane / 16;
      aptr[i] = a + (int64_t)(ti.row0 + (row < ti.mcount ? row : 0)) * K;
    }
  };
#pragma unroll
  for (int i = 0; i < 8; ++i) lcol[i] = ((lane % 16) ^ ((32 * wave + 4 * i + lane / 16) & 15)) * 8;
  set_rows();
  auto advance_issue = [&]() {
    if (++ci < nchunk) return;
    if (ji + 1 < ntiles) {
      ++ji;
      ci = 0;
      ti = g_tile(first + ji * nq, off, E, mt_total, ntn, lane);
      set_rows();
    } else {
      ci = nchunk - 1;  // past the end: keep re-loading the last chunk (into a free slot)
    }
  };
  // DMA i (0 .. kDma - 1) of the issue-side chunk into ring slot `slot`:
  //   0..7            activation rows 32 wave + 4 i .. + 3;
  //   8..8+RGW-1      1 KB of weight codes: tile m / 2, half m % 2, m = RGW wave + i - 8;
  //   8+RGW           256 bytes of the scale block (2 RGW tiles x 128 bytes, then padding);
  //   8+RGW+1         waves 0, 1: 256 bytes of the tile's bias run (2 x 64 RGW bytes);
  //                   waves 2, 3: a dummy.
  const uint8_t *ccode = pcodes + lane * 16;
  auto dma = [&](int i, int slot) {
    unsigned char *st = lds + slot * kGStageBytes;
    const int gt0 = ti.nt * 2 * RGW;
    const int64_t ebase = (int64_t)ti.e * NG * nchunk;
    if (i < 8) {
      int kk = ci * 128 + lcol[i];
      kk = kk < K ? kk : 0;  // past K: any in-bounds element (its weight is an exact zero)
      __builtin_amdgcn_global_load_lds(aptr[i] + kk, st + (32 * wave + 4 * i) * kGRowBytes, 16, 0, 0);
    } else if (i < 8 + RGW) {
      const int m = RGW * wave + i - 8;
      const int g = gt0 + m / 2;
      const int64_t t = (g < NG) ? ebase + (int64_t)g * nchunk + ci : 0;
      __builtin_amdgcn_global_load_lds(ccode + t * 2048 + (m % 2) * 1024, st + kGActBytes + m * 1024, 16, 0, 0);
    } else if (i == 8 + RGW) {
      const int o = 256 * wave + 4 * lane;
      const int tt = o / 128, g = gt0 + tt;
      const int64_t t = (tt < 2 * RGW && g < NG) ? ebase + (int64_t)g * nchunk + ci : 0;
      __builtin_amdgcn_global_load_lds(pscales + t * 128 + (o % 128), st + kGActBytes + kGWBytes + 256 * wave, 4, 0,
                                       0);
    } else {
      const int o = 256 * wave + 4 * lane;  // byte of the tile's bias run
      const int n = ti.nt * kGRows + o / 2;
      const uint16_t *src = (bias != nullptr && o < 2 * kGRows && n < N) ? bias + (int64_t)ti.e * N + n
                                                                         : reinterpret_cast<const uint16_t *>(pscales);
      __builtin_amdgcn_global_load_lds(src, st + kGActBytes + kGWBytes + kGSBytes + 256 * wave, 4, 0, 0);
    }
  };

  // ---- compute side
  GTile tc = ti;
  f32x16_t acc[RGW][2];
  auto zero = [&]() {
#pragma unroll
    for (int g = 0; g < RGW; ++g)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][b][i] = 0.f;
  };
  zero();

  // epilogue of the compute-side tile from ring slot `slot` (its last chunk's stage holds the
  // tile's bias): lane holds slot column wx*64 + 32b + r32 and rows 8i + 4kh + jj of tile g
  auto epilogue = [&](int slot) {
    const unsigned char *bb = lds + slot * kGStageBytes + kGActBytes + kGWBytes + kGSBytes;
    const int nloc0 = wy * 32 * RGW;
    const uint32_t bmask = bias != nullptr ? 0xffffffffu : 0u;  // without bias the run holds junk
    uint2 bq[RGW][4];
#pragma unroll
    for (int g = 0; g < RGW; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint2 v = lds_read_b64_sync(bb + 2 * (nloc0 + 32 * g + 8 * i + 4 * kh));
        bq[g][i] = uint2{v.x & bmask, v.y & bmask};
      }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int col = wx * 64 + 32 * b + r32;
      if (col >= tc.mcount) continue;
      const int64_t r = tc.row0 + col;
#pragma unroll
      for (int g = 0; g < RGW; ++g) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = tc.nt * kGRows + nloc0 + 32 * g + 8 * i + 4 * kh;
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
            *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(out) + r * N + n) =
                f32x4_t{h[0], h[1], h[2], h[3]};
          }
        }
      }
    }
  };

  // prologue: stages 0 and 1
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int i = 0; i < kGDma; ++i) dma(i, s);
    advance_issue();
  }
  int G = 0;  // global chunk counter: ring slot G % 3
  for (int jc = 0; jc < ntiles; ++jc) {
    for (int cc = 0; cc < nchunk; ++cc, ++G) {
      // this wave's 13 loads of stage G are the oldest outstanding but for stage G+1's 13
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kGDma));
      __builtin_amdgcn_s_barrier();
      const int slot = G % kGStages, nslot = (G + 2) % kGStages;
      const unsigned char *abuf = lds + slot * kGStageBytes;
      const unsigned char *wbuf = abuf + kGActBytes + (wy * RGW) * 2048 + lane * 16;
      const unsigned char *sbuf = abuf + kGActBytes + kGWBytes + (wy * RGW) * 128 + r32 * 4;
      uint32_t swd[RGW];
#pragma unroll
      for (int g = 0; g < RGW; ++g) swd[g] = *reinterpret_cast<const uint32_t *>(sbuf + g * 128);
      auto bload = [&](int p, int j, bf16x8_t *bv) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
          bv[b] = as_bf16x8(
              *reinterpret_cast<const u32x4_t *>(abuf + g_off(wx * 64 + 32 * b + r32, 4 * (2 * p + kh) + j)));
      };
      bf16x8_t bcur[2], bnext[2];
      bload(0, 0, bcur);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        u32x4_t cw[RGW];
        float sc[RGW];
#pragma unroll
        for (int g = 0; g < RGW; ++g) {
          cw[g] = *reinterpret_cast<const u32x4_t *>(wbuf + g * 2048 + p * 1024);
          sc[g] = e8m0_to_f32((swd[g] >> (8 * (2 * p + kh))) & 0xffu);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int s = 4 * p + j;
          const int nj = (j + 1) & 3, np = p + (j == 3 ? 1 : 0);
          if (np < 2) bload(np, nj, bnext);
          // this k-step's share of the stage-after-next DMAs, in the shadow of its MFMAs
          dma(s, nslot);
          if (s < RGW + 2) dma(8 + s, nslot);
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
      advance_issue();
    }
    epilogue((G - 1) % kGStages);  // the tile's last chunk is still in its ring slot
    zero();
    if (jc + 1 < ntiles) tc = g_tile(first + (jc + 1) * nq, off, E, mt_total, ntn, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no DMA may still target this workgroup's LDS when it ends
}

int gemm_grid_cap() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// Tile height: 256 weight rows (fewer bytes per flop and more time to hide each stage's
// loads: 624 vs 674 us for the 5760-row gate_up at 16,384 slots) unless that pads more than
// a tenth of the 32-row tiles; then 192 if it pads less.
hipError_t launch_ffn_gemm(const uint16_t *a_sorted, const int32_t *offsets, int E, int64_t S, const MxWeight &w,
                           int epilogue, void *out, float limit, float alpha, hipStream_t stream) {
  if (E > kGMaxExperts) return hipErrorInvalidValue;
  const int NG = w.N / 32;
  const int pad4 = (NG + 7) / 8 * 8 - NG, pad3 = (NG + 5) / 6 * 6 - NG;
  const bool tall = pad4 * 10 <= NG || pad4 <= pad3;
  const int rows = tall ? GShape<4>::kRows : GShape<3>::kRows;
  const int64_t busy = (S < E) ? S : E;
  const int64_t mtiles = (S + kGCols - 1) / kGCols + busy;  // bound on the real m-tile count
  const int ntn = (w.N + rows - 1) / rows;
  const int64_t bound = mtiles * ntn;
  const int cap = gemm_grid_cap();  // one workgroup per CU (the LDS ring takes most of a CU)
  dim3 grid((unsigned)(bound < cap ? bound : cap));
#define MOE_LAUNCH_GEMM(EPI, RG)                                                                               \
  hipLaunchKernelGGL((ffn_gemm_kernel<EPI, RG>), grid, dim3(256), GShape<RG>::kLds, stream, a_sorted, offsets, E, \
                     w.codes, w.scales, w.bias, w.N, w.K, ntn, out, limit, alpha)
#define MOE_LAUNCH_GEMM_EPI(RG)                                               \
  switch (epilogue) {                                                         \
    case kEpiSwigluBf16: MOE_LAUNCH_GEMM(kEpiSwigluBf16, RG); break;          \
    case kEpiPreactF32: MOE_LAUNCH_GEMM(kEpiPreactF32, RG); break;            \
    case kEpiActF32: MOE_LAUNCH_GEMM(kEpiActF32, RG); break;                  \
    default: MOE_LAUNCH_GEMM(kEpiLinearF32, RG); break;                       \
  }
  if (tall) {
    MOE_LAUNCH_GEMM_EPI(4)
  } else {
    MOE_LAUNCH_GEMM_EPI(3)
  }
#undef MOE_LAUNCH_GEMM_EPI
#undef MOE_LAUNCH_GEMM
  return hipGetLastError();
}

}  // namespace moe
