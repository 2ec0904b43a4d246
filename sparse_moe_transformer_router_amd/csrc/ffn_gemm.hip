// Expert FFN projections for prefill-sized batches: a persistent grouped GEMM on the matrix
// cores.
//
// Each expert's slots (review of the from-scratch gpt-oss-20B at pomoai.com, section 3.4)
// are multiplied by its MXFP4 weights (gpt-oss walkthrough at pnsm.cn, sections 1 and 4),
// with the clamped SwiGLU (+1 on the linear branch) fused into the gate_up epilogue
// (walkthrough section 2.2; review section 3.3). Weights must be in the tiled layout; the
// activations are expert-sorted rows (x gathered by launch_gather_rows, or the act rows), or
// on the block-scaled path optionally rows picked through a row map (sorted row r reads
// a_rows[r] / a_div: a slot's token record, so x is converted once per token).
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
// Each wave issues exactly 10 + RGW DMAs per stage (11 + RGW block-scaled), two stages
// ahead, spread over the MFMAs of the chunk before; a stage is consumed after an explicit
// s_waitcnt vmcnt of that count and a bare s_barrier (a fence would drain the prefetches).
// With a row map, one more DMA a chunk before each tile brings the wave's 32 map entries;
// it is older than the chunk's own DMAs, so the same waits cover it. Every DMA reads a clamped,
// in-bounds address (past the end of the list the last chunk is re-loaded into the ring
// slot nobody reads), so the count is exact. Rows past N read tile 0 and are never stored;
// slots past an m-tile's count re-read its first slot and are never stored.
//
// Tile order: workgroups are dispatched round-robin over the 8 XCDs (block b to XCD b % 8),
// each with its own L2. The tile list runs over groups of kGGroupN n-tiles; within a group,
// m-tile by m-tile (experts in order), each m-tile's kGGroupN n-tiles in a row. XCD x owns a
// contiguous range of the list and its 32 workgroups sweep it together, so the tiles an XCD
// works on at a time are 4 m-tiles x the group's 8 n-tiles: an expert's 8 weight tiles (2.9 MB
// at 256 rows) stay in its L2 while the XCD walks that expert's m-tiles, and each m-tile's
// activations are fetched once for the 8 n-tiles. (Against 4 m-tiles x all n-tiles: 4.59
// instead of 5.19 GB fetched per prefill120b call, 1-2% faster; the GEMM is bound by the
// matrix cores, not by this traffic.)
//
// Lane l of a weight tile holds MX block 4c + 2p + l/32 of row l%32 (p = 0, 1), split into
// four 8-element k-steps; the B operand reads the same k-assignment from LDS.
//
// Block-scaled variant (MX = true): the activations arrive as two MXFP8 (E4M3) terms with one
// E8M0 scale per 32 elements each (the layout in mx_act.h), and the MXFP4 weight tile is
// the A operand of gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 as it sits in memory: no
// conversion of the weights at all, their E8M0 scales go to the instruction's scale operand
// and the activation terms' scales to the other. Per 128-element chunk a wave issues
// 2 (terms) x 2 (64-element halves) x RGW x 2 scaled MFMAs. The activation stage holds
// 128 slot rows x (128 hi + 128 lo bytes), the same 32 KB as the bf16 rows, plus 1 KB of
// term scales. Its accumulators start from the bias; the gate_up epilogue writes the
// activation in the same two-term form, the down epilogue stages its fp32 rows through LDS.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mx_act.h"

namespace moe {

constexpr int kGCols = 128;       // slots per tile
constexpr int kGStages = 3;       // LDS ring depth
constexpr int kGRowBytes = 256;   // one 128-element bf16 chunk of a slot row
constexpr int kGActBytes = kGCols * kGRowBytes;
constexpr int kGSBytes = 1024;    // the tiles' scales (2 RGW x 128 bytes, padded)
constexpr int kGBBytes = 1024;    // the tile's bias (64 RGW rows x 2 bytes, padded)
constexpr int kGBiasAreas = 3;    // tile j's bias lives in area j % 3 (the DMA side is at most
                                  // two tiles ahead of the epilogue that reads it)
constexpr int kGGroupN = 8;       // n-tiles per group of the tile order
constexpr int kXcds = 8;
constexpr int kGMaxExperts = 256;
// RGW = 32-row weight tiles per wave: a tile is 64 RGW weight rows x 128 slots. The block-scaled
// forms add the activation terms' scales (128 slots x 2 dwords) after the activation rows. An
// MXFP6 stage holds 128 rows x 192 bytes: the records' 16-byte parts as 128-byte rows (kM6A,
// the 8 units of a row XOR-swizzled by (row >> 1) & 7), then their 8-byte parts (kM6B bytes per
// row) as, per 32-row group, four planes (t, g) of 32 16-byte units (unit (t, g) of the record:
// half 0's and half 1's 8-byte pieces of lane group g, term t). A wave's operand reads then hit
// distinct banks: 16 lanes of a 16-byte read cover 16 rows = 256 distinct bytes (with the rows'
// former swizzle by row & 7, or 8-byte pieces in 64-byte rows, 2 and 4 lanes shared a bank).
template <int RGW, int AF>
struct GShape {
  static constexpr bool kMx = AF != kActBf16;
  static constexpr int kRows = 64 * RGW;
  static constexpr int kActBytes = AF == kActMx6 ? kGCols * kMx6RecBytes : kGActBytes;
  static constexpr int kAScBytes = kMx ? kGCols * 8 : 0;
  static constexpr int kWOff = kActBytes + kAScBytes;  // weight codes, then scales, then bias
  static constexpr int kWBytes = 2 * RGW * 2048;       // codes of the 2 RGW weight tiles
  static constexpr int kStageBytes = kWOff + kWBytes + kGSBytes;
  static constexpr int kBiasOff = kGStages * kStageBytes;  // 3 tile-bias areas after the ring
  static constexpr int kActDma = AF == kActMx6 ? 6 : 8;    // activation DMAs per wave per stage
  static constexpr int kDma = kActDma + RGW + 2 + (kMx ? 1 : 0);  // DMAs per wave per stage
  // the expert offsets, then (block-scaled) each wave's 256-byte area for row-map entries
  static constexpr int kMapOff = kBiasOff + kGBiasAreas * kGBBytes + (kGMaxExperts + 4) * 4;
  static constexpr size_t kLds = (size_t)kMapOff + (kMx ? 4 * 256 : 0);
};
constexpr int kM6A = kMx6BPart;             // bytes of a row's 16-byte parts in an MXFP6 stage
constexpr int kM6B = kMx6RecBytes - kMx6BPart;  // bytes of its 8-byte parts
constexpr int kM6BOff = kGCols * kM6A;     // the 8-byte parts' area in an MXFP6 stage

__device__ __forceinline__ int g_off(int row, int col16) { return row * kGRowBytes + ((col16 ^ (row & 15)) << 4); }

__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
  // s_waitcnt immediate with vmcnt = n (split field) and expcnt / lgkmcnt left at their maxima
  return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8);
}

// A 4-byte LDS read that waits for its own result inside the asm block (a plain read of a
// DMA-written area makes the compiler wait for every DMA in flight). Early-clobber output.
__device__ __forceinline__ int lds_read_b32_sync(const void *p) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(a) : "memory");
  return v;
}

// The epilogue's bias pieces in one LDS round trip: 16 dwords-pairs at 16-byte steps from p
// (tile g, row group i of the wave: offset 64 g + 16 i; pieces past RGW tiles stay inside the
// bias area and are ignored). The reads wait for themselves inside the asm block (the compiler
// would take plain reads for possible targets of the DMAs in flight and wait for all of them);
// the outputs are early-clobber, since later reads of the block still use the address register.
__device__ __forceinline__ void lds_read_bias16(const void *p, uint2 (&v)[16]) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
  asm volatile(
      "ds_read_b64 %0, %16\n\tds_read_b64 %1, %16 offset:16\n\tds_read_b64 %2, %16 offset:32\n\t"
      "ds_read_b64 %3, %16 offset:48\n\tds_read_b64 %4, %16 offset:64\n\tds_read_b64 %5, %16 offset:80\n\t"
      "ds_read_b64 %6, %16 offset:96\n\tds_read_b64 %7, %16 offset:112\n\tds_read_b64 %8, %16 offset:128\n\t"
      "ds_read_b64 %9, %16 offset:144\n\tds_read_b64 %10, %16 offset:160\n\tds_read_b64 %11, %16 offset:176\n\t"
      "ds_read_b64 %12, %16 offset:192\n\tds_read_b64 %13, %16 offset:208\n\tds_read_b64 %14, %16 offset:224\n\t"
      "ds_read_b64 %15, %16 offset:240\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
        "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]),
        "=&v"(v[15])
      : "v"(a)
      : "memory");
}

struct GTile {
  int e, nt, row0, mcount;  // expert, weight-row tile, first sorted row, slots (1..128)
};

// Tile L of the global list -> its expert and rows, from the expert offsets held in LDS.
__device__ GTile g_tile(int L, const int32_t *off, int E, int mt_total, int ntn, int lane) {
  const int ngrp = L / (kGGroupN * mt_total);
  const int gn = (ntn - ngrp * kGGroupN < kGGroupN) ? ntn - ngrp * kGGroupN : kGGroupN;
  const int rem = L - ngrp * kGGroupN * mt_total;
  const int mt = rem / gn;
  GTile t{0, ngrp * kGGroupN + rem % gn, 0, 1};
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

// One workgroup per CU (the LDS ring takes most of it): the compiler is told so, and schedules
// for one wave per SIMD instead of saving registers for more.
template <int EPI, int RGW, int AF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void ffn_gemm_kernel(const void *__restrict__ a_src, const uint8_t *__restrict__ a_scales,
                                                       const int32_t *__restrict__ a_rows, int a_div,
                                                       const int32_t *__restrict__ offsets, int E,
                                                       const uint8_t *__restrict__ pcodes,
                                                       const uint8_t *__restrict__ pscales,
                                                       const uint16_t *__restrict__ bias, int N, int K, int ntn,
                                                       void *__restrict__ out, uint8_t *__restrict__ out_scales,
                                                       float limit, float alpha) {
  using SH = GShape<RGW, AF>;
  constexpr bool MX = AF != kActBf16, M6 = AF == kActMx6;
  constexpr int kGRows = SH::kRows, kGWBytes = SH::kWBytes, kGStageBytes = SH::kStageBytes, kGDma = SH::kDma;
  constexpr int kWOff = SH::kWOff, kActDma = SH::kActDma;
  static_assert((EPI != kEpiMxAct && EPI != kEpiMx6Act) || (AF == kActMx8 && RGW == 4),
                "two-term output: one 128-element record per n-tile, from the MXFP8 gate_up");
  static_assert(!M6 || EPI == kEpiLinearF32, "MXFP6 input: the down projection");
  static_assert(EPI != kEpiSwigluBf16 || !MX, "bf16 activation output belongs to the bf16 path");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  int32_t *off = reinterpret_cast<int32_t *>(lds + SH::kBiasOff + kGBiasAreas * kGBBytes);
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
  // bytes per activation row: K bf16, or nchunk two-term records
  const int64_t arow = M6 ? (int64_t)nchunk * kMx6RecBytes : MX ? (int64_t)nchunk * kMxRecBytes : (int64_t)K * 2;
  // DMA i (0 .. kDma - 1) of the issue-side chunk into ring slot `slot`:
  //   0..7            activation rows 32 wave + 4 i .. + 3 (bf16 elements, or a two-term record);
  //   8..8+RGW-1      1 KB of weight codes: tile m / 2, half m % 2, m = RGW wave + i - 8;
  //   8+RGW           256 bytes of the scale block (2 RGW tiles x 128 bytes, then padding);
  //   8+RGW+1         waves 0, 1: 256 bytes of the tile's bias run (2 x 64 RGW bytes) into
  //                   bias area ji % 3 (outside the ring); waves 2, 3: a dummy;
  //   8+RGW+2 (MX)    256 bytes of term scales: slots 32 wave .. 32 wave + 31, 8 bytes each.
  // Sources are set once per tile as a byte offset and a per-chunk stride, so the chunk loop
  // computes each address without a branch (branches would cut the loop body into blocks the
  // instruction scheduler cannot interleave). Rows past N read weight tile 0 with stride 0;
  // slots past an m-tile's count re-read its first slot; neither is ever stored.
  const uint8_t *aptr[8];
  int lcol[8];                    // byte offset of the lane's 16 bytes within a 256-byte row chunk
  int64_t woff[RGW];              // weight codes of this wave's DMA m, chunk 0 (from pcodes)
  int wstr[RGW];                  // 2048, or 0 for tiles past N
  int64_t soff;                   // scale block, chunk 0 (from pscales)
  int sstr;                       // 128, or 0
  int64_t boff;                   // the tile's bias run (from bias), or -1: no bias here
  const uint8_t *sptr = nullptr;  // MX: this lane's term-scale dword of slot (64 wave + lane) / 2, chunk 0
  // Block-scaled path with a row map: the map entries of the wave's 32 rows of an issue-side
  // tile come by LDS DMA (lane j: tile row 32 wave + j; lanes 32.. repeat them) into the
  // wave's own area, issued at the top of the chunk before the tile starts, so the wait for
  // the next stage covers them; at the switch the wave reads its area back.
  const bool mapped = MX && a_rows != nullptr;
  unsigned char *mapl = lds + SH::kMapOff + 256 * wave;
  auto dma_map = [&](const GTile &t) {
    const int rr = 32 * wave + (lane & 31);
    __builtin_amdgcn_global_load_lds(a_rows + t.row0 + (rr < t.mcount ? rr : 0), mapl, 4, 0, 0);
  };
  auto set_rows = [&]() {
    // source row of each tile row: the row itself, or with the row map the two-term row
    // a_rows[r] / a_div (e.g. a slot's token); lane j holds tile row 32 wave + j's source,
    // and each lane takes its rows' entries with a cross-lane read
    int srcv = 0;
    if (mapped) {
      srcv = lds_read_b32_sync(mapl + (lane & 31) * 4) / a_div;
    } else {
      srcv = ti.row0 + ((32 * wave + (lane & 31)) < ti.mcount ? 32 * wave + (lane & 31) : 0);
    }
#pragma unroll
    for (int i = 0; i < kActDma; ++i) {
      // tile row (within the wave's 32) of the lane's piece of activation DMA i
      const int rw = M6 ? (i < 4 ? 8 * i + lane / 8 : lane % 32) : 4 * i + lane / 16;
      const int src = __builtin_amdgcn_ds_bpermute(rw * 4, srcv);
      aptr[i] = static_cast<const uint8_t *>(a_src) + (int64_t)src * arow;
    }
    const int gt0 = ti.nt * 2 * RGW;
    const int64_t ebase = (int64_t)ti.e * NG * nchunk;
#pragma unroll
    for (int m = 0; m < RGW; ++m) {
      const int mm = RGW * wave + m, g = gt0 + mm / 2;
      const bool ok = g < NG;
      woff[m] = (ok ? ebase + (int64_t)g * nchunk : 0) * 2048 + (mm % 2) * 1024 + lane * 16;
      wstr[m] = ok ? 2048 : 0;
    }
    {
      const int o = 256 * wave + 4 * lane;
      const int tt = o / 128, g = gt0 + tt;
      const bool ok = tt < 2 * RGW && g < NG;
      soff = (ok ? ebase + (int64_t)g * nchunk : 0) * 128 + (o % 128);
      sstr = ok ? 128 : 0;
      const int n = ti.nt * kGRows + o / 2;  // byte o of the tile's bias run
      boff = (bias != nullptr && o < 2 * kGRows && n < N) ? ((int64_t)ti.e * N + n) * 2 : -1;
    }
    if constexpr (MX) {
      const int sl = (64 * wave + lane) >> 1;
      const int src = __builtin_amdgcn_ds_bpermute((sl - 32 * wave) * 4, srcv);
      sptr = a_scales + (int64_t)src * nchunk * kMxScBytes + (lane & 1) * 4;
    }
  };
  // (MXFP6: a 16-byte part's row holds 8 units, swizzled by (row >> 1) & 7; the 8-byte parts go
  // to planes (t, g) of 16-byte units, DMA 4 + j bringing planes 2j and 2j + 1 of the wave's 32
  // rows, lane l plane 2j + l / 32, row l % 32)
#pragma unroll
  for (int i = 0; i < 8; ++i)
    lcol[i] = M6 ? (i < 4 ? ((lane % 8) ^ (((8 * i + lane / 8) >> 1) & 7)) * 16 : kM6A + (2 * (i - 4) + lane / 32) * 16)
                 : ((lane % 16) ^ ((32 * wave + 4 * i + lane / 16) & 15)) * 16;
  if (mapped) {
    dma_map(ti);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's map entries are in its area
  }
  set_rows();
  // Called before a stage is issued (the chunk counter ci was advanced after the previous
  // one): moves the issue side to its next tile when the chunks of this one are all issued.
  // It runs at the top of a chunk, so no branch follows the chunk's MFMAs (the compiler would
  // otherwise sink them past it, away from the loads they should hide).
  GTile tnext = ti;
  auto advance_issue = [&]() {
    if (ci >= nchunk) {
      if (ji + 1 < ntiles) {
        ++ji;
        ci = 0;
        if (mapped)
          ti = tnext;
        else
          ti = g_tile(first + ji * nq, off, E, mt_total, ntn, lane);
        set_rows();
      } else {
        ci = nchunk - 1;  // past the end: keep re-loading the last chunk (into a free slot)
      }
    }
    // the next tile's row map, a chunk ahead (its DMA is older than the chunk's own DMAs, so
    // the chunk's wait for the next stage covers it)
    if (mapped && ci == nchunk - 1 && ji + 1 < ntiles) {
      tnext = g_tile(first + (ji + 1) * nq, off, E, mt_total, ntn, lane);
      dma_map(tnext);
    }
  };
  auto dma = [&](int i, int slot) {
    unsigned char *st = lds + slot * kGStageBytes;
    if (i < kActDma) {
      if constexpr (M6) {
        // 16-byte parts: 8 rows x 128 bytes per DMA; 8-byte parts: two planes of the wave's 32 rows
        unsigned char *dst = i < 4 ? st + (32 * wave + 8 * i) * kM6A : st + kM6BOff + wave * (32 * kM6B) + (i - 4) * 1024;
        __builtin_amdgcn_global_load_lds(aptr[i] + ci * kMx6RecBytes + lcol[i], dst, 16, 0, 0);
      } else {
        const uint8_t *src;
        if constexpr (MX) {
          src = aptr[i] + ci * kMxRecBytes + lcol[i];
        } else {
          int kk = ci * 128 + lcol[i] / 2;
          kk = kk < K ? kk : 0;  // past K: any in-bounds element (its weight is an exact zero)
          src = aptr[i] + 2 * (int64_t)kk;
        }
        __builtin_amdgcn_global_load_lds(src, st + (32 * wave + 4 * i) * kGRowBytes, 16, 0, 0);
      }
    } else if (i < kActDma + RGW) {
      const int m = i - kActDma;
      // (the offset goes through a local: with the array reads inside the builtin's argument
      // the host compilation silently drops the kernel's launch stub)
      const int64_t wo = woff[m] + ci * wstr[m];
      __builtin_amdgcn_global_load_lds(pcodes + wo, st + kWOff + (RGW * wave + m) * 1024, 16, 0, 0);
    } else if (i == kActDma + RGW) {
      __builtin_amdgcn_global_load_lds(pscales + soff + ci * sstr, st + kWOff + kGWBytes + 256 * wave, 4, 0, 0);
    } else if (i == kActDma + RGW + 1) {
      const uint8_t *src = boff >= 0 ? reinterpret_cast<const uint8_t *>(bias) + boff : pscales;  // else a dummy
      __builtin_amdgcn_global_load_lds(src, lds + SH::kBiasOff + (ji % kGBiasAreas) * kGBBytes + 256 * wave, 4, 0, 0);
    } else {
      __builtin_amdgcn_global_load_lds(sptr + ci * kMxScBytes, st + SH::kActBytes + 256 * wave, 4, 0, 0);
    }
  };

  // ---- compute side
  // A wave's two 32-slot column groups b = 0, 1 are slots 32 (wx + 2b) .. + 31 of the tile, so
  // a tile of at most 64 slots gives every wave one group and half the MFMAs (no imbalance).
  auto scol = [&](int b) { return 32 * (wx + 2 * b) + r32; };
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

  // The bias of compute tile jc from bias area jc % 3: lane holds slot column scol(b) and rows
  // 8i + 4kh + jj of tile g.
  const int nloc0 = wy * 32 * RGW;
  auto bias_regs = [&](int jc, uint2 (&bq)[RGW][4]) {
    const unsigned char *bb = lds + SH::kBiasOff + (jc % kGBiasAreas) * kGBBytes;
    const uint32_t bmask = bias != nullptr ? 0xffffffffu : 0u;  // without bias the run holds junk
    uint2 v[16];
    lds_read_bias16(bb + 2 * (nloc0 + 4 * kh), v);
#pragma unroll
    for (int g = 0; g < RGW; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) bq[g][i] = uint2{v[4 * g + i].x & bmask, v[4 * g + i].y & bmask};
  };
  // Block-scaled path: the accumulators of compute tile jc start from its bias (rows are the
  // same for both column groups), so the epilogues add none. Called once the tile's bias area
  // is complete: after the barrier that completes the tile's first stage.
  auto init_acc = [&](int jc) {
    uint2 bq[RGW][4];
    bias_regs(jc, bq);
#pragma unroll
    for (int g = 0; g < RGW; ++g)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[g][b][4 * i + 0] = __uint_as_float(bq[g][i].x << 16);
          acc[g][b][4 * i + 1] = __uint_as_float(bq[g][i].x & 0xffff0000u);
          acc[g][b][4 * i + 2] = __uint_as_float(bq[g][i].y << 16);
          acc[g][b][4 * i + 3] = __uint_as_float(bq[g][i].y & 0xffff0000u);
        }
  };
  // fp32 rows of the block-scaled path (the down projection) leave through LDS: a lane holds
  // 16-byte pieces of 32 different slot rows, so storing them straight makes every store
  // instruction touch 32 rows 32 bytes each. Staged per wave in the 8 KB of LDS that only its
  // own DMAs write (its activation rows of ring slot fs, which the ring does not refill before
  // this wave's next chunk), 32 slots x 64 rows per round (two 32-row tiles, XOR-swizzled
  // 16-byte units), each store then writes 4 slots x 256 contiguous bytes.
  auto epilogue_staged = [&](int fs) {
    unsigned char *stg = lds + fs * kGStageBytes + wave * 32 * kGRowBytes;
    float *outp = static_cast<float *>(out);
    const int nb_live = tc.mcount > 64 ? 2 : 1;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (b >= nb_live) break;
#pragma unroll
      for (int gp = 0; gp < (RGW + 1) / 2; ++gp) {
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const int g = 2 * gp + gg;
          if (g >= RGW) break;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int u = 8 * gg + 2 * i + kh;
            *reinterpret_cast<f32x4_t *>(stg + r32 * 256 + ((u ^ (r32 & 15)) << 4)) =
                f32x4_t{acc[g][b][4 * i], acc[g][b][4 * i + 1], acc[g][b][4 * i + 2], acc[g][b][4 * i + 3]};
          }
        }
        f32x4_t v[8];  // all reads before the first (conditional) store
        const int u = lane % 16;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int sl = 4 * j + lane / 16;
          v[j] = *reinterpret_cast<const f32x4_t *>(stg + sl * 256 + ((u ^ (sl & 15)) << 4));
        }
        const int n = tc.nt * kGRows + nloc0 + 64 * gp + 4 * u;
        const bool n_ok = n < N && (u < 8 || 2 * gp + 1 < RGW);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = 32 * (wx + 2 * b) + 4 * j + lane / 16;
          if (n_ok && col < tc.mcount) *reinterpret_cast<f32x4_t *>(outp + (int64_t)(tc.row0 + col) * N + n) = v[j];
        }
      }
    }
  };
  auto epilogue = [&](int jc) {
    uint2 bq[RGW][4];
    if constexpr (!MX) bias_regs(jc, bq);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int col = scol(b);
      if (col >= tc.mcount) continue;
      const int64_t r = tc.row0 + col;
#pragma unroll
      for (int g = 0; g < RGW; ++g) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = tc.nt * kGRows + nloc0 + 32 * g + 8 * i + 4 * kh;
          if (n >= N) continue;
          float h[4];
          if constexpr (MX) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) h[jj] = acc[g][b][4 * i + jj];
          } else {
            h[0] = acc[g][b][4 * i + 0] + __uint_as_float(bq[g][i].x << 16);
            h[1] = acc[g][b][4 * i + 1] + __uint_as_float(bq[g][i].x & 0xffff0000u);
            h[2] = acc[g][b][4 * i + 2] + __uint_as_float(bq[g][i].y << 16);
            h[3] = acc[g][b][4 * i + 3] + __uint_as_float(bq[g][i].y & 0xffff0000u);
          }
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
  // Two-term activation output (gate_up, 256-row tiles): the n-tile's 128 activations are
  // record nt of each slot row; this wave's 64 of them (blocks 2 wy, 2 wy + 1 of the record)
  // come from tiles g = 0, 1 (block 2 wy) and g = 2, 3 (block 2 wy + 1). A lane holds, per
  // block, 16 of the 32 values (bytes 16 gg + 4 i + 2 kh + {0, 1} for tile 2j + gg); the
  // lane pair l, l ^ 32 shares the block maximum, then swaps half its codes so that lane kh
  // stores bytes 16 kh .. 16 kh + 15 of the block. Rows past N (the last n-tile) are zeros.
  auto epilogue_mx = [&](int jc) {
    (void)jc;
    uint8_t *orec = static_cast<uint8_t *>(out);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int col = scol(b);
      const bool live = col < tc.mcount;  // same for the lane pair; shuffles run on every lane
      const int64_t r = tc.row0 + (live ? col : 0);
      float av[RGW][4][2];
#pragma unroll
      for (int g = 0; g < RGW; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = tc.nt * kGRows + nloc0 + 32 * g + 8 * i + 4 * kh;
          const float h0 = acc[g][b][4 * i + 0], h1 = acc[g][b][4 * i + 1];  // bias included
          const float h2 = acc[g][b][4 * i + 2], h3 = acc[g][b][4 * i + 3];
          const float a0 = bf16_to_f32(f32_to_bf16_rne(swiglu_unit(h0, h1, limit, alpha)));
          const float a1 = bf16_to_f32(f32_to_bf16_rne(swiglu_unit(h2, h3, limit, alpha)));
          av[g][i][0] = n < N ? a0 : 0.0f;
          av[g][i][1] = n < N ? a1 : 0.0f;
        }
      uint8_t *rec = orec + (r * ntn + tc.nt) * kMxRecBytes + 2 * wy * 32 + 16 * kh;
      uint32_t sc_hi = 0, sc_lo = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float m = 0.0f;
#pragma unroll
        for (int gg = 0; gg < 2; ++gg)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(av[2 * j + gg][i][0]), fabsf(av[2 * j + gg][i][1])));
        {  // the block maximum over the lane pair (l, l + 32): one half swap, no LDS round trip
          const auto mm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
          m = fmaxf(__uint_as_float(mm[0]), __uint_as_float(mm[1]));
        }
        const MxBlockScale s = mx_block_scale(m);
        sc_hi |= s.sh << (8 * j);
        sc_lo |= s.sl << (8 * j);
        uint32_t hp[2][4], lp[2][4];
#pragma unroll
        for (int gg = 0; gg < 2; ++gg)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx_split2(av[2 * j + gg][i][0], av[2 * j + gg][i][1], s, hp[gg][i], lp[gg][i]);
        // Lane kh of the pair stores half gg = kh: its own pairs hp[kh] and the partner's
        // hp[kh]. permlane32_swap(x = hp[0], y = hp[1]) returns [x lanes 0-31, y lanes 0-31] and
        // [x lanes 32-63, y lanes 32-63]: in the low lanes own hp[0], then the partner's; in the
        // high lanes the partner's hp[1], then own -- so both store r0 | r1 << 16.
        u32x4_t wh, wl;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const uint32_t xh = hp[0][2 * d] | (hp[0][2 * d + 1] << 16), yh = hp[1][2 * d] | (hp[1][2 * d + 1] << 16);
          const uint32_t xl = lp[0][2 * d] | (lp[0][2 * d + 1] << 16), yl = lp[1][2 * d] | (lp[1][2 * d + 1] << 16);
          const auto rh = __builtin_amdgcn_permlane32_swap(xh, yh, false, false);
          const auto rl = __builtin_amdgcn_permlane32_swap(xl, yl, false, false);
          wh[2 * d] = (rh[0] & 0xffffu) | (rh[1] << 16);
          wh[2 * d + 1] = (rh[0] >> 16) | (rh[1] & 0xffff0000u);
          wl[2 * d] = (rl[0] & 0xffffu) | (rl[1] << 16);
          wl[2 * d + 1] = (rl[0] >> 16) | (rl[1] & 0xffff0000u);
        }
        if (live) {
          *reinterpret_cast<u32x4_t *>(rec + 32 * j) = wh;
          *reinterpret_cast<u32x4_t *>(rec + 32 * j + 128) = wl;
        }
      }
      if (live)
        *reinterpret_cast<uint16_t *>(out_scales + (r * ntn + tc.nt) * kMxScBytes + 4 * kh + 2 * wy) =
            (uint16_t)(kh ? sc_lo : sc_hi);
    }
  };

  // MXFP6 form of the fp32 staging above: the wave's own 16-byte-part rows of ring slot fs are
  // 4 KB (32 rows x 128 bytes), so a round is 32 slots x one 32-row tile (XOR-swizzled 16-byte
  // units), and each store writes 8 slots x 128 contiguous bytes.
  auto epilogue_staged6 = [&](int fs) {
    unsigned char *stg = lds + fs * kGStageBytes + wave * 32 * kM6A;
    float *outp = static_cast<float *>(out);
    const int nb_live = tc.mcount > 64 ? 2 : 1;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (b >= nb_live) break;
#pragma unroll
      for (int g = 0; g < RGW; ++g) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int u = 2 * i + kh;
          *reinterpret_cast<f32x4_t *>(stg + r32 * kM6A + ((u ^ (r32 & 7)) << 4)) =
              f32x4_t{acc[g][b][4 * i], acc[g][b][4 * i + 1], acc[g][b][4 * i + 2], acc[g][b][4 * i + 3]};
        }
        f32x4_t v[4];  // all reads before the first (conditional) store
        const int u = lane % 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int sl = 8 * j + lane / 8;
          v[j] = *reinterpret_cast<const f32x4_t *>(stg + sl * kM6A + ((u ^ (sl & 7)) << 4));
        }
        const int n = tc.nt * kGRows + nloc0 + 32 * g + 4 * u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = 32 * (wx + 2 * b) + 8 * j + lane / 8;
          if (n < N && col < tc.mcount) *reinterpret_cast<f32x4_t *>(outp + (int64_t)(tc.row0 + col) * N + n) = v[j];
        }
      }
    }
  };
  // Two-term MXFP6 activation output (gate_up, 256-row tiles): as epilogue_mx, the n-tile's 128
  // activations are record nt of each slot row and this wave's 64 are blocks 2 wy, 2 wy + 1. A
  // lane holds 16 of each block's 32 values (elements 16 gg + 4 i + 2 kh + {0, 1} of block j from
  // tile 2 j + gg); one permlane32_swap per bf16 pair gives lane kh all 32 of block 2 wy + kh,
  // which it splits and stores alone (no cross-lane maximum).
  auto epilogue_mx6 = [&]() {
    uint8_t *orec = static_cast<uint8_t *>(out);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int col = scol(b);
      const bool live = col < tc.mcount;  // same for the lane pair; the swaps run on every lane
      const int64_t r = tc.row0 + (live ? col : 0);
      uint32_t pk[2][2][4];  // [block j][tile gg][i]: elements 16 gg + 4 i + 2 kh + {0, 1}
#pragma unroll
      for (int g = 0; g < RGW; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = tc.nt * kGRows + nloc0 + 32 * g + 8 * i + 4 * kh;
          const uint32_t a0 = f32_to_bf16_rne(swiglu_unit(acc[g][b][4 * i], acc[g][b][4 * i + 1], limit, alpha));
          const uint32_t a1 = f32_to_bf16_rne(swiglu_unit(acc[g][b][4 * i + 2], acc[g][b][4 * i + 3], limit, alpha));
          pk[g / 2][g % 2][i] = n < N ? (a0 | (a1 << 16)) : 0u;
        }
      float v[32];
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // [own j = 0 | the low lanes' j = 1] and [the high lanes' j = 0 | own j = 1]: lane kh
          // now has elements 16 gg + 4 i + 2 kk + {0, 1} of its block from swap result kk
          const auto rr = __builtin_amdgcn_permlane32_swap(pk[0][gg][i], pk[1][gg][i], false, false);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            v[16 * gg + 4 * i + 2 * kk] = __uint_as_float((uint32_t)rr[kk] << 16);
            v[16 * gg + 4 * i + 2 * kk + 1] = __uint_as_float((uint32_t)rr[kk] & 0xffff0000u);
          }
        }
      uint32_t hi[6], lo[6], sh, sl;
      mx6_split_block(v, hi, lo, sh, sl);
      const int blk = 2 * wy + kh;
      if (live) {
        mx6_store_block(orec + (r * ntn + tc.nt) * kMx6RecBytes, blk, hi, lo);
        out_scales[(r * ntn + tc.nt) * kMxScBytes + blk] = (uint8_t)sh;
        out_scales[(r * ntn + tc.nt) * kMxScBytes + 4 + blk] = (uint8_t)sl;
      }
    }
  };

  // prologue: stages 0 and 1
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    advance_issue();
#pragma unroll
    for (int i = 0; i < kGDma; ++i) dma(i, s);
    ++ci;
  }
  int G = 0;  // global chunk counter: ring slot G % 3

  // Block-scaled path. Operands of a chunk's step 0 and its scale operands are read at the end
  // of the chunk before (step 3), right after the barrier that makes that stage complete: the
  // LDS round trip after the barrier then overlaps the last step's MFMAs instead of stalling
  // every wave at the top of the chunk. They live across chunks (and tiles), so they are
  // declared here. Lane group kh of the FP8 operand holds elements 16 kh .. 16 kh + 15 and
  // 32 + 16 kh .. of a 64-element half, i.e. 16-byte columns 4p + kh and 4p + 2 + kh of the
  // term's 128 bytes.
  // MXFP6: the lane's block 2p + kh of term t is its record's 16-byte unit (t, 2p + kh) in the
  // 16-byte-part rows and half p of unit (t, kh) in the 8-byte-part planes (read whole at half
  // 0, half 1's piece kept for the step of half 1); the operand's dwords 6 and 7 are unused.
  i32x8_t bv[2][2] = {};
  uint32_t m6h1[2][2][2] = {};  // MXFP6: half 1's 8-byte piece of column group b, term t (read with half 0's)
  u32x4_t wv[2][RGW];
  uint32_t swd[RGW], ash[2][2];
  // half h of the FP8 operand (16-byte columns 4p + kh, 4p + 2 + kh of term t), or the MXFP6
  // operand's part h (h = 0: dwords 0-3, h = 1: dwords 4-5), of slot row `row` into b8
  auto act_read = [&](const unsigned char *abuf, int row, int p, int t, int h, int b, i32x8_t &b8) {
    if constexpr (M6) {
      if (h == 0) {
        const u32x4_t u =
            *reinterpret_cast<const u32x4_t *>(abuf + row * kM6A + (((4 * t + 2 * p + kh) ^ ((row >> 1) & 7)) << 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) b8[i] = (int)u[i];
      } else if (p == 0) {
        // the 16-byte unit (t, kh) of the row in its plane: half 0's piece now, half 1's kept
        const u32x4_t u = *reinterpret_cast<const u32x4_t *>(abuf + kM6BOff + (row >> 5) * (32 * kM6B) +
                                                             (2 * t + kh) * 512 + (row & 31) * 16);
        b8[4] = (int)u[0];
        b8[5] = (int)u[1];
        m6h1[b][t][0] = u[2];
        m6h1[b][t][1] = u[3];
      } else {
        b8[4] = (int)m6h1[b][t][0];
        b8[5] = (int)m6h1[b][t][1];
      }
    } else {
      const u32x4_t u = *reinterpret_cast<const u32x4_t *>(abuf + g_off(row, 8 * t + 4 * p + 2 * h + kh));
#pragma unroll
      for (int i = 0; i < 4; ++i) b8[4 * h + i] = (int)u[i];
    }
  };
  auto bload = [&](const unsigned char *abuf, int p, int t, i32x8_t *b8, int nb) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (b >= nb) break;
      act_read(abuf, scol(b), p, t, 0, b, b8[b]);
      act_read(abuf, scol(b), p, t, 1, b, b8[b]);
    }
  };
  auto wload = [&](const unsigned char *abuf, int p, u32x4_t *w4) {
#pragma unroll
    for (int g = 0; g < RGW; ++g)
      w4[g] = *reinterpret_cast<const u32x4_t *>(abuf + kWOff + (wy * RGW + g) * 2048 + p * 1024 + lane * 16);
  };
  // the scales of the stage at abuf (one asm block that waits for itself: a plain LDS read of
  // the term scales makes the compiler wait for every DMA in flight)
  // The scale operands of the stage at abuf, unshifted (shifted where a chunk starts, after the
  // wait its first MFMA needs anyway). The term scales are read as two dwords each: written as
  // one 8-byte read, the compiler took them for a possible target of the DMAs in flight and
  // waited for all of them.
  auto sload = [&](const unsigned char *abuf) {
#pragma unroll
    for (int g = 0; g < RGW; ++g)
      swd[g] = *reinterpret_cast<const uint32_t *>(abuf + kWOff + kGWBytes + (wy * RGW + g) * 128 + r32 * 4);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      ash[b][0] = *reinterpret_cast<const uint32_t *>(abuf + SH::kActBytes + scol(b) * 8);
      ash[b][1] = *reinterpret_cast<const uint32_t *>(abuf + SH::kActBytes + scol(b) * 8 + 4);
    }
  };
  // Wait for stage G + 1 while stage G + 2's DMAs of steps 0..2 (the youngest) may still fly.
  constexpr int kPerStep = (kGDma + 3) / 4;  // DMAs issued per step
  constexpr int kYounger = (3 * kPerStep < kGDma) ? 3 * kPerStep : kGDma;
  if constexpr (MX) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kGDma));  // stage 0 complete (this wave)
    __builtin_amdgcn_s_barrier();                  // ... and every wave's
    asm volatile("" ::: "memory");
    sload(lds);
    bload(lds, 0, 0, bv[0], 2);
    wload(lds, 0, wv[0]);
    init_acc(0);
  }

  // The chunk loop of one tile with NB column groups per wave (1 for tiles of at most 64
  // slots). Chosen once per tile: a choice per chunk made the compiler copy the accumulators
  // between the two loop bodies every chunk.
  auto tile_chunks = [&](auto NBC) {
    constexpr int NB = decltype(NBC)::value;
    for (int cc = 0; cc < nchunk; ++cc, ++G) {
      if constexpr (!MX) {
        // this wave's kDma loads of stage G are the oldest outstanding but for stage G+1's
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kGDma));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");  // no LDS read of this stage may be hoisted above the barrier
      }
      advance_issue();
      const int slot = G % kGStages, nslot = (G + 2) % kGStages;
      const unsigned char *abuf = lds + slot * kGStageBytes;
      const unsigned char *wbuf = abuf + kWOff + (wy * RGW) * 2048 + lane * 16;
      const unsigned char *sbuf = abuf + kWOff + kGWBytes + (wy * RGW) * 128 + r32 * 4;
      if constexpr (MX) {
        // Four steps (64-element half p, term t), each RGW x NB scaled MFMAs. Each step issues
        // its first MFMA, then the next step's LDS reads and its share of the DMAs spread over
        // its other MFMAs: with LDS DMA in flight the compiler can only wait for all LDS reads
        // (lgkmcnt(0)), which it does before a step's first MFMA. Step 3 instead waits for the
        // next stage, passes the barrier, and reads the next chunk's step-0 operands and scales;
        // its own DMAs go out after the barrier, so the wait's count of younger DMAs is exact.
        const unsigned char *nbuf = lds + ((G + 1) % kGStages) * kGStageBytes;
        // this chunk's scale operands (sload overwrites swd / ash), shifted by 8 kh so that the
        // instruction's byte select 2p picks block 2p + kh
        uint32_t sw_c[RGW], as_c[2][2];
#pragma unroll
        for (int g = 0; g < RGW; ++g) sw_c[g] = swd[g] >> (8 * kh);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          as_c[b][0] = ash[b][0] >> (8 * kh);
          as_c[b][1] = ash[b][1] >> (8 * kh);
        }
        // Read k of a step's LDS reads into the next operands: k < nw, weight tile k of half pw;
        // then half (k - nw) % 2 of the FP8 operand of column group (k - nw) / 2 (64-element half
        // p, term t).
        auto read_op = [&](const unsigned char *buf, int k, int nw, int p, int t, i32x8_t *bd, int pw, u32x4_t *wd) {
          if (k < nw) {
            wd[k] = *reinterpret_cast<const u32x4_t *>(buf + kWOff + (wy * RGW + k) * 2048 + pw * 1024 + lane * 16);
          } else {
            const int b = (k - nw) / 2, h = (k - nw) % 2;
            act_read(buf, scol(b), p, t, h, b, bd[b]);
          }
        };
        auto step = [&](auto SC) {
          constexpr int s = decltype(SC)::value, p = s / 2, t = s % 2;
          constexpr int NM = RGW * NB;
          // this step's reads (of the next step's operands, or at step 3 of the next chunk's
          // first) and DMAs
          constexpr int NR = s < 3 ? 2 * NB + (s == 0 ? RGW : 0) : 4 + RGW;
          constexpr int D0 = s < 3 ? s * kPerStep : 3 * kPerStep;
          constexpr int ND = s < 3 ? (kGDma - D0 < kPerStep ? kGDma - D0 : kPerStep) : kGDma - D0;
          constexpr int kPerR = (NR + NM - 2) / (NM - 1), kPerD = (ND + NM - 3) / (NM - 2);
          auto mfma = [&](int g, int b) {
            const u32x4_t u = wv[p][g];
            const i32x8_t wa = i32x8_t{(int)u[0], (int)u[1], (int)u[2], (int)u[3], 0, 0, 0, 0};
            // A: FP4 (format 4); B: FP8 E4M3 (0) or FP6 E2M3 (2)
            acc[g][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                wa, bv[s % 2][b], acc[g][b], 4, M6 ? 2 : 0, 2 * p, (int)sw_c[g], 2 * p, (int)as_c[b][t]);
          };
          mfma(0, 0);
          if constexpr (s == 3) {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): every read of this stage has landed
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(kYounger));
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            sload(nbuf);
          }
          // Issue order, held by scheduling fences: before MFMA j (j >= 1) up to kPerR reads and,
          // from j = 2 on, up to kPerD DMAs. A wave stalled issuing a run of them would leave the
          // matrix core idle; spread out, each issues in the shadow of an MFMA.
#pragma unroll
          for (int j = 1; j <= NM; ++j) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = (j - 1) * kPerR; k < j * kPerR && k < NR; ++k) {
              if constexpr (s < 3)
                read_op(abuf, k, s == 0 ? RGW : 0, (s + 1) / 2, (s + 1) % 2, bv[(s + 1) % 2], 1, wv[1]);
              else
                read_op(nbuf, k, RGW, 0, 0, bv[0], 0, wv[0]);  // both column groups: the next tile may be full
            }
            if (j >= 2) {
#pragma unroll
              for (int i = (j - 2) * kPerD; i < (j - 1) * kPerD && i < ND; ++i) dma(D0 + i, nslot);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (j < NM) mfma(j / NB, j % NB);
          }
        };
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
        (void)wbuf;
        (void)sbuf;
      } else {
        {
          uint32_t swd[RGW];
#pragma unroll
          for (int g = 0; g < RGW; ++g) swd[g] = *reinterpret_cast<const uint32_t *>(sbuf + g * 128);
          auto bload = [&](int p, int j, bf16x8_t *bv) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
              bv[b] = as_bf16x8(*reinterpret_cast<const u32x4_t *>(abuf + g_off(scol(b), 4 * (2 * p + kh) + j)));
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
                for (int b = 0; b < NB; ++b)
                  acc[g][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, bcur[b], acc[g][b], 0, 0, 0);
              }
#pragma unroll
              for (int b = 0; b < NB; ++b) bcur[b] = bnext[b];
            }
          }
        }
      }
      ++ci;
    }
  };
  for (int jc = 0; jc < ntiles; ++jc) {
    if (tc.mcount > 64)
      tile_chunks(std::integral_constant<int, 2>{});
    else
      tile_chunks(std::integral_constant<int, 1>{});
    if constexpr (EPI == kEpiMx6Act) {
      epilogue_mx6();
    } else if constexpr (EPI == kEpiMxAct) {
      epilogue_mx(jc);
    } else {
      // the slot of the tile's last chunk, free until the next chunk's DMAs
      if constexpr (M6 && EPI == kEpiLinearF32)
        epilogue_staged6((G + 2) % kGStages);
      else if constexpr (MX && EPI == kEpiLinearF32)
        epilogue_staged((G + 2) % kGStages);
      else
        epilogue(jc);
    }
    if constexpr (MX)
      init_acc(jc + 1);  // (past the last tile: a harmless read of a bias area)
    else
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
// a tenth of the 32-row tiles; then 192 if it pads less. The two-term activation output
// always uses 256 rows (one 128-element record per n-tile).
hipError_t launch_ffn_gemm(const void *a, const uint8_t *a_scales, const int32_t *a_rows, int a_div, int af,
                           const int32_t *offsets, int E, int64_t S, const MxWeight &w, int epilogue, void *out,
                           uint8_t *out_scales, float limit, float alpha, hipStream_t stream) {
  const bool mx = af != kActBf16;
  if (af < kActBf16 || af > kActMx6) return hipErrorInvalidValue;
  if (a_rows != nullptr && (!mx || a_div < 1)) return hipErrorInvalidValue;
  if (E > kGMaxExperts) return hipErrorInvalidValue;
  if (epilogue == kEpiMxAct && !mx) return hipErrorInvalidValue;
  if (epilogue == kEpiSwigluBf16 && mx) return hipErrorInvalidValue;
  const int NG = w.N / 32;
  const int pad4 = (NG + 7) / 8 * 8 - NG, pad3 = (NG + 5) / 6 * 6 - NG;
  const bool rec_out = epilogue == kEpiMxAct || epilogue == kEpiMx6Act;
  if (rec_out && af != kActMx8) return hipErrorInvalidValue;
  if (af == kActMx6 && epilogue != kEpiLinearF32) return hipErrorInvalidValue;
  const bool tall = rec_out || pad4 * 10 <= NG || pad4 <= pad3;
  const int rows = tall ? 256 : 192;
  const int64_t busy = (S < E) ? S : E;
  const int64_t mtiles = (S + kGCols - 1) / kGCols + busy;  // bound on the real m-tile count
  const int ntn = (w.N + rows - 1) / rows;
  const int64_t bound = mtiles * ntn;
  const int cap = gemm_grid_cap();  // one workgroup per CU (the LDS ring takes most of a CU)
  dim3 grid((unsigned)(bound < cap ? bound : cap));
#define MOE_LAUNCH_GEMM(EPI, RG, M)                                                                          \
  hipLaunchKernelGGL((ffn_gemm_kernel<EPI, RG, M>), grid, dim3(256), (GShape<RG, M>::kLds), stream, a, a_scales, \
                     a_rows, a_div, offsets, E, w.codes, w.scales, w.bias, w.N, w.K, ntn, out, out_scales, limit, alpha)
  if (af == kActMx6) {  // the down projection on MXFP6 activation records
    if (tall)
      MOE_LAUNCH_GEMM(kEpiLinearF32, 4, kActMx6);
    else
      MOE_LAUNCH_GEMM(kEpiLinearF32, 3, kActMx6);
  } else if (af == kActMx8) {
    if (tall) {
      switch (epilogue) {
        case kEpiMxAct: MOE_LAUNCH_GEMM(kEpiMxAct, 4, kActMx8); break;
        case kEpiMx6Act: MOE_LAUNCH_GEMM(kEpiMx6Act, 4, kActMx8); break;
        case kEpiPreactF32: MOE_LAUNCH_GEMM(kEpiPreactF32, 4, kActMx8); break;
        case kEpiActF32: MOE_LAUNCH_GEMM(kEpiActF32, 4, kActMx8); break;
        default: MOE_LAUNCH_GEMM(kEpiLinearF32, 4, kActMx8); break;
      }
    } else {
      switch (epilogue) {
        case kEpiPreactF32: MOE_LAUNCH_GEMM(kEpiPreactF32, 3, kActMx8); break;
        case kEpiActF32: MOE_LAUNCH_GEMM(kEpiActF32, 3, kActMx8); break;
        default: MOE_LAUNCH_GEMM(kEpiLinearF32, 3, kActMx8); break;
      }
    }
  } else {
#define MOE_LAUNCH_GEMM_EPI(RG)                                                  \
  switch (epilogue) {                                                            \
    case kEpiSwigluBf16: MOE_LAUNCH_GEMM(kEpiSwigluBf16, RG, kActBf16); break;   \
    case kEpiPreactF32: MOE_LAUNCH_GEMM(kEpiPreactF32, RG, kActBf16); break;     \
    case kEpiActF32: MOE_LAUNCH_GEMM(kEpiActF32, RG, kActBf16); break;           \
    default: MOE_LAUNCH_GEMM(kEpiLinearF32, RG, kActBf16); break;                \
  }
    if (tall) {
      MOE_LAUNCH_GEMM_EPI(4)
    } else {
      MOE_LAUNCH_GEMM_EPI(3)
    }
#undef MOE_LAUNCH_GEMM_EPI
  }
#undef MOE_LAUNCH_GEMM
  return hipGetLastError();
}

}  // namespace moe
