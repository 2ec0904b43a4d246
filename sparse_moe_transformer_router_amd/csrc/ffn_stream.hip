// Expert FFN projections for decode-sized batches: a weight-streaming grouped GEMM.
//
// Each expert's projection y = W x (+ b) runs only on the slots routed to it (review of the
// from-scratch gpt-oss-20B at pomoai.com, section 3.4), with W in MXFP4 (gpt-oss
// walkthrough at pnsm.cn, sections 1 and 4) and the clamped SwiGLU with +1 on the linear
// branch fused into the gate_up epilogue (walkthrough section 2.2; review section 3.3).
//
// With few slots per expert the product is bound by streaming the 4.25-bit weights from
// HBM, so the weights take the MFMA's 16-row A operand straight from global memory:
//   * a workgroup owns 64 weight rows (four 16-row groups) of one expert and up to 16 of
//     that expert's slots (one "m-tile"); its four waves split the input dimension in
//     128-wide chunks, round robin;
//   * lane l reads 16 code bytes = one 32-element MX block of row (l % 16) in each row
//     group and converts them with the block's scale into bf16 in registers (gfx950's
//     scaled FP4 convert; E2M1 times a power of two is exact in bf16), lanes l / 16 = q
//     taking consecutive blocks;
//   * the slot activations (bf16) come from global memory through L1/L2, 64 bytes per lane
//     per chunk, matching the k-range of the lane's weight block;
//   * v_mfma_f32_16x16x32_bf16 accumulates in fp32; the four waves' partial sums are added
//     in LDS in a fixed order, so results are deterministic.
// The m-tile -> (expert, first slot) map is recomputed by every wave from expert_offsets
// (a wave-wide scan over experts), so no tile list is materialised and the grid is sized
// from host-known bounds only; surplus workgroups exit at once.
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

constexpr int kSRows = 64;   // weight rows per workgroup
constexpr int kSCols = 16;   // slots per m-tile
constexpr int kSWaves = 4;

template <int EPI>
__global__ __launch_bounds__(kSWaves *kWave) void ffn_stream_kernel(
    const uint16_t *__restrict__ a_src, int a_by_token, const int32_t *__restrict__ sorted_slot, int k,
    const int32_t *__restrict__ offsets, int E, const uint8_t *__restrict__ codes,
    const uint8_t *__restrict__ scales, const uint16_t *__restrict__ bias, int N, int K,
    void *__restrict__ out, float limit, float alpha) {
  __shared__ float red[kSWaves][kSRows][kSCols + 1];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int n0 = blockIdx.y * kSRows;
  const int mt = blockIdx.x;

  // ---- which expert and which 16 of its slots this m-tile covers
  int e = -1, m0 = 0, rbase = 0, mcount = 0;
  {
    int carry = 0;
    for (int eb = 0; eb < E; eb += kWave) {
      const int ex = eb + lane;
      const int cnt = (ex < E) ? offsets[ex + 1] - offsets[ex] : 0;
      const int tiles = (cnt + kSCols - 1) / kSCols;
      const int inc = wave_inclusive_scan(tiles);
      const int excl = inc - tiles + carry;
      const uint64_t hit = __ballot(tiles > 0 && mt >= excl && mt < excl + tiles);
      if (hit) {
        const int src = __ffsll((unsigned long long)hit) - 1;
        const int sel_excl = wave_read(excl, src);
        e = eb + src;
        m0 = (mt - sel_excl) * kSCols;
        rbase = offsets[e];
        const int cnt_e = offsets[e + 1] - rbase;
        mcount = (cnt_e - m0 < kSCols) ? cnt_e - m0 : kSCols;
        break;
      }
      carry += wave_read(inc, kWave - 1);
    }
  }
  if (e < 0) return;  // same decision in every wave: the whole workgroup leaves

  const int rl = lane % 16, q = lane / 16;
  const bool col_ok = rl < mcount;
  const uint16_t *arow = a_src;
  if (col_ok) {
    const int r = rbase + m0 + rl;
    const int64_t src_row = a_by_token ? (int64_t)(sorted_slot[r] / k) : (int64_t)r;
    arow = a_src + src_row * K;
  }

  const int KB = K / 32;
  const int nchunk = (KB + 3) / 4;
  const int64_t row_bytes = K / 2;
  const uint8_t *cexp = codes + (int64_t)e * N * row_bytes;
  const uint8_t *sexp = scales + (int64_t)e * N * KB;

  f32x4_t acc[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int c = wave; c < nchunk; c += kSWaves) {
    const int b = c * 4 + q;  // this lane's MX block along K
    const bool bvalid = b < KB;
    u32x4_t cw[4];
    uint32_t sw[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int row = n0 + 16 * g + rl;
      if (bvalid && row < N) {
        cw[g] = *reinterpret_cast<const u32x4_t *>(cexp + row * row_bytes + b * 16);
        sw[g] = sexp[(int64_t)row * KB + b];
      } else {
        cw[g] = u32x4_t{0u, 0u, 0u, 0u};
        sw[g] = 127u;
      }
    }
    u32x4_t av[4];
    if (bvalid && col_ok) {
      const u32x4_t *ap = reinterpret_cast<const u32x4_t *>(arow + b * 32);
#pragma unroll
      for (int j = 0; j < 4; ++j) av[j] = ap[j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) av[j] = u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float sc = e8m0_to_f32(sw[g]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t wa = fp4x8_to_bf16x8(cw[g][j], sc);
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, as_bf16x8(av[j]), acc[g], 0, 0, 0);
      }
    }
  }

  // ---- cross-wave reduction (fixed order) and epilogue
  // mfma 16x16 output: lane l holds rows 4*(l/16) + i, column l % 16
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][16 * g + 4 * q + i][rl] = acc[g][i];
  __syncthreads();

  const int col = threadIdx.x % kSCols;
  const int r0 = (threadIdx.x / kSCols) * 4;  // 4 consecutive rows of the 64
  if (col >= mcount) return;
  float h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float s = red[0][r0 + i][col];
#pragma unroll
    for (int w = 1; w < kSWaves; ++w) s += red[w][r0 + i][col];
    const int n = n0 + r0 + i;
    if (bias != nullptr && n < N) s += bf16_to_f32(bias[(int64_t)e * N + n]);
    h[i] = s;
  }
  const int64_t r = rbase + m0 + col;  // sorted row of this slot
  if (EPI == kEpiSwigluBf16 || EPI == kEpiActF32) {
    const int half = N / 2;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int n = n0 + r0 + 2 * p;
      if (n < N) {
        const uint16_t ab = f32_to_bf16_rne(swiglu_unit(h[2 * p], h[2 * p + 1], limit, alpha));
        if (EPI == kEpiSwigluBf16)
          reinterpret_cast<uint16_t *>(out)[r * half + n / 2] = ab;
        else
          reinterpret_cast<float *>(out)[r * half + n / 2] = bf16_to_f32(ab);
      }
    }
  } else {
    float *o = reinterpret_cast<float *>(out) + r * N + n0 + r0;
    if (n0 + r0 + 3 < N) {
      *reinterpret_cast<f32x4_t *>(o) = f32x4_t{h[0], h[1], h[2], h[3]};
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n0 + r0 + i < N) o[i] = h[i];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Same product on the tiled weight layout (moe_mxfp4_pack), on v_mfma_f32_32x32x16_bf16 (which
// issues at twice the rate of the 16x16x32 form on gfx950): a workgroup owns 64 weight rows
// (two 32-row tiles) of one expert and up to 32 of its slots; four waves split the chunks.
// Every weight load is one contiguous 1 KB per wave; a lane's two 16-byte loads per tile and
// chunk are MX blocks 4c + 2p + lane/32 (p = 0, 1) of row lane%32, each split into four
// 8-element MFMA k-steps; the slot activations for a step are read with the same
// k-assignment (64 contiguous bytes per lane and block). PF = chunks of register prefetch.
constexpr int kTRows = 64;   // weight rows per workgroup (two 32-row tiles)
constexpr int kTCols = 32;   // slots per m-tile
constexpr int kTiledPrefetch = 2;  // chunks in flight per wave

// One token's routing inside the gate_up launch (R1 = k, its pick count; 0: off): the slots
// are the token's k picks, and m-tile j is pick j alone. Every wave sums the router's split-K
// partials and picks the experts exactly as the router's top-k kernels do (the same helpers,
// so the same picks and weights), and workgroup 0's first wave publishes the routing (picks,
// weights, offsets, the stable sort of the k slots) for the down projection and the combine.
// No workgroup reads what another writes.
template <int R1>
__device__ __forceinline__ int route1_rank(const int (&pe)[R1], int e) {
  int rank = 0;
#pragma unroll
  for (int j = 0; j < R1; ++j) rank += (pe[j] >= 0 && pe[j] < e) ? 1 : 0;
  return rank;
}

template <int R1>
__device__ __forceinline__ void route1_publish(const int (&pe)[R1], const float (&pw)[R1], int E, int lane,
                                               const Route1 &r1) {
  int ej = -1;
  float wj = 0.f;
#pragma unroll
  for (int j = 0; j < R1; ++j) {
    ej = lane == j ? pe[j] : ej;
    wj = lane == j ? pw[j] : wj;
  }
  if (lane < R1) {
    const int rank = route1_rank<R1>(pe, ej);
    r1.topk_idx[lane] = ej;
    r1.topk_w[lane] = wj;
    r1.slot_row[lane] = ej >= 0 ? rank : -1;  // a pick with no expert (NaN logits) gets no row
    if (ej >= 0) r1.sorted_slot[rank] = lane;
  }
  for (int x = lane; x <= E; x += kWave) r1.offsets[x] = route1_rank<R1>(pe, x);
}

template <int EPI, int PF, int R1 = 0>
__global__ __launch_bounds__(kSWaves *kWave) void ffn_stream_tiled_kernel(
    const uint16_t *__restrict__ a_src, int a_by_token, const int32_t *__restrict__ sorted_slot, int k,
    const int32_t *__restrict__ offsets, int E, const uint8_t *__restrict__ pcodes,
    const uint8_t *__restrict__ pscales, const uint16_t *__restrict__ bias, int N, int K, int ntiles_n,
    void *__restrict__ out, float limit, float alpha, Route1 r1) {
  constexpr int RG = kTRows / 32;
  __shared__ float red[kSWaves][kTRows][kTCols + 1];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int mt = blockIdx.x / ntiles_n, nt = blockIdx.x % ntiles_n;
  const int g0 = nt * RG;
  const int n0 = nt * kTRows;

  int e = -1, m0 = 0, rbase = 0, mcount = 0;
  if constexpr (R1 > 0) {
    float v[4];
    router_logits_wave<false>(r1.partial, r1.nsplit, r1.bias, 0, 1, E, lane, v);
    int pe[R1];
    float pw[R1];
    topk_picks_wave_k<R1>(v, E, lane, pe, pw);
    if (blockIdx.x == 0 && wave == 0) route1_publish<R1>(pe, pw, E, lane, r1);
    int sel = -1;
#pragma unroll
    for (int j = 0; j < R1; ++j) sel = j == mt ? pe[j] : sel;
    if (sel >= 0) {
      e = sel;
      rbase = route1_rank<R1>(pe, sel);
      mcount = 1;
    }
  } else {
    int carry = 0;
    for (int eb = 0; eb < E; eb += kWave) {
      const int ex = eb + lane;
      const int cnt = (ex < E) ? offsets[ex + 1] - offsets[ex] : 0;
      const int tiles = (cnt + kTCols - 1) / kTCols;
      const int inc = wave_inclusive_scan(tiles);
      const int excl = inc - tiles + carry;
      const uint64_t hit = __ballot(tiles > 0 && mt >= excl && mt < excl + tiles);
      if (hit) {
        const int src = __ffsll((unsigned long long)hit) - 1;
        const int sel_excl = wave_read(excl, src);
        e = eb + src;
        m0 = (mt - sel_excl) * kTCols;
        rbase = offsets[e];
        const int cnt_e = offsets[e + 1] - rbase;
        mcount = (cnt_e - m0 < kTCols) ? cnt_e - m0 : kTCols;
        break;
      }
      carry += wave_read(inc, kWave - 1);
    }
  }
  if (e < 0) return;

  const int r32 = lane % 32, kh = lane / 32;
  const bool col_ok = r32 < mcount;
  // slot-order output: the epilogue thread's slot row, looked up now, not after the loop
  const int ycol = threadIdx.x % kTCols;
  const int yrow = EPI == kEpiLinearSlotF32 ? sorted_slot[rbase + m0 + (ycol < mcount ? ycol : 0)] : 0;
  const uint16_t *arow = a_src;  // R1: the one token's row
  if (R1 == 0 && col_ok) {
    const int r = rbase + m0 + r32;
    arow = a_src + (a_by_token ? (int64_t)(sorted_slot[r] / k) : (int64_t)r) * K;
  }
  const int KB = K / 32;
  const int nchunk = (KB + 3) / 4;
  const int NG = N / 32;
  const uint8_t *cbase = pcodes + (int64_t)e * NG * nchunk * 2048 + lane * 16;
  const uint8_t *sbase = pscales + (int64_t)e * NG * nchunk * 128 + r32 * 4;

  f32x16_t acc[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;
  // this wave's chunks c = wave + kSWaves i, i < nmine, PF of them in flight. Every load is
  // issued unconditionally from a clamped in-bounds address (a tile past N reads tile 0 and is
  // never stored; a block past K reads block 0 and is zeroed at its use; a chunk past the
  // wave's last re-reads that last one, from cache), and the loop body has no path that skips
  // its loads: with a load under a branch the compiler waits for every load in flight at the
  // top of each iteration, which serialises the prefetch.
  const int nmine = wave < nchunk ? (nchunk - wave + kSWaves - 1) / kSWaves : 0;
  u32x4_t cw[PF][RG][2];
  uint32_t sw[PF][RG];
  u32x4_t av[PF][2][4];
  auto load = [&](int i, int s) {
    const int c = nmine > 0 ? wave + kSWaves * (i < nmine ? i : nmine - 1) : 0;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const int gg = (g0 + g) < NG ? g0 + g : 0;
      const int64_t t = (int64_t)gg * nchunk + c;
#pragma unroll
      for (int p = 0; p < 2; ++p)
        cw[s][g][p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(cbase + t * 2048 + p * 1024));
      sw[s][g] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(sbase + t * 128));
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int blk = 4 * c + 2 * p + kh;  // this lane's MX block of half p
      const u32x4_t *a4 = reinterpret_cast<const u32x4_t *>(arow + (blk < KB ? blk : 0) * 32);
#pragma unroll
      for (int j = 0; j < 4; ++j) av[s][p][j] = a4[j];
    }
  };
  auto body = [&](int i, int s) {
    const int c = wave + kSWaves * i;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const bool ok = col_ok && (4 * c + 2 * p + kh) < KB;
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        const float sc = e8m0_to_f32((sw[s][g] >> (8 * (2 * p + kh))) & 0xffu);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8_t wa = fp4x8_to_bf16x8(cw[s][g][p][j], sc);
          const u32x4_t a = ok ? av[s][p][j] : u32x4_t{0u, 0u, 0u, 0u};
          acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, as_bf16x8(a), acc[g], 0, 0, 0);
        }
      }
    }
    load(i + PF, s);
  };
#pragma unroll
  for (int s = 0; s < PF; ++s) load(s, s);
  int i = 0;
  for (; i + PF <= nmine; i += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) body(i + s, s);
  }
#pragma unroll
  for (int s = 0; s < PF - 1; ++s)
    if (i + s < nmine) body(i + s, s);

  // 32x32 output: lane holds slot column lane%32, rows 8i + 4*(lane/32) + j (i, j = 0..3)
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[wave][32 * g + 8 * i + 4 * kh + j][r32] = acc[g][4 * i + j];
  __syncthreads();

  const int col = threadIdx.x % kTCols;
  const int rq = (threadIdx.x / kTCols) * 8;  // 8 consecutive rows of the 64
  if (col >= mcount) return;
  const int64_t r = EPI == kEpiLinearSlotF32 ? (int64_t)yrow : rbase + m0 + col;
  uint2 bq[2] = {uint2{0u, 0u}, uint2{0u, 0u}};  // bias of the 8 rows (rows past N: row 0)
  if (bias != nullptr) {
#pragma unroll
    for (int h4 = 0; h4 < 2; ++h4) {
      const int n = n0 + rq + 4 * h4;
      bq[h4] = *reinterpret_cast<const uint2 *>(bias + (int64_t)e * N + (n < N ? n : 0));
    }
  }
#pragma unroll
  for (int h4 = 0; h4 < 2; ++h4) {
    const int r0 = rq + 4 * h4;
    const float bv[4] = {__uint_as_float(bq[h4].x << 16), __uint_as_float(bq[h4].x & 0xffff0000u),
                         __uint_as_float(bq[h4].y << 16), __uint_as_float(bq[h4].y & 0xffff0000u)};
    float h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float sum = red[0][r0 + i][col];
#pragma unroll
      for (int w = 1; w < kSWaves; ++w) sum += red[w][r0 + i][col];
      h[i] = sum + bv[i];
    }
    if (EPI == kEpiSwigluBf16 || EPI == kEpiActF32) {
      const int half = N / 2;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int n = n0 + r0 + 2 * p;
        if (n < N) {
          const uint16_t ab = f32_to_bf16_rne(swiglu_unit(h[2 * p], h[2 * p + 1], limit, alpha));
          if (EPI == kEpiSwigluBf16)
            reinterpret_cast<uint16_t *>(out)[r * half + n / 2] = ab;
          else
            reinterpret_cast<float *>(out)[r * half + n / 2] = bf16_to_f32(ab);
        }
      }
    } else {
      float *o = reinterpret_cast<float *>(out) + r * N + n0 + r0;
      if (n0 + r0 + 3 < N) {
        *reinterpret_cast<f32x4_t *>(o) = f32x4_t{h[0], h[1], h[2], h[3]};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n0 + r0 + i < N) o[i] = h[i];
      }
    }
  }
}


// ---------------------------------------------------------------------------------------
// Row-split form for more than a handful of slots, tiled weights: the four waves of a
// workgroup own four different 32-row tiles (128 rows) of one expert and walk the whole
// input dimension together, so the 32-slot activation chunk is fetched once per workgroup
// and shared through LDS, and no cross-wave reduction is needed. Each chunk's activations
// go global -> registers (two 16-byte pieces per lane, loaded three chunks ahead) ->
// ds_write into a 2-deep LDS ring (16-byte columns XOR-swizzled by slot); weights stream
// into registers D chunks ahead with non-temporal loads (each weight byte is read once per
// layer; on this part non-temporal streaming reads reach ~7.1 TB/s against ~6.3 TB/s for
// plain ones, and they keep the reused activations in the caches). No LDS DMA here: the compiler's wait counting for the
// register loads stays exact only without it. All loads are issued unconditionally from
// clamped in-bounds addresses (values past K or of absent slots are zeroed after the
// load), so no control path skips a load and the compiler's waits stay tight.
// Chunks c + J of a D-deep weight ring, fully unrolled: weight set J % D, activation register
// set (J + 1) % 2 (D is even).
template <int D, typename F, int... J>
__device__ __forceinline__ void ring_unroll(F &&body, int c, std::integer_sequence<int, J...>) {
  (body(c + J, std::integral_constant<int, J % D>{}, std::integral_constant<int, (J + 1) % 2>{}), ...);
}
template <int D, typename F, int... J>
__device__ __forceinline__ void ring_tail(F &&body, int c, int nchunk, std::integer_sequence<int, J...>) {
  ((c + J < nchunk ? (body(c + J, std::integral_constant<int, J % D>{}, std::integral_constant<int, (J + 1) % 2>{}),
                      0)
                   : 0),
   ...);
}

constexpr int kRWaves = 4;
constexpr int kRCols = 32;            // slots per m-tile
// below this many slots the K-split form keeps more waves busy (FFN, decode20b: 16 slots 45.0
// against 47.5 us for the row-split form; 24 slots 52.9 against 51.4, 32 slots 74.1 against 70.7)
constexpr int kRowSplitMinSlots = 20;

template <int EPI, int D>
__global__ __launch_bounds__(kRWaves *kWave) void ffn_stream_rows_kernel(
    const uint16_t *__restrict__ a_src, int a_by_token, const int32_t *__restrict__ sorted_slot, int k,
    const int32_t *__restrict__ offsets, int E, const uint8_t *__restrict__ pcodes,
    const uint8_t *__restrict__ pscales, const uint16_t *__restrict__ bias, int N, int K, int ntiles_n,
    void *__restrict__ out, float limit, float alpha) {
  static_assert(D % 2 == 0, "the weight ring period must be even");
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kRCols * 256];
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int mt = blockIdx.x / ntiles_n, nt = blockIdx.x % ntiles_n;
  int e = -1, m0 = 0, rbase = 0, mcount = 0;
  {
    int carry = 0;
    for (int eb = 0; eb < E; eb += kWave) {
      const int ex = eb + lane;
      const int cnt = (ex < E) ? offsets[ex + 1] - offsets[ex] : 0;
      const int tiles = (cnt + kRCols - 1) / kRCols;
      const int inc = wave_inclusive_scan(tiles);
      const int excl = inc - tiles + carry;
      const uint64_t hit = __ballot(tiles > 0 && mt >= excl && mt < excl + tiles);
      if (hit) {
        const int src = __ffsll((unsigned long long)hit) - 1;
        const int sel_excl = wave_read(excl, src);
        e = eb + src;
        m0 = (mt - sel_excl) * kRCols;
        rbase = offsets[e];
        const int cnt_e = offsets[e + 1] - rbase;
        mcount = (cnt_e - m0 < kRCols) ? cnt_e - m0 : kRCols;
        break;
      }
      carry += wave_read(inc, kWave - 1);
    }
  }
  if (e < 0) return;
  const int r32 = lane % 32, kh = lane / 32;
  // slot-order output: this lane's row goes to its slot's row, looked up now, not after the loop
  const int yrow = EPI == kEpiLinearSlotF32 ? sorted_slot[rbase + m0 + (r32 < mcount ? r32 : 0)] : 0;
  const int KB = K / 32;
  const int nchunk = (KB + 3) / 4;
  const int NG = N / 32;
  const int g = nt * kRWaves + wave;
  const int gc = g < NG ? g : 0;  // a wave past N streams tile 0 again and stores nothing

  // activation staging: piece i of this wave is slot 8 wave + 4 i + lane / 16, logical
  // 16-byte column lane % 16, stored at column (lane % 16) ^ (slot & 15)
  const uint16_t *rowp[2];
  int soff[2];
  bool sok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int slot = 8 * wave + 4 * i + lane / 16;
    sok[i] = slot < mcount;
    const int r = rbase + m0 + (sok[i] ? slot : 0);
    rowp[i] = a_src + (a_by_token ? (int64_t)(sorted_slot[r] / k) : (int64_t)r) * K;  // row start
    soff[i] = slot * 256 + (((lane % 16) ^ (slot & 15)) << 4);
  }
  u32x4_t ar[2][2];
  auto aload = [&](int c, int s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      // in range: elements c*128 + 8 (lane % 16) .. +7 of the row; otherwise the row's first 8
      const int off = c * 128 + (lane % 16) * 8;
      const bool ok = sok[i] && c < nchunk && off < K;
      const u32x4_t v = *reinterpret_cast<const u32x4_t *>(rowp[i] + (ok ? off : 0));
      ar[s][i] = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto awrite = [&](int c, int s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4_t *>(lds + (c & 1) * 8192 + soff[i]) = ar[s][i];
  };
  const uint8_t *cb = pcodes + ((int64_t)e * NG + gc) * nchunk * 2048 + lane * 16;
  const uint32_t *sb = reinterpret_cast<const uint32_t *>(pscales + ((int64_t)e * NG + gc) * nchunk * 128) + r32;
  u32x4_t cw[D][2];
  uint32_t sw[D];
  auto wload = [&](int c, int s) {
    const int cc = c < nchunk ? c : 0;
    cw[s][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(cb + (int64_t)cc * 2048));
    cw[s][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(cb + (int64_t)cc * 2048 + 1024));
    sw[s] = __builtin_nontemporal_load(sb + cc * 32);
  };
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  // prologue: chunk 0 into LDS, chunks 1 and 2 in register sets 1 and 0, weights 0..D-1
  aload(0, 0);
#pragma unroll
  for (int s = 0; s < D; ++s) wload(s, s);
  awrite(0, 0);
  aload(1, 1);
  aload(2, 0);
  // chunk c: barrier; MFMAs on LDS stage c & 1 with weight set u; write chunk c + 1 (register
  // set a) to stage (c + 1) & 1, reload set a with chunk c + 3, reload weight set u with c + D
  auto body = [&](int c, auto U_, auto A_) {
    constexpr int u = decltype(U_)::value;
    constexpr int a = decltype(A_)::value;
    __syncthreads();
    const unsigned char *abuf = lds + (c & 1) * 8192;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float sc = e8m0_to_f32((sw[u] >> (8 * (2 * p + kh))) & 0xffu);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col16 = 4 * (2 * p + kh) + j;
        const bf16x8_t bv =
            as_bf16x8(*reinterpret_cast<const u32x4_t *>(abuf + r32 * 256 + ((col16 ^ (r32 & 15)) << 4)));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp4x8_to_bf16x8(cw[u][p][j], sc), bv, acc, 0, 0, 0);
      }
    }
    awrite(c + 1, a);
    aload(c + 3, a);
    wload(c + D, u);
  };
  // D chunks per iteration (weight set J % D, activation register set (J + 1) % 2), then the
  // remainder peeled
  int c = 0;
  for (; c + D <= nchunk; c += D) ring_unroll<D>(body, c, std::make_integer_sequence<int, D>{});
  ring_tail<D>(body, c, nchunk, std::make_integer_sequence<int, D - 1>{});

  // epilogue: lane holds slot lane % 32 and rows 32 g + 8 i + 4 kh + jj of the output
  if (g >= NG || r32 >= mcount) return;
  const int64_t r = EPI == kEpiLinearSlotF32 ? (int64_t)yrow : rbase + m0 + r32;
  uint2 bq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    bq[i] = bias ? *reinterpret_cast<const uint2 *>(bias + (int64_t)e * N + 32 * g + 8 * i + 4 * kh) : uint2{0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = 32 * g + 8 * i + 4 * kh;
    const float h0 = acc[4 * i + 0] + __uint_as_float(bq[i].x << 16);
    const float h1 = acc[4 * i + 1] + __uint_as_float(bq[i].x & 0xffff0000u);
    const float h2 = acc[4 * i + 2] + __uint_as_float(bq[i].y << 16);
    const float h3 = acc[4 * i + 3] + __uint_as_float(bq[i].y & 0xffff0000u);
    if (EPI == kEpiSwigluBf16 || EPI == kEpiActF32) {
      const uint16_t a0 = f32_to_bf16_rne(swiglu_unit(h0, h1, limit, alpha));
      const uint16_t a1 = f32_to_bf16_rne(swiglu_unit(h2, h3, limit, alpha));
      if (EPI == kEpiSwigluBf16)
        *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(out) + r * (N / 2) + n / 2) =
            (uint32_t)a0 | ((uint32_t)a1 << 16);
      else
        *reinterpret_cast<float2 *>(reinterpret_cast<float *>(out) + r * (N / 2) + n / 2) =
            float2{bf16_to_f32(a0), bf16_to_f32(a1)};
    } else {
      *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(out) + r * N + n) = f32x4_t{h0, h1, h2, h3};
    }
  }
}

hipError_t launch_ffn_stream(const uint16_t *a_src, bool a_by_token, const int32_t *sorted_slot,
                             int k, const int32_t *offsets, int E, int64_t S, const MxWeight &w,
                             int epilogue, void *out, float limit, float alpha, hipStream_t stream) {
  const int64_t busy = (S < E) ? S : E;  // experts with at least one slot, at most
  const int64_t mtiles = (S + kSCols - 1) / kSCols + busy;
  // m-tiles along x (unbounded), weight-row tiles along y (at most 512)
  dim3 grid((unsigned)mtiles, (unsigned)((w.N + kSRows - 1) / kSRows));
  dim3 block(kSWaves * kWave);
#define MOE_LAUNCH_STREAM(EPI)                                                                   \
  hipLaunchKernelGGL(ffn_stream_kernel<EPI>, grid, block, 0, stream, a_src, a_by_token ? 1 : 0,    \
                     sorted_slot, k, offsets, E, w.codes, w.scales, w.bias, w.N, w.K, out, limit, \
                     alpha)
  if (w.tiled && S >= kRowSplitMinSlots) {
    const int64_t mt32 = (S + kRCols - 1) / kRCols + busy;
    const int ntn = (w.N / 32 + kRWaves - 1) / kRWaves;
    dim3 g1((unsigned)(mt32 * ntn));
    // a 4-chunk weight ring from 80 slots (FFN, decode20b: 20 tokens 77.6 against 81.3 us, 28 tokens 81.7
    // against 85.1; at 16 tokens and fewer the 2-chunk ring, with a wave more per SIMD, is faster: 73.0
    // against 75.8 us at 16, 69.0 against 71.1 at 8)
    const bool deep = S >= 80;
#define MOE_LAUNCH_ROWS(EPI)                                                                           \
  do {                                                                                                 \
    if (deep)                                                                                          \
      hipLaunchKernelGGL((ffn_stream_rows_kernel<EPI, 4>), g1, dim3(kRWaves * kWave), 0, stream, a_src, \
                         a_by_token ? 1 : 0, sorted_slot, k, offsets, E, w.codes, w.scales, w.bias, w.N, \
                         w.K, ntn, out, limit, alpha);                                                 \
    else                                                                                               \
      hipLaunchKernelGGL((ffn_stream_rows_kernel<EPI, 2>), g1, dim3(kRWaves * kWave), 0, stream, a_src, \
                         a_by_token ? 1 : 0, sorted_slot, k, offsets, E, w.codes, w.scales, w.bias, w.N, \
                         w.K, ntn, out, limit, alpha);                                                 \
  } while (0)
    switch (epilogue) {
      case kEpiSwigluBf16: MOE_LAUNCH_ROWS(kEpiSwigluBf16); break;
      case kEpiPreactF32: MOE_LAUNCH_ROWS(kEpiPreactF32); break;
      case kEpiActF32: MOE_LAUNCH_ROWS(kEpiActF32); break;
      case kEpiLinearSlotF32: MOE_LAUNCH_ROWS(kEpiLinearSlotF32); break;
      default: MOE_LAUNCH_ROWS(kEpiLinearF32); break;
    }
#undef MOE_LAUNCH_ROWS
    return hipGetLastError();
  }
  if (w.tiled) {
    // m-tile-major 1-D grid; each wave keeps kTiledPrefetch of its chunks in flight
    const int64_t mt32 = (S + kTCols - 1) / kTCols + busy;
    const int ntn = (w.N + kTRows - 1) / kTRows;
    dim3 g1((unsigned)(mt32 * ntn));
#define MOE_LAUNCH_TILED(EPI)                                                                       \
  hipLaunchKernelGGL((ffn_stream_tiled_kernel<EPI, kTiledPrefetch>), g1, block, 0, stream, a_src,   \
                     a_by_token ? 1 : 0, sorted_slot, k, offsets, E, w.codes, w.scales, w.bias, w.N, \
                     w.K, ntn, out, limit, alpha, Route1{})
    switch (epilogue) {
      case kEpiSwigluBf16: MOE_LAUNCH_TILED(kEpiSwigluBf16); break;
      case kEpiPreactF32: MOE_LAUNCH_TILED(kEpiPreactF32); break;
      case kEpiActF32: MOE_LAUNCH_TILED(kEpiActF32); break;
      case kEpiLinearSlotF32: MOE_LAUNCH_TILED(kEpiLinearSlotF32); break;
      default: MOE_LAUNCH_TILED(kEpiLinearF32); break;
    }
#undef MOE_LAUNCH_TILED
    return hipGetLastError();
  }
  if (epilogue == kEpiLinearSlotF32) return hipErrorInvalidValue;  // tiled weights only
  switch (epilogue) {
    case kEpiSwigluBf16: MOE_LAUNCH_STREAM(kEpiSwigluBf16); break;
    case kEpiPreactF32: MOE_LAUNCH_STREAM(kEpiPreactF32); break;
    case kEpiActF32: MOE_LAUNCH_STREAM(kEpiActF32); break;
    default: MOE_LAUNCH_STREAM(kEpiLinearF32); break;
  }
#undef MOE_LAUNCH_STREAM
  return hipGetLastError();
}

bool ffn_route1_fits(int64_t T, int E, int k, const MxWeight &w) {
  return T == 1 && w.tiled && k >= 1 && k <= 8 && E >= k && E <= 256 && (int64_t)k < kRowSplitMinSlots;
}

hipError_t launch_ffn_stream_route1(const uint16_t *x, int k, int E, const MxWeight &w, void *act, float limit,
                                    float alpha, const Route1 &r1, hipStream_t stream) {
  // one m-tile per pick, the weight rows of gate_up in 64-row tiles
  const int ntn = (w.N + kTRows - 1) / kTRows;
  const dim3 grid((unsigned)(k * ntn)), block(kSWaves * kWave);
#define MOE_LAUNCH_ROUTE1(K1)                                                                                      \
  hipLaunchKernelGGL((ffn_stream_tiled_kernel<kEpiSwigluBf16, kTiledPrefetch, K1>), grid, block, 0, stream, x, 0, \
                     nullptr, k, nullptr, E, w.codes, w.scales, w.bias, w.N, w.K, ntn, act, limit, alpha, r1)
  switch (k) {
    case 1: MOE_LAUNCH_ROUTE1(1); break;
    case 2: MOE_LAUNCH_ROUTE1(2); break;
    case 3: MOE_LAUNCH_ROUTE1(3); break;
    case 4: MOE_LAUNCH_ROUTE1(4); break;
    case 5: MOE_LAUNCH_ROUTE1(5); break;
    case 6: MOE_LAUNCH_ROUTE1(6); break;
    case 7: MOE_LAUNCH_ROUTE1(7); break;
    case 8: MOE_LAUNCH_ROUTE1(8); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_LAUNCH_ROUTE1
  return hipGetLastError();
}

}  // namespace moe
