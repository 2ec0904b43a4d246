// Expert FFN for a decode batch of one token: the gate_up projection, the clamped SwiGLU and
// the down projection in one launch. Decode time goes to moving expert weights (gpt-oss review
// at pomoai.com, section 4: decode dominates generation time; launch retrospective at
// youniszhang.com, "当时发生了什么": weight movement is the cost); with four slots the
// two-kernel form leaves the chip idle between its two launches and streams each matrix on too
// few workgroups, so here every weight byte a workgroup needs is requested at its start and the
// activation never leaves the workgroup.
//
// A workgroup owns one (expert e, block b) pair: the 32 activations 32 b .. 32 b + 31 of every
// slot routed to e (at most MT slots; tiled weights only, moe_mxfp4_pack):
//   * gate_up: W1's rows 64 b .. 64 b + 63 (tiles 2 b and 2 b + 1; gate and linear rows
//     interleaved, gpt-oss walkthrough at pnsm.cn, section 2.2) over the whole input
//     dimension. Eight waves: wave w takes tile w & 1 over quarter w >> 1 of the chunks, all of
//     its chunks requested at once; the expert's slot rows of x sit in LDS (zero-padded to whole
//     chunks). The quarters are added in a fixed order in LDS, then the bias, the clamp, the
//     SwiGLU with +1 on the linear branch (review, section 3.3), rounded to bf16: the block's
//     activations, in LDS only.
//   * down: MX block b of every row of W2, i.e. in each 32-row tile of W2 the 512 contiguous
//     bytes of chunk b / 4, half (b / 2) % 2, lanes 32 (b % 2) .. 32 (b % 2) + 31. One wave
//     load covers two tiles (lanes 0-31 one tile, lanes 32-63 the next); wave w takes loads
//     w, w + 8, ..., requested at the start with the gate_up weights. Lane l's product is row
//     32 G + l % 32 of its tile G against the block's 32 activations, complete in the lane:
//     y_b = W2[:, block b] a_b (plus b2 in block 0) goes to part[b][sorted row][H].
// With so few slots the matrix cores would spend almost all of their work on absent columns, so
// the products are VALU dot products: a lane turns its 16 code bytes (one row's MX block) into
// 16 bf16 pairs with gfx950's scaled FP4 convert (exact) and, per slot, adds 16
// v_dot2_f32_bf16 products of those pairs with the slot's matching activations into four fp32
// partial sums. Sums run in a fixed order everywhere (the four partials, the lane pair holding
// a row's two halves of a chunk, the four chunk quarters), and the per-block partial rows are
// added in a fixed order by the combine, so results are deterministic. Weight bytes are read
// once per touched expert; the partials (I / 32 x slots x H fp32, written once and read once)
// are the extra traffic.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int kSmWaves = 8;
constexpr int kSmMaxH = 3072;  // 24 chunks: at most 6 per wave and quarter
constexpr int kSmW1 = 6;       // gate_up chunks per wave
constexpr int kSmW2 = 6;       // down wave loads per wave (H / 64 loads over 8 waves)
}  // namespace

// MT: the most slots an expert can hold (the batch's token count); every per-slot array and
// loop is sized by it. Launched with MT = 1: with more slots the VALU products grow with them
// while the matrix-core form does not. (Measured on MI355X at one token, decode20b: this
// kernel 19.7 us plus a 5.5 us sliced combine, against 13.3 + 7.7 us for the two weight-
// streaming kernels plus a 3.8 us plain combine; layer 34.3 against 32.6 us. So it is opt-in.)
template <int MT>
__global__ __launch_bounds__(kSmWaves *kWave) void ffn_small_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ sorted_slot, int k, const int32_t *__restrict__ offsets,
    int E, int nblk, const uint8_t *__restrict__ c1, const uint8_t *__restrict__ s1, const uint16_t *__restrict__ b1,
    const uint8_t *__restrict__ c2, const uint8_t *__restrict__ s2, const uint16_t *__restrict__ b2, int H, int I,
    int64_t S, float *__restrict__ part, float limit, float alpha) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r32 = lane % 32, kh = lane / 32;
  const int ei = blockIdx.x / nblk, b = blockIdx.x % nblk;

  // ---- the ei-th expert that has slots (every wave finds the same one)
  int e = -1;
  {
    int carry = 0;
    for (int eb = 0; eb < E; eb += kWave) {
      const int ex = eb + lane;
      const int nz = (ex < E && offsets[ex + 1] > offsets[ex]) ? 1 : 0;
      const int inc = wave_inclusive_scan(nz) + carry;
      const uint64_t hit = __ballot(nz && inc == ei + 1);
      if (hit) {
        e = eb + __ffsll((unsigned long long)hit) - 1;
        break;
      }
      carry = wave_read(inc, kWave - 1);
    }
  }
  if (e < 0) return;  // the same in every wave: the whole workgroup leaves
  const int rbase = offsets[e];
  // at most MT (one slot per token); the clamp only keeps a malformed routing inside the
  // staged rows
  const int cnt = offsets[e + 1] - rbase;
  const int mcount = cnt < MT ? cnt : MT;

  const int nch1 = (H / 32 + 3) / 4;  // gate_up chunks (128 input elements each)
  const int NG1 = 2 * I / 32, NG2 = H / 32, nch2 = (I / 32 + 3) / 4;
  const int xrow = nch1 * 128;  // staged x row, zero-padded to whole chunks
  uint16_t *xs = reinterpret_cast<uint16_t *>(lds);
  float *red = reinterpret_cast<float *>(lds + MT * xrow * 2);          // [4 quarters][2 tiles][MT][32 rows]
  uint16_t *act = reinterpret_cast<uint16_t *>(red + 4 * 2 * MT * 32);  // [MT][32]

  // ---- every load up front: this wave's gate_up chunks and down tiles, then the slot rows of x
  const int tt = wave & 1, qq = wave >> 1;
  const int G1 = 2 * b + tt;
  const int per = (nch1 + 3) / 4;
  const int c_lo = qq * per;
  const int c_hi = c_lo + per < nch1 ? c_lo + per : nch1;
  const int nmine = c_hi > c_lo ? c_hi - c_lo : 0;
  const uint8_t *cb1 = c1 + ((int64_t)e * NG1 + G1) * nch1 * 2048 + lane * 16;
  const uint32_t *sb1 = reinterpret_cast<const uint32_t *>(s1 + ((int64_t)e * NG1 + G1) * nch1 * 128) + r32;
  u32x4_t cw[kSmW1][2];
  uint32_t sw[kSmW1];
#pragma unroll
  for (int i = 0; i < kSmW1; ++i) {
    int c = c_lo + (i < nmine ? i : 0);
    c = c < nch1 ? c : nch1 - 1;  // a quarter with no chunks (tiny H) still reads inside the tile
    cw[i][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(cb1 + (int64_t)c * 2048));
    cw[i][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(cb1 + (int64_t)c * 2048 + 1024));
    sw[i] = __builtin_nontemporal_load(sb1 + c * 32);
  }
  const int cbk = b >> 2, pp = (b >> 1) & 1, kh0 = b & 1;  // block b's place in W2's tiles
  const int nload2 = (NG2 + 1) / 2;
  u32x4_t w2v[kSmW2];
  uint32_t w2s[kSmW2];
#pragma unroll
  for (int i = 0; i < kSmW2; ++i) {
    const int j = wave + kSmWaves * i;
    int G = 2 * j + kh;
    G = G < NG2 ? G : NG2 - 1;  // (loads past the last tile are never used)
    const int64_t t = ((int64_t)e * NG2 + G) * nch2 + cbk;
    w2v[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_t *>(c2 + t * 2048 + pp * 1024 + (kh0 * 32 + r32) * 16));
    w2s[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(s2 + t * 128 + r32 * 4));
  }
  {
    constexpr int kXPieces = (MT * kSmMaxH / 8 + kSmWaves * kWave - 1) / (kSmWaves * kWave);
    const int xp = xrow / 8;  // 16-byte pieces per staged row
    int tok[MT];
#pragma unroll
    for (int r = 0; r < MT; ++r) tok[r] = r < mcount ? sorted_slot[rbase + r] / k : 0;
#pragma unroll
    for (int q = 0; q < kXPieces; ++q) {
      const int idx = threadIdx.x + q * kSmWaves * kWave;
      const int r = idx / xp, c8 = idx - r * xp;
      if (r < MT) {
        int tr = 0;
#pragma unroll
        for (int rr = 0; rr < MT; ++rr) tr = rr == r ? tok[rr] : tr;
        const bool ok = r < mcount && 8 * c8 < H;  // H % 32 == 0: a piece is wholly inside or past H
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(x + (int64_t)tr * H + (ok ? 8 * c8 : 0));
        *reinterpret_cast<u32x4_t *>(xs + r * xrow + 8 * c8) = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }
  __syncthreads();

  // ---- products of one lane's 32 weights (16 code bytes, one MX block of one row) with the
  // same 32 elements of each slot's activation row (bf16 in LDS at `a`, row stride `astride`)
  auto dot_block = [&](const u32x4_t &code, float sc, const uint16_t *a, int astride, float (&acc)[MT][4]) {
    bf16x2_t w[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {  // (the byte select must be a constant)
      w[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code[d], sc, 0);
      w[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code[d], sc, 1);
      w[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code[d], sc, 2);
      w[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code[d], sc, 3);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= mcount) break;  // wave-uniform
      // (the pairs are read as bf16x2 values: reading dword vectors and bit-casting their
      // elements made this compiler use element 0 for every pair)
      const bf16x2_t *ap = reinterpret_cast<const bf16x2_t *>(a + m * astride);
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[m][i] = __builtin_amdgcn_fdot2_f32_bf16(w[4 * v + i], ap[4 * v + i], acc[m][i], false);
    }
  };

  // ---- gate_up: lane (row r32, half kh) of chunk c, half p holds block 4c + 2p + kh of tile row r32
  float acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[m][i] = 0.f;
#pragma unroll
  for (int i = 0; i < kSmW1; ++i) {
    if (i >= nmine) break;  // wave-uniform
    const int c = c_lo + i;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float sc = e8m0_to_f32((sw[i] >> (8 * (2 * p + kh))) & 0xffu);
      dot_block(cw[i][p], sc, xs + 128 * c + 32 * (2 * p + kh), xrow, acc);
    }
  }
  // a row's total: its four partials, then the lane l ^ 32 partner's (the row's other blocks),
  // the same two values in the same order on both lanes
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= mcount) break;
    const float v = (acc[m][0] + acc[m][1]) + (acc[m][2] + acc[m][3]);
    const auto sv = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    if (kh == 0) red[((qq * 2 + tt) * MT + m) * 32 + r32] = __uint_as_float(sv[0]) + __uint_as_float(sv[1]);
  }
  __syncthreads();
  // the four quarters in order, the bias, the SwiGLU of (gate, linear) = rows (2i, 2i + 1): the
  // even lane of each pair computes activation 16 tt + r32 / 2 of the block
  if (wave < 2) {
    const float bias = b1 != nullptr ? bf16_to_f32(b1[(int64_t)e * 2 * I + 32 * G1 + r32]) : 0.f;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= mcount) break;
      const float *rq = red + (tt * MT + m) * 32 + r32;
      const float h = (((rq[0] + rq[2 * MT * 32]) + rq[4 * MT * 32]) + rq[6 * MT * 32]) + bias;
      const float hl = __shfl_down(h, 1, kWave);  // the linear half, from the odd lane
      if (kh == 0 && (r32 & 1) == 0) act[m * 32 + 16 * tt + r32 / 2] = f32_to_bf16_rne(swiglu_unit(h, hl, limit, alpha));
    }
  }
  __syncthreads();

  // ---- down: lane l of load j holds block b of row r32 of tile G = 2 j + l / 32
#pragma unroll
  for (int i = 0; i < kSmW2; ++i) {
    const int j = wave + kSmWaves * i;
    if (j >= nload2) break;  // wave-uniform
    const int G = 2 * j + kh;
    const float sc = e8m0_to_f32((w2s[i] >> (8 * (b & 3))) & 0xffu);
    float y[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) y[m][q] = 0.f;
    dot_block(w2v[i], sc, act, 32, y);
    if (G < NG2) {
      const int n = 32 * G + r32;
      const float bias = (b == 0 && b2 != nullptr) ? bf16_to_f32(b2[(int64_t)e * H + n]) : 0.f;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m >= mcount) break;
        part[((int64_t)b * S + rbase + m) * H + n] = ((y[m][0] + y[m][1]) + (y[m][2] + y[m][3])) + bias;
      }
    }
  }
}

int small_slices(int I) { return I / 32; }

bool small_ffn_fits(int64_t T, int H, int I) {
  return T >= 1 && T <= kSmallMaxT && H <= kSmMaxH && I >= 32 && I / 32 <= kSmallMaxSlices;
}

size_t small_partial_floats(int64_t T, int k, int H, int I) {
  return small_ffn_fits(T, H, I) ? (size_t)small_slices(I) * (size_t)(T * k) * (size_t)H : 0;
}

hipError_t launch_ffn_small(const uint16_t *x, const int32_t *sorted_slot, int k, const int32_t *offsets, int E,
                            int64_t S, const MxWeight &w1, const MxWeight &w2, float *part, float limit, float alpha,
                            hipStream_t stream) {
  const int H = w1.K, I = w2.K;
  const int64_t T = S / k;
  if (!small_ffn_fits(T, H, I)) return hipErrorInvalidValue;
  const int nblk = small_slices(I);
  const int64_t busy = S < E ? S : E;  // experts with slots, at most
  const int nch1 = (H / 32 + 3) / 4;
  const size_t lds = (size_t)kSmallMaxT * nch1 * 128 * 2 + 4 * 2 * kSmallMaxT * 32 * 4 + kSmallMaxT * 32 * 2;
  hipLaunchKernelGGL(ffn_small_kernel<kSmallMaxT>, dim3((unsigned)(busy * nblk)), dim3(kSmWaves * kWave), lds, stream,
                     x, sorted_slot, k, offsets, E, nblk, w1.codes, w1.scales, w1.bias, w2.codes, w2.scales, w2.bias,
                     H, I, S, part, limit, alpha);
  return hipGetLastError();
}

}  // namespace moe
