// Host-side launchers of the layer's HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Output modes of the expert-FFN kernels' epilogues.
enum FfnEpilogue : int {
  kEpiSwigluBf16 = 0,  // gate_up: SwiGLU(h) -> bf16 act [S][N/2]
  kEpiPreactF32 = 1,   // gate_up: h -> fp32 [S][N]
  kEpiActF32 = 2,      // gate_up: bf16-rounded SwiGLU(h) widened to fp32 [S][N/2]
  kEpiLinearF32 = 3,   // down: W a + b -> fp32 [S][N]
  kEpiMxAct = 4,       // gate_up: bf16-rounded SwiGLU(h) -> two-term MXFP8 records (mx_act.h)
  kEpiMx6Act = 5,      // gate_up: bf16-rounded SwiGLU(h) -> two-term MXFP6 records (mx_act.h)
  kEpiLinearSlotF32 = 6,  // down, tiled weights: W a + b -> fp32 [S][N] in slot order (sorted row r
                          // goes to row sorted_slot[r]), for launch_combine's by_slot form
};

struct MxWeight {
  const uint8_t *codes;   // row-major [E][N][K/2], or tiled (moe_mxfp4_pack)
  const uint8_t *scales;  // row-major [E][N][K/32], or tiled
  const uint16_t *bias;   // [E][N] bf16 or nullptr
  int N, K;
  bool tiled;
};

hipError_t launch_pack(const uint8_t *codes, const uint8_t *scales, int E, int N, int K, uint8_t *pcodes,
                       uint8_t *pscales, hipStream_t stream);

hipError_t launch_dequant(const uint8_t *codes, const uint8_t *scales, int64_t n, float *out,
                          hipStream_t stream);

// Router: split-K partial logits into `partial` (router_partial_floats() floats), then top-k.
// launch_router_partial zeroes *counter too when it is given.
size_t router_partial_floats(int64_t T, int E, int H);
int router_splits(int64_t T, int E, int H);
hipError_t launch_router_partial(const uint16_t *x, int64_t T, int H, const float *w, int E, float *partial,
                                 hipStream_t stream, int *counter = nullptr);
hipError_t launch_router(const uint16_t *x, int64_t T, int H, const float *w, const float *b, int E, int k,
                         float *partial, int32_t *topk_idx, float *topk_w, hipStream_t stream);

// Stable counting sort of the S slots by expert. More than 8192 slots use several workgroups
// and need permute_scratch_ints(S, E) int32 of scratch (else one workgroup sorts them all).
int64_t permute_scratch_ints(int64_t S, int E);
hipError_t launch_permute(const int32_t *topk_idx, int64_t S, int E, int32_t *offsets,
                          int32_t *sorted_slot, int32_t *slot_row, int32_t *scratch, hipStream_t stream);

// Decode-sized batches (topk_permute_fits): the top-k step of launch_router on the partials of
// launch_router_partial (token-major; counter zeroed by that launch), and the permutation of
// launch_permute, in one launch. Same outputs as the two separate steps. Up to 16 tokens one
// workgroup does both (the counter is not used).
bool topk_permute_fits(int64_t T, int E, int k);
hipError_t launch_router_topk_permute(const float *partial, int nsplit, const float *bias, int64_t T, int E, int k,
                                      int32_t *topk_idx, float *topk_w, int *counter, int32_t *offsets,
                                      int32_t *sorted_slot, int32_t *slot_row, hipStream_t stream);


// One expert GEMM over all sorted rows, weight-streaming kernel family.
// a_src: bf16 rows; if a_by_token, sorted row r reads a_src[(sorted_slot[r] / k) * K], else
// a_src[r * K]. Output rows are sorted rows.
hipError_t launch_ffn_stream(const uint16_t *a_src, bool a_by_token, const int32_t *sorted_slot,
                             int k, const int32_t *offsets, int E, int64_t S, const MxWeight &w,
                             int epilogue, void *out, float limit, float alpha, hipStream_t stream);

// One token (ffn_route1_fits: T = 1, tiled weights, k <= 8, E <= 256): the gate_up launch of
// launch_ffn_stream (SwiGLU bf16 epilogue, act rows in sorted order) that also does the top-k of
// launch_router_topk_permute on the router's partials (launch_router_partial, token-major) and
// writes its outputs (topk_idx, topk_w, offsets, sorted_slot, slot_row; a pick without an
// expert gets slot_row -1), so the routing needs no launch of its own. The down launch and the
// combine then run as usual on those outputs.
struct Route1 {
  const float *partial;
  int nsplit;
  const float *bias;
  int32_t *topk_idx;
  float *topk_w;
  int32_t *offsets;
  int32_t *sorted_slot;
  int32_t *slot_row;
};
bool ffn_route1_fits(int64_t T, int E, int k, const MxWeight &w);
hipError_t launch_ffn_stream_route1(const uint16_t *x, int k, int E, const MxWeight &w, void *act, float limit,
                                    float alpha, const Route1 &r1, hipStream_t stream);

// Activation forms of the grouped GEMM's input rows: bf16, or two-term block-scaled records
// (MXFP8 or MXFP6 terms, mx_act.h).
enum ActForm : int { kActBf16 = 0, kActMx8 = 1, kActMx6 = 2 };

// One expert GEMM, persistent LDS-tiled grouped-GEMM family (tiled weights only): the
// activations are expert-sorted rows (r = sorted row), either bf16 a[r * K] (af kActBf16) or
// two-term records with their scale array a_scales (kActMx8, kActMx6; layouts in mx_act.h);
// with a_rows (records only), sorted row r reads record row a_rows[r] / a_div instead (a slot's
// token: a_rows = sorted_slot, a_div = k). Output rows are sorted rows. kEpiMxAct / kEpiMx6Act
// (MXFP8 input only) write MXFP8 / MXFP6 records to out and their scales to out_scales; an
// MXFP6 input takes the linear epilogue only (the down projection). E at most 256.
hipError_t launch_ffn_gemm(const void *a, const uint8_t *a_scales, const int32_t *a_rows, int a_div, int af,
                           const int32_t *offsets, int E, int64_t S, const MxWeight &w, int epilogue, void *out,
                           uint8_t *out_scales, float limit, float alpha, hipStream_t stream);

// Smallest decode batches (T <= kSmallMaxT, H <= 3072, I <= 32 kSmallMaxSlices, tiled weights):
// gate_up, SwiGLU and the down projection in one launch (ffn_small.hip), one workgroup per
// (expert, 32-activation block). Writes per-block partial outputs part[block][sorted row][H]
// (small_partial_floats floats; b2 in block 0); the combine adds the blocks in order. Every
// expert must hold at most kSmallMaxT slots (top-k routing picks distinct experts per token,
// so T <= kSmallMaxT does). One token only: the kernel's VALU products grow with the slots.
// Opt-in (MOE_PATH_DECODE_FUSED): the two-kernel form is faster on this part even at one token.
constexpr int kSmallMaxT = 1;
constexpr int kSmallMaxSlices = 128;  // the sliced combine's limit
bool small_ffn_fits(int64_t T, int H, int I);
int small_slices(int I);
size_t small_partial_floats(int64_t T, int k, int H, int I);
hipError_t launch_ffn_small(const uint16_t *x, const int32_t *sorted_slot, int k, const int32_t *offsets, int E,
                            int64_t S, const MxWeight &w1, const MxWeight &w2, float *part, float limit, float alpha,
                            hipStream_t stream);
// y[r][h] = the sum over s = 0 .. nslice-1 of part[s][r][h] (S rows of H), in the fixed order of
// launch_combine_sliced.
hipError_t launch_slice_sum(const float *part, int nslice, int64_t S, int H, float *y, hipStream_t stream);

// xs[r] = x[sorted_slot[r] / k] for every sorted row r (rows of H bf16).
hipError_t launch_gather_rows(const uint16_t *x, const int32_t *sorted_slot, int k, int64_t S, int H,
                              uint16_t *xs, hipStream_t stream);

// The same gather, written as two-term MXFP8 records (mx_act.h): rec [S][ceil(H/128)][256],
// scales [S][ceil(H/128)][8]. With sorted_slot null, row r is x's row r (records per token).
hipError_t launch_gather_rows_mx(const uint16_t *x, const int32_t *sorted_slot, int k, int64_t S, int H,
                                 uint8_t *rec, uint8_t *scales, hipStream_t stream);

// The fixed device array behind moe_forward_noalloc (noalloc.hip): its size, and this device's
// address of it (looked up once per device, then kept).
size_t scratch_bytes();
hipError_t scratch_address(void **ptr);

// residual (bf16 [T][H], nullable) is added to the weighted sum before the rounding.
// by_slot: y's rows are in slot order (y[t * k + j], kEpiLinearSlotF32), so no row is looked up
// before its load; slot_row still marks the picks that have a row.
hipError_t launch_combine(const float *y, const int32_t *slot_row, const float *topk_w, int64_t T,
                          int k, int H, void *out, bool out_f32, hipStream_t stream,
                          const uint16_t *residual = nullptr, bool by_slot = false);
// The same combine when each picked expert's output row is the sum of nslice partial rows
// (part + s * S * H, s = 0 .. nslice-1; the smallest-batch path), summed in the fixed order that
// launch_slice_sum uses. nslice <= kSmallMaxSlices.
hipError_t launch_combine_sliced(const float *part, int nslice, const int32_t *slot_row, const float *topk_w,
                                 int64_t T, int k, int H, void *out, bool out_f32, hipStream_t stream,
                                 const uint16_t *residual);

// xn = bf16(x / sqrt(mean(x^2) + eps) * scale) per row of H; with rec non-null also the rows'
// two-term MXFP8 records and scales (as launch_gather_rows_mx with sorted_slot null, of xn).
// scale: fp32 [H], 16-byte aligned.
hipError_t launch_rmsnorm(const uint16_t *x, int64_t T, int H, const float *scale, float eps, uint16_t *xn,
                          uint8_t *rec, uint8_t *rec_scales, hipStream_t stream);

// One decode step of grouped-query attention with per-head sinks (attn.hip). q [B][Hq][64],
// kc / vc [B][Hkv][L][64] bf16, lens [B], sinks [Hq] fp32 or null, window 0 = dense; out
// [B][Hq][64] bf16 or fp32; ws: attn_partial_floats(B, Hkv, L, window) floats. Hq / Hkv <= 16.
int attn_splits(int64_t L, int window);
size_t attn_partial_floats(int64_t B, int Hkv, int64_t L, int window);
hipError_t launch_attn_decode(const uint16_t *q, const uint16_t *kc, const uint16_t *vc, const int32_t *lens,
                              const float *sinks, int64_t B, int Hq, int Hkv, int64_t L, int window, void *out,
                              bool out_f32, float *ws, hipStream_t stream);

}  // namespace moe
