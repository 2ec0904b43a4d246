// extern "C" entry points of the MXFP4 top-k MoE layer: argument checks (all before the first
// HIP call), workspace layout, kernel-family choice, and launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <new>
#include <map>
#include <utility>

#include "kernels.h"
#include "moe_mxfp4.h"
#include "mx_act.h"

namespace {

constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 256;
constexpr int kMaxDim = 16384;
constexpr size_t kWsAlign = 256;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t align_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

// One workspace layout serves every entry point (each uses a subset of the regions).
struct WsLayout {
  size_t logits, topk_idx, topk_w, offsets, counter, sorted_slot, slot_row, act, y, xs, xn, pscratch, ypart, total;
};

// Bytes of S activation rows of K elements: bf16, or the two-term records and their scales
// (mx_act.h), whichever is larger; the records come first, their scales after S records.
size_t act_rows_bytes(size_t S, int K) {
  const size_t bf16 = S * (size_t)K * sizeof(uint16_t);
  const size_t mx = S * (size_t)moe::mx_records(K) * (moe::kMxRecBytes + moe::kMxScBytes);
  return bf16 > mx ? bf16 : mx;
}
size_t mx_scales_offset(size_t S, int K) { return S * (size_t)moe::mx_records(K) * moe::kMxRecBytes; }

bool ws_layout(int64_t T, int E, int k, int H, int I, WsLayout *L) {
  if (T < 0 || E < 1 || k < 1 || H < 1 || I < 1) return false;
  const size_t S = (size_t)T * (size_t)k;
  size_t off = 0;
  L->logits = off;      off = align_up(off + moe::router_partial_floats(T, E, H) * sizeof(float));
  L->topk_idx = off;    off = align_up(off + S * sizeof(int32_t));
  L->topk_w = off;      off = align_up(off + S * sizeof(float));
  L->offsets = off;     off = align_up(off + (size_t)(E + 1) * sizeof(int32_t));
  L->counter = off;     off = align_up(off + sizeof(int32_t));
  L->sorted_slot = off; off = align_up(off + S * sizeof(int32_t));
  L->slot_row = off;    off = align_up(off + S * sizeof(int32_t));
  L->act = off;         off = align_up(off + act_rows_bytes(S, I));
  L->y = off;           off = align_up(off + S * (size_t)H * sizeof(float));
  L->xs = off;          off = align_up(off + act_rows_bytes(S, H));  // sorted x (GEMM paths)
  L->xn = off;          off = align_up(off + (size_t)T * (size_t)H * sizeof(uint16_t));  // normalised x (block)
  L->pscratch = off;    off = align_up(off + (size_t)moe::permute_scratch_ints((int64_t)S, E) * sizeof(int32_t));
  L->ypart = off;       off = align_up(off + moe::small_partial_floats(T, k, H, I) * sizeof(float));  // smallest batches
  L->total = off;
  return true;
}

template <typename P>
P *at(void *base, size_t off) {
  return reinterpret_cast<P *>(static_cast<char *>(base) + off);
}

int check_common(int64_t T, int E, int k) {
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (k < 1 || k > kMaxTopK || E < k || E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (T * (int64_t)k >= ((int64_t)1 << 31))) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_dim(int64_t d) { return (d >= 32 && d <= kMaxDim && d % 32 == 0) ? MOE_OK : MOE_ERR_UNSUPPORTED; }

int check_weight(const moe_mxfp4_weight_t *w) {
  if (w == nullptr || w->codes == nullptr || w->scales == nullptr) return MOE_ERR_INVALID_ARG;
  if (w->layout != MOE_LAYOUT_ROWMAJOR && w->layout != MOE_LAYOUT_TILED) return MOE_ERR_INVALID_ARG;
  if (!aligned(w->codes, 16) || !aligned(w->bias, 2)) return MOE_ERR_INVALID_ARG;
  if (w->layout == MOE_LAYOUT_TILED && (!aligned(w->scales, 4) || !aligned(w->bias, 8))) return MOE_ERR_INVALID_ARG;
  if (check_dim(w->k) != MOE_OK || w->n < 1 || w->n > 2 * kMaxDim) return MOE_ERR_UNSUPPORTED;
  if (w->layout == MOE_LAYOUT_TILED && w->n % 32 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe::MxWeight mx(const moe_mxfp4_weight_t &w) {
  return moe::MxWeight{w.codes, w.scales, w.bias, w.n, w.k, w.layout == MOE_LAYOUT_TILED};
}

moe_options_t default_options() {
  moe_options_t o;
  o.swiglu_limit = 7.0f;
  o.swiglu_alpha = 1.0f;
  o.out_dtype = MOE_DTYPE_BF16;
  o.path = MOE_PATH_AUTO;
  o.flags = 0;
  return o;
}

int check_options(const moe_options_t &o) {
  if (o.out_dtype != MOE_DTYPE_BF16 && o.out_dtype != MOE_DTYPE_F32) return MOE_ERR_INVALID_ARG;
  if (o.path < MOE_PATH_AUTO || o.path > MOE_PATH_DECODE_FUSED) return MOE_ERR_INVALID_ARG;
  if (!(o.swiglu_limit > 0.0f) || !(o.swiglu_alpha == o.swiglu_alpha)) return MOE_ERR_INVALID_ARG;
  if (o.flags & ~(MOE_FLAG_EMIT_PREACT | MOE_FLAG_EMIT_ACT)) return MOE_ERR_INVALID_ARG;
  if ((o.flags & MOE_FLAG_EMIT_PREACT) && (o.flags & MOE_FLAG_EMIT_ACT)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Which expert-GEMM family runs: a grouped GEMM (tiled weights only) when asked for, or on
// AUTO when the batch averages at least kGemmSlotsPerExpert slots per expert; otherwise the
// weight-streaming kernels. AUTO's grouped GEMM takes the exact two-term MXFP8 activation for
// gate_up, and for down the two-term MXFP6 one from kMx6MinI activations on: its error (below
// 2^-9 of each 32-element block's maximum, the order of the activation's own bf16 rounding)
// averages over many blocks there (measured max |err| / RMS against the fp64 layer: 7.7e-3
// against 6.4e-3 at 4096 tokens of the 2880-wide layer, 1.1e-2 against 9.5e-3 at I = 1024,
// under the 2e-2 bar; three blocks, I = 96, reach 2.04e-2), and the down GEMM runs ~12% faster
// (FFN 703 against 742 us at 4096 tokens, 1536 against 1603 us at 8192 x 128 experts).
// Measured crossover (FFN time, stream vs block-scaled GEMM): E = 32 at 24 slots per expert
// 105 vs 142 us, at 32: 150 vs 145 us; E = 128 at 16: 354 vs 467 us, at 32: 544 vs 485 us.
constexpr int64_t kGemmSlotsPerExpert = 32;
constexpr int kMx6MinI = 1024;

enum class Family { kStream, kGemm, kGemmMx, kGemmMx6 };

bool is_gemm_path(int path) {
  return path == MOE_PATH_PREFILL_BF16 || path == MOE_PATH_PREFILL_MX8SPLIT || path == MOE_PATH_PREFILL_MX6SPLIT;
}
bool needs_tiled(int path) { return is_gemm_path(path) || path == MOE_PATH_DECODE_FUSED; }

int check_path(const moe_options_t &o, const moe_mxfp4_weight_t &gu, const moe_mxfp4_weight_t &dn) {
  if (needs_tiled(o.path) && (gu.layout != MOE_LAYOUT_TILED || dn.layout != MOE_LAYOUT_TILED))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

Family family(const moe_options_t &o, const moe_mxfp4_weight_t &gu, const moe_mxfp4_weight_t &dn, int64_t S,
              int E) {
  const bool tiled = gu.layout == MOE_LAYOUT_TILED && dn.layout == MOE_LAYOUT_TILED;
  if (o.path == MOE_PATH_PREFILL_BF16) return Family::kGemm;
  if (o.path == MOE_PATH_PREFILL_MX8SPLIT) return Family::kGemmMx;
  if (o.path == MOE_PATH_PREFILL_MX6SPLIT) return Family::kGemmMx6;
  if (o.path == MOE_PATH_DECODE || o.path == MOE_PATH_DECODE_FUSED || !tiled || S < kGemmSlotsPerExpert * (int64_t)E)
    return Family::kStream;
  return dn.k >= kMx6MinI ? Family::kGemmMx6 : Family::kGemmMx;
}

// The expert GEMMs that follow the permutation. Arguments already validated. The GEMM
// families read their gate_up activations from an expert-sorted copy of x in the xs region
// (S x H bf16, or two-term records); the act region holds the activation between the
// projections (bf16 or two-term records).
// x_records_ready: the block-scaled families' per-token MXFP8 records of x are already in xs
// (the block's normalisation writes them), so the gather is skipped.
// part / nslice_out: on MOE_PATH_DECODE_FUSED with tiled weights and the smallest batches
// (small_ffn_fits; the routing picks distinct experts per token, so an expert holds at most T
// slots), the expert FFNs run as one launch (launch_ffn_small) writing per-block partial rows
// into part; then *nslice_out = the block count (1 or more), and y is written (the blocks'
// in-order sum) only if want_y. Otherwise y is written and *nslice_out = 0.
// y_slot: non-null when the caller takes y in slot order (row t * k + j, for launch_combine's
// by_slot form); *y_slot then says whether y was written that way (the weight-streaming family
// with tiled down weights) or in sorted order.
int run_ffn(const uint16_t *x, int64_t T, int k, int E, const int32_t *offsets, const int32_t *sorted_slot,
            const moe_mxfp4_weight_t &gu, const moe_mxfp4_weight_t &dn, const moe_options_t &o, float *y,
            void *act, void *xs, float *part, bool want_y, int *nslice_out, hipStream_t stream,
            bool x_records_ready = false, bool *y_slot = nullptr) {
  if (y_slot != nullptr) *y_slot = false;
  const int64_t S = T * k;
  const int H = gu.k, I = dn.k;
  const moe::MxWeight w1 = mx(gu);
  const moe::MxWeight w2 = mx(dn);
  const Family f = family(o, gu, dn, S, E);
  const float lim = o.swiglu_limit, alpha = o.swiglu_alpha;
  const int first_epi = (o.flags & MOE_FLAG_EMIT_PREACT) ? moe::kEpiPreactF32
                        : (o.flags & MOE_FLAG_EMIT_ACT)  ? moe::kEpiActF32
                                                         : -1;
  *nslice_out = 0;
  if (f == Family::kStream && o.path == MOE_PATH_DECODE_FUSED && first_epi < 0 && w1.tiled && w2.tiled &&
      moe::small_ffn_fits(T, H, I)) {
    if (moe::launch_ffn_small(x, sorted_slot, k, offsets, E, S, w1, w2, part, lim, alpha, stream) != hipSuccess)
      return MOE_ERR_HIP;
    *nslice_out = moe::small_slices(I);
    if (want_y && moe::launch_slice_sum(part, *nslice_out, S, H, y, stream) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
  }
  if (f == Family::kStream) {
    auto launch = [&](const uint16_t *a, bool by_token, const moe::MxWeight &w, int epi, void *out) {
      return moe::launch_ffn_stream(a, by_token, sorted_slot, k, offsets, E, S, w, epi, out, lim, alpha, stream);
    };
    if (first_epi >= 0) return launch(x, true, w1, first_epi, y) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    if (launch(x, true, w1, moe::kEpiSwigluBf16, act) != hipSuccess) return MOE_ERR_HIP;
    const bool slot = y_slot != nullptr && w2.tiled;
    if (launch(static_cast<uint16_t *>(act), false, w2, slot ? moe::kEpiLinearSlotF32 : moe::kEpiLinearF32, y) !=
        hipSuccess)
      return MOE_ERR_HIP;
    if (slot) *y_slot = true;
    return MOE_OK;
  }
  // block-scaled families: x's T rows become exact two-term MXFP8 records once, and gate_up reads
  // each sorted row's token record (a_rows = sorted_slot, a_div = k); its epilogue writes the
  // activation as MXFP8 records, or as MXFP6 records for the MXFP6 down GEMM. bf16: an
  // expert-sorted copy of x. (The scale arrays sit at the same offset for both record forms:
  // the regions are sized for the larger MXFP8 records.)
  const bool mxp = f == Family::kGemmMx || f == Family::kGemmMx6;
  const int af_x = mxp ? moe::kActMx8 : moe::kActBf16;
  const int af_act = f == Family::kGemmMx6 ? moe::kActMx6 : af_x;
  const int epi_act = f == Family::kGemmMx6 ? moe::kEpiMx6Act : mxp ? moe::kEpiMxAct : moe::kEpiSwigluBf16;
  uint8_t *xs_sc = mxp ? static_cast<uint8_t *>(xs) + mx_scales_offset((size_t)S, H) : nullptr;
  uint8_t *act_sc = mxp ? static_cast<uint8_t *>(act) + mx_scales_offset((size_t)S, I) : nullptr;
  const hipError_t g =
      mxp ? (x_records_ready ? hipSuccess
                             : moe::launch_gather_rows_mx(x, nullptr, 1, T, H, static_cast<uint8_t *>(xs), xs_sc, stream))
          : moe::launch_gather_rows(x, sorted_slot, k, S, H, static_cast<uint16_t *>(xs), stream);
  if (g != hipSuccess) return MOE_ERR_HIP;
  const int32_t *rows = mxp ? sorted_slot : nullptr;
  if (first_epi >= 0)
    return moe::launch_ffn_gemm(xs, xs_sc, rows, k, af_x, offsets, E, S, w1, first_epi, y, nullptr, lim, alpha,
                                stream) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
  if (moe::launch_ffn_gemm(xs, xs_sc, rows, k, af_x, offsets, E, S, w1, epi_act, act, act_sc, lim, alpha, stream) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return moe::launch_ffn_gemm(act, act_sc, nullptr, 1, af_act, offsets, E, S, w2, moe::kEpiLinearF32, y, nullptr,
                              lim, alpha, stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

int check_layer(const uint16_t *x, const moe_router_t *router, const moe_mxfp4_weight_t *gu,
                const moe_mxfp4_weight_t *dn, int64_t T, int E, int k, const void *out) {
  int st = check_common(T, E, k);
  if (st != MOE_OK) return st;
  if (router == nullptr || gu == nullptr || dn == nullptr) return MOE_ERR_INVALID_ARG;
  if ((st = check_weight(gu)) != MOE_OK || (st = check_weight(dn)) != MOE_OK) return st;
  const int H = gu->k, I = dn->k;
  if (gu->n != 2 * I || dn->n != H) return MOE_ERR_UNSUPPORTED;
  if ((st = check_dim(H)) != MOE_OK || (st = check_dim(I)) != MOE_OK) return st;
  if (T > 0) {
    if (x == nullptr || out == nullptr || router->weight == nullptr) return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(router->weight, 16))
      return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

// The layer; with norm_scale non-null, the block around it: the layer runs on
// xn = bf16(RMSNorm(x)) and x is added to its output.
int forward_impl(const uint16_t *x, const moe_router_t *router, const moe_mxfp4_weight_t *gu,
                 const moe_mxfp4_weight_t *dn, int64_t T, int E, int k, const moe_options_t &o, void *out,
                 void *ws, size_t ws_bytes, hipStream_t stream, const float *norm_scale = nullptr,
                 float norm_eps = 0.0f) {
  const int H = gu->k, I = dn->k;
  WsLayout L;
  ws_layout(T, E, k, H, I, &L);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, kWsAlign)) return MOE_ERR_INVALID_ARG;
  const int64_t S = T * k;
  const uint16_t *residual = nullptr;
  bool records_ready = false;
  if (norm_scale != nullptr) {
    // the block-scaled families read x as per-token records: the normalisation writes them
    const Family f = family(o, *gu, *dn, S, E);
    const bool mxp = f == Family::kGemmMx || f == Family::kGemmMx6;
    uint8_t *xs = at<uint8_t>(ws, L.xs);
    uint16_t *xn = at<uint16_t>(ws, L.xn);
    if (moe::launch_rmsnorm(x, T, H, norm_scale, norm_eps, xn, mxp ? xs : nullptr,
                            mxp ? xs + mx_scales_offset((size_t)S, H) : nullptr, stream) != hipSuccess)
      return MOE_ERR_HIP;
    residual = x;
    x = xn;
    records_ready = mxp;
  }
  float *logits = at<float>(ws, L.logits);
  int32_t *idx = at<int32_t>(ws, L.topk_idx);
  float *wts = at<float>(ws, L.topk_w);
  int32_t *offsets = at<int32_t>(ws, L.offsets);
  int32_t *sorted_slot = at<int32_t>(ws, L.sorted_slot);
  int32_t *slot_row = at<int32_t>(ws, L.slot_row);
  void *act = at<void>(ws, L.act);
  float *y = at<float>(ws, L.y);
  const moe::MxWeight w1 = mx(*gu);
  if (o.path != MOE_PATH_DECODE_FUSED && o.flags == 0 && family(o, *gu, *dn, S, E) == Family::kStream &&
      moe::ffn_route1_fits(T, E, k, w1)) {
    // one token: the top-k and the permutation of its k slots run inside the gate_up launch
    const moe::Route1 r1{logits, moe::router_splits(T, E, H), router->bias, idx, wts, offsets, sorted_slot, slot_row};
    const moe::MxWeight w2 = mx(*dn);
    if (moe::launch_router_partial(x, T, H, router->weight, E, logits, stream) != hipSuccess ||
        moe::launch_ffn_stream_route1(x, k, E, w1, act, o.swiglu_limit, o.swiglu_alpha, r1, stream) != hipSuccess ||
        moe::launch_ffn_stream(static_cast<uint16_t *>(act), false, sorted_slot, k, offsets, E, S, w2,
                               w2.tiled ? moe::kEpiLinearSlotF32 : moe::kEpiLinearF32, y, o.swiglu_limit,
                               o.swiglu_alpha, stream) != hipSuccess ||
        moe::launch_combine(y, slot_row, wts, T, k, H, out, o.out_dtype == MOE_DTYPE_F32, stream, residual,
                            w2.tiled) != hipSuccess)
      return MOE_ERR_HIP;
    return MOE_OK;
  }
  if (moe::topk_permute_fits(T, E, k)) {  // decode batches: top-k and permutation in one launch
    int *counter = at<int>(ws, L.counter);
    if (moe::launch_router_partial(x, T, H, router->weight, E, logits, stream, counter) != hipSuccess ||
        moe::launch_router_topk_permute(logits, moe::router_splits(T, E, H), router->bias, T, E, k, idx, wts,
                                        counter, offsets, sorted_slot, slot_row, stream) != hipSuccess)
      return MOE_ERR_HIP;
  } else {
    if (moe::launch_router(x, T, H, router->weight, router->bias, E, k, logits, idx, wts, stream) != hipSuccess)
      return MOE_ERR_HIP;
    if (moe::launch_permute(idx, S, E, offsets, sorted_slot, slot_row, at<int32_t>(ws, L.pscratch), stream) !=
        hipSuccess)
      return MOE_ERR_HIP;
  }
  int nslice = 0;
  float *part = at<float>(ws, L.ypart);
  bool y_slot = false;
  int st = run_ffn(x, T, k, E, offsets, sorted_slot, *gu, *dn, o, y, act, at<void>(ws, L.xs), part, false, &nslice,
                   stream, records_ready, &y_slot);
  if (st != MOE_OK) return st;
  // the experts' outputs: y, or the per-slice partial rows of the smallest-batch path
  const hipError_t ce =
      nslice > 0 ? moe::launch_combine_sliced(part, nslice, slot_row, wts, T, k, H, out, o.out_dtype == MOE_DTYPE_F32,
                                              stream, residual)
                 : moe::launch_combine(y, slot_row, wts, T, k, H, out, o.out_dtype == MOE_DTYPE_F32, stream, residual,
                                       y_slot);
  if (ce != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

struct OwnedWorkspace {
  void *ptr = nullptr;
  size_t bytes = 0;
};
// moe_forward's workspaces, one per (device, stream): calls on different streams never share
// one, so they do not race; calls on one stream are ordered by the stream itself.
std::mutex g_ws_mutex;
std::map<std::pair<int, uintptr_t>, OwnedWorkspace> g_ws;

}  // namespace

#define MOE_GUARD_BEGIN try {
#define MOE_GUARD_END                   \
  }                                     \
  catch (const std::bad_alloc &) {      \
    return MOE_ERR_HIP;                 \
  }                                     \
  catch (...) {                         \
    return MOE_ERR_HIP;                 \
  }

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument (null, negative, misaligned or bad enum)";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape (k, E, H, I or T*k outside the limits)";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime or kernel launch error";
    case MOE_ERR_SCRATCH: return "the call needs more workspace than moe_forward_noalloc's fixed scratch holds";
    default: return "unknown status";
  }
}

size_t moe_workspace_size(int64_t T, int32_t E, int32_t k, int32_t H, int32_t I, int32_t path) {
  if (path < MOE_PATH_AUTO || path > MOE_PATH_DECODE_FUSED) return 0;
  if (check_common(T, E, k) != MOE_OK || check_dim(H) != MOE_OK || check_dim(I) != MOE_OK) return 0;
  WsLayout L;
  if (!ws_layout(T, E, k, H, I, &L)) return 0;
  return L.total;
}

int moe_mxfp4_tiled_bytes(int32_t E, int32_t n, int32_t k, size_t *codes_bytes, size_t *scales_bytes) {
  MOE_GUARD_BEGIN
  if (E < 1 || E > kMaxExperts || n < 32 || n % 32 != 0 || n > 2 * kMaxDim || check_dim(k) != MOE_OK)
    return MOE_ERR_UNSUPPORTED;
  const size_t tiles = (size_t)E * (size_t)(n / 32) * (size_t)((k / 32 + 3) / 4);
  if (codes_bytes) *codes_bytes = tiles * 2048;
  if (scales_bytes) *scales_bytes = tiles * 128;
  return MOE_OK;
  MOE_GUARD_END
}

int moe_mxfp4_pack(const moe_mxfp4_weight_t *src, int32_t E, uint8_t *codes_out, uint8_t *scales_out,
                   moe_stream_t stream) {
  MOE_GUARD_BEGIN
  if (src == nullptr || codes_out == nullptr || scales_out == nullptr) return MOE_ERR_INVALID_ARG;
  if (src->layout != MOE_LAYOUT_ROWMAJOR) return MOE_ERR_INVALID_ARG;
  int st = check_weight(src);
  if (st != MOE_OK) return st;
  size_t cb = 0, sb = 0;
  if ((st = moe_mxfp4_tiled_bytes(E, src->n, src->k, &cb, &sb)) != MOE_OK) return st;
  if (!aligned(codes_out, 16) || !aligned(scales_out, 16)) return MOE_ERR_INVALID_ARG;
  return moe::launch_pack(src->codes, src->scales, E, src->n, src->k, codes_out, scales_out,
                          (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
  MOE_GUARD_END
}

int moe_mxfp4_dequant(const uint8_t *codes, const uint8_t *scales, int64_t n, float *out,
                      moe_stream_t stream) {
  MOE_GUARD_BEGIN
  if (n < 0 || n % 32 != 0) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (codes == nullptr || scales == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(codes, 16) || !aligned(out, 16)) return MOE_ERR_INVALID_ARG;
  return moe::launch_dequant(codes, scales, n, out, (hipStream_t)stream) == hipSuccess ? MOE_OK
                                                                                        : MOE_ERR_HIP;
  MOE_GUARD_END
}

int moe_route(const uint16_t *x, int64_t T, int32_t H, const moe_router_t *router, int32_t E,
              int32_t k, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
              moe_stream_t stream) {
  MOE_GUARD_BEGIN
  int st = check_common(T, E, k);
  if (st != MOE_OK) return st;
  if (router == nullptr) return MOE_ERR_INVALID_ARG;
  if ((st = check_dim(H)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (x == nullptr || router->weight == nullptr || topk_idx == nullptr || topk_w == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(router->weight, 16)) return MOE_ERR_INVALID_ARG;
  WsLayout L;
  ws_layout(T, E, k, H, H, &L);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, kWsAlign)) return MOE_ERR_INVALID_ARG;
  float *logits = at<float>(ws, L.logits);
  return moe::launch_router(x, T, H, router->weight, router->bias, E, k, logits, topk_idx, topk_w,
                            (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
  MOE_GUARD_END
}

int moe_permute(const int32_t *topk_idx, int64_t T, int32_t E, int32_t k, int32_t *expert_offsets,
                int32_t *sorted_slot, int32_t *slot_row, void *ws, size_t ws_bytes,
                moe_stream_t stream) {
  MOE_GUARD_BEGIN
  int st = check_common(T, E, k);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (topk_idx == nullptr || expert_offsets == nullptr || sorted_slot == nullptr || slot_row == nullptr)
    return MOE_ERR_INVALID_ARG;
  // the multi-workgroup sort keeps its per-range counts at the start of the workspace (this
  // call uses no other region); without a large enough workspace one workgroup sorts
  int32_t *scratch = nullptr;
  if (ws != nullptr) {
    if (!aligned(ws, kWsAlign)) return MOE_ERR_INVALID_ARG;
    const size_t need = (size_t)moe::permute_scratch_ints(T * k, E) * sizeof(int32_t);
    if (need > 0 && ws_bytes >= need) scratch = static_cast<int32_t *>(ws);
  }
  return moe::launch_permute(topk_idx, T * k, E, expert_offsets, sorted_slot, slot_row, scratch,
                             (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
  MOE_GUARD_END
}

int moe_mxfp4_ffn(const uint16_t *x, int64_t T, int32_t k, int32_t E, const int32_t *expert_offsets,
                  const int32_t *sorted_slot, const moe_mxfp4_weight_t *gate_up,
                  const moe_mxfp4_weight_t *down, const moe_options_t *opts, float *y, void *ws,
                  size_t ws_bytes, moe_stream_t stream) {
  MOE_GUARD_BEGIN
  int st = check_common(T, E, k);
  if (st != MOE_OK) return st;
  if (gate_up == nullptr || down == nullptr) return MOE_ERR_INVALID_ARG;
  if ((st = check_weight(gate_up)) != MOE_OK || (st = check_weight(down)) != MOE_OK) return st;
  const int H = gate_up->k, I = down->k;
  if (gate_up->n != 2 * I || down->n != H) return MOE_ERR_UNSUPPORTED;
  if ((st = check_dim(H)) != MOE_OK || (st = check_dim(I)) != MOE_OK) return st;
  const moe_options_t o = opts ? *opts : default_options();
  if ((st = check_options(o)) != MOE_OK) return st;
  if ((st = check_path(o, *gate_up, *down)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (x == nullptr || expert_offsets == nullptr || sorted_slot == nullptr || y == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
  WsLayout L;
  ws_layout(T, E, k, H, I, &L);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, kWsAlign)) return MOE_ERR_INVALID_ARG;
  int nslice = 0;
  return run_ffn(x, T, k, E, expert_offsets, sorted_slot, *gate_up, *down, o, y, at<void>(ws, L.act),
                 at<void>(ws, L.xs), at<float>(ws, L.ypart), true, &nslice, (hipStream_t)stream);
  MOE_GUARD_END
}

int moe_combine(const float *y, const int32_t *slot_row, const float *topk_w, int64_t T, int32_t k,
                int32_t H, void *out, int32_t out_dtype, moe_stream_t stream) {
  MOE_GUARD_BEGIN
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (k < 1 || k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  int st = check_dim(H);
  if (st != MOE_OK) return st;
  if (out_dtype != MOE_DTYPE_BF16 && out_dtype != MOE_DTYPE_F32) return MOE_ERR_INVALID_ARG;
  if (T * (int64_t)k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (y == nullptr || slot_row == nullptr || topk_w == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(out, 16)) return MOE_ERR_INVALID_ARG;
  return moe::launch_combine(y, slot_row, topk_w, T, k, H, out, out_dtype == MOE_DTYPE_F32,
                             (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
  MOE_GUARD_END
}

int moe_forward_ex(const uint16_t *x, const moe_router_t *router,
                   const moe_mxfp4_weight_t *w_gate_up, const moe_mxfp4_weight_t *w_down,
                   int64_t T, int32_t E, int32_t k, const moe_options_t *opts, void *out, void *ws,
                   size_t ws_bytes, moe_stream_t stream) {
  MOE_GUARD_BEGIN
  int st = check_layer(x, router, w_gate_up, w_down, T, E, k, out);
  if (st != MOE_OK) return st;
  const moe_options_t o = opts ? *opts : default_options();
  if ((st = check_options(o)) != MOE_OK) return st;
  if (o.flags != 0) return MOE_ERR_INVALID_ARG;
  if ((st = check_path(o, *w_gate_up, *w_down)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  return forward_impl(x, router, w_gate_up, w_down, T, E, k, o, out, ws, ws_bytes, (hipStream_t)stream);
  MOE_GUARD_END
}

int moe_rmsnorm(const uint16_t *x, int64_t T, int32_t H, const float *scale, float eps, uint16_t *out,
                moe_stream_t stream) {
  MOE_GUARD_BEGIN
  if (T < 0 || !(eps >= 0.0f) || !std::isfinite(eps)) return MOE_ERR_INVALID_ARG;
  int st = check_dim(H);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (x == nullptr || scale == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(scale, 16) || !aligned(out, 16)) return MOE_ERR_INVALID_ARG;
  return moe::launch_rmsnorm(x, T, H, scale, eps, out, nullptr, nullptr, (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
  MOE_GUARD_END
}

int moe_block_forward_ex(const uint16_t *x, const float *norm_scale, float norm_eps, const moe_router_t *router,
                         const moe_mxfp4_weight_t *w_gate_up, const moe_mxfp4_weight_t *w_down, int64_t T,
                         int32_t E, int32_t k, const moe_options_t *opts, void *out, void *ws, size_t ws_bytes,
                         moe_stream_t stream) {
  MOE_GUARD_BEGIN
  int st = check_layer(x, router, w_gate_up, w_down, T, E, k, out);
  if (st != MOE_OK) return st;
  const moe_options_t o = opts ? *opts : default_options();
  if ((st = check_options(o)) != MOE_OK) return st;
  if (o.flags != 0) return MOE_ERR_INVALID_ARG;
  if ((st = check_path(o, *w_gate_up, *w_down)) != MOE_OK) return st;
  if (!(norm_eps >= 0.0f) || !std::isfinite(norm_eps)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (norm_scale == nullptr || !aligned(norm_scale, 16)) return MOE_ERR_INVALID_ARG;
  return forward_impl(x, router, w_gate_up, w_down, T, E, k, o, out, ws, ws_bytes, (hipStream_t)stream,
                      norm_scale, norm_eps);
  MOE_GUARD_END
}

size_t moe_attn_workspace_size(int64_t B, int32_t n_kv_heads, int64_t max_len, int32_t window) {
  if (B < 0 || n_kv_heads < 1 || max_len < 1 || window < 0) return 0;
  return moe::attn_partial_floats(B, n_kv_heads, max_len, window) * sizeof(float);
}

int moe_attn_decode(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache, const int32_t *lens,
                    const float *sinks, int64_t B, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                    int64_t max_len, int32_t window, void *out, int32_t out_dtype, void *ws, size_t ws_bytes,
                    moe_stream_t stream) {
  MOE_GUARD_BEGIN
  if (B < 0 || n_kv_heads < 1 || n_q_heads < 1 || max_len < 1 || window < 0) return MOE_ERR_INVALID_ARG;
  if (out_dtype != MOE_DTYPE_BF16 && out_dtype != MOE_DTYPE_F32) return MOE_ERR_INVALID_ARG;
  if (head_dim != 64 || n_q_heads % n_kv_heads != 0 || n_q_heads / n_kv_heads > 16) return MOE_ERR_UNSUPPORTED;
  if (B > 65535 || n_kv_heads > 65535 || max_len > ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (B == 0) return MOE_OK;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || lens == nullptr || out == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) || !aligned(lens, 4) ||
      !aligned(sinks, 4))
    return MOE_ERR_INVALID_ARG;
  const size_t need = moe::attn_partial_floats(B, n_kv_heads, max_len, window) * sizeof(float);
  if (ws == nullptr || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, kWsAlign)) return MOE_ERR_INVALID_ARG;
  return moe::launch_attn_decode(q, k_cache, v_cache, lens, sinks, B, n_q_heads, n_kv_heads, max_len, window, out,
                                 out_dtype == MOE_DTYPE_F32, static_cast<float *>(ws), (hipStream_t)stream) ==
                 hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
  MOE_GUARD_END
}

int moe_forward(const uint16_t *x, const moe_router_t *router, const moe_mxfp4_weight_t *w_gate_up,
                const moe_mxfp4_weight_t *w_down, int64_t T, int32_t E, int32_t k, uint16_t *out,
                moe_stream_t stream) {
  MOE_GUARD_BEGIN
  int st = check_layer(x, router, w_gate_up, w_down, T, E, k, out);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  WsLayout L;
  ws_layout(T, E, k, w_gate_up->k, w_down->k, &L);
  hipStream_t s = (hipStream_t)stream;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  void *ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    OwnedWorkspace &w = g_ws[{dev, reinterpret_cast<uintptr_t>(s)}];
    if (w.bytes < L.total) {
      // stream-ordered: the old buffer is released after the work already queued on s, the new
      // one is ready for the work queued next; no host synchronisation
      if (w.ptr != nullptr) {
        if (hipFreeAsync(w.ptr, s) != hipSuccess) return MOE_ERR_HIP;
        w.ptr = nullptr;
        w.bytes = 0;
      }
      if (hipMallocAsync(&w.ptr, L.total, s) != hipSuccess) {
        w.ptr = nullptr;
        return MOE_ERR_HIP;
      }
      w.bytes = L.total;
    }
    ws = w.ptr;
  }
  const moe_options_t o = default_options();
  return forward_impl(x, router, w_gate_up, w_down, T, E, k, o, out, ws, L.total, s);
  MOE_GUARD_END
}

int moe_forward_noalloc(const uint16_t *x, const moe_router_t *router, const moe_mxfp4_weight_t *w_gate_up,
                        const moe_mxfp4_weight_t *w_down, int64_t T, int32_t E, int32_t k, uint16_t *out,
                        moe_stream_t stream) {
  MOE_GUARD_BEGIN
  int st = check_layer(x, router, w_gate_up, w_down, T, E, k, out);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  WsLayout L;
  ws_layout(T, E, k, w_gate_up->k, w_down->k, &L);
  if (L.total > moe::scratch_bytes()) return MOE_ERR_SCRATCH;
  void *ws = nullptr;
  if (moe::scratch_address(&ws) != hipSuccess) return MOE_ERR_HIP;
  return forward_impl(x, router, w_gate_up, w_down, T, E, k, default_options(), out, ws, L.total,
                      (hipStream_t)stream);
  MOE_GUARD_END
}

size_t moe_noalloc_scratch_bytes(void) { return moe::scratch_bytes(); }

int moe_release_workspace(void) {
  MOE_GUARD_BEGIN
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  bool synced = false;
  hipError_t err = hipSuccess;
  for (auto it = g_ws.begin(); it != g_ws.end();) {
    if (it->first.first != dev) {
      ++it;
      continue;
    }
    if (it->second.ptr != nullptr) {
      if (!synced) {
        if (hipDeviceSynchronize() != hipSuccess) return MOE_ERR_HIP;
        synced = true;
      }
      // stream-ordered memory goes back the same way (its stream may no longer exist; after the
      // device synchronisation the null stream orders the release)
      if (hipFreeAsync(it->second.ptr, nullptr) != hipSuccess) err = hipErrorInvalidValue;
    }
    it = g_ws.erase(it);
  }
  if (synced && hipStreamSynchronize(nullptr) != hipSuccess) err = hipErrorInvalidValue;
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  MOE_GUARD_END
}

}  // extern "C"
