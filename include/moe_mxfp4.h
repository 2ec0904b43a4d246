/*
 * moe_mxfp4.h -- C ABI of a top-k routed mixture-of-experts feed-forward layer with
 * MXFP4 expert weights, written for AMD Instinct MI355X (gfx950).
 *
 * The layer (gpt-oss pages: architecture walkthrough at pnsm.cn/news/1975454, sections 1,
 * 2.2 and 2.4; review of the from-scratch gpt-oss-20B at pomoai.com, sections 3.3-3.4):
 *   logits = x W_r^T + b_r                  linear router, one score per expert
 *   idx    = the k best experts per token   (k = 4 in both gpt-oss sizes)
 *   w      = softmax over those k scores
 *   h      = W1_e x + b1_e                  fused gate/linear projection, 2I outputs
 *   a      = clamp(g) * sigmoid(alpha * clamp(g)) * (clamp(l) + 1)   clamped SwiGLU, +1 residual
 *   y      = W2_e a + b2_e
 *   out    = sum_j w_j y_{idx_j}
 * Expert weights are MXFP4: 4-bit E2M1 elements with one E8M0 power-of-two scale per 32
 * consecutive input features (4.25 bits per weight; walkthrough sections 1 and 4).
 *
 * Conventions for every entry point:
 *  - Every pointer argument is DEVICE memory owned by the caller, except the descriptor
 *    structs (moe_router_t, moe_mxfp4_weight_t, moe_options_t), which are HOST structs
 *    read during the call and not retained. Nothing is freed or retained by the library
 *    except moe_forward's internal workspace (see there).
 *  - bf16 tensors are passed as uint16_t bit patterns. All tensors are dense row-major.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default (null) stream.
 *    Calls are asynchronous with respect to the host; device faults surface at the
 *    caller's next synchronisation, as for any HIP kernel.
 *  - All argument checks happen before the first HIP call, so an error return leaves no
 *    partial work queued. T == 0 returns MOE_OK without launching anything.
 *  - NaN/Inf inputs are not checked; results for them are unspecified.
 *  - Return value: MOE_OK (0) or one of the negative MOE_ERR_* codes below.
 *  - Limits: 1 <= k <= 8, k <= E <= 256, H and I multiples of 32 and at most 16384,
 *    T * k < 2^31. x and code pointers must be 16-byte aligned, fp32 outputs 16-byte aligned.
 */
#ifndef MOE_MXFP4_H_
#define MOE_MXFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

/* status codes */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1)  /* NULL pointer, negative size, misaligned pointer, bad enum */
#define MOE_ERR_UNSUPPORTED (-2)  /* shape outside the limits above */
#define MOE_ERR_WORKSPACE (-3)    /* caller workspace smaller than moe_workspace_size() */
#define MOE_ERR_HIP (-4)          /* a HIP runtime call or kernel launch failed */
#define MOE_ERR_SCRATCH (-5)      /* moe_forward_noalloc: the sizes need more than its fixed scratch */

/* output element types */
#define MOE_DTYPE_BF16 0
#define MOE_DTYPE_F32 1

/* expert-FFN kernel family (moe_options_t.path) */
#define MOE_PATH_AUTO 0  /* chosen from T*k and E on the host */
#define MOE_PATH_DECODE 1 /* weight-streaming kernels for decode-sized batches */
#define MOE_PATH_PREFILL_BF16 2 /* LDS-tiled grouped GEMM for prefill-sized batches, bf16
                                   activations times MXFP4 weights decoded to bf16 in registers;
                                   needs MOE_LAYOUT_TILED weights (else MOE_ERR_UNSUPPORTED). */
#define MOE_PATH_PREFILL_MX8SPLIT 3 /* the same grouped GEMM on gfx950's block-scaled MFMA: the
                                   MXFP4 weights are an operand as stored, each bf16 activation is
                                   split exactly into two MXFP8 (E4M3) terms with E8M0 block
                                   scales. Needs MOE_LAYOUT_TILED weights. AUTO picks it for
                                   tiled weights when T*k >= 32*E and I < 1024. */
#define MOE_PATH_PREFILL_MX6SPLIT 4 /* gate_up as MX8SPLIT; the down projection's input (the
                                   bf16-rounded activation) as two MXFP6 (E2M3) terms with E8M0
                                   block scales, on the FP6 x FP4 scaled MFMA, which issues faster
                                   than FP8 x FP4. That split is exact for activations within 2^3
                                   of their 32-element block's maximum, else off by less than 2^-9
                                   of that maximum (so not bit-equal to the bf16 GEMM). Needs
                                   MOE_LAYOUT_TILED weights. AUTO picks it for tiled weights
                                   when T*k >= 32*E and I >= 1024 (the gpt-oss widths). */
#define MOE_PATH_DECODE_FUSED 5 /* a batch of one token (H <= 3072, I <= 4096, tiled weights):
                                   gate_up, SwiGLU and down in one launch, one workgroup per
                                   (picked expert, 32-activation block), each writing its block's
                                   share of the expert's output, the shares added in a fixed
                                   order by the combine; other batches run as MOE_PATH_DECODE.
                                   Opt-in: on MI355X the two-kernel form of MOE_PATH_DECODE is
                                   faster at one token. Needs MOE_LAYOUT_TILED weights. */
/* earlier names of the same paths */
#define MOE_PATH_STREAM MOE_PATH_DECODE
#define MOE_PATH_GEMM MOE_PATH_PREFILL_BF16
#define MOE_PATH_GEMM_MX MOE_PATH_PREFILL_MX8SPLIT

/* moe_mxfp4_weight_t.layout */
#define MOE_LAYOUT_ROWMAJOR 0 /* codes [E][n][k/2], scales [E][n][k/32] as described below */
#define MOE_LAYOUT_TILED 1    /* the kernel layout written by moe_mxfp4_pack */

/* moe_options_t.flags: test hooks for per-step checks of the expert FFN */
#define MOE_FLAG_EMIT_PREACT 1u /* stop after gate_up: y <- h = W1 x + b1, fp32 [T*k][2I] */
#define MOE_FLAG_EMIT_ACT 2u    /* stop after the SwiGLU: y <- a (bf16-rounded, as fp32) [T*k][I] */

typedef void *moe_stream_t; /* a hipStream_t */

/* Linear router [review section 3.4]. */
typedef struct moe_router {
  const float *weight; /* fp32 [E][H] */
  const float *bias;   /* fp32 [E], or NULL for zero */
} moe_router_t;

/*
 * One MXFP4 weight matrix for all E experts [walkthrough sections 1 and 4].
 * Expert e's matrix has `n` rows (output features) of `k` elements (input features).
 * codes:  uint8 [E][n][k/2]; byte j of a row holds element 2j in its low nibble and
 *         element 2j+1 in its high nibble; a nibble is an E2M1 code (sign, 2 exponent
 *         bits with bias 1, 1 mantissa bit; OCP MX v1.0).
 * scales: uint8 [E][n][k/32]; byte b is the E8M0 scale 2^(byte-127) of elements
 *         32b..32b+31 of the row (0xFF is NaN).
 * bias:   bf16 [E][n], or NULL for zero.
 * For the gate_up matrix n = 2I with rows interleaved: row 2i is unit i's gate, row
 * 2i+1 its linear branch; k = H. For the down matrix n = H, k = I.
 * layout MOE_LAYOUT_TILED: codes and scales hold the same values re-ordered by
 * moe_mxfp4_pack into 32-row x 128-element tiles (see there); bias is unchanged but
 * must be 8-byte aligned (codes 16-byte, scales 4-byte); row-major: codes 16-byte,
 * bias 2-byte. Misaligned pointers are rejected with MOE_ERR_INVALID_ARG.
 */
typedef struct moe_mxfp4_weight {
  const uint8_t *codes;
  const uint8_t *scales;
  const uint16_t *bias;
  int32_t n;
  int32_t k;
  int32_t layout; /* MOE_LAYOUT_ROWMAJOR or MOE_LAYOUT_TILED */
} moe_mxfp4_weight_t;

/* Options for the _ex entry points; NULL selects the defaults shown. */
typedef struct moe_options {
  float swiglu_limit; /* 7.0: clamp bound of both halves [review section 3.3] */
  float swiglu_alpha; /* 1.0: sigmoid slope; 1 is plain SiLU */
  int32_t out_dtype;  /* MOE_DTYPE_BF16 */
  int32_t path;       /* MOE_PATH_AUTO */
  uint32_t flags;     /* 0; see MOE_FLAG_* (moe_mxfp4_ffn only) */
} moe_options_t;

/* ABI version of the loaded library (MOE_ABI_VERSION of its build). */
int moe_abi_version(void);

/* Static, never-NULL description of a status code. */
const char *moe_status_string(int status);

/*
 * Bytes of caller workspace that moe_route, moe_permute, moe_mxfp4_ffn and moe_forward_ex
 * need for these sizes and this path (one size serves them all). Returns 0 for invalid
 * sizes.
 * A workspace passed to those calls must be 256-byte aligned.
 */
size_t moe_workspace_size(int64_t T, int32_t E, int32_t k, int32_t H, int32_t I, int32_t path);

/*
 * Decode n MXFP4 elements to fp32 (an exported test of the decode step; the layer never
 * writes decoded weights to memory). codes: uint8 [n/2], scales: uint8 [n/32],
 * out: fp32 [n]. n must be a multiple of 32. Exact: E2M1 value times 2^(scale-127),
 * with fp32 overflow giving +-inf, fp32 subnormals kept, and scale 0xFF giving NaN.
 */
int moe_mxfp4_dequant(const uint8_t *codes, const uint8_t *scales, int64_t n, float *out,
                      moe_stream_t stream);

/*
 * Bytes of the tiled copies of one MXFP4 matrix (E experts, n x k each) that
 * moe_mxfp4_pack writes: *codes_bytes = E * (n/32) * ceil(k/128) * 2048 and
 * *scales_bytes = E * (n/32) * ceil(k/128) * 128. Returns MOE_ERR_UNSUPPORTED unless
 * n is a positive multiple of 32 and k a positive multiple of 32.
 */
int moe_mxfp4_tiled_bytes(int32_t E, int32_t n, int32_t k, size_t *codes_bytes, size_t *scales_bytes);

/*
 * Re-order a row-major MXFP4 matrix (src->layout must be MOE_LAYOUT_ROWMAJOR) into the
 * tiled kernel layout, on the device. A one-time, load-time conversion: the values and
 * their MX blocks are unchanged, only their order in memory. Tile (G, c) of expert e covers
 * rows 32G..32G+31 and elements 128c..128c+127 (MX blocks 4c..4c+3) and is stored as two
 * 1 KB halves p = 0, 1 of 64 lanes x 16 bytes, lane l holding the 16 code bytes of block
 * 4c + 2p + l/32 of row 32G + l%32; the scales array holds 32 rows x 4 scale bytes (blocks
 * 4c..4c+3) per tile. Elements past k are zero codes with scale 127. Requires n % 32 == 0.
 * codes_out / scales_out: device buffers of moe_mxfp4_tiled_bytes() bytes, 16-byte aligned.
 */
int moe_mxfp4_pack(const moe_mxfp4_weight_t *src, int32_t E, uint8_t *codes_out, uint8_t *scales_out,
                   moe_stream_t stream);

/*
 * Router [review section 3.4; walkthrough sections 2.2 and 4; config.json read-through at
 * m.youleyou.com, Part.01: experts_per_token = 4].
 * x: bf16 [T][H]. router->weight fp32 [E][H], router->bias fp32 [E] or NULL.
 * Outputs topk_idx int32 [T][k] (the k largest fp32 logits, largest first, ties to the
 * lower expert id) and topk_w fp32 [T][k] (softmax over those k logits).
 * Logits are accumulated in fp32. ws: at least moe_workspace_size(T, E, k, H, H, 0)
 * bytes (the fp32 logits are staged there).
 */
int moe_route(const uint16_t *x, int64_t T, int32_t H, const moe_router_t *router, int32_t E,
              int32_t k, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
              moe_stream_t stream);

/*
 * Group the T*k slots (slot s = t*k + j) by expert [review section 3.4: only the picked
 * experts run]. topk_idx int32 [T][k] with values in [0, E).
 * Outputs: expert_offsets int32 [E+1] (exclusive prefix sum of per-expert slot counts,
 * expert_offsets[E] = T*k), sorted_slot int32 [T*k] (slots ordered by expert, then by
 * slot id), slot_row int32 [T*k] (position of slot s in that order).
 * ws/ws_bytes: a workspace of moe_workspace_size bytes for these T, E, k; with more than
 * 8192 slots the sort spreads over several workgroups and keeps per-range counts there.
 * ws may be NULL (then one workgroup sorts every slot: same result, slower for large T).
 * Deterministic.
 */
int moe_permute(const int32_t *topk_idx, int64_t T, int32_t E, int32_t k, int32_t *expert_offsets,
                int32_t *sorted_slot, int32_t *slot_row, void *ws, size_t ws_bytes,
                moe_stream_t stream);

/*
 * Expert FFNs of all slots [walkthrough sections 2.2 and 2.4; review section 3.3].
 * For sorted row r (slot s = sorted_slot[r], token t = s / k, expert e with
 * expert_offsets[e] <= r < expert_offsets[e+1]):
 *   y[r] = W2_e (swiglu(W1_e x[t] + b1_e)) + b2_e,      y fp32 [T*k][H]
 * The activation a is rounded to bf16 between the two products; accumulation is fp32.
 * x bf16 [T][H]; gate_up->n = 2 * down->k, gate_up->k = down->n = H.
 * opts->flags may stop early (MOE_FLAG_EMIT_PREACT: y is [T*k][2I]; MOE_FLAG_EMIT_ACT:
 * y is [T*k][I]). ws: at least moe_workspace_size(T, E, k, H, I, opts->path) bytes.
 * The routing must give each expert at most one slot per token (distinct experts in each
 * token's k picks, as moe_route's top-k and moe_permute produce): on MOE_PATH_DECODE_FUSED with
 * one token the FFNs run fused per (expert, 32-activation block) with the token's row staged on
 * chip, and an expert holding more than one slot there gives unspecified values for its slots
 * (never an access outside the buffers).
 */
int moe_mxfp4_ffn(const uint16_t *x, int64_t T, int32_t k, int32_t E, const int32_t *expert_offsets,
                  const int32_t *sorted_slot, const moe_mxfp4_weight_t *gate_up,
                  const moe_mxfp4_weight_t *down, const moe_options_t *opts, float *y, void *ws,
                  size_t ws_bytes, moe_stream_t stream);

/*
 * Weighted combine [review section 3.4]: out[t] = sum over j = 0..k-1, in that order, of
 * topk_w[t][j] * y[slot_row[t*k + j]], accumulated in fp32, then rounded to nearest-even
 * bf16 (out_dtype MOE_DTYPE_BF16, out is uint16 [T][H]) or stored as fp32 (MOE_DTYPE_F32).
 */
int moe_combine(const float *y, const int32_t *slot_row, const float *topk_w, int64_t T, int32_t k,
                int32_t H, void *out, int32_t out_dtype, moe_stream_t stream);

/*
 * The whole layer: route, permute, expert FFNs, combine; out bf16 [T][H].
 * Uses a workspace owned by the library, one per (device, stream), grown on demand and kept
 * until moe_release_workspace() or process exit; growing it is stream-ordered (hipFreeAsync of
 * the old buffer and hipMallocAsync of the new one on `stream`, no host synchronisation). Calls
 * on different streams use different workspaces; calls on one stream are ordered by that
 * stream. Concurrent calls from several host threads are safe (a mutex guards
 * the table of workspaces), but callers that cannot afford the first call's allocation, or
 * that capture the call in a HIP graph, use moe_forward_ex with their own workspace.
 */
int moe_forward(const uint16_t *x, const moe_router_t *router, const moe_mxfp4_weight_t *w_gate_up,
                const moe_mxfp4_weight_t *w_down, int64_t T, int32_t E, int32_t k, uint16_t *out,
                moe_stream_t stream);

/*
 * moe_forward with options and a caller workspace of at least
 * moe_workspace_size(T, E, k, H, I, opts->path) bytes (256-byte aligned). out is bf16
 * [T][H] or fp32 [T][H] per opts->out_dtype. opts->flags must be 0.
 */
int moe_forward_ex(const uint16_t *x, const moe_router_t *router,
                   const moe_mxfp4_weight_t *w_gate_up, const moe_mxfp4_weight_t *w_down,
                   int64_t T, int32_t E, int32_t k, const moe_options_t *opts, void *out, void *ws,
                   size_t ws_bytes, moe_stream_t stream);

/*
 * RMSNorm of each row [review section 3.2: the row over its root mean square, times a
 * per-feature scale; walkthrough section 2.3: RMSNorm without bias]:
 *   out[t][h] = bf16( x[t][h] / sqrt(mean_h x[t][h]^2 + eps) * scale[h] )
 * x bf16 [T][H]; scale fp32 [H]; out bf16 [T][H], rounded to nearest-even once. The mean of
 * squares is an fp32 sum, the root and the divisions are correctly rounded fp32, and the
 * products are (x * r) * scale, so an element can differ by one bf16 step from the exactly
 * rounded value when the exact value lies within fp32 rounding of a rounding boundary.
 * eps >= 0 and finite (else MOE_ERR_INVALID_ARG); eps = 0 is the pages' plain RMS, for which
 * an all-zero row gives NaN. x, scale and out 16-byte aligned; H a multiple of 32.
 */
int moe_rmsnorm(const uint16_t *x, int64_t T, int32_t H, const float *scale, float eps, uint16_t *out,
                moe_stream_t stream);

/*
 * The MoE half of a decoder block around the layer [walkthrough section 2: each block
 * normalises its input before the MoE layer; review section 3.3: a residual path joins the
 * FFN's output and its input]:
 *   xn  = moe_rmsnorm(x, norm_scale, norm_eps)          (bf16, as above)
 *   out = x + layer(xn)                                 (the layer of moe_forward_ex on xn)
 * The residual x is added to the fp32 weighted sum of the experts' outputs, after it, and the
 * result is rounded once (out bf16 or fp32 per opts->out_dtype). norm_scale fp32 [H], 16-byte
 * aligned; norm_eps as for moe_rmsnorm. Workspace, options and limits as moe_forward_ex (the
 * same moe_workspace_size covers the normalised copy of x). With a bf16 output, out may be x
 * itself (an in-place residual update): x is last read by the kernel that writes out, element
 * by element before the write.
 */
int moe_block_forward_ex(const uint16_t *x, const float *norm_scale, float norm_eps, const moe_router_t *router,
                         const moe_mxfp4_weight_t *w_gate_up, const moe_mxfp4_weight_t *w_down, int64_t T,
                         int32_t E, int32_t k, const moe_options_t *opts, void *out, void *ws, size_t ws_bytes,
                         moe_stream_t stream);

/*
 * One decode step of grouped-query attention with per-head sink logits, the other per-layer
 * hot path of the same model [walkthrough section 2.1: 64 query heads share 8 key/value
 * heads, layers alternate between a 128-token banded window and dense attention, each head
 * learns a logit added to the softmax's denominator; review section 3.5; retrospective
 * "工程影响": head dimension 64, 2-byte cache]. For sequence b and query head h (key/value
 * head h / (n_q_heads / n_kv_heads): consecutive query heads share one), over the visible
 * positions j (0 <= j < lens[b]; with window > 0 only lens[b] - window <= j):
 *   s_j = q[b][h] . k[b][kvh][j] / sqrt(64)
 *   out[b][h] = sum_j e^(s_j) v[b][kvh][j] / (sum_j e^(s_j) + e^(sinks[h]))
 * (without the sink term when sinks is NULL; 0 for a sequence with no visible position).
 * q bf16 [B][n_q_heads][64] (positional rotation already applied); k_cache, v_cache bf16
 * [B][n_kv_heads][max_len][64] (the new token's key and value already written at position
 * lens[b] - 1); lens int32 [B], values clamped into [0, max_len]; sinks fp32 [n_q_heads] or
 * NULL; out bf16 or fp32 [B][n_q_heads][64] per out_dtype. Scores, exponentials and sums are
 * fp32; the weights enter the weighted sum of values as two bf16 terms (relative error about
 * 2^-17). head_dim must be 64 and n_q_heads / n_kv_heads at most 16 (else
 * MOE_ERR_UNSUPPORTED). ws: at least moe_attn_workspace_size(B, n_kv_heads, max_len, window)
 * bytes, 256-byte aligned. Deterministic.
 */
size_t moe_attn_workspace_size(int64_t B, int32_t n_kv_heads, int64_t max_len, int32_t window);
int moe_attn_decode(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache, const int32_t *lens,
                    const float *sinks, int64_t B, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                    int64_t max_len, int32_t window, void *out, int32_t out_dtype, void *ws, size_t ws_bytes,
                    moe_stream_t stream);

/*
 * moe_forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same layer, the same kernels and
 * the same result as moe_forward, with its workspace in a fixed device array of
 * moe_noalloc_scratch_bytes() bytes (64 MiB) that each GPU the library runs on holds until the
 * process ends. The call itself allocates nothing, never synchronises and records no memset.
 * Sizes whose workspace (moe_workspace_size(T, E, k, H, I, MOE_PATH_AUTO)) exceeds the array are
 * rejected with MOE_ERR_SCRATCH before anything is launched; at H = I = 2880, k = 4 that allows
 * about 650 tokens. Every call on one GPU uses that GPU's one array, and the array keeps the last
 * call's contents (each call zeroes, by a kernel of its own, what it needs zeroed): calls that
 * overlap on one GPU (other streams, other host threads) race on it and must be serialised by
 * the caller, e.g. issued on one stream.
 */
int moe_forward_noalloc(const uint16_t *x, const moe_router_t *router, const moe_mxfp4_weight_t *w_gate_up,
                        const moe_mxfp4_weight_t *w_down, int64_t T, int32_t E, int32_t k, uint16_t *out,
                        moe_stream_t stream);
size_t moe_noalloc_scratch_bytes(void);

/* Free moe_forward's workspaces (every stream's) on the current device (synchronises the
 * device first). */
int moe_release_workspace(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H_ */
