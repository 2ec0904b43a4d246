"""fp64 reference for the top-k routed MoE feed-forward layer with MXFP4 expert weights.

TEST INFRASTRUCTURE: imported only by tests/, the smoke check and the benchmark's CPU
baseline. It shares no code, table or constant with the GPU library.

What it computes, and where each step comes from:

* Sources ("pages"):
  - [walkthrough] the gpt-oss architecture walkthrough at pnsm.cn/news/1975454
    (sections 1, 2.2 "MoE layer", 2.4 "comparison with GPT-2 / Qwen3", 4 "config.toml").
  - [review] the review of the from-scratch PyTorch gpt-oss-20B at
    pomoai.com/hubs/HamzaElshafie/gpt-oss-20B (sections 3.2 "RMSNorm", 3.3 "SwiGLU",
    3.4 "MoE", 3.5 "GQA + sliding window + attention sinks", 5).
  - [config] the config.json read-through at m.youleyou.com/wenzhang/3183859 (Part.01).
  - [retrospective] the gpt-oss launch retrospective at youniszhang.com ("工程影响": KV
    heads, head dimension and cache bytes).
  - [OCP-MX] OCP Microscaling Formats (MX) Specification v1.0 -- the public definition of
    the MXFP4 element (E2M1) and scale (E8M0) encodings; the pages only name the format.
* Every floating-point step runs in float64 on exact inputs (bf16 and fp32 inputs widen
  exactly), including the one place floating point decides an integer: which experts a
  token picks is decided on the float64 logits.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional, Sequence, Tuple

import numpy as np

E2M1_BIAS = 1  # exponent bias of the FP4 E2M1 element [OCP-MX, FP4 element definition]
E8M0_BIAS = 127  # exponent bias of the E8M0 shared scale [OCP-MX, scale definition]
E8M0_NAN = 0xFF


def e2m1_value(code: int) -> float:
    """Value of one 4-bit E2M1 element [OCP-MX FP4 definition; walkthrough §1, §4 name MXFP4].

    Bit 3 is the sign, bits 2..1 the exponent (bias 1), bit 0 the mantissa. Exponent
    field 0 encodes subnormals (0 and 0.5); the format has no infinity and no NaN.
    """
    code = int(code) & 0xF
    sign = (code >> 3) & 1
    exp_field = (code >> 1) & 3
    man = code & 1
    if exp_field == 0:
        mag = (man / 2.0) * 2.0 ** (1 - E2M1_BIAS)
    else:
        mag = (1.0 + man / 2.0) * 2.0 ** (exp_field - E2M1_BIAS)
    return -mag if sign else mag


def e8m0_value(byte: int) -> float:
    """Value of one E8M0 scale byte: a bare power of two, 2^(byte-127); 0xFF is NaN [OCP-MX]."""
    byte = int(byte) & 0xFF
    if byte == E8M0_NAN:
        return float("nan")
    return 2.0 ** (byte - E8M0_BIAS)


_E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E8M0_TABLE = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)


def mxfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode an MXFP4 tensor to float64 [walkthrough §1, §4: MoE weights in MXFP4, ~4.25 bit].

    codes  uint8 [..., K/2]: element 2j is the low nibble of byte j, element 2j+1 the high one.
    scales uint8 [..., K/32]: one E8M0 scale per 32 consecutive elements along the last axis.
    4 bits per element plus 8 bits per 32 elements gives the pages' 4.25 bits per weight.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    K = codes.shape[-1] * 2
    if scales.shape[-1] * 32 != K or scales.shape[:-1] != codes.shape[:-1]:
        raise ValueError("scales must hold one byte per 32 elements of each row")
    elem = np.empty(codes.shape[:-1] + (K,), dtype=np.float64)
    elem[..., 0::2] = _E2M1_TABLE[codes & 0xF]
    elem[..., 1::2] = _E2M1_TABLE[codes >> 4]
    blk = _E8M0_TABLE[scales]
    elem = elem.reshape(codes.shape[:-1] + (K // 32, 32)) * blk[..., None]
    return elem.reshape(codes.shape[:-1] + (K,))


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact): the pattern is the top half of a float32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def router_logits(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """One score per (token, expert) from a linear projection of the token [review §3.4].

    x float64 [T][H]; w fp32 [E][H]; b fp32 [E] or None. Returns float64 [T][E].
    """
    logits = np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
    if b is not None:
        logits = logits + np.asarray(b, np.float64)[None, :]
    return logits


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """The k highest-scoring experts per token, highest first [review §3.4; walkthrough §2.2, §4;
    config Part.01 experts_per_token = 4].

    The pages do not say how ties break or in which order the k experts are listed. Reading
    taken: ties go to the lower expert id, and the list is in descending score order. The
    ranking is the plain one of the float64 scores.
    """
    lg = np.asarray(logits, np.float64)
    order = np.argsort(-lg, axis=-1, kind="stable")  # stable: equal scores keep id order
    return order[..., :k].astype(np.int32)


def softmax_selected(sel_logits: np.ndarray) -> np.ndarray:
    """Mixing weights: softmax over the k selected experts' scores only [walkthrough §2.2;
    review §3.4]. They sum to one for every token."""
    sel = np.asarray(sel_logits, np.float64)
    z = np.exp(sel - sel.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def route(x_bits: np.ndarray, w: np.ndarray, b: Optional[np.ndarray], k: int,
          forced_idx: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Router: logits, top-k ids, softmax weights. ``forced_idx`` replaces the selection
    (used to grade tokens whose k-th and (k+1)-th scores nearly tie)."""
    logits = router_logits(bf16_to_f64(x_bits), w, b)
    idx = topk_select(logits, k) if forced_idx is None else np.asarray(forced_idx, np.int32)
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=-1)
    return logits, idx, softmax_selected(sel)


def permute(topk_idx: np.ndarray, E: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Group the T*k (token, rank) slots by expert [review §3.4: only the picked experts run;
    retrospective "当时发生了什么": all expert weights stay resident].

    Slot s = t*k + j. Returns counts[E], offsets[E+1] (exclusive prefix sum of counts),
    sorted_slot[T*k] (slots ordered by expert, then by slot id) and slot_row[T*k], the
    position of each slot in that order (the inverse permutation).
    """
    flat = np.asarray(topk_idx, np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_slot = np.argsort(flat, kind="stable").astype(np.int32)
    slot_row = np.empty_like(sorted_slot)
    slot_row[sorted_slot] = np.arange(flat.size, dtype=np.int32)
    return counts, offsets, sorted_slot, slot_row


def swiglu_clamped(h: np.ndarray, limit: float = 7.0, alpha: float = 1.0) -> np.ndarray:
    """Clamped gated SwiGLU with the +1 on the linear branch [walkthrough §1, §2.2;
    review §3.3].

    h [..., 2I] holds the fused projection with gate and linear interleaved (2i = gate,
    2i+1 = linear; the pages leave the order open). Both halves are clamped to
    [-limit, limit] (the pages give +-7.0 without saying which half or side), then
    a = g * sigmoid(alpha*g) * (l + 1). alpha = 1 is plain SiLU, the only slope the pages
    imply; other values are accepted for parity runs.
    """
    h = np.asarray(h, np.float64)
    g = np.clip(h[..., 0::2], -limit, limit)
    lin = np.clip(h[..., 1::2], -limit, limit)
    sig = 1.0 / (1.0 + np.exp(-alpha * g))
    return g * sig * (lin + 1.0)


def expert_ffn(x: np.ndarray, w1: np.ndarray, b1: Optional[np.ndarray], w2: np.ndarray,
               b2: Optional[np.ndarray], limit: float = 7.0, alpha: float = 1.0
               ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One expert on rows x [n][H]: h = x W1^T + b1 (2I outputs), a = swiglu(h), y = a W2^T + b2
    [walkthrough §2.4: embedding and expert projection widths are both 2880]. Returns (h, a, y)."""
    h = np.asarray(x, np.float64) @ np.asarray(w1, np.float64).T
    if b1 is not None:
        h = h + b1[None, :]
    a = swiglu_clamped(h, limit, alpha)
    y = a @ np.asarray(w2, np.float64).T
    if b2 is not None:
        y = y + b2[None, :]
    return h, a, y


ExpertTensors = Tuple[np.ndarray, np.ndarray, Optional[np.ndarray],
                      np.ndarray, np.ndarray, Optional[np.ndarray]]


def experts_from_arrays(w1_codes, w1_scales, w1_bias, w2_codes, w2_scales, w2_bias
                        ) -> Callable[[int], ExpertTensors]:
    """Adapter: stacked [E][...] arrays -> per-expert tuple getter (bias arrays may be None)."""
    def get(e: int) -> ExpertTensors:
        return (w1_codes[e], w1_scales[e], None if w1_bias is None else w1_bias[e],
                w2_codes[e], w2_scales[e], None if w2_bias is None else w2_bias[e])
    return get


@dataclasses.dataclass
class MoEResult:
    out: np.ndarray          # float64 [n_tok][H]
    tokens: np.ndarray       # int64 [n_tok], which rows of x these are
    logits: np.ndarray       # float64 [n_tok][E]
    idx: np.ndarray          # int32 [n_tok][k]
    w: np.ndarray            # float64 [n_tok][k]
    h: Optional[np.ndarray] = None    # float64 [n_tok][k][2I]
    act: Optional[np.ndarray] = None  # float64 [n_tok][k][I]
    y: Optional[np.ndarray] = None    # float64 [n_tok][k][H]


def moe_layer(x_bits: np.ndarray, router_w: np.ndarray, router_b: Optional[np.ndarray],
              get_expert: Callable[[int], ExpertTensors], k: int,
              limit: float = 7.0, alpha: float = 1.0,
              tokens: Optional[Sequence[int]] = None,
              forced_idx: Optional[np.ndarray] = None,
              keep_intermediates: bool = False) -> MoEResult:
    """The whole layer for the rows ``tokens`` of x (all rows if None).

    Route each token to its top-k experts with softmax weights over the selected scores,
    run only the selected experts, and sum their outputs weighted by those weights
    [review §3.4; walkthrough §2.2]. Tokens are independent, so any subset can be computed.
    """
    x_bits = np.asarray(x_bits, np.uint16)
    tok = np.arange(x_bits.shape[0]) if tokens is None else np.asarray(tokens, np.int64)
    x = bf16_to_f64(x_bits[tok])
    logits, idx, w = route(x_bits[tok], router_w, router_b, k, forced_idx)
    n, H = x.shape
    y_slots = np.zeros((n, k, H), np.float64)
    h_slots = a_slots = None
    for e in np.unique(idx):
        rows, ranks = np.nonzero(idx == e)
        w1c, w1s, b1, w2c, w2s, b2 = get_expert(int(e))
        W1 = mxfp4_decode(w1c, w1s)
        W2 = mxfp4_decode(w2c, w2s)
        h, a, y = expert_ffn(x[rows], W1, None if b1 is None else bf16_to_f64(b1),
                             W2, None if b2 is None else bf16_to_f64(b2), limit, alpha)
        y_slots[rows, ranks] = y
        if keep_intermediates:
            if h_slots is None:
                h_slots = np.zeros((n, k, h.shape[1]), np.float64)
                a_slots = np.zeros((n, k, a.shape[1]), np.float64)
            h_slots[rows, ranks] = h
            a_slots[rows, ranks] = a
    out = np.zeros((n, H), np.float64)
    for j in range(k):  # weighted sum over the k picks, rank order
        out += w[:, j:j + 1] * y_slots[:, j, :]
    return MoEResult(out, tok, logits, idx, w, h_slots, a_slots,
                     y_slots if keep_intermediates else None)


def rms_norm(x: np.ndarray, scale: np.ndarray, eps: float = 0.0) -> np.ndarray:
    """RMSNorm of each row [review §3.2; walkthrough §2.3]: the row divided by its root mean
    square, times a per-feature scale, with no mean subtraction and no bias.

    x float64 [..., H]; scale [H]. RMS(x) = sqrt(mean over the row of x^2 + eps): the pages
    give RMS(x) with no epsilon; eps (0 = the pages' form) is the usual guard against an
    all-zero row and is a caller's parameter.
    """
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(scale, np.float64)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits, fp32's exponent range), to
    nearest with ties to even, in one rounding; returns the uint16 bit patterns.

    The quantum of v is 2^(e-8) for v = m 2^e with m in [0.5, 1), and never below 2^-133,
    the spacing of bf16 subnormals. Magnitudes that round to 2^128 or above become inf.
    """
    v = np.asarray(v, np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("finite values only")
    _, e = np.frexp(v)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(v / q) * q  # v / q is exact (a power-of-two scaling); rint ties to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@dataclasses.dataclass
class BlockResult:
    out: np.ndarray       # float64 [n_tok][H]: x + MoE(xn)
    xn_bits: np.ndarray   # uint16 [n_tok][H]: the normalised rows as the layer's bf16 input
    moe: MoEResult        # the layer on xn (its .tokens are rows of x)


def moe_block(x_bits: np.ndarray, norm_scale: np.ndarray, norm_eps: float,
              router_w: np.ndarray, router_b: Optional[np.ndarray],
              get_expert: Callable[[int], ExpertTensors], k: int,
              limit: float = 7.0, alpha: float = 1.0,
              tokens: Optional[Sequence[int]] = None,
              forced_idx: Optional[np.ndarray] = None,
              forced_xn_bits: Optional[np.ndarray] = None) -> BlockResult:
    """The MoE half of a decoder block around the layer: out = x + MoE(RMSNorm(x))
    [walkthrough §2 and §2.3: each block normalises the stream before the MoE layer;
    review §3.2 RMSNorm, §3.3: a residual path joins the FFN's output and its input].

    Reading taken: the normalised row is the layer's bf16 input, so it is rounded to bf16
    once (to nearest, ties to even) before the router and the experts see it; the residual
    adds the un-normalised x to the layer's output. ``forced_xn_bits`` (rows of the selected
    tokens) replaces that rounding: used to grade rows where an element lies so close to a
    bf16 rounding boundary that a float32 evaluation of the norm rounds it the other way.
    """
    x_bits = np.asarray(x_bits, np.uint16)
    tok = np.arange(x_bits.shape[0]) if tokens is None else np.asarray(tokens, np.int64)
    x = bf16_to_f64(x_bits[tok])
    if forced_xn_bits is None:
        xn_bits = f64_to_bf16_bits(rms_norm(x, norm_scale, norm_eps))
    else:
        xn_bits = np.asarray(forced_xn_bits, np.uint16)
    res = moe_layer(xn_bits, router_w, router_b, get_expert, k, limit, alpha,
                    forced_idx=forced_idx)
    res.tokens = tok
    return BlockResult(x + res.out, xn_bits, res)


# --------------------------------------------------------------------------- decode attention
def attention_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, lens: np.ndarray,
                     sinks: Optional[np.ndarray], window: int = 0) -> np.ndarray:
    """One decode step of grouped-query attention with per-head sink logits
    [walkthrough §2.1: 64 query heads share 8 key/value heads; layers alternate between a
    128-token banded window and dense attention; each head learns a logit that joins the
    softmax's denominator, so a head can attend to nothing; review §3.5 the same three;
    retrospective "工程影响": 8 KV heads of dimension 64 with a 2-byte cache].

    q       [B][Hq][D]     the new token's queries (positional rotation already applied)
    k_cache [B][Hkv][L][D] keys of positions 0..L-1; v_cache the same for values
    lens    [B]            sequence b's tokens in the cache (the new one is position lens[b]-1)
    sinks   [Hq] or None   the per-head sink logit (None: no sink)
    window  0 for dense attention, else the band: the query at position i sees keys
            i-window+1 .. i (the last `window` tokens, itself included)

    Readings taken: query head h reads key/value head h // (Hq / Hkv) (consecutive query heads
    share one); the score is q.k / sqrt(D); the sink is one more logit in the softmax whose
    value vector is zero, so the weights of the real keys sum to less than one. A sequence with
    no visible position (lens[b] = 0) gives 0: with a sink every real key's weight is 0, and
    without one the weighted sum has no terms (the pages do not reach this case).
    Returns float64 [B][Hq][D].
    """
    q = np.asarray(q, np.float64)
    kc = np.asarray(k_cache, np.float64)
    vc = np.asarray(v_cache, np.float64)
    B, Hq, D = q.shape
    Hkv = kc.shape[1]
    group = Hq // Hkv
    out = np.zeros((B, Hq, D), np.float64)
    for b in range(B):
        n = int(lens[b])
        lo = 0 if window <= 0 else max(0, n - window)
        if n <= lo:
            continue  # nothing visible: the output row stays 0
        for h in range(Hq):
            g = h // group
            keys = kc[b, g, lo:n]      # [n - lo][D]
            vals = vc[b, g, lo:n]
            s = keys @ q[b, h] / np.sqrt(D)
            if sinks is not None:
                s_all = np.concatenate([s, [float(sinks[h])]])
            else:
                s_all = s
            m = s_all.max()
            e = np.exp(s_all - m)
            w = e[:n - lo] / e.sum()
            out[b, h] = w @ vals
    return out
