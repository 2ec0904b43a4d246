"""Plant plausible mistakes in the oracle (CPU only) and check that some pin catches each.

A pin set that lets one of these through would let the same mistake through in the oracle
itself, so this is the evidence that the pins constrain every step of the oracle.
"""
import numpy as np
import pytest

import oracle.moe_oracle as om
import pins

_orig_decode = om.mxfp4_decode
_orig_swiglu = om.swiglu_clamped
_orig_topk = om.topk_select
_orig_softmax = om.softmax_selected
_orig_logits = om.router_logits
_orig_ffn = om.expert_ffn
_orig_permute = om.permute
_orig_route = om.route
_orig_e2m1 = om.e2m1_value
_orig_e8m0 = om.e8m0_value
_orig_rms = om.rms_norm
_orig_bf16 = om.f64_to_bf16_bits
_orig_block = om.moe_block
_orig_attn = om.attention_decode


def _decode_nibbles_swapped(codes, scales):
    c = np.asarray(codes, np.uint8)
    swapped = ((c & 0xF) << 4) | (c >> 4)
    return _orig_decode(swapped.astype(np.uint8), scales)


def _decode_block16(codes, scales):
    """Mistake: scale index taken as element // 16 (clamped), i.e. 16-element blocks."""
    c = np.asarray(codes, np.uint8)
    K = c.shape[-1] * 2
    table = np.array([om.e2m1_value(v) for v in range(16)])
    el = np.empty(c.shape[:-1] + (K,))
    el[..., 0::2] = table[c & 0xF]
    el[..., 1::2] = table[c >> 4]
    s = np.array([om.e8m0_value(b) for b in range(256)])[np.asarray(scales)]
    sidx = np.minimum(np.arange(K) // 16, K // 32 - 1)
    return el * s[..., sidx]


def _decode_scale_bias128(codes, scales):
    return _orig_decode(codes, scales) * 0.5


def _swiglu_swapped(h, limit=7.0, alpha=1.0):
    h = np.asarray(h, float).copy()
    g = h[..., 0::2].copy()
    h[..., 0::2] = h[..., 1::2]
    h[..., 1::2] = g
    return _orig_swiglu(h, limit, alpha)


def _swiglu_no_plus1(h, limit=7.0, alpha=1.0):
    h = np.asarray(h, float)
    g = np.clip(h[..., 0::2], -limit, limit)
    lin = np.clip(h[..., 1::2], -limit, limit)
    return g / (1 + np.exp(-alpha * g)) * lin


def _swiglu_sig_sign(h, limit=7.0, alpha=1.0):
    h = np.asarray(h, float)
    g = np.clip(h[..., 0::2], -limit, limit)
    lin = np.clip(h[..., 1::2], -limit, limit)
    return g / (1 + np.exp(alpha * g)) * (lin + 1)


def _swiglu_gate_clamp_only(h, limit=7.0, alpha=1.0):
    h = np.asarray(h, float)
    g = np.clip(h[..., 0::2], -limit, limit)
    lin = h[..., 1::2]
    return g / (1 + np.exp(-alpha * g)) * (lin + 1)


def _swiglu_no_clamp(h, limit=7.0, alpha=1.0):
    h = np.asarray(h, float)
    g = h[..., 0::2]
    lin = h[..., 1::2]
    return g / (1 + np.exp(-alpha * g)) * (lin + 1)


def _swiglu_alpha_ignored(h, limit=7.0, alpha=1.0):
    return _orig_swiglu(h, limit, 1.0)


def _topk_ascending(logits, k):
    l32 = np.asarray(logits, np.float64)
    return np.argsort(l32, axis=-1, kind="stable")[..., :k].astype(np.int32)


def _topk_high_id_ties(logits, k):
    l32 = np.asarray(logits, np.float64)
    E = l32.shape[-1]
    order = np.argsort(-l32[..., ::-1], axis=-1, kind="stable")
    return (E - 1 - order[..., :k]).astype(np.int32)


def _topk_unsorted(logits, k):
    return np.sort(_orig_topk(logits, k), axis=-1).astype(np.int32)


def _softmax_not_renormalised(sel):
    sel = np.asarray(sel, float)
    return np.exp(sel) / (np.exp(sel).sum(-1, keepdims=True) + 1.0)


def _logits_no_bias(x, w, b):
    return _orig_logits(x, w, None)


def _ffn_no_b1(x, w1, b1, w2, b2, limit=7.0, alpha=1.0):
    return _orig_ffn(x, w1, None, w2, b2, limit, alpha)


def _ffn_no_b2(x, w1, b1, w2, b2, limit=7.0, alpha=1.0):
    return _orig_ffn(x, w1, b1, w2, None, limit, alpha)


def _permute_unstable(topk_idx, E):
    counts, offsets, sorted_slot, slot_row = _orig_permute(topk_idx, E)
    ss = sorted_slot.copy()
    for e in range(E):
        ss[offsets[e]:offsets[e + 1]] = ss[offsets[e]:offsets[e + 1]][::-1]
    sr = np.empty_like(ss)
    sr[ss] = np.arange(ss.size, dtype=ss.dtype)
    return counts, offsets, ss, sr


def _route_weights_reversed(x_bits, w, b, k, forced_idx=None):
    logits, idx, wt = _orig_route(x_bits, w, b, k, forced_idx)
    return logits, idx, wt[..., ::-1].copy()


def _rms_no_sqrt(x, scale, eps=0.0):
    x = np.asarray(x, float)
    return x / (np.mean(x * x, axis=-1, keepdims=True) + eps) * scale


def _rms_sum_not_mean(x, scale, eps=0.0):
    x = np.asarray(x, float)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * scale


def _rms_eps_outside(x, scale, eps=0.0):
    x = np.asarray(x, float)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * scale


def _rms_over_tokens(x, scale, eps=0.0):
    x = np.asarray(x, float)
    return x / np.sqrt(np.mean(x * x, axis=0, keepdims=True) + eps) * scale


def _bf16_via_f32(v):
    return _orig_bf16(np.asarray(v, np.float64).astype(np.float32).astype(np.float64))


def _bf16_truncate(v):
    return (np.asarray(v, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _block_residual_of_xn(x_bits, norm_scale, norm_eps, *a, **kw):
    r = _orig_block(x_bits, norm_scale, norm_eps, *a, **kw)
    tok = r.moe.tokens
    r.out = r.out - om.bf16_to_f64(np.asarray(x_bits, np.uint16)[tok]) + om.bf16_to_f64(r.xn_bits)
    return r


def _block_no_residual(x_bits, norm_scale, norm_eps, *a, **kw):
    r = _orig_block(x_bits, norm_scale, norm_eps, *a, **kw)
    r.out = r.moe.out
    return r


def _block_norm_skipped(x_bits, norm_scale, norm_eps, *a, **kw):
    return _orig_block(x_bits, np.ones(np.asarray(x_bits).shape[-1]), 0.0, *a, **kw)


def _attn_generic(q, k, v, lens, sinks, window, *, scale=None, head_map=None, lo_shift=0, sink_mode="denominator",
                  ignore_lens=False):
    """The decode step with one planted change (a compact second formulation)."""
    q, k, v = (np.asarray(a, float) for a in (q, k, v))
    B, Hq, D = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = L if ignore_lens else int(lens[b])
        lo = 0 if window <= 0 else max(0, n - window + lo_shift)
        for h in range(Hq):
            g = head_map(h, Hq, Hkv) if head_map else h // (Hq // Hkv)
            sc = k[b, g, lo:n] @ q[b, h] * (scale if scale is not None else 1 / np.sqrt(D))
            m = sc.max()
            e = np.exp(sc - m)
            den = e.sum()
            if sinks is not None and sink_mode == "denominator":
                den += np.exp(float(sinks[h]) - m)
            out[b, h] = (e / den) @ v[b, g, lo:n]
    return out


MUTATIONS = {
    "decode_nibbles_swapped": ("mxfp4_decode", _decode_nibbles_swapped),
    "decode_scale_per_16": ("mxfp4_decode", _decode_block16),
    "decode_scale_bias_128": ("mxfp4_decode", _decode_scale_bias128),
    "e2m1_bias_0": ("e2m1_value", lambda c: 2.0 * _orig_e2m1(c)),
    "e8m0_bias_126": ("e8m0_value", lambda b: 2.0 * _orig_e8m0(b)),
    "swiglu_gate_linear_swapped": ("swiglu_clamped", _swiglu_swapped),
    "swiglu_no_plus_one": ("swiglu_clamped", _swiglu_no_plus1),
    "swiglu_sigmoid_sign": ("swiglu_clamped", _swiglu_sig_sign),
    "swiglu_clamp_gate_only": ("swiglu_clamped", _swiglu_gate_clamp_only),
    "swiglu_no_clamp": ("swiglu_clamped", _swiglu_no_clamp),
    "swiglu_alpha_ignored": ("swiglu_clamped", _swiglu_alpha_ignored),
    "topk_ascending": ("topk_select", _topk_ascending),
    "topk_ties_to_high_id": ("topk_select", _topk_high_id_ties),
    "topk_not_in_score_order": ("topk_select", _topk_unsorted),
    "softmax_not_renormalised": ("softmax_selected", _softmax_not_renormalised),
    "router_bias_dropped": ("router_logits", _logits_no_bias),
    "ffn_gate_up_bias_dropped": ("expert_ffn", _ffn_no_b1),
    "ffn_down_bias_dropped": ("expert_ffn", _ffn_no_b2),
    "permute_unstable": ("permute", _permute_unstable),
    "combine_weights_reversed": ("route", _route_weights_reversed),
    "rmsnorm_no_sqrt": ("rms_norm", _rms_no_sqrt),
    "rmsnorm_sum_not_mean": ("rms_norm", _rms_sum_not_mean),
    "rmsnorm_eps_outside_root": ("rms_norm", _rms_eps_outside),
    "rmsnorm_over_tokens": ("rms_norm", _rms_over_tokens),
    "rmsnorm_scale_dropped": ("rms_norm", lambda x, scale, eps=0.0: _orig_rms(x, np.ones_like(scale), eps)),
    "bf16_double_rounding": ("f64_to_bf16_bits", _bf16_via_f32),
    "bf16_truncation": ("f64_to_bf16_bits", _bf16_truncate),
    "block_residual_of_normed_x": ("moe_block", _block_residual_of_xn),
    "block_no_residual": ("moe_block", _block_no_residual),
    "block_norm_skipped": ("moe_block", _block_norm_skipped),
    "attn_sink_dropped": ("attention_decode", lambda *a: _attn_generic(*a, sink_mode="none")),
    "attn_no_score_scale": ("attention_decode", lambda *a: _attn_generic(*a, scale=1.0)),
    "attn_heads_interleaved": ("attention_decode",
                               lambda *a: _attn_generic(*a, head_map=lambda h, hq, hkv: h % hkv)),
    "attn_window_one_wider": ("attention_decode", lambda *a: _attn_generic(*a, lo_shift=-1)),
    "attn_window_one_narrower": ("attention_decode", lambda *a: _attn_generic(*a, lo_shift=1)),
    "attn_lens_ignored": ("attention_decode", lambda *a: _attn_generic(*a, ignore_lens=True)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(om, attr, bad)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except Exception as exc:  # an assertion, or the mistake breaking a shape
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"planted mistake {name!r} passed every pin"
