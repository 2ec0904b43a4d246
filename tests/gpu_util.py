"""Helpers for the GPU parity tests: device copies of seeded inputs, and oracle comparisons.

The oracle is test infrastructure; it is called here on the CPU with the same seeded
inputs that are copied to the GPU. Nothing computed on the GPU feeds the oracle except,
for tokens whose k-th and (k+1)-th fp64 logits nearly tie, the GPU's choice of experts
(the oracle then recomputes those tokens with that choice forced).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

import oracle
import synth
import sparse_moe_transformer_router_amd as moe

TIE_GAP = 1e-3        # k-th vs (k+1)-th logit gap below which either choice is accepted
OUT_TOL = 2e-2        # max-abs error <= OUT_TOL * RMS(oracle output)
W_TOL = 1e-5          # routing weights


def to_dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def to_dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@dataclasses.dataclass
class DevLayer:
    inp: synth.MoEInputs
    x: torch.Tensor
    router: moe.Router
    w1: moe.MXFP4Weight
    w2: moe.MXFP4Weight

    @property
    def k(self) -> int:
        return self.inp.cfg.k

    @property
    def E(self) -> int:
        return self.inp.cfg.E


def device_layer(inp: synth.MoEInputs, with_bias: bool = True, tiled: bool = False) -> DevLayer:
    x = to_dev_bf16(inp.x)
    router = moe.Router(to_dev_f32(inp.router_w), to_dev_f32(inp.router_b))
    w1 = moe.MXFP4Weight(to_dev_u8(inp.w1_codes), to_dev_u8(inp.w1_scales),
                         to_dev_bf16(inp.w1_bias) if with_bias else None)
    w2 = moe.MXFP4Weight(to_dev_u8(inp.w2_codes), to_dev_u8(inp.w2_scales),
                         to_dev_bf16(inp.w2_bias) if with_bias else None)
    if tiled:
        w1, w2 = moe.moe_mxfp4_pack(w1), moe.moe_mxfp4_pack(w2)
    return DevLayer(inp, x, router, w1, w2)


def tiled_reference(codes: np.ndarray, scales: np.ndarray):
    """The tiled layout re-derived with numpy reshapes, independently of the library:
    tile (e, G, c) = half p, lane l -> block 4c + 2p + l//32 of row 32G + l%32; scales per
    tile: 32 rows x 4 blocks."""
    E, N, KH = codes.shape
    KB = scales.shape[2]
    nchunk = (KB + 3) // 4
    c = np.zeros((E, N, nchunk * 64), np.uint8)
    c[:, :, :KH] = codes
    sc = np.full((E, N, nchunk * 4), 127, np.uint8)
    sc[:, :, :KB] = scales
    # row bytes of chunk c: block (2p + kh) * 16 + byte; tile order: e, G, c, p, lane (kh, r), byte
    c = c.reshape(E, N // 32, 32, nchunk, 2, 2, 16).transpose(0, 1, 3, 4, 5, 2, 6)
    sc = sc.reshape(E, N // 32, 32, nchunk, 4).transpose(0, 1, 3, 2, 4)
    return np.ascontiguousarray(c).reshape(-1), np.ascontiguousarray(sc).reshape(-1)


def oracle_experts(inp: synth.MoEInputs, with_bias: bool = True):
    b1 = inp.w1_bias if with_bias else None
    b2 = inp.w2_bias if with_bias else None
    return oracle.experts_from_arrays(inp.w1_codes, inp.w1_scales, b1, inp.w2_codes, inp.w2_scales, b2)


def near_tie_tokens(logits: np.ndarray, k: int, gap: float = TIE_GAP) -> np.ndarray:
    """Tokens whose k-th and (k+1)-th largest fp64 logits differ by less than ``gap``."""
    E = logits.shape[1]
    if k >= E:
        return np.zeros(logits.shape[0], bool)
    s = -np.sort(-logits, axis=1)
    return (s[:, k - 1] - s[:, k]) < gap


def check_routing(gpu_idx: np.ndarray, gpu_w: np.ndarray, ref_logits: np.ndarray, k: int):
    """Indices bit-exact except near-tie tokens (checked for validity instead); weights within
    W_TOL of the softmax of the fp64 logits at the GPU's picks."""
    ref_idx = oracle.topk_select(ref_logits, k)
    tie = near_tie_tokens(ref_logits, k)
    bad = np.nonzero((gpu_idx != ref_idx).any(1) & ~tie)[0]
    assert bad.size == 0, f"{bad.size} tokens route differently, first {bad[:5]}: " \
                          f"gpu {gpu_idx[bad[:1]]} oracle {ref_idx[bad[:1]]}"
    for t in np.nonzero(tie)[0]:  # any valid top-k choice: distinct ids, scores within the gap
        assert len(set(gpu_idx[t].tolist())) == k
        kth = -np.sort(-ref_logits[t])[k - 1]
        assert np.all(ref_logits[t, gpu_idx[t]] >= kth - TIE_GAP)
    sel = np.take_along_axis(ref_logits, gpu_idx.astype(np.int64), axis=1)
    ref_w = oracle.softmax_selected(sel)
    assert np.abs(gpu_w - ref_w).max() <= W_TOL, np.abs(gpu_w - ref_w).max()
    assert np.abs(gpu_w.sum(1) - 1.0).max() <= 1e-6
    return tie


def oracle_forward(inp: synth.MoEInputs, gpu_idx: Optional[np.ndarray], tokens: Optional[Sequence[int]] = None,
                   with_bias: bool = True, limit: float = 7.0, alpha: float = 1.0,
                   keep_intermediates: bool = False) -> oracle.MoEResult:
    """Oracle output; tokens whose routing nearly ties are recomputed with the GPU's picks."""
    get = oracle_experts(inp, with_bias)
    res = oracle.moe_layer(inp.x, inp.router_w, inp.router_b, get, inp.cfg.k, limit, alpha, tokens=tokens,
                           keep_intermediates=keep_intermediates)
    if gpu_idx is None:
        return res
    tok = res.tokens
    tie = near_tie_tokens(res.logits, inp.cfg.k) & (gpu_idx[tok] != res.idx).any(1)
    if tie.any():
        sub = tok[tie]
        forced = oracle.moe_layer(inp.x, inp.router_w, inp.router_b, get, inp.cfg.k, limit, alpha,
                                  tokens=sub, forced_idx=gpu_idx[sub], keep_intermediates=keep_intermediates)
        res.out[tie] = forced.out
        res.idx[tie] = forced.idx
        res.w[tie] = forced.w
        if keep_intermediates:
            res.h[tie] = forced.h
            res.act[tie] = forced.act
    return res


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |v| (the rounding bound of a bf16 output)."""
    a = np.abs(v).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 1e-38)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def check_output(gpu_out: np.ndarray, ref_out: np.ndarray, bf16: bool, tol: float = OUT_TOL):
    """max|gpu - ref| <= tol * RMS(ref) (+ half a bf16 ulp of ref for bf16 outputs)."""
    rms = float(np.sqrt(np.mean(ref_out ** 2)))
    err = np.abs(gpu_out.astype(np.float64) - ref_out)
    bound = tol * rms + (bf16_half_ulp(ref_out) if bf16 else 0.0)
    worst = float((err - bound).max())
    assert worst <= 0.0, f"max err {err.max():.4g} (rms {rms:.4g}, rel {err.max() / rms:.4g}) exceeds bound"
    return float(err.max() / rms)


def act_rounded_layer(inp: synth.MoEInputs, res: oracle.MoEResult, with_bias: bool = True) -> np.ndarray:
    """The layer's output with the activation rounded to bf16 between the two products (the
    layer's specified precision, which the oracle does not apply), built here from the oracle's
    own intermediates (res needs keep_intermediates): y = W2 bf16(a) + b2, summed over the picks
    in rank order. Used only as the reference of degenerate shapes (one expert, a down projection
    of at most 64 terms), where that rounding alone can move an output by ~2% of the RMS."""
    a = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(res.act))  # [n][k][I]
    n, k = res.idx.shape
    y = np.zeros((n, k, res.out.shape[1]), np.float64)
    for e in np.unique(res.idx):
        rows, ranks = np.nonzero(res.idx == e)
        W2 = oracle.mxfp4_decode(inp.w2_codes[e], inp.w2_scales[e])
        ye = a[rows, ranks] @ W2.T
        if with_bias:
            ye = ye + oracle.bf16_to_f64(inp.w2_bias[e])[None, :]
        y[rows, ranks] = ye
    out = np.zeros_like(res.out)
    for j in range(k):
        out += res.w[:, j:j + 1] * y[:, j, :]
    return out
