"""torch-tensor front end of the C ABI: one function per entry point, same names.

Argument marshalling only (device pointers, sizes, the current HIP stream); every step of
the layer runs in libmoe_mxfp4.so. Tensors must already live on the GPU; bf16 tensors are
torch.bfloat16 (passed as their bit patterns).
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional, Tuple

import torch

from . import _lib as L


@dataclasses.dataclass
class MXFP4Weight:
    """One MXFP4 matrix for all experts. Row-major: codes uint8 [E][n][k/2], scales uint8
    [E][n][k/32]; tiled (from moe_mxfp4_pack): flat uint8 buffers, with n and k given.
    bias bf16 [E][n] or None."""
    codes: torch.Tensor
    scales: torch.Tensor
    bias: Optional[torch.Tensor]
    layout: int = L.MOE_LAYOUT_ROWMAJOR
    shape_nk: Optional[Tuple[int, int]] = None  # (n, k) for the tiled layout

    @property
    def n(self) -> int:
        return self.shape_nk[0] if self.shape_nk else int(self.codes.shape[1])

    @property
    def k(self) -> int:
        return self.shape_nk[1] if self.shape_nk else int(self.codes.shape[2]) * 2

    def desc(self) -> L.MoeMxfp4Weight:
        return L.MoeMxfp4Weight(_ptr(self.codes), _ptr(self.scales), _ptr(self.bias), self.n, self.k,
                                self.layout)


@dataclasses.dataclass
class Router:
    """Linear router: weight fp32 [E][H], bias fp32 [E] or None."""
    weight: torch.Tensor
    bias: Optional[torch.Tensor]

    def desc(self) -> L.MoeRouter:
        return L.MoeRouter(_ptr(self.weight), _ptr(self.bias))


@dataclasses.dataclass
class Options:
    swiglu_limit: float = 7.0
    swiglu_alpha: float = 1.0
    out_dtype: int = L.MOE_DTYPE_BF16
    path: int = L.MOE_PATH_AUTO
    flags: int = 0

    def desc(self) -> L.MoeOptions:
        return L.MoeOptions(self.swiglu_limit, self.swiglu_alpha, self.out_dtype, self.path, self.flags)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the MoE library must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr() or None


def _stream(stream: Optional[torch.cuda.Stream]) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _empty(shape, dtype, device, stream: Optional[torch.cuda.Stream]) -> torch.Tensor:
    """A new device tensor allocated on the stream the library will launch on. torch's caching
    allocator ties a block to the stream it was allocated on: a temporary allocated on another
    stream and freed when the call returns could be handed to that stream's next work while the
    library's kernels, queued on `stream`, still use it."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def abi_version() -> int:
    return int(L.lib().moe_abi_version())


def moe_workspace_size(T: int, E: int, k: int, H: int, I: int, path: int = L.MOE_PATH_AUTO) -> int:
    return int(L.lib().moe_workspace_size(T, E, k, H, I, path))


def workspace(T: int, E: int, k: int, H: int, I: int, path: int = L.MOE_PATH_AUTO,
              device=None, stream=None) -> torch.Tensor:
    """A caller-owned workspace tensor of the size the library asks for (torch's allocator
    returns 256-byte aligned blocks), allocated on `stream` (None: the current stream)."""
    n = moe_workspace_size(T, E, k, H, I, path)
    if n == 0:
        raise ValueError("invalid sizes for a workspace")
    return _empty(n, torch.uint8, device or "cuda", stream)


def moe_mxfp4_tiled_bytes(E: int, n: int, k: int) -> Tuple[int, int]:
    cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    L.check("moe_mxfp4_tiled_bytes", L.lib().moe_mxfp4_tiled_bytes(E, n, k, ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def moe_mxfp4_pack(w: MXFP4Weight, stream=None) -> MXFP4Weight:
    """A tiled copy of a row-major weight (new device buffers; the bias tensor is shared)."""
    E = int(w.codes.shape[0])
    cb, sb = moe_mxfp4_tiled_bytes(E, w.n, w.k)
    codes = _empty(cb, torch.uint8, w.codes.device, stream)
    scales = _empty(sb, torch.uint8, w.codes.device, stream)
    d = w.desc()
    L.check("moe_mxfp4_pack", L.lib().moe_mxfp4_pack(ctypes.byref(d), E, _ptr(codes), _ptr(scales),
                                                        _stream(stream)))
    return MXFP4Weight(codes, scales, w.bias, L.MOE_LAYOUT_TILED, (w.n, w.k))


def moe_mxfp4_dequant(codes: torch.Tensor, scales: torch.Tensor, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    n = codes.numel() * 2
    if out is None:
        out = _empty(n, torch.float32, codes.device, stream)
    L.check("moe_mxfp4_dequant", L.lib().moe_mxfp4_dequant(_ptr(codes), _ptr(scales), n, _ptr(out),
                                                              _stream(stream)))
    return out


def moe_route(x: torch.Tensor, router: Router, k: int, topk_idx=None, topk_w=None, ws=None,
              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    T, H = x.shape
    E = int(router.weight.shape[0])
    if topk_idx is None:
        topk_idx = _empty((T, k), torch.int32, x.device, stream)
    if topk_w is None:
        topk_w = _empty((T, k), torch.float32, x.device, stream)
    if ws is None:
        ws = workspace(T, E, k, H, H, device=x.device, stream=stream)
    r = router.desc()
    L.check("moe_route", L.lib().moe_route(_ptr(x), T, H, ctypes.byref(r), E, k, _ptr(topk_idx),
                                              _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream)))
    return topk_idx, topk_w


def moe_permute(topk_idx: torch.Tensor, E: int, out=None, ws=None, stream=None
                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """ws: optional workspace (uint8 tensor); with it, more than 8192 slots are sorted by
    several workgroups (same result)."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    if out is None:
        out = (_empty(E + 1, torch.int32, dev, stream), _empty(T * k, torch.int32, dev, stream),
               _empty(T * k, torch.int32, dev, stream))
    offsets, sorted_slot, slot_row = out
    L.check("moe_permute", L.lib().moe_permute(_ptr(topk_idx), T, E, k, _ptr(offsets), _ptr(sorted_slot),
                                                  _ptr(slot_row), _ptr(ws), 0 if ws is None else ws.numel(),
                                                  _stream(stream)))
    return offsets, sorted_slot, slot_row


def moe_mxfp4_ffn(x: torch.Tensor, k: int, E: int, expert_offsets: torch.Tensor, sorted_slot: torch.Tensor,
                  gate_up: MXFP4Weight, down: MXFP4Weight, opts: Optional[Options] = None,
                  y: Optional[torch.Tensor] = None, ws=None, stream=None) -> torch.Tensor:
    T, H = x.shape
    I = down.k
    o = opts or Options()
    width = {L.MOE_FLAG_EMIT_PREACT: 2 * I, L.MOE_FLAG_EMIT_ACT: I}.get(o.flags, H)
    if y is None:
        y = _empty((T * k, width), torch.float32, x.device, stream)
    if ws is None:
        ws = workspace(T, E, k, H, I, o.path, device=x.device, stream=stream)
    g, d, od = gate_up.desc(), down.desc(), o.desc()
    L.check("moe_mxfp4_ffn", L.lib().moe_mxfp4_ffn(
        _ptr(x), T, k, E, _ptr(expert_offsets), _ptr(sorted_slot), ctypes.byref(g), ctypes.byref(d),
        ctypes.byref(od), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))
    return y


def moe_combine(y: torch.Tensor, slot_row: torch.Tensor, topk_w: torch.Tensor,
                out_dtype: int = L.MOE_DTYPE_BF16, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    T, k = topk_w.shape
    H = int(y.shape[1])
    if out is None:
        dt = torch.bfloat16 if out_dtype == L.MOE_DTYPE_BF16 else torch.float32
        out = _empty((T, H), dt, y.device, stream)
    L.check("moe_combine", L.lib().moe_combine(_ptr(y), _ptr(slot_row), _ptr(topk_w), T, k, H, _ptr(out),
                                                  out_dtype, _stream(stream)))
    return out


def moe_forward(x: torch.Tensor, router: Router, w_gate_up: MXFP4Weight, w_down: MXFP4Weight, k: int,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    T, H = x.shape
    E = int(router.weight.shape[0])
    if out is None:
        out = _empty((T, H), torch.bfloat16, x.device, stream)
    r, g, d = router.desc(), w_gate_up.desc(), w_down.desc()
    L.check("moe_forward", L.lib().moe_forward(_ptr(x), ctypes.byref(r), ctypes.byref(g), ctypes.byref(d),
                                                  T, E, k, _ptr(out), _stream(stream)))
    return out


def moe_forward_noalloc(x: torch.Tensor, router: Router, w_gate_up: MXFP4Weight, w_down: MXFP4Weight, k: int,
                        out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_forward with the library's fixed device scratch as its workspace (no allocation in the
    library; `out` is allocated here only if it is not given)."""
    T, H = x.shape
    E = int(router.weight.shape[0])
    if out is None:
        out = _empty((T, H), torch.bfloat16, x.device, stream)
    r, g, d = router.desc(), w_gate_up.desc(), w_down.desc()
    L.check("moe_forward_noalloc", L.lib().moe_forward_noalloc(_ptr(x), ctypes.byref(r), ctypes.byref(g),
                                                                  ctypes.byref(d), T, E, k, _ptr(out),
                                                                  _stream(stream)))
    return out


def moe_forward_ex(x: torch.Tensor, router: Router, w_gate_up: MXFP4Weight, w_down: MXFP4Weight, k: int,
                   opts: Optional[Options] = None, out: Optional[torch.Tensor] = None, ws=None,
                   stream=None) -> torch.Tensor:
    T, H = x.shape
    E = int(router.weight.shape[0])
    o = opts or Options()
    if out is None:
        dt = torch.bfloat16 if o.out_dtype == L.MOE_DTYPE_BF16 else torch.float32
        out = _empty((T, H), dt, x.device, stream)
    if ws is None:
        ws = workspace(T, E, k, H, w_down.k, o.path, device=x.device, stream=stream)
    r, g, d, od = router.desc(), w_gate_up.desc(), w_down.desc(), o.desc()
    L.check("moe_forward_ex", L.lib().moe_forward_ex(
        _ptr(x), ctypes.byref(r), ctypes.byref(g), ctypes.byref(d), T, E, k, ctypes.byref(od), _ptr(out),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out


def moe_rmsnorm(x: torch.Tensor, scale: torch.Tensor, eps: float = 1e-5, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """bf16(x / sqrt(mean(x^2) + eps) * scale) per row; x bf16 [T][H], scale fp32 [H]."""
    T, H = x.shape
    if out is None:
        out = _empty((T, H), torch.bfloat16, x.device, stream)
    L.check("moe_rmsnorm", L.lib().moe_rmsnorm(_ptr(x), T, H, _ptr(scale), float(eps), _ptr(out),
                                                  _stream(stream)))
    return out


def moe_block_forward_ex(x: torch.Tensor, norm_scale: torch.Tensor, norm_eps: float, router: Router,
                         w_gate_up: MXFP4Weight, w_down: MXFP4Weight, k: int, opts: Optional[Options] = None,
                         out: Optional[torch.Tensor] = None, ws=None, stream=None) -> torch.Tensor:
    """x + layer(bf16(RMSNorm(x))): the MoE half of a decoder block."""
    T, H = x.shape
    E = int(router.weight.shape[0])
    o = opts or Options()
    if out is None:
        dt = torch.bfloat16 if o.out_dtype == L.MOE_DTYPE_BF16 else torch.float32
        out = _empty((T, H), dt, x.device, stream)
    if ws is None:
        ws = workspace(T, E, k, H, w_down.k, o.path, device=x.device, stream=stream)
    r, g, d, od = router.desc(), w_gate_up.desc(), w_down.desc(), o.desc()
    L.check("moe_block_forward_ex", L.lib().moe_block_forward_ex(
        _ptr(x), _ptr(norm_scale), float(norm_eps), ctypes.byref(r), ctypes.byref(g), ctypes.byref(d), T, E, k,
        ctypes.byref(od), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def moe_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, lens: torch.Tensor,
                    sinks: Optional[torch.Tensor] = None, window: int = 0, out_dtype: int = L.MOE_DTYPE_BF16,
                    out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """One decode step of grouped-query attention with per-head sinks: q [B][Hq][64] bf16, caches
    [B][Hkv][L][64] bf16, lens [B] int32, sinks [Hq] fp32 or None; window 0 = dense."""
    B, Hq, D = q.shape
    Hkv, Lmax = int(k_cache.shape[1]), int(k_cache.shape[2])
    if out is None:
        dt = torch.bfloat16 if out_dtype == L.MOE_DTYPE_BF16 else torch.float32
        out = _empty((B, Hq, D), dt, q.device, stream)
    if ws is None:
        ws = _empty(int(L.lib().moe_attn_workspace_size(B, Hkv, Lmax, window)), torch.uint8, q.device, stream)
    L.check("moe_attn_decode", L.lib().moe_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens), _ptr(sinks), B, Hq, Hkv, D, Lmax, window, _ptr(out),
        out_dtype, _ptr(ws), ws.numel(), _stream(stream)))
    return out


def moe_release_workspace() -> None:
    L.check("moe_release_workspace", L.lib().moe_release_workspace())
