"""ctypes loader for libmoe_mxfp4.so, the HIP library of the MXFP4 top-k MoE layer.

torch is imported first so that the process holds one HIP runtime (torch's), which the
library then shares: device pointers and streams from torch are valid inside it. There is
no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # noqa: F401  (must precede the library load: one HIP runtime per process)

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_MXFP4_LIBRARY selects another build of the same library (the host-sanitizer build of the
# C ABI's tests); by default the in-tree build.
LIB_PATH = os.environ.get("MOE_MXFP4_LIBRARY") or os.path.join(_PKG, "lib", "libmoe_mxfp4.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_SCRATCH = -5

MOE_DTYPE_BF16 = 0
MOE_DTYPE_F32 = 1

MOE_PATH_AUTO = 0
MOE_PATH_DECODE = 1
MOE_PATH_PREFILL_BF16 = 2
MOE_PATH_PREFILL_MX8SPLIT = 3
MOE_PATH_PREFILL_MX6SPLIT = 4
MOE_PATH_DECODE_FUSED = 5
# earlier names of the same paths
MOE_PATH_STREAM = MOE_PATH_DECODE
MOE_PATH_GEMM = MOE_PATH_PREFILL_BF16
MOE_PATH_GEMM_MX = MOE_PATH_PREFILL_MX8SPLIT

MOE_LAYOUT_ROWMAJOR = 0
MOE_LAYOUT_TILED = 1

MOE_FLAG_EMIT_PREACT = 1
MOE_FLAG_EMIT_ACT = 2

c_void_p = ctypes.c_void_p
c_int32 = ctypes.c_int32
c_int64 = ctypes.c_int64
c_size_t = ctypes.c_size_t


class MoeRouter(ctypes.Structure):
    _fields_ = [("weight", c_void_p), ("bias", c_void_p)]


class MoeMxfp4Weight(ctypes.Structure):
    _fields_ = [("codes", c_void_p), ("scales", c_void_p), ("bias", c_void_p),
                ("n", c_int32), ("k", c_int32), ("layout", c_int32)]


class MoeOptions(ctypes.Structure):
    _fields_ = [("swiglu_limit", ctypes.c_float), ("swiglu_alpha", ctypes.c_float),
                ("out_dtype", c_int32), ("path", c_int32), ("flags", ctypes.c_uint32)]


# name -> (restype, argtypes); the declarations of include/moe_mxfp4.h
SIGNATURES = {
    "moe_abi_version": (c_int32, []),
    "moe_status_string": (ctypes.c_char_p, [c_int32]),
    "moe_workspace_size": (c_size_t, [c_int64, c_int32, c_int32, c_int32, c_int32, c_int32]),
    "moe_mxfp4_dequant": (c_int32, [c_void_p, c_void_p, c_int64, c_void_p, c_void_p]),
    "moe_mxfp4_tiled_bytes": (c_int32, [c_int32, c_int32, c_int32, ctypes.POINTER(c_size_t),
                                        ctypes.POINTER(c_size_t)]),
    "moe_mxfp4_pack": (c_int32, [ctypes.POINTER(MoeMxfp4Weight), c_int32, c_void_p, c_void_p, c_void_p]),
    "moe_route": (c_int32, [c_void_p, c_int64, c_int32, ctypes.POINTER(MoeRouter), c_int32, c_int32,
                            c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_permute": (c_int32, [c_void_p, c_int64, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_size_t, c_void_p]),
    "moe_mxfp4_ffn": (c_int32, [c_void_p, c_int64, c_int32, c_int32, c_void_p, c_void_p,
                                ctypes.POINTER(MoeMxfp4Weight), ctypes.POINTER(MoeMxfp4Weight),
                                ctypes.POINTER(MoeOptions), c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_combine": (c_int32, [c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_int32, c_void_p,
                              c_int32, c_void_p]),
    "moe_forward": (c_int32, [c_void_p, ctypes.POINTER(MoeRouter), ctypes.POINTER(MoeMxfp4Weight),
                              ctypes.POINTER(MoeMxfp4Weight), c_int64, c_int32, c_int32, c_void_p,
                              c_void_p]),
    "moe_forward_ex": (c_int32, [c_void_p, ctypes.POINTER(MoeRouter), ctypes.POINTER(MoeMxfp4Weight),
                                 ctypes.POINTER(MoeMxfp4Weight), c_int64, c_int32, c_int32,
                                 ctypes.POINTER(MoeOptions), c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_rmsnorm": (c_int32, [c_void_p, c_int64, c_int32, c_void_p, ctypes.c_float, c_void_p, c_void_p]),
    "moe_block_forward_ex": (c_int32, [c_void_p, c_void_p, ctypes.c_float, ctypes.POINTER(MoeRouter),
                                       ctypes.POINTER(MoeMxfp4Weight), ctypes.POINTER(MoeMxfp4Weight),
                                       c_int64, c_int32, c_int32, ctypes.POINTER(MoeOptions), c_void_p,
                                       c_void_p, c_size_t, c_void_p]),
    "moe_attn_workspace_size": (c_size_t, [c_int64, c_int32, c_int64, c_int32]),
    "moe_attn_decode": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_int32,
                                  c_int32, c_int64, c_int32, c_void_p, c_int32, c_void_p, c_size_t, c_void_p]),
    "moe_forward_noalloc": (c_int32, [c_void_p, ctypes.POINTER(MoeRouter), ctypes.POINTER(MoeMxfp4Weight),
                                      ctypes.POINTER(MoeMxfp4Weight), c_int64, c_int32, c_int32, c_void_p,
                                      c_void_p]),
    "moe_noalloc_scratch_bytes": (c_size_t, []),
    "moe_release_workspace": (c_int32, []),
}

_lock = threading.Lock()
_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m sparse_moe_transformer_router_amd.build` (there is no fallback path)")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
        return _lib


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status, lib().moe_status_string(status).decode())
