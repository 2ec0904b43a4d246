"""Seeded generators for the layer's inputs.

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence([seed, tensor_id, ...]))``
so that the order in which tensors are generated never changes their values, and any
single expert can be regenerated on its own.

Distributions (the workloads of the gpt-oss pages, stood in for by random data because
trained weights and real hidden states are not available):

* x: bf16(N(0, 1)) per element, a stand-in for RMS-normalised hidden states.
* decode attention (the model's other per-layer hot path): q, k, v = bf16(N(0, 1)) per
  element (q times ``q_scale`` for sharper score distributions), sink logits fp32 N(0, 1),
  per-sequence lengths uniform over 1..L with the first sequence at L.
* block input (the residual stream before the block's RMSNorm): bf16(N(0, 1) * 2^u) with
  one u ~ U(-2, 2) per token, so tokens differ in scale by up to 16x and the normalisation
  matters; RMSNorm scale: fp32 U(0.5, 1.5) per feature.
* router weight: fp32 N(0, 0.02^2); router bias: zero, or a stored calibration vector.
* expert weights: MXFP4 -- every 4-bit code uniform over all 16 codes (so every packed
  byte is uniform over 0..255), one E8M0 scale byte per 32 consecutive input features,
  uniform over ``scale_bytes`` (123..127 means 2^-4 .. 2^0); biases bf16(N(0, 0.01^2)).

Byte layout delivered (the layout the library's weight descriptors expect):

* codes  uint8 [E][N][K/2]: byte j of a row holds element 2j in its low nibble and
  element 2j+1 in its high nibble.
* scales uint8 [E][N][K/32]: byte b scales elements 32b .. 32b+31 of the row.
* gate_up has N = 2*I rows, interleaved: row 2i is the gate of unit i, row 2i+1 its
  linear branch. down has N = H rows and K = I.
"""
from __future__ import annotations

import dataclasses
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

_DATA_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "data")

# tensor ids for SeedSequence keys
_TID_X = 1
_TID_ROUTER_W = 2
_TID_W1_CODES = 10
_TID_W1_SCALES = 11
_TID_W1_BIAS = 12
_TID_W2_CODES = 20
_TID_W2_SCALES = 21
_TID_W2_BIAS = 22
_TID_BLOCK_X = 30
_TID_BLOCK_TOKEN_SCALE = 31
_TID_NORM_SCALE = 32
_TID_ATTN = 40


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(v) for v in key]))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T_list: Tuple[int, ...]
    H: int
    I: int
    E: int
    k: int
    seed: int
    scale_bytes: Tuple[int, int] = (123, 127)  # inclusive range of E8M0 bytes
    router_bias: str = "zero"                  # "zero" or the stem of a file in synth/data
    description: str = ""

    def with_(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny parity case, the 20b-shaped layer at decode and prefill
# batch sizes, the 120b-shaped layer at prefill, and a skewed 120b decode sweep.
CONFIGS: Dict[str, LayerConfig] = {
    "tiny": LayerConfig("tiny", (16,), 256, 256, 8, 4, 0,
                        description="T=16, hidden 256, width 256, E=8, top-4, router bias 0"),
    "decode20b": LayerConfig("decode20b", (1, 8, 32, 64), 2880, 2880, 32, 4, 1,
                             description="20b-shaped layer, decode batches, E=32, top-4"),
    "prefill20b": LayerConfig("prefill20b", (4096,), 2880, 2880, 32, 4, 2,
                              router_bias="balance_prefill20b",
                              description="20b-shaped layer, 4096-token prefill, E=32, "
                                          "per-expert load within +-20% of T*4/32"),
    "prefill120b": LayerConfig("prefill120b", (8192,), 2880, 2880, 128, 4, 3,
                               router_bias="balance_prefill120b",
                               description="120b-shaped layer, 8192-token prefill, E=128, "
                                           "near-uniform routing"),
    "decode120b_zipf": LayerConfig("decode120b_zipf", (1, 16, 64, 256), 2880, 2880, 128, 4, 4,
                                   router_bias="zipf_decode120b",
                                   description="120b-shaped layer, decode batches, E=128, "
                                               "expert popularity ~ Zipf(1.2)"),
}


def get_config(name: str) -> LayerConfig:
    return CONFIGS[name]


def load_router_bias(stem: str, E: int) -> np.ndarray:
    """Read a stored fp32 router-bias vector (one value per line, '#' comments)."""
    path = os.path.join(_DATA_DIR, stem + ".txt")
    vals: List[float] = []
    with open(path, "r", encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.append(float.fromhex(line) if line.startswith(("0x", "-0x")) else float(line))
    b = np.asarray(vals, dtype=np.float32)
    if b.shape != (E,):
        raise ValueError(f"router bias file {path} holds {b.shape[0]} values, expected {E}")
    return b


@dataclasses.dataclass
class ExpertWeights:
    """One expert's MXFP4 tensors (gate_up and down) in the delivered byte layout."""
    w1_codes: np.ndarray   # uint8 [2I][H/2]
    w1_scales: np.ndarray  # uint8 [2I][H/32]
    w1_bias: np.ndarray    # uint16 bf16 bits [2I]
    w2_codes: np.ndarray   # uint8 [H][I/2]
    w2_scales: np.ndarray  # uint8 [H][I/32]
    w2_bias: np.ndarray    # uint16 bf16 bits [H]


@dataclasses.dataclass
class MoEInputs:
    cfg: LayerConfig
    T: int
    x: np.ndarray           # uint16 bf16 bits [T][H]
    router_w: np.ndarray    # float32 [E][H]
    router_b: np.ndarray    # float32 [E]
    w1_codes: np.ndarray    # uint8 [E][2I][H/2]
    w1_scales: np.ndarray   # uint8 [E][2I][H/32]
    w1_bias: np.ndarray     # uint16 [E][2I]
    w2_codes: np.ndarray    # uint8 [E][H][I/2]
    w2_scales: np.ndarray   # uint8 [E][H][I/32]
    w2_bias: np.ndarray     # uint16 [E][H]

    def expert(self, e: int) -> ExpertWeights:
        return ExpertWeights(self.w1_codes[e], self.w1_scales[e], self.w1_bias[e],
                             self.w2_codes[e], self.w2_scales[e], self.w2_bias[e])


def make_x(cfg: LayerConfig, T: int, offset: int = 0) -> np.ndarray:
    """bf16 bits [T][H] ~ N(0,1). ``offset`` selects an independent stream (calibration batches)."""
    g = _rng(cfg.seed, _TID_X, T, offset)
    return bf16_bits_from_f32(g.standard_normal((T, cfg.H), dtype=np.float32))


def make_block_x(cfg: LayerConfig, T: int) -> np.ndarray:
    """bf16 bits [T][H]: the block's input, N(0,1) per element times 2^u per token, u ~ U(-2, 2)."""
    z = _rng(cfg.seed, _TID_BLOCK_X, T).standard_normal((T, cfg.H), dtype=np.float32)
    u = _rng(cfg.seed, _TID_BLOCK_TOKEN_SCALE, T).uniform(-2.0, 2.0, size=(T, 1))
    return bf16_bits_from_f32(z * np.exp2(u).astype(np.float32))


def make_norm_scale(cfg: LayerConfig) -> np.ndarray:
    """fp32 [H]: the RMSNorm's per-feature scale, U(0.5, 1.5)."""
    return _rng(cfg.seed, _TID_NORM_SCALE).uniform(0.5, 1.5, size=cfg.H).astype(np.float32)


@dataclasses.dataclass
class AttnInputs:
    q: np.ndarray       # uint16 bf16 bits [B][Hq][D]
    k: np.ndarray       # uint16 bf16 bits [B][Hkv][L][D]
    v: np.ndarray       # uint16 bf16 bits [B][Hkv][L][D]
    lens: np.ndarray    # int32 [B]
    sinks: np.ndarray   # float32 [Hq]


def make_attn_inputs(B: int, L: int, Hq: int = 64, Hkv: int = 8, D: int = 64, seed: int = 0,
                     q_scale: float = 1.0, full: bool = False) -> AttnInputs:
    """One decode step's attention inputs (key/value caches filled at every position; positions
    at or past lens[b] are not visible). ``full``: every sequence at length L."""
    g = _rng(seed, _TID_ATTN, B, L, Hq, Hkv)
    q = bf16_bits_from_f32(g.standard_normal((B, Hq, D), dtype=np.float32) * np.float32(q_scale))
    k = bf16_bits_from_f32(g.standard_normal((B, Hkv, L, D), dtype=np.float32))
    v = bf16_bits_from_f32(g.standard_normal((B, Hkv, L, D), dtype=np.float32))
    lens = np.full(B, L, np.int32) if full else g.integers(1, L + 1, B).astype(np.int32)
    lens[0] = L
    sinks = g.standard_normal(Hq).astype(np.float32)
    return AttnInputs(q, k, v, lens, sinks)


def make_router(cfg: LayerConfig, bias: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    g = _rng(cfg.seed, _TID_ROUTER_W)
    w = (g.standard_normal((cfg.E, cfg.H), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    if bias is not None:
        b = np.asarray(bias, dtype=np.float32)
    elif cfg.router_bias == "zero":
        b = np.zeros(cfg.E, dtype=np.float32)
    else:
        b = load_router_bias(cfg.router_bias, cfg.E)
    return w, b


def _mx_tensor(cfg: LayerConfig, tid_codes: int, tid_scales: int, tid_bias: int, e: int,
               N: int, K: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    lo, hi = cfg.scale_bytes
    codes = _rng(cfg.seed, tid_codes, e).integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = _rng(cfg.seed, tid_scales, e).integers(lo, hi + 1, size=(N, K // 32), dtype=np.uint8)
    bias = bf16_bits_from_f32(
        _rng(cfg.seed, tid_bias, e).standard_normal(N, dtype=np.float32) * np.float32(0.01))
    return codes, scales, bias


def make_expert(cfg: LayerConfig, e: int) -> ExpertWeights:
    """Regenerate expert ``e`` alone (identical to slice e of make_inputs' tensors)."""
    if cfg.H % 32 or cfg.I % 32:
        raise ValueError("H and I must be multiples of 32")
    c1, s1, b1 = _mx_tensor(cfg, _TID_W1_CODES, _TID_W1_SCALES, _TID_W1_BIAS, e, 2 * cfg.I, cfg.H)
    c2, s2, b2 = _mx_tensor(cfg, _TID_W2_CODES, _TID_W2_SCALES, _TID_W2_BIAS, e, cfg.H, cfg.I)
    return ExpertWeights(c1, s1, b1, c2, s2, b2)


def make_inputs(cfg: LayerConfig, T: Optional[int] = None, experts: Optional[Sequence[int]] = None,
                router_bias: Optional[np.ndarray] = None) -> MoEInputs:
    """All inputs of one layer call. ``experts`` limits weight generation (others left zero)."""
    if T is None:
        T = cfg.T_list[-1]
    x = make_x(cfg, T)
    rw, rb = make_router(cfg, router_bias)
    E, H, I = cfg.E, cfg.H, cfg.I
    w1c = np.zeros((E, 2 * I, H // 2), np.uint8)
    w1s = np.zeros((E, 2 * I, H // 32), np.uint8)
    w1b = np.zeros((E, 2 * I), np.uint16)
    w2c = np.zeros((E, H, I // 2), np.uint8)
    w2s = np.zeros((E, H, I // 32), np.uint8)
    w2b = np.zeros((E, H), np.uint16)
    for e in (range(E) if experts is None else experts):
        ew = make_expert(cfg, e)
        w1c[e], w1s[e], w1b[e] = ew.w1_codes, ew.w1_scales, ew.w1_bias
        w2c[e], w2s[e], w2b[e] = ew.w2_codes, ew.w2_scales, ew.w2_bias
    return MoEInputs(cfg, T, x, rw, rb, w1c, w1s, w1b, w2c, w2s, w2b)
