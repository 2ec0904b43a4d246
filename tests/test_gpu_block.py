"""GPU parity of the block wrap around the layer: RMSNorm (moe_rmsnorm) and
out = x + layer(bf16(RMSNorm(x))) (moe_block_forward_ex), called through the C ABI, against
the fp64 oracle.

Bars: the normalised row bit-exact except elements whose exact value lies within fp32
rounding of a bf16 rounding boundary (those one bf16 step away); routing and outputs as for
the layer (indices bit-exact except near-ties, outputs within 2e-2 x RMS of the layer's
output plus half a bf16 ulp for bf16 outputs); and, kernel against kernel, the block equal
bit for bit to the layer run on the normalised rows with x added in fp32.
"""
import sys

import numpy as np
import pytest
import torch

import gpu_util as gu
import oracle
import synth

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("sparse_moe_transformer_router_amd")

EPS = 1e-5


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def _check_norm_bits(gpu_bits, x_bits, scale, eps=EPS):
    """GPU normalised rows against the exactly rounded oracle values."""
    ref = oracle.rms_norm(oracle.bf16_to_f64(x_bits), scale, eps)
    want = oracle.f64_to_bf16_bits(ref)
    diff = gpu_bits != want
    if diff.any():
        g = gpu_bits[diff].astype(np.int64)
        w = want[diff].astype(np.int64)
        assert np.all(np.abs(g - w) == 1), "normalised values more than one bf16 step apart"
        mid = (oracle.bf16_to_f64(gpu_bits[diff]) + oracle.bf16_to_f64(want[diff])) / 2
        r = ref[diff]
        assert np.all(np.abs(r - mid) <= 2.0 ** -17 * np.abs(r)), "a differing element is not near a tie"
    assert diff.sum() <= max(2, 2e-3 * diff.size), diff.sum()
    return int(diff.sum())


WIDE = synth.LayerConfig("wide", (20,), 4608, 64, 4, 2, 41, scale_bytes=(119, 123))  # rows past 4096


def _block_layer(name, T, tiled=True):
    cfg = WIDE if name == "wide" else synth.get_config(name)
    inp = synth.make_inputs(cfg, T)
    inp.x = synth.make_block_x(cfg, T)
    scale = synth.make_norm_scale(cfg)
    dev = gu.device_layer(inp, tiled=tiled)
    return inp, scale, dev, gu.to_dev_f32(scale)


@pytest.mark.parametrize("name,T", [("tiny", 16), ("decode20b", 1), ("decode20b", 37), ("decode20b", 64),
                                    ("prefill20b", 4096)])
def test_rmsnorm_matches_oracle(name, T):
    cfg = synth.get_config(name)
    x = synth.make_block_x(cfg, T)
    scale = synth.make_norm_scale(cfg)
    out = moe.moe_rmsnorm(gu.to_dev_bf16(x), gu.to_dev_f32(scale), EPS)
    _check_norm_bits(gu.bf16_bits(out), x, scale)


@pytest.mark.parametrize("H", [32, 160, 2880, 4096, 8192])
def test_rmsnorm_edge_rows(H):
    """Rows of one repeated value, a zero row with eps > 0 (zeros out), large and small
    magnitudes (2^+-40: the fp32 sum of squares stays finite and normal), and eps = 0 (the
    pages' plain RMS)."""
    rng = np.random.default_rng(H)
    scale = rng.uniform(0.5, 1.5, H).astype(np.float32)
    rows = [np.full(H, 3.0), np.full(H, -0.015625), np.zeros(H),
            rng.standard_normal(H) * 2.0 ** 40, rng.standard_normal(H) * 2.0 ** -40]
    x = synth.bf16_bits_from_f32(np.stack(rows).astype(np.float32))
    for eps in (EPS, 0.0):
        take = slice(None) if eps > 0 else [0, 1, 3, 4]  # eps = 0 on a zero row is 0 / 0
        xs = np.ascontiguousarray(x[take])
        out = gu.bf16_bits(moe.moe_rmsnorm(gu.to_dev_bf16(xs), gu.to_dev_f32(scale), eps))
        _check_norm_bits(out, xs, scale, eps)
    zero_row = gu.bf16_bits(moe.moe_rmsnorm(gu.to_dev_bf16(x[2:3]), gu.to_dev_f32(scale), EPS))
    assert np.all(zero_row == 0)


def _gpu_block(dev, scale_d, out_dtype, path=0):
    return moe.moe_block_forward_ex(dev.x, scale_d, EPS, dev.router, dev.w1, dev.w2, dev.k,
                                    moe.Options(out_dtype=out_dtype, path=path))


@pytest.mark.parametrize("name,T,path", [("tiny", 16, 0), ("tiny", 16, 1), ("tiny", 16, 2), ("tiny", 16, 3),
                                         ("decode20b", 64, 0), ("decode20b", 1024, 2), ("decode20b", 1024, 3),
                                         ("decode20b", 3, 3), ("prefill20b", 4096, 0), ("wide", 20, 0),
                                         ("wide", 20, 3), ("tiny", 16, 4), ("decode20b", 1024, 4),
                                         ("wide", 20, 4), ("decode20b", 1, 0), ("decode20b", 1, 5)])
# (paths 4 and 5: kernel against kernel, any shape)
def test_block_equals_layer_on_normalised_rows(name, T, path):
    """Kernel against kernel: the block's fp32 output is the layer's fp32 output on
    moe_rmsnorm's rows plus x, bit for bit (so the records the normalisation writes for the
    block-scaled GEMM equal the gather's, and the residual is one fp32 add); the bf16 output
    is that fp32 value rounded to nearest even."""
    inp, scale, dev, scale_d = _block_layer(name, T)
    xn = moe.moe_rmsnorm(dev.x, scale_d, EPS)
    lay = moe.moe_forward_ex(xn, dev.router, dev.w1, dev.w2, dev.k,
                             moe.Options(out_dtype=moe.MOE_DTYPE_F32, path=path))
    want = (lay + dev.x.float()).cpu().numpy()
    got = _gpu_block(dev, scale_d, moe.MOE_DTYPE_F32, path).cpu().numpy()
    assert np.array_equal(got, want)
    got16 = gu.bf16_bits(_gpu_block(dev, scale_d, moe.MOE_DTYPE_BF16, path))
    assert np.array_equal(got16, synth.bf16_bits_from_f32(want))


def _check_block(name, T, path=0, tokens=None, tiled=True):
    inp, scale, dev, scale_d = _block_layer(name, T, tiled)
    k = inp.cfg.k
    xn_d = moe.moe_rmsnorm(dev.x, scale_d, EPS)
    xn = gu.bf16_bits(xn_d)
    nerr = _check_norm_bits(xn, inp.x, scale)
    gidx, gw = moe.moe_route(xn_d, dev.router, k)
    gidx = gidx.cpu().numpy()
    get = gu.oracle_experts(inp)
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    ref = oracle.moe_block(inp.x, scale, EPS, inp.router_w, inp.router_b, get, k, tokens=tok)
    # rows where the GPU rounded an element of the normalised row the other way (checked just
    # above: one step, at an element within fp32 rounding of a tie) are recomputed on the GPU's
    # row, as tokens whose experts nearly tie are recomputed with the GPU's choice below
    xn_used = ref.xn_bits.copy()
    dif = (xn[tok] != ref.xn_bits).any(1)
    if dif.any():
        f = oracle.moe_block(inp.x, scale, EPS, inp.router_w, inp.router_b, get, k, tokens=tok[dif],
                             forced_xn_bits=xn[tok[dif]])
        xn_used[dif] = f.xn_bits
        ref.out[dif] = f.out
        for a in ("out", "logits", "idx", "w"):
            getattr(ref.moe, a)[dif] = getattr(f.moe, a)
    gu.check_routing(gidx[tok], gw.cpu().numpy()[tok], ref.moe.logits, k)
    tie = gu.near_tie_tokens(ref.moe.logits, k) & (gidx[tok] != ref.moe.idx).any(1)
    if tie.any():
        forced = oracle.moe_block(inp.x, scale, EPS, inp.router_w, inp.router_b, get, k, tokens=tok[tie],
                                  forced_idx=gidx[tok[tie]],
                                  forced_xn_bits=xn_used[tie] if dif[tie].any() else None)
        ref.out[tie] = forced.out
        ref.moe.out[tie] = forced.moe.out
    x64 = oracle.bf16_to_f64(inp.x[tok])
    out32 = _gpu_block(dev, scale_d, moe.MOE_DTYPE_F32, path).cpu().numpy()[tok]
    assert np.isfinite(out32).all()
    # the residual is exact, so the bar is the layer's: 2e-2 x RMS of the layer's output
    gu.check_output(out32 - x64, ref.moe.out, bf16=False)
    out16 = synth.f32_from_bf16_bits(gu.bf16_bits(_gpu_block(dev, scale_d, moe.MOE_DTYPE_BF16, path)))[tok]
    err = np.abs(out16.astype(np.float64) - ref.out)
    bound = gu.OUT_TOL * float(np.sqrt(np.mean(ref.moe.out ** 2))) + gu.bf16_half_ulp(ref.out)
    assert float((err - bound).max()) <= 0.0, err.max()
    return nerr


@pytest.mark.parametrize("tiled,path", [(False, 0), (True, 0), (True, 2), (True, 3)])
def test_block_tiny(tiled, path):
    _check_block("tiny", 16, path, tiled=tiled)


@pytest.mark.parametrize("T", [1, 64])
def test_block_decode20b(T):
    _check_block("decode20b", T)


def test_block_wide_rows():
    _check_block("wide", 20, 3)


def test_block_decode120b_zipf():
    _check_block("decode120b_zipf", 256)


@pytest.mark.parametrize("path", [0, 4])
def test_block_prefill20b_full(path):
    """All 4096 tokens of the block at the 20b prefill shape (AUTO: the normalisation writes
    the block-scaled GEMM's records; path 4 gathers MXFP6 records from the normalised rows)."""
    _check_block("prefill20b", 4096, path)


def test_block_in_place():
    """out = x: the residual update in place gives the same bits as a separate output."""
    for name, T in [("decode20b", 64), ("prefill20b", 4096)]:
        inp, scale, dev, scale_d = _block_layer(name, T)
        want = gu.bf16_bits(_gpu_block(dev, scale_d, moe.MOE_DTYPE_BF16))
        x = dev.x.clone()
        moe.moe_block_forward_ex(x, scale_d, EPS, dev.router, dev.w1, dev.w2, dev.k, moe.Options(), out=x)
        assert np.array_equal(gu.bf16_bits(x), want), name
