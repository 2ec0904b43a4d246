"""GPU parity of the decode attention step (moe_attn_decode: grouped-query attention with
per-head sink logits, banded or dense window), called through the C ABI, against the fp64
oracle.

Bar (derived from the arithmetic: fp32 scores of exact bf16 products, fp32 exponentials and
sums, weights entering the value sum as two bf16 terms, ~2^-17 relative): max-abs error
<= 1e-4 x RMS of the oracle output for fp32 outputs, plus half a bf16 ulp of the oracle
value for bf16 outputs.
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

ATTN_TOL = 1e-4


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def _dev(inp):
    return (gu.to_dev_bf16(inp.q), gu.to_dev_bf16(inp.k), gu.to_dev_bf16(inp.v),
            torch.from_numpy(inp.lens).to("cuda"), gu.to_dev_f32(inp.sinks))


def _check(inp, window, with_sink=True, check_bf16=True):
    q, k, v, lens, sinks = _dev(inp)
    ref = oracle.attention_decode(oracle.bf16_to_f64(inp.q), oracle.bf16_to_f64(inp.k), oracle.bf16_to_f64(inp.v),
                                  inp.lens, inp.sinks if with_sink else None, window)
    out = moe.moe_attn_decode(q, k, v, lens, sinks if with_sink else None, window,
                              out_dtype=moe.MOE_DTYPE_F32).cpu().numpy()
    assert np.isfinite(out).all()
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(out.astype(np.float64) - ref)
    assert err.max() <= ATTN_TOL * rms, (err.max(), rms)
    if check_bf16:
        o16 = synth.f32_from_bf16_bits(gu.bf16_bits(moe.moe_attn_decode(q, k, v, lens, sinks if with_sink else None,
                                                                         window)))
        err16 = np.abs(o16.astype(np.float64) - ref)
        assert float((err16 - ATTN_TOL * rms - gu.bf16_half_ulp(ref)).max()) <= 0.0
        # the bf16 output is the fp32 one rounded to nearest even
        assert np.array_equal(gu.bf16_bits(moe.moe_attn_decode(q, k, v, lens, sinks if with_sink else None, window)),
                              synth.bf16_bits_from_f32(out))
    return float(err.max() / rms)


@pytest.mark.parametrize("B,L", [(1, 1), (3, 37), (5, 300), (16, 1000), (2, 4096)])
@pytest.mark.parametrize("window", [0, 128])
def test_attn_gpt_oss_heads(B, L, window):
    """64 query heads over 8 key/value heads, head dimension 64, dense and 128-token band."""
    _check(synth.make_attn_inputs(B, L, seed=B * 7 + L), window)


@pytest.mark.parametrize("window", [1, 7, 255, 256, 257])
def test_attn_window_edges(window):
    """Bands of one position, a few, and around the per-wave range of 256 positions."""
    _check(synth.make_attn_inputs(6, 700, seed=window), window)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 1), (12, 4), (64, 4)])
def test_attn_group_sizes(Hq, Hkv):
    _check(synth.make_attn_inputs(4, 333, Hq=Hq, Hkv=Hkv, seed=Hq + Hkv), 0)


@pytest.mark.parametrize("q_scale", [0.25, 4.0])
def test_attn_score_spread_and_no_sink(q_scale):
    inp = synth.make_attn_inputs(4, 513, seed=11, q_scale=q_scale)
    _check(inp, 0, with_sink=True)
    _check(inp, 0, with_sink=False, check_bf16=False)
    _check(inp, 128, with_sink=False, check_bf16=False)


def test_attn_invisible_positions_are_never_read_into_the_result():
    """Cache positions at or past lens[b] hold NaN: the output stays finite and equal to the
    oracle's, which never sees them."""
    inp = synth.make_attn_inputs(5, 600, seed=3)
    for b in range(5):
        inp.k[b, :, inp.lens[b]:] = 0x7FC0
        inp.v[b, :, inp.lens[b]:] = 0x7FC0
    _check(inp, 0)
    _check(inp, 128)


@pytest.mark.parametrize("with_sink", [True, False])
@pytest.mark.parametrize("window", [0, 128])
def test_attn_zero_length_and_determinism(with_sink, window):
    """A sequence with no visible position gives 0 (with or without sinks, as the oracle does);
    the others match the oracle; a second call gives the same bits."""
    inp = synth.make_attn_inputs(3, 64, seed=5)
    inp.lens[1] = 0
    q, k, v, lens, sinks = _dev(inp)
    out = moe.moe_attn_decode(q, k, v, lens, sinks if with_sink else None, window,
                              out_dtype=moe.MOE_DTYPE_F32).cpu().numpy()
    assert np.all(out[1] == 0.0)
    _check(inp, window, with_sink=with_sink)
    again = moe.moe_attn_decode(q, k, v, lens, sinks if with_sink else None, window,
                                out_dtype=moe.MOE_DTYPE_F32).cpu().numpy()
    assert np.array_equal(out, again)


def test_attn_longest_context():
    """One sequence at the gpt-oss context length (131072 positions: 512 ranges, the
    four-wave merge)."""
    _check(synth.make_attn_inputs(1, 131072, seed=2, full=True), 0)


@pytest.mark.parametrize("window", [0, 128])
def test_attn_bench_configuration(window):
    """The benchmark's launch configuration: 64 sequences, every one at 4096 positions."""
    _check(synth.make_attn_inputs(64, 4096, seed=1, full=True), window)
