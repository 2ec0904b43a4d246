"""The seeded input generators: determinism, layout, and the routing shape of each workload."""
import numpy as np

import oracle
import synth


def test_expert_regeneration_matches_stack():
    cfg = synth.get_config("tiny")
    full = synth.make_inputs(cfg)
    for e in (0, 3, cfg.E - 1):
        ew = synth.make_expert(cfg, e)
        assert np.array_equal(ew.w1_codes, full.w1_codes[e])
        assert np.array_equal(ew.w1_scales, full.w1_scales[e])
        assert np.array_equal(ew.w2_bias, full.w2_bias[e])
    again = synth.make_inputs(cfg)
    assert np.array_equal(again.x, full.x) and np.array_equal(again.router_w, full.router_w)


def test_shapes_and_ranges():
    cfg = synth.get_config("tiny")
    inp = synth.make_inputs(cfg)
    E, H, I = cfg.E, cfg.H, cfg.I
    assert inp.x.shape == (16, H) and inp.x.dtype == np.uint16
    assert inp.w1_codes.shape == (E, 2 * I, H // 2) and inp.w1_scales.shape == (E, 2 * I, H // 32)
    assert inp.w2_codes.shape == (E, H, I // 2) and inp.w2_scales.shape == (E, H, I // 32)
    assert inp.w1_scales.min() >= 123 and inp.w1_scales.max() <= 127
    x = oracle.bf16_to_f64(inp.x)
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05
    assert abs(inp.router_w.std() - 0.02) < 0.002
    # every nibble value occurs (uniform codes)
    nib = np.concatenate([(inp.w1_codes & 15).ravel(), (inp.w1_codes >> 4).ravel()])
    assert np.bincount(nib, minlength=16).min() > 0


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -7 + 2 ** -9, -2.5], np.float32)
    got = synth.f32_from_bf16_bits(synth.bf16_bits_from_f32(v))
    assert got.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5]


def test_prefill_loads_within_band():
    for name in ("prefill20b", "prefill120b"):
        cfg = synth.get_config(name)
        T = cfg.T_list[-1]
        x = synth.make_x(cfg, T)
        w, b = synth.make_router(cfg)
        _, idx, _ = oracle.route(x, w, b, cfg.k)
        c = np.bincount(idx.ravel(), minlength=cfg.E)
        mean = T * cfg.k / cfg.E
        assert c.min() >= 0.8 * mean and c.max() <= 1.2 * mean, (name, c.min(), c.max())


def test_zipf_decode_is_skewed():
    cfg = synth.get_config("decode120b_zipf")
    w, b = synth.make_router(cfg)
    x = synth.make_x(cfg, 256)
    _, idx, _ = oracle.route(x, w, b, cfg.k)
    c = np.bincount(idx.ravel(), minlength=cfg.E)
    assert c.max() >= 0.2 * 256  # the hot expert sees (almost) every token
    assert (c == 0).sum() >= 10  # many cold experts
