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


def test_block_and_attention_generators():
    """Seeded, order-independent draws with the documented shapes and laws."""
    import numpy as np
    import synth
    cfg = synth.get_config("decode20b")
    x = synth.make_block_x(cfg, 8)
    assert x.shape == (8, cfg.H) and x.dtype == np.uint16
    assert np.array_equal(x, synth.make_block_x(cfg, 8))
    rms = np.sqrt(np.mean(synth.f32_from_bf16_bits(x).astype(np.float64) ** 2, axis=1))
    assert rms.min() > 0.2 and rms.max() < 4.5 and rms.max() / rms.min() > 1.5  # per-token scales 2^U(-2,2)
    s = synth.make_norm_scale(cfg)
    assert s.shape == (cfg.H,) and s.dtype == np.float32 and 0.5 <= s.min() and s.max() <= 1.5
    a = synth.make_attn_inputs(3, 40, Hq=16, Hkv=2, seed=5)
    assert a.q.shape == (3, 16, 64) and a.k.shape == (3, 2, 40, 64) and a.v.shape == a.k.shape
    assert a.lens[0] == 40 and a.lens.min() >= 1 and a.lens.max() <= 40 and a.sinks.shape == (16,)
    b = synth.make_attn_inputs(3, 40, Hq=16, Hkv=2, seed=5)
    assert all(np.array_equal(getattr(a, f), getattr(b, f)) for f in ("q", "k", "v", "lens", "sinks"))
    assert np.all(synth.make_attn_inputs(4, 10, seed=1, full=True).lens == 10)
