"""Pins that tie the fp64 oracle to facts outside itself.

Each pin is a plain function that raises AssertionError when the oracle disagrees with
what the pages, the OCP MX specification or mathematics fix. The pins look the oracle's
functions up at call time, so tests/test_oracle_mutations.py can plant a mistake in the
oracle and check that some pin catches it.
"""
from __future__ import annotations

import itertools
import math
import os

import numpy as np

import oracle.moe_oracle as om

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------- fixtures
def _lines(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line.split()


def golden_e2m1():
    return {int(c, 2): float(v) for c, v in _lines("e2m1_table.txt")}


def golden_e8m0():
    out = {}
    for b, v in _lines("e8m0_special.txt"):
        out[int(b)] = float("nan") if v == "nan" else 2.0 ** int(v.split("^")[1])
    return out


def golden_row_example():
    scales, bytes_, elems = None, {}, {}
    for parts in _lines("mxfp4_row_example.txt"):
        if parts[0] == "scales":
            scales = [int(p) for p in parts[1:]]
        elif parts[0] == "byte":
            bytes_[int(parts[1])] = int(parts[2], 16)
        elif parts[0] == "elem":
            elems[int(parts[1])] = float(parts[2])
    return scales, bytes_, elems


def _same(a, b):
    """Equal as floats, including the sign of zero and NaN == NaN."""
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


# --------------------------------------------------------------------------- a0 decode
def pin_e2m1_table():
    table = golden_e2m1()
    assert len(table) == 16
    for c, v in table.items():
        got = om.e2m1_value(c)
        assert _same(got, v), f"E2M1 code {c:04b}: oracle {got}, spec {v}"


def pin_e8m0_special():
    for b, v in golden_e8m0().items():
        got = om.e8m0_value(b)
        assert _same(got, v), f"E8M0 byte {b}: oracle {got}, spec {v}"


def pin_e8m0_ieee_bits():
    """For bytes 1..254 an E8M0 scale is the float32 whose exponent field is that byte and
    whose mantissa is zero -- a route through the IEEE bit layout, not the formula."""
    for b in range(1, 255):
        ieee = float(np.array([b << 23], np.uint32).view(np.float32)[0])
        assert om.e8m0_value(b) == ieee, f"E8M0 byte {b}"


def pin_mxfp4_row_example():
    scales, bytes_, elems = golden_row_example()
    codes = np.zeros((1, 32), np.uint8)
    for i, v in bytes_.items():
        codes[0, i] = v
    dec = om.mxfp4_decode(codes, np.array([scales], np.uint8))
    assert dec.shape == (1, 64)
    for i in range(64):
        want = elems.get(i, 0.0)
        assert _same(float(dec[0, i]), want), f"element {i}: oracle {dec[0, i]}, by hand {want}"


def pin_mxfp4_grid():
    """All 16 codes under all 256 scale bytes, against the spec tables element by element."""
    table = golden_e2m1()
    special = golden_e8m0()
    codes = np.zeros((256, 16), np.uint8)
    codes[:, :8] = np.array([c0 | (c1 << 4) for c0, c1 in zip(range(0, 16, 2), range(1, 16, 2))],
                            np.uint8)
    scales = np.arange(256, dtype=np.uint8)[:, None]
    dec = om.mxfp4_decode(codes, scales)
    for s in range(256):
        if s in special:
            sc = special[s]
        else:
            sc = float(np.array([s << 23], np.uint32).view(np.float32)[0])
        for c in range(16):
            want = table[c] * sc if not math.isnan(sc) else float("nan")
            assert _same(float(dec[s, c]), want), f"scale {s} code {c}"


def pin_bits_per_weight(H=2880, I=2880):
    """4 bits per element + 8 bits per 32 elements = 4.25 bits [walkthrough §1, §4]."""
    n_el = 2 * I * H
    code_bytes = n_el // 2
    scale_bytes = n_el // 32
    assert (code_bytes + scale_bytes) * 8 / n_el == 4.25
    dec = om.mxfp4_decode(np.zeros((3, H // 2), np.uint8), np.full((3, H // 32), 127, np.uint8))
    assert dec.shape == (3, H)


# --------------------------------------------------------------------------- a1/a2 routing
def pin_router_bruteforce(seed=0):
    """Logits against exactly-rounded sums of exact products (pure-Python brute force)."""
    rng = np.random.default_rng(seed)
    T, E, H = 3, 5, 40
    x_bits = (rng.standard_normal((T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = rng.standard_normal((E, H)).astype(np.float32) * np.float32(0.02)
    b = rng.standard_normal(E).astype(np.float32)
    got = om.router_logits(om.bf16_to_f64(x_bits), w, b)
    for t in range(T):
        xs = [float(np.array([int(v) << 16], np.uint32).view(np.float32)[0]) for v in x_bits[t]]
        for e in range(E):
            want = math.fsum([xs[h] * float(w[e, h]) for h in range(H)] + [float(b[e])])
            assert abs(got[t, e] - want) <= 1e-13 * (1 + abs(want)), (t, e, got[t, e], want)


def pin_topk_bruteforce(seed=1):
    """The chosen set maximises the sum over all k-subsets; the list is in descending order."""
    rng = np.random.default_rng(seed)
    for _ in range(40):
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        logits = rng.standard_normal((2, E))
        idx = om.topk_select(logits, k)
        for t in range(2):
            best = max(itertools.combinations(range(E), k),
                       key=lambda c: sum(logits[t, list(c)]))
            assert sorted(idx[t].tolist()) == sorted(best), (logits[t], idx[t], best)
            vals = logits[t, idx[t]]
            assert all(vals[i] >= vals[i + 1] for i in range(k - 1))


def pin_topk_ties():
    """Ties go to the lower expert id (reading of the pages' silence); the ranking is of the
    float64 scores, so a difference far below float32 resolution still decides."""
    lg = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]])
    assert om.topk_select(lg, 2).tolist() == [[1, 2]]
    assert om.topk_select(lg, 4).tolist() == [[1, 2, 4, 3]]
    # a difference below float32 resolution is not a tie in float64
    lg = np.array([[1.0, 1.0 + 1e-12, 0.5]])
    assert om.topk_select(lg, 1).tolist() == [[1]]
    assert om.topk_select(lg, 3).tolist() == [[1, 0, 2]]


def pin_softmax(seed=2):
    from scipy.special import softmax as sp_softmax
    rng = np.random.default_rng(seed)
    # closed form: scores ln4, ln2, 0, 0 -> 4/8, 2/8, 1/8, 1/8
    w = om.softmax_selected(np.array([[math.log(4), math.log(2), 0.0, 0.0]]))
    assert np.allclose(w, [[0.5, 0.25, 0.125, 0.125]], rtol=0, atol=1e-15)
    for _ in range(20):
        E = int(rng.integers(1, 12))
        k = int(rng.integers(1, E + 1))
        lg = rng.standard_normal((3, E)) * 3
        idx = om.topk_select(lg, k)
        w = om.softmax_selected(np.take_along_axis(lg, idx.astype(np.int64), axis=-1))
        assert np.allclose(w.sum(-1), 1.0, rtol=0, atol=1e-14)
        # softmax over all experts, then renormalised over the picked ones: a second route
        full = sp_softmax(lg, axis=-1)
        sel = np.take_along_axis(full, idx.astype(np.int64), axis=-1)
        assert np.allclose(w, sel / sel.sum(-1, keepdims=True), rtol=1e-13, atol=1e-15)
        if k == E:  # every expert picked: plain softmax (in pick order)
            assert np.allclose(w, sel, rtol=1e-13, atol=1e-15)
        # shift invariance
        w2 = om.softmax_selected(np.take_along_axis(lg + 123.0, idx.astype(np.int64), axis=-1))
        assert np.allclose(w, w2, rtol=1e-12, atol=1e-15)


def pin_route_end_to_end():
    """route() with a router whose scores are known exactly: one-hot x, bias ln-values."""
    H, E, k = 32, 6, 4
    x_bits = np.zeros((1, H), np.uint16)
    x_bits[0, 3] = 0x3F80  # 1.0
    w = np.zeros((E, H), np.float32)
    w[:, 3] = [0.0, 5.0, -1.0, 2.0, 4.0, 0.0]
    b = np.array([math.log(1), math.log(2) - 5.0, 0.0, math.log(4) - 2.0, math.log(8) - 4.0,
                  math.log(1)], np.float32)
    logits, idx, wts = om.route(x_bits, w, b, k)
    # scores: 0, ln2, -1, ln4, ln8, 0 -> top-4 = 4, 3, 1, then tie 0/5 -> 0
    assert idx.tolist() == [[4, 3, 1, 0]]
    want = np.array([8, 4, 2, 1], float) / 15.0
    assert np.allclose(wts[0], want, rtol=1e-6, atol=0)  # bias stored in float32


# --------------------------------------------------------------------------- a3 permute
def pin_permute_bruteforce(seed=3):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        E = int(rng.integers(1, 10))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(0, 30))
        idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32).reshape(T, k)
        counts, offsets, sorted_slot, slot_row = om.permute(idx, E)
        flat = idx.reshape(-1).tolist()
        want_sorted = [s for e in range(E) for s in range(len(flat)) if flat[s] == e]
        assert sorted_slot.tolist() == want_sorted
        assert counts.tolist() == [flat.count(e) for e in range(E)]
        assert offsets[0] == 0 and offsets[-1] == len(flat)
        for e in range(E):
            assert offsets[e + 1] - offsets[e] == counts[e]
            assert all(flat[s] == e for s in sorted_slot[offsets[e]:offsets[e + 1]])
        for s in range(len(flat)):
            assert sorted_slot[slot_row[s]] == s


# --------------------------------------------------------------------------- a4 epilogue
def pin_swiglu_identities(limit=7.0):
    rng = np.random.default_rng(4)
    for alpha in (1.0, 1.702):
        g = rng.uniform(-limit, limit, 200)
        lin = rng.uniform(-limit, limit, 200)

        def A(gg, ll):
            gg, ll = np.broadcast_arrays(np.asarray(gg, float), np.asarray(ll, float))
            h = np.stack([gg.ravel(), ll.ravel()], axis=1)  # one unit per row: [gate, linear]
            return om.swiglu_clamped(h, limit, alpha).reshape(gg.shape)

        assert np.all(A(g, -1.0) == 0.0), "linear branch -1 must zero the unit (the +1)"
        assert np.all(A(0.0 * g, lin) == 0.0), "gate 0 must zero the unit"
        # silu(g) - silu(-g) = g for any slope: catches a flipped sigmoid argument
        assert np.allclose(A(g, lin) - A(-g, lin), g * (lin + 1.0), rtol=1e-12, atol=1e-12)
        # saturation: both halves clamp to +-limit
        assert np.allclose(A(g * 0 + 50.0, lin), A(g * 0 + limit, lin), rtol=0, atol=0)
        assert np.allclose(A(g * 0 - 50.0, lin), A(g * 0 - limit, lin), rtol=0, atol=0)
        assert np.allclose(A(g, lin * 0 + 50.0), A(g, lin * 0 + limit), rtol=0, atol=0)
        assert np.allclose(A(g, lin * 0 - 50.0), A(g, lin * 0 - limit), rtol=0, atol=0)
        # closed form: sigmoid(ln 3) = 3/4, so a(ln3/alpha, 0) = (3/4) ln3 / alpha
        assert abs(A(np.array([math.log(3) / alpha]), np.array([0.0]))[0]
                   - 0.75 * math.log(3) / alpha) < 1e-15
        # bound: |a| <= limit * sigmoid(alpha*limit) * (limit + 1)
        big = rng.uniform(-100, 100, (500,))
        a = om.swiglu_clamped(big.reshape(-1, 2), limit, alpha)
        assert np.all(np.abs(a) <= limit / (1 + math.exp(-alpha * limit)) * (limit + 1) + 1e-12)


def pin_swiglu_interleave():
    """Gate at even positions, linear at odd positions (the reading of the fused layout)."""
    h = np.array([[2.0, -1.0, 0.0, 5.0, 3.0, 0.0]])
    a = om.swiglu_clamped(h)
    assert a[0, 0] == 0.0 and a[0, 1] == 0.0 and a[0, 2] > 0.0
    assert abs(a[0, 2] - 3.0 / (1.0 + math.exp(-3.0))) < 1e-15


# --------------------------------------------------------------------------- a4-a6 layer
def _tiny_layer(seed, T, E, k, H, I, scale_bytes=(120, 124)):
    rng = np.random.default_rng(seed)
    x_bits = (rng.standard_normal((T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    rw = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    rb = rng.standard_normal(E).astype(np.float32)
    w1c = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w1s = rng.integers(scale_bytes[0], scale_bytes[1] + 1, (E, 2 * I, H // 32), dtype=np.uint8)
    w1b = (rng.standard_normal((E, 2 * I)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w2c = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w2s = rng.integers(scale_bytes[0], scale_bytes[1] + 1, (E, H, I // 32), dtype=np.uint8)
    w2b = (rng.standard_normal((E, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return x_bits, rw, rb, (w1c, w1s, w1b, w2c, w2s, w2b)


def pin_single_expert_reduction():
    """E = 1, k = 1: the layer is one clamped-SwiGLU FFN applied to every token, weight 1."""
    T, H, I = 5, 64, 96
    x_bits, rw, rb, ws = _tiny_layer(5, T, 1, 1, H, I)
    res = om.moe_layer(x_bits, rw, rb, om.experts_from_arrays(*ws), 1)
    assert np.all(res.w == 1.0) and np.all(res.idx == 0)
    w1c, w1s, w1b, w2c, w2s, w2b = ws
    x = om.bf16_to_f64(x_bits)
    W1 = om.mxfp4_decode(w1c[0], w1s[0])
    W2 = om.mxfp4_decode(w2c[0], w2s[0])
    # dense expression per token, written with explicit loops over units
    for t in range(T):
        h = W1 @ x[t] + om.bf16_to_f64(w1b[0])
        act = np.empty(I)
        for i in range(I):
            g = min(max(h[2 * i], -7.0), 7.0)
            lin = min(max(h[2 * i + 1], -7.0), 7.0)
            act[i] = g / (1.0 + math.exp(-g)) * (lin + 1.0)
        y = W2 @ act + om.bf16_to_f64(w2b[0])
        assert np.allclose(res.out[t], y, rtol=1e-12, atol=1e-9 * np.abs(y).max())


def pin_dense_masked_bruteforce(seed=6):
    """Sparse top-k output equals the dense sum over all experts, masked to the top k and
    weighted by the renormalised softmax -- every expert evaluated, no grouping."""
    for trial in range(6):
        rng = np.random.default_rng(seed + trial)
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, min(E, 4) + 1))
        T = int(rng.integers(1, 17))
        H, I = 64, 96
        x_bits, rw, rb, ws = _tiny_layer(seed * 100 + trial, T, E, k, H, I)
        res = om.moe_layer(x_bits, rw, rb, om.experts_from_arrays(*ws), k)
        x = om.bf16_to_f64(x_bits)
        logits = x @ rw.astype(np.float64).T + rb.astype(np.float64)
        dense = np.zeros((T, E, H))
        for e in range(E):
            W1 = om.mxfp4_decode(ws[0][e], ws[1][e])
            W2 = om.mxfp4_decode(ws[3][e], ws[4][e])
            _, _, y = om.expert_ffn(x, W1, om.bf16_to_f64(ws[2][e]), W2, om.bf16_to_f64(ws[5][e]))
            dense[:, e] = y
        for t in range(T):
            l32 = logits[t]
            # top-k by repeated removal of the current maximum (lowest id on ties)
            remaining = list(range(E))
            picked = []
            for _ in range(k):
                best = remaining[0]
                for e in remaining:
                    if l32[e] > l32[best]:
                        best = e
                picked.append(best)
                remaining.remove(best)
            mask = np.zeros(E)
            mask[picked] = 1.0
            ex = np.exp(logits[t] - logits[t][picked].max()) * mask
            wts = ex / ex.sum()
            want = (wts[:, None] * dense[t]).sum(0)
            assert np.allclose(res.out[t], want, rtol=1e-12, atol=1e-12 * np.abs(want).max()), (trial, t)


def pin_token_subset():
    T, E, k, H, I = 9, 5, 3, 64, 32
    x_bits, rw, rb, ws = _tiny_layer(11, T, E, k, H, I)
    full = om.moe_layer(x_bits, rw, rb, om.experts_from_arrays(*ws), k)
    sub = [7, 2, 5]
    part = om.moe_layer(x_bits, rw, rb, om.experts_from_arrays(*ws), k, tokens=sub)
    # BLAS may block a 3-row product differently from a 9-row one: fp64 rounding only
    assert np.allclose(part.out, full.out[sub], rtol=1e-12, atol=1e-12 * np.abs(full.out).max())
    assert np.array_equal(part.idx, full.idx[sub])


# --------------------------------------------------------------------------- block wrap
def pin_rms_norm_closed_forms():
    """RMSNorm (review §3.2: the row over its root mean square, times a scale): closed forms.

    A row of one repeated value c has RMS |c|, so it maps to sign(c) * scale; with eps the
    RMS is sqrt(c^2 + eps) (1 and eps 3 give 2, so 0.5 * scale: eps inside the root, not
    added after it). A row (3, 4) has mean square 12.5. Rows are normalised separately."""
    scale = np.array([0.5, -2.0, 3.0, 1.25])
    rows = np.array([[2.0] * 4, [-0.75] * 4, [1e-3] * 4])
    out = om.rms_norm(rows, scale)
    assert np.array_equal(out, np.sign(rows) * scale[None, :])
    assert np.allclose(om.rms_norm(np.ones((1, 4)), scale, 3.0), 0.5 * scale, rtol=0, atol=1e-15)
    assert np.allclose(om.rms_norm(np.full((1, 4), 2.0), scale, 12.0), 0.5 * scale, rtol=0, atol=1e-15)
    two = om.rms_norm(np.array([[3.0, 4.0]]), np.ones(2))
    assert abs(two[0, 0] - 3.0 / math.sqrt(12.5)) < 1e-15 and abs(two[0, 1] - 4.0 / math.sqrt(12.5)) < 1e-15


def pin_rms_norm_invariants(seed=21):
    """Unit scale and no eps: every output row has mean square 1; the map ignores a positive
    factor on the row and commutes with a permutation of the features (scale permuted too)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((7, 96)) * rng.uniform(0.1, 10.0, (7, 1))
    out = om.rms_norm(x, np.ones(96))
    assert np.allclose(np.mean(out * out, axis=1), 1.0, rtol=1e-14)
    scale = rng.standard_normal(96)
    base = om.rms_norm(x, scale)
    assert np.allclose(om.rms_norm(3.5 * x, scale), base, rtol=1e-13, atol=1e-15)
    perm = rng.permutation(96)
    assert np.allclose(om.rms_norm(x[:, perm], scale[perm]), base[:, perm], rtol=1e-13, atol=1e-15)


def pin_bf16_rounding():
    """One rounding to bf16, to nearest with ties to even: hand cases (a tie on each side of
    an even mantissa, just past a tie, subnormals, overflow), then torch's float32 -> bfloat16
    cast (round to nearest even) on random float32 values, which reach it without a prior
    rounding."""
    import torch
    cases = {1.0: 0x3F80, 1.0 + 2.0 ** -8: 0x3F80, 1.0 + 3 * 2.0 ** -8: 0x3F82,
             1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81, -2.0: 0xC000, math.pi: 0x4049,
             1.5 * 2.0 ** -133: 0x0002, 2.0 ** -134: 0x0000, 3 * 2.0 ** -135: 0x0001,
             3.4e38: 0x7F80, -3.39e38: 0xFF7F, 3.38e38: 0x7F7E, 0.0: 0x0000}
    got = om.f64_to_bf16_bits(np.array(list(cases.keys())))
    assert [int(g) for g in got] == list(cases.values()), [hex(int(g)) for g in got]
    rng = np.random.default_rng(22)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-80, 80, 20000))).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(om.f64_to_bf16_bits(v.astype(np.float64)), want)


def pin_block_reductions():
    """The block out = x + MoE(bf16(RMSNorm(x))) in three special cases: experts with all-zero
    weights and biases give out = x exactly (the residual is the un-normalised x); a zero
    norm scale feeds every expert a zero row, so E = 1, k = 1 gives x + W2 swiglu(b1) + b2;
    and the normalised input handed to the layer is the bf16 rounding of the norm."""
    T, E, k, H, I = 6, 4, 2, 64, 32
    x_bits, rw, rb, ws = _tiny_layer(23, T, E, k, H, I)
    x = om.bf16_to_f64(x_bits)
    rng = np.random.default_rng(24)
    scale = rng.uniform(0.5, 2.0, H)
    zeros = (np.zeros_like(ws[0]), np.full_like(ws[1], 127), None,
             np.zeros_like(ws[3]), np.full_like(ws[4], 127), None)
    blk = om.moe_block(x_bits, scale, 1e-5, rw, rb, om.experts_from_arrays(*zeros), k)
    assert np.array_equal(blk.out, x)
    ms = np.array([sum(float(v) ** 2 for v in row) / H for row in x])
    for t in range(T):
        for h in range(H):
            ref = float(x[t, h]) / math.sqrt(ms[t] + 1e-5) * scale[h]
            got = float(om.bf16_to_f64(blk.xn_bits[t:t + 1, h:h + 1])[0, 0])
            # the bf16 neighbours of ref: the rounding must pick the nearer one
            assert abs(got - ref) <= abs(ref) * 2.0 ** -8 * (1 + 1e-9), (t, h, got, ref)
    x_bits1, rw1, rb1, ws1 = _tiny_layer(25, T, 1, 1, H, I)
    blk1 = om.moe_block(x_bits1, np.zeros(H), 1e-5, rw1, rb1, om.experts_from_arrays(*ws1), 1)
    b1 = om.bf16_to_f64(ws1[2][0])
    g = np.clip(b1[0::2], -7, 7)
    lin = np.clip(b1[1::2], -7, 7)
    act = g / (1.0 + np.exp(-g)) * (lin + 1.0)
    const = om.mxfp4_decode(ws1[3][0], ws1[4][0]) @ act + om.bf16_to_f64(ws1[5][0])
    want = om.bf16_to_f64(x_bits1) + const[None, :]
    assert np.allclose(blk1.out, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


# --------------------------------------------------------------------------- decode attention
def _attn_case(seed, B=3, Hq=16, Hkv=2, D=64, L=40):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D))
    lens = rng.integers(1, L + 1, B)
    lens[0] = L
    return q, k, v, lens


def _sdpa(q, k, v, lens, window, sink_keys=None):
    """torch's scaled_dot_product_attention (float64, CPU) with the key/value heads repeated
    for their query-head groups and an explicit boolean mask of the visible positions; with
    sink_keys ([B][Hq][D]), one extra key per query head whose value is zero."""
    import torch
    import torch.nn.functional as F
    B, Hq, D = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    kk = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)  # [B][Hq][L][D]
    vv = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1)
    qq = torch.from_numpy(q)[:, :, None, :]                       # [B][Hq][1][D]
    pos = torch.arange(L)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(lens[b])
        lo = 0 if window <= 0 else max(0, n - window)
        mask = ((pos >= lo) & (pos < n))[None, None, :].expand(1, Hq, L)
        kb, vb = kk[b:b + 1], vv[b:b + 1]
        if sink_keys is not None:
            kb = torch.cat([kb, torch.from_numpy(sink_keys[b])[None, :, None, :]], dim=2)
            vb = torch.cat([vb, torch.zeros(1, Hq, 1, D, dtype=vb.dtype)], dim=2)
            mask = torch.cat([mask, torch.ones(1, Hq, 1, dtype=torch.bool)], dim=2)
        o = F.scaled_dot_product_attention(qq[b:b + 1], kb, vb, attn_mask=mask[:, :, None, :])
        out[b] = o[0, :, 0, :].numpy()
    return out


def pin_attention_library_reductions(seed=41):
    """Without sinks the decode step is torch's scaled_dot_product_attention over the visible
    positions (dense, and windows of 1, 7 and 128); with sinks it is the same attention with
    one more key per head whose score is the sink logit and whose value is zero."""
    q, k, v, lens = _attn_case(seed)
    for window in (0, 1, 7, 128):
        got = om.attention_decode(q, k, v, lens, None, window)
        assert np.allclose(got, _sdpa(q, k, v, lens, window), rtol=1e-12, atol=1e-12), window
    rng = np.random.default_rng(seed + 1)
    sinks = rng.standard_normal(q.shape[1]) * 2.0
    D = q.shape[2]
    # a key k_s with q.k_s / sqrt(D) = sink: k_s = sink * sqrt(D) * q / |q|^2
    ks = sinks[None, :, None] * math.sqrt(D) * q / np.sum(q * q, axis=2, keepdims=True)
    for window in (0, 5):
        got = om.attention_decode(q, k, v, lens, sinks, window)
        assert np.allclose(got, _sdpa(q, k, v, lens, window, ks), rtol=1e-11, atol=1e-11), window


def pin_attention_closed_forms():
    """One visible key whose score equals the sink: half the value; a sink far below: the value
    itself; n equal keys of score s with sink c: the value times n e^s / (n e^s + e^c)."""
    D = 64
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 8.0                      # score = 8 * key[0] / 8 = key[0]
    k = np.zeros((1, 1, 5, D))
    k[0, 0, :, 0] = 1.5                   # every score 1.5
    v = np.tile(np.linspace(-1, 1, D), (1, 1, 5, 1))
    out = om.attention_decode(q, k, v, np.array([1]), np.array([1.5]), 0)
    assert np.allclose(out[0, 0], 0.5 * v[0, 0, 0], rtol=0, atol=1e-15)
    out = om.attention_decode(q, k, v, np.array([1]), np.array([-1e4]), 0)
    assert np.allclose(out[0, 0], v[0, 0, 0], rtol=0, atol=1e-15)
    out = om.attention_decode(q, k, v, np.array([5]), np.array([0.25]), 0)
    want = v[0, 0, 0] * 5 * math.exp(1.5) / (5 * math.exp(1.5) + math.exp(0.25))
    assert np.allclose(out[0, 0], want, rtol=1e-14, atol=1e-15)
    out = om.attention_decode(q, k, v, np.array([5]), np.array([0.25]), 2)  # only 2 keys in view
    want = v[0, 0, 0] * 2 * math.exp(1.5) / (2 * math.exp(1.5) + math.exp(0.25))
    assert np.allclose(out[0, 0], want, rtol=1e-14, atol=1e-15)


def pin_attention_empty_sequence():
    """No visible position (lens = 0): the output row is 0, with a sink (every real key's weight
    is 0) and without one (an empty weighted sum); the other sequence is unaffected."""
    rng = np.random.default_rng(43)
    q = rng.standard_normal((2, 4, 64))
    k = rng.standard_normal((2, 2, 3, 64))
    v = rng.standard_normal((2, 2, 3, 64))
    lens = np.array([0, 3])
    for sinks in (None, np.array([0.5, -1.0, 2.0, 0.0])):
        out = om.attention_decode(q, k, v, lens, sinks, 0)
        assert np.all(out[0] == 0.0)
        alone = om.attention_decode(q[1:], k[1:], v[1:], lens[1:], sinks, 0)
        assert np.array_equal(out[1], alone[0])


# --------------------------------------------------------------------------- shapes vs pages
GIB = 2.0 ** 30


def model_sizes(layers, experts, H=2880, I=2880, vocab=201088, q_heads=64, kv_heads=8, head_dim=64):
    """Bytes and parameter counts of a gpt-oss-shaped model from its shapes.

    MoE experts in MXFP4 (4.25 bits per weight) with bf16 biases; everything else in bf16.
    Attention: q, k, v and o projections with biases, plus one sink logit per head.
    """
    expert_w = 2 * I * H + H * I
    expert_b = 2 * I + H
    router = experts * H + experts
    attn = H * q_heads * head_dim + 2 * H * kv_heads * head_dim + q_heads * head_dim * H
    attn += q_heads * head_dim + 2 * kv_heads * head_dim + H + q_heads
    norms = 2 * H
    per_layer_dense = attn + router + norms
    emb = 2 * vocab * H + H
    moe_params = layers * experts * (expert_w + expert_b)
    dense_params = layers * per_layer_dense + emb
    total = moe_params + dense_params
    active = layers * 4 * (expert_w + expert_b) + dense_params - vocab * H  # unembed only
    moe_bytes = layers * experts * (expert_w * 4.25 / 8 + expert_b * 2)
    dense_bytes = dense_params * 2
    return dict(total=total, active=active, bytes=moe_bytes + dense_bytes,
                expert_bytes=expert_w * 4.25 / 8 + expert_b * 2)


def pin_shapes_against_pages():
    """Widths 2880/2880 with a fused 5760-wide gate_up at 4.25 bits reproduce the pages'
    checkpoint sizes (walkthrough §1, §4: ~12.8 GiB and ~60.8 GiB) and parameter counts
    (retrospective "时间与证据": 21B/3.6B and 117B/5.1B); 24 and 36 layers come from the
    retrospective's KV-cache estimate ("工程影响")."""
    s20 = model_sizes(24, 32)
    s120 = model_sizes(36, 128)
    assert s20["expert_bytes"] == 13_236_480
    assert abs(s20["bytes"] / GIB - 12.8) < 0.05, s20["bytes"] / GIB
    assert abs(s120["bytes"] / GIB - 60.8) < 0.1, s120["bytes"] / GIB
    assert abs(s20["total"] / 1e9 - 21) < 0.2 and abs(s20["active"] / 1e9 - 3.6) < 0.05
    assert abs(s120["total"] / 1e9 - 117) < 0.5 and abs(s120["active"] / 1e9 - 5.1) < 0.05


ALL_PINS = [
    pin_e2m1_table, pin_e8m0_special, pin_e8m0_ieee_bits, pin_mxfp4_row_example, pin_mxfp4_grid,
    pin_bits_per_weight, pin_router_bruteforce, pin_topk_bruteforce, pin_topk_ties, pin_softmax,
    pin_route_end_to_end, pin_permute_bruteforce, pin_swiglu_identities, pin_swiglu_interleave,
    pin_single_expert_reduction, pin_dense_masked_bruteforce, pin_token_subset,
    pin_shapes_against_pages, pin_rms_norm_closed_forms, pin_rms_norm_invariants,
    pin_bf16_rounding, pin_block_reductions, pin_attention_library_reductions,
    pin_attention_closed_forms, pin_attention_empty_sequence,
]
