"""Write the stored router-bias vectors that shape the synthetic routing of two workloads.

Run from the repository root:  python -m oracle.calibrate_router_bias

It uses only this package's routing (fp64 logits, top-k in float32) on the seeded
synthetic inputs, and writes plain-text fp32 vectors (hex floats, one per line) under
synth/data/, which the input generator reads. Nothing here runs on the GPU.

* balance_prefill120b: near-uniform load for the 8192-token, 128-expert prefill batch.
  Iterate b_e -= 0.1 * ln(count_e / mean) on that batch until every count is within
  +-20% of T*k/E (the load-balance band the 20b prefill workload is specified with; the
  config.json read-through, Part.01, reports a strong balancing loss, coefficient 0.9).
* zipf_decode120b: skewed routing for the 128-expert decode sweep. The expert ranked r
  (over a seeded random permutation of experts) should receive a share of routed slots
  proportional to r^-1.2. Fixed-point iteration b += 0.5 * (ln target - ln freq) on a
  16384-token calibration batch drawn from an independent stream, 60 iterations. With
  top-4, no expert can take more than 1/4 of the slots, so the head of the curve caps there.
* balance_prefill20b: the zero vector already keeps the 4096-token, 32-expert batch in
  the +-20% band; the file is written so the workload names its bias explicitly.
"""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle.moe_oracle import bf16_to_f64, router_logits, topk_select  # noqa: E402

DATA = os.path.join(ROOT, "synth", "data")


def _counts(xf, w, b, k, E):
    idx = topk_select(router_logits(xf, w, b), k)
    return np.bincount(idx.reshape(-1), minlength=E)


def balance(cfg, T, band=0.2, max_iter=200):
    x = bf16_to_f64(synth.make_x(cfg, T))
    w, _ = synth.make_router(cfg, np.zeros(cfg.E, np.float32))
    b = np.zeros(cfg.E, np.float32)
    mean = T * cfg.k / cfg.E
    for it in range(max_iter):
        c = _counts(x, w, b, cfg.k, cfg.E)
        if c.min() >= (1 - band) * mean and c.max() <= (1 + band) * mean:
            return b, c, it
        b = (b - 0.1 * np.log(np.maximum(c, 1) / mean)).astype(np.float32)
    raise RuntimeError("load balancing did not converge")


def zipf(cfg, s=1.2, n_cal=16384, iters=60, step=0.5):
    x = bf16_to_f64(synth.make_x(cfg, n_cal, offset=1))  # calibration stream, not the eval batches
    w, _ = synth.make_router(cfg, np.zeros(cfg.E, np.float32))
    perm = np.random.default_rng(np.random.SeedSequence([cfg.seed, 99])).permutation(cfg.E)
    target = np.empty(cfg.E)
    target[perm] = np.arange(1, cfg.E + 1, dtype=np.float64) ** (-s)
    target /= target.sum()
    b = np.zeros(cfg.E, np.float64)
    for _ in range(iters):
        freq = _counts(x, w, b.astype(np.float32), cfg.k, cfg.E) / (n_cal * cfg.k)
        b += step * (np.log(target) - np.log(np.maximum(freq, 0.5 / (n_cal * cfg.k))))
        b -= b.max()
    b = b.astype(np.float32)
    freq = _counts(x, w, b, cfg.k, cfg.E) / (n_cal * cfg.k)
    return b, freq, target


def write(stem, b, header):
    os.makedirs(DATA, exist_ok=True)
    with open(os.path.join(DATA, stem + ".txt"), "w", encoding="utf-8") as f:
        for line in header:
            f.write("# " + line + "\n")
        for v in b:
            f.write(float(v).hex() + "\n")


def main():
    cfg = synth.get_config("prefill20b")
    b, c, it = balance(cfg, cfg.T_list[-1])
    write("balance_prefill20b", b, [
        "router bias, 20b-shaped prefill (T=4096, E=32, top-4); written by oracle/calibrate_router_bias.py",
        f"iterations {it}; per-expert slot counts min {c.min()} max {c.max()} (mean {4096 * 4 / 32:.0f})"])
    print("prefill20b", it, c.min(), c.max())

    cfg = synth.get_config("prefill120b")
    b, c, it = balance(cfg, cfg.T_list[-1])
    write("balance_prefill120b", b, [
        "router bias, 120b-shaped prefill (T=8192, E=128, top-4); written by oracle/calibrate_router_bias.py",
        f"iterations {it}; per-expert slot counts min {c.min()} max {c.max()} (mean {8192 * 4 / 128:.0f})"])
    print("prefill120b", it, c.min(), c.max())

    cfg = synth.get_config("decode120b_zipf")
    b, freq, target = zipf(cfg)
    l1 = float(np.abs(freq - target).sum())
    write("zipf_decode120b", b, [
        "router bias, 120b-shaped decode sweep, expert popularity ~ rank^-1.2 over a seeded",
        "permutation of the 128 experts; written by oracle/calibrate_router_bias.py",
        f"calibration batch 16384 tokens: L1(freq, target) = {l1:.4f}; top share {freq.max():.4f}"])
    print("zipf", l1, freq.max(), np.sort(freq)[::-1][:8])


if __name__ == "__main__":
    main()
