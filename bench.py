"""Benchmark of the MXFP4 top-k MoE layer on one MI355X; prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode20b] [--T 64]

A step is one call of the whole layer (router, top-k/softmax, permutation, expert
gate_up + SwiGLU, down, weighted combine) over one batch of T tokens, with inputs
resident in HBM. Steps rotate over L distinct copies of the layer's weights (24 for the
20b-shaped layer, 36 for the 120b-shaped one, like the models' depth) so the 256 MB
last-level cache cannot hold the weights between steps.

With --workload attn_decode a step is one decode step of the model's attention instead
(moe_attn_decode over --T sequences of --context positions, dense or --window).
With --block a step is the block around the layer instead: RMSNorm of the residual-stream
rows, the layer on the normalised rows, and the residual add (moe_block_forward_ex).

The roofline object covers the dominant step, the expert FFN (moe_mxfp4_ffn: the gate_up
and down kernels), timed with HIP events on the stream it runs on. cpu_baseline times
the fp64 oracle on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s; % HBM BW at T≤64, % MXFP4 MFMA peak at T=4096"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
MXFP4_PEAK_TFLOPS = 10100.0

NORM_EPS = 1e-5  # the block's RMSNorm epsilon

EXPERT_BYTES_PER_ROW = lambda K: K // 2 + K // 32 + 2  # codes + scales + bf16 bias


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode20b",
                   choices=["decode20b", "prefill20b", "prefill120b", "decode120b_zipf", "attn_decode"])
    p.add_argument("--context", type=int, default=4096,
                   help="attn_decode: positions in every sequence's cache (all visible unless --window)")
    p.add_argument("--window", type=int, default=0, help="attn_decode: 0 dense, else the band (gpt-oss: 128)")
    p.add_argument("--T", type=int, default=0, help="batch size (default: the workload's largest)")
    p.add_argument("--layers", type=int, default=0, help="rotated weight copies (default 24 / 36)")
    p.add_argument("--path", type=int, default=0, help="0 auto, 1 stream, 2 gemm (bf16), 3 gemm (block-scaled)")
    p.add_argument("--layout", default="tiled", choices=["tiled", "rowmajor"],
                   help="weights prepacked once (untimed) into the kernel layout, or row-major")
    p.add_argument("--block", action="store_true",
                   help="time the block around the layer, x + layer(RMSNorm(x)) (moe_block_forward_ex), "
                        "on residual-stream inputs with per-token scales")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--pmc-summary", nargs=4, metavar=("COPY_FETCH", "COPY_WRITE", "FETCH", "WRITE"),
                   help="only print the traffic line for --workload/--T from four rocprofv3 --pmc csv "
                        "output folders (FETCH_SIZE and WRITE_SIZE of --copy-calibration 1024, then of "
                        "this benchmark) and exit")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only copy MIB MiB device-to-device 4 times and exit: the known-size copy "
                        "that scales the FETCH_SIZE / WRITE_SIZE counters of a profiled run")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.md")
CALIBRATION_MIB = 1024
FFN_KERNELS = ("ffn_", "gather_rows")  # kernels one moe_mxfp4_ffn call launches, once each


# the sources of what one moe_mxfp4_ffn call runs at decode (the weight-streaming kernels) and
# at prefill (the gather and the grouped GEMM): kernels, their headers and the host code that
# picks and launches them
FFN_SOURCES = {
    "stream": ("ffn_stream.hip", "common.h", "kernels.h", "moe_abi.cpp"),
    "gemm": ("ffn_gemm.hip", "gather.hip", "common.h", "mx_act.h", "kernels.h", "moe_abi.cpp"),
}


def kernel_source_hash(workload):
    """Hash of the expert-FFN sources the workload runs: a stored traffic figure is valid for
    these only."""
    import hashlib
    csrc = os.path.join(ROOT, "sparse_moe_transformer_router_amd", "csrc")
    h = hashlib.sha256()
    for name in FFN_SOURCES["stream" if workload.startswith("decode") else "gemm"]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def pmc_means(folder, counter):
    """Mean counter value per dispatch, per kernel name, from a rocprofv3 --pmc csv folder."""
    import csv
    import glob
    sums = {}
    for path in glob.glob(os.path.join(folder, "*counter_collection.csv")):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"].split("(")[0].replace("void ", "").strip()
                tot, n = sums.get(name, (0.0, 0))
                sums[name] = (tot + float(r["Counter_Value"]), n + 1)
    return {k: t / n for k, (t, n) in sums.items()}


def pmc_summary(args, T):
    cal = CALIBRATION_MIB << 10  # KiB the copy moves each way
    cf = pmc_means(args.pmc_summary[0], "FETCH_SIZE")
    cw = pmc_means(args.pmc_summary[1], "WRITE_SIZE")
    copy = [k for k in cf if "copyBuffer" in k]
    fetch_scale = cal / cf[copy[0]]
    write_scale = cal / cw[copy[0]]
    f = pmc_means(args.pmc_summary[2], "FETCH_SIZE")
    w = pmc_means(args.pmc_summary[3], "WRITE_SIZE")
    names = sorted(k for k in f if any(t in k for t in FFN_KERNELS))
    fk = sum(f[k] for k in names)
    wk = sum(w.get(k, 0.0) for k in names)
    nbytes = int(round((fk * fetch_scale + wk * write_scale) * 1024))
    print(f"traffic workload={args.workload} T={T} src={kernel_source_hash(args.workload)} bytes={nbytes} "
          f"fetch_kib={fk:.0f} write_kib={wk:.0f} fetch_scale={fetch_scale:.4f} write_scale={write_scale:.4f} "
          f"kernels={'+'.join(n.replace(' ', '') for n in names)}", flush=True)


def stored_traffic(workload, T):
    """HBM bytes per expert-FFN call measured by rocprofv3 for these exact kernel sources, or None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    src = kernel_source_hash(workload)
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if not line.startswith("traffic "):
                continue
            kv = dict(t.split("=", 1) for t in line.split()[1:])
            if kv.get("workload") == workload and kv.get("T") == str(T) and kv.get("src") == src:
                return int(kv["bytes"])
    return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}), flush=True)
        sys.exit(2)

    import torch
    import synth
    import sparse_moe_transformer_router_amd as moe

    if args.pmc_summary:
        cfg = synth.get_config(args.workload)
        pmc_summary(args, args.T or cfg.T_list[-1])
        return
    torch.cuda.init()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 4}), flush=True)
        return
    if args.workload == "attn_decode":
        attn_main(args, torch, synth, moe, dev)
        return
    cfg = synth.get_config(args.workload)
    T = args.T or cfg.T_list[-1]
    L = args.layers or (24 if cfg.E <= 32 else 36)
    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    t0 = time.time()
    inp = synth.make_inputs(cfg, T)
    log(f"generated {cfg.name} T={T} in {time.time() - t0:.1f}s")

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    base_w1 = moe.MXFP4Weight(u8(inp.w1_codes), u8(inp.w1_scales), bf16(inp.w1_bias))
    base_w2 = moe.MXFP4Weight(u8(inp.w2_codes), u8(inp.w2_scales), bf16(inp.w2_bias))
    if args.layout == "tiled":  # one-time load-time conversion, outside the timed region
        base_w1, base_w2 = moe.moe_mxfp4_pack(base_w1), moe.moe_mxfp4_pack(base_w2)
    base_rt = moe.Router(torch.from_numpy(inp.router_w).to(dev), torch.from_numpy(inp.router_b).to(dev))
    layers = [(base_rt, base_w1, base_w2)]
    def clone(w):
        return moe.MXFP4Weight(w.codes.clone(), w.scales.clone(), w.bias.clone(), w.layout, w.shape_nk)

    for _ in range(L - 1):  # device-side copies at distinct addresses
        layers.append((moe.Router(base_rt.weight.clone(), base_rt.bias.clone()), clone(base_w1), clone(base_w2)))
    x = bf16(inp.x)
    if args.block:  # the block's input: the residual stream, normalised inside the timed step
        x = bf16(synth.make_block_x(cfg, T))
        inp.x = synth.make_block_x(cfg, T)
        norm_scale_np = synth.make_norm_scale(cfg)
        norm_scale = torch.from_numpy(norm_scale_np).to(dev)
    opts = moe.Options(path=args.path)
    ws = moe.workspace(T, E, k, H, I, args.path, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"{L} layer copies resident ({L * (base_w1.codes.numel() + base_w1.scales.numel() + base_w2.codes.numel() + base_w2.scales.numel()) / 1e9:.1f} GB)")

    # realised routing of this batch (same for every copy); the block routes the normalised rows
    x_layer = moe.moe_rmsnorm(x, norm_scale, NORM_EPS) if args.block else x
    idx, _ = moe.moe_route(x_layer, base_rt, k)
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=E)
    touched = int((counts > 0).sum())

    def step(i):
        rt, w1, w2 = layers[i % L]
        if args.block:
            moe.moe_block_forward_ex(x, norm_scale, NORM_EPS, rt, w1, w2, k, opts, out=out, ws=ws)
        else:
            moe.moe_forward_ex(x, rt, w1, w2, k, opts, out=out, ws=ws)

    def timed_steps(n, warm):
        for i in range(warm):
            step(i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(n):
            step(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n  # ms per step

    ms = timed_steps(args.steps, args.warmup)
    tok_s = T / (ms * 1e-3)
    log(f"T={T}: {ms * 1e3:.1f} us/step, {tok_s:.0f} tok/s, touched {touched}/{E}")

    # ---- dominant step: the expert FFN (gate_up + down), timed with events on its stream. The
    # routing is the same for every weight copy (same router, same x), so it is computed once
    # and n_ffn FFN calls run back to back between two events (no event or routing kernel
    # between the timed calls).
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_slot = torch.empty(T * k, dtype=torch.int32, device=dev)
    slot_row = torch.empty(T * k, dtype=torch.int32, device=dev)
    y = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    ti = torch.empty((T, k), dtype=torch.int32, device=dev)
    moe.moe_route(x_layer, base_rt, k, topk_idx=ti, topk_w=tw, ws=ws)
    moe.moe_permute(ti, E, out=(offsets, sorted_slot, slot_row))
    n_ffn = max(20, min(args.steps, 200))
    ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for rep in range(2):  # first pass warms up
        torch.cuda.synchronize()
        if rep:
            ev_a.record()
        for i in range(n_ffn):
            _, w1, w2 = layers[i % L]
            moe.moe_mxfp4_ffn(x_layer, k, E, offsets, sorted_slot, w1, w2, opts, y=y, ws=ws)
        if rep:
            ev_b.record()
        torch.cuda.synchronize()
    ffn_ms = ev_a.elapsed_time(ev_b) / n_ffn

    expert_bytes = 2 * I * EXPERT_BYTES_PER_ROW(H) + H * EXPERT_BYTES_PER_ROW(I)
    ffn_bytes = touched * expert_bytes + T * H * 2
    ffn_flops = 2.0 * T * k * (2 * I * H + H * I)
    decode_like = cfg.name.startswith("decode")
    if decode_like:
        achieved = ffn_bytes / (ffn_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(cfg.name, T)}
    else:
        # Both grouped-GEMM paths do the algorithmic flops at a 2.5 PFLOP/s ceiling: the bf16 one
        # on the bf16 MFMA; the block-scaled one on the FP8xFP4 scaled MFMA (5.0 PFLOP/s) with two
        # E4M3 terms per bf16 activation, i.e. two instruction flops per algorithmic flop.
        mx = args.path in (0, 3)
        basis = ("FP8xFP4 scaled MFMA 5.0 PFLOP/s / 2 (two E4M3 terms per bf16 activation)" if mx
                 else "bf16 MFMA 2.5 PFLOP/s")
        achieved = ffn_flops / (ffn_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                    "traffic": stored_traffic(cfg.name, T), "peak_basis": basis,
                    "frac_of_mxfp4_peak": round(achieved / MXFP4_PEAK_TFLOPS, 4)}
    roofline.update({"kernel": "moe_mxfp4_ffn (gate_up + down)", "ms_per_launch": round(ffn_ms, 5),
                     "algorithmic_bytes": int(ffn_bytes), "algorithmic_flops": ffn_flops})
    log(f"ffn: {ffn_ms * 1e3:.1f} us, {roofline['achieved']} {roofline['unit']} ({roofline['frac']:.1%})")

    sweep = []
    if not args.no_sweep and decode_like and not args.block:
        for Ts in cfg.T_list:
            if Ts == T:
                continue
            xs = bf16(synth.make_x(cfg, Ts))
            wss = moe.workspace(Ts, E, k, H, I, args.path, device=dev)
            outs = torch.empty((Ts, H), dtype=torch.bfloat16, device=dev)
            ids, _ = moe.moe_route(xs, base_rt, k)
            tch = int((np.bincount(ids.cpu().numpy().ravel(), minlength=E) > 0).sum())

            def step_s(i):
                rt, w1, w2 = layers[i % L]
                moe.moe_forward_ex(xs, rt, w1, w2, k, opts, out=outs, ws=wss)
            for i in range(args.warmup):
                step_s(i)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(args.steps):
                step_s(i)
            b.record()
            torch.cuda.synchronize()
            ms_s = a.elapsed_time(b) / args.steps
            layer_bytes = tch * expert_bytes + E * H * 4 + E * 4 + Ts * H * 4 + Ts * k * 8
            sweep.append({"T": Ts, "ms_per_step": round(ms_s, 5), "tokens_per_s": round(Ts / (ms_s * 1e-3), 1),
                          "touched_experts": tch, "layer_GBps": round(layer_bytes / (ms_s * 1e-3) / 1e9, 1)})
            log(f"sweep T={Ts}: {ms_s * 1e3:.1f} us/step, touched {tch}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, inp, T, log, norm_scale_np if args.block else None)

    layer_bytes = touched * expert_bytes + E * H * 4 + E * 4 + T * H * 4 + T * k * 8
    line = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "E": E, "k": k, "hidden": H, "expert_width": I,
                   "weights": "MXFP4 (E2M1 + E8M0 per 32)", "weight_layout": args.layout,
                   "layers_rotated": L, "path": args.path,
                   "touched_experts": touched, "per_expert_slots_min_max": [int(counts.min()), int(counts.max())],
                   "layer_GBps": round(layer_bytes / (ms * 1e-3) / 1e9, 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if args.block:
        line["config"]["block"] = f"x + layer(RMSNorm(x)), eps {NORM_EPS:g}"
    if sweep:
        line["sweep"] = sweep
    print(json.dumps(line), flush=True)


def attn_main(args, torch, synth, moe, dev):
    """One decode step of the model's attention (64 query heads over 8 key/value heads of
    dimension 64, per-head sinks) for a batch of T sequences with `--context` cached positions;
    steps rotate over cache copies larger together than the last-level cache."""
    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    B = args.T or 64
    Lctx, W = args.context, args.window
    Hq, Hkv, D = 64, 8, 64
    t0 = time.time()
    inp = synth.make_attn_inputs(B, Lctx, Hq, Hkv, D, seed=1, full=True)
    log(f"generated attention inputs B={B} context={Lctx} in {time.time() - t0:.1f}s")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    cache_bytes = 2 * inp.k.nbytes
    copies = args.layers or max(2, int(np.ceil(2e9 / cache_bytes)))
    kv = [(bf16(inp.k), bf16(inp.v))]
    for _ in range(copies - 1):
        kv.append((kv[0][0].clone(), kv[0][1].clone()))
    q = bf16(inp.q)
    lens = torch.from_numpy(inp.lens).to(dev)
    sinks = torch.from_numpy(inp.sinks).to(dev)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(int(moe.lib().moe_attn_workspace_size(B, Hkv, Lctx, W)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"{copies} cache copies resident ({copies * cache_bytes / 1e9:.1f} GB)")

    def step(i):
        k, v = kv[i % copies]
        moe.moe_attn_decode(q, k, v, lens, sinks, W, out=out, ws=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(args.steps):
        step(i)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    visible = min(W, Lctx) if W > 0 else Lctx
    nbytes = B * Hkv * visible * D * 2 * 2 + 2 * B * Hq * D * 2
    achieved = nbytes / (ms * 1e-3) / 1e9
    log(f"B={B} context={Lctx} window={W}: {ms * 1e3:.1f} us/step, {achieved:.0f} GB/s")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "moe_attn_decode (split + merge)", "ms_per_launch": round(ms, 5),
                "algorithmic_bytes": int(nbytes)}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        n = min(B, 2)
        qf, kf, vf = (oracle.bf16_to_f64(x[:n]) for x in (inp.q, inp.k, inp.v))
        threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
        reps, dt = 0, 0.0
        while reps < 16 and (reps == 0 or dt < 10.0):
            t1 = time.perf_counter()
            oracle.attention_decode(qf, kf, vf, inp.lens[:n], inp.sinks, W)
            dt += time.perf_counter() - t1
            reps += 1
        log(f"oracle: {reps} x {n} sequences in {dt:.1f}s")
        cpu = {"value": round(reps * n / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"first {n} of the {B} sequences, {reps} repetitions, fp64 numpy decode attention; {dt:.1f} s"}
    line = {
        "metric": "decode attention tokens/s (one new token per sequence)",
        "value": round(B / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "attn_decode", "sequences": B, "context": Lctx, "window": W, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "sinks": True, "cache_copies": copies},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, inp, T, log, norm_scale=None, min_seconds=10.0, max_reps=16):
    """The fp64 oracle as it stands, on a bounded token sample of the same batch, repeated
    until about min_seconds of host work have been timed (the block around the layer when
    norm_scale is given)."""
    import oracle
    n = min(T, 64 if cfg.E <= 32 else 16)
    tokens = np.arange(n)
    get = oracle.experts_from_arrays(inp.w1_codes, inp.w1_scales, inp.w1_bias, inp.w2_codes,
                                     inp.w2_scales, inp.w2_bias)
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    reps, dt = 0, 0.0
    while reps < max_reps and (reps == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        if norm_scale is None:
            oracle.moe_layer(inp.x, inp.router_w, inp.router_b, get, cfg.k, tokens=tokens)
        else:
            oracle.moe_block(inp.x, norm_scale, NORM_EPS, inp.router_w, inp.router_b, get, cfg.k, tokens=tokens)
        dt += time.perf_counter() - t0
        reps += 1
    log(f"oracle: {reps} x {n} tokens in {dt:.1f}s on {threads} threads")
    return {"value": round(reps * n / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of the {T} tokens, {reps} repetitions, full {'block' if norm_scale is not None else 'layer'} in fp64 numpy (router, "
                      f"top-{cfg.k}, per-expert MXFP4 decode, FFN, combine); {dt:.1f} s"}


if __name__ == "__main__":
    main()
