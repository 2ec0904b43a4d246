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
    p.add_argument("--path", type=int, default=0,
                   help="0 auto, 1 decode (weight streaming), 2 prefill bf16 GEMM, 3 prefill two-term MXFP8 GEMM, "
                        "4 prefill with MXFP6 down input, 5 decode with one token in one launch")
    p.add_argument("--layout", default="tiled", choices=["tiled", "rowmajor"],
                   help="weights prepacked once (untimed) into the kernel layout, or row-major")
    p.add_argument("--block", action="store_true",
                   help="time the block around the layer, x + layer(RMSNorm(x)) (moe_block_forward_ex), "
                        "on residual-stream inputs with per-token scales")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-prefill", action="store_true",
                   help="decode workloads: skip the 4096-token prefill20b record added to the line")
    p.add_argument("--chain", type=int, default=0, metavar="L",
                   help="multi-layer decode: a step is L chained blocks x <- x + layer_l(RMSNorm_l(x)) over L "
                        "distinct layers, each router reading the previous block's output")
    p.add_argument("--prefetch-hot", type=int, default=0, metavar="N",
                   help="with --chain: at the start of each block, read the layer's N most popular experts' "
                        "weights (by the previous step's routing) on a side stream while the block routes")
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
# instances that only the layer steps launch (the down projection writing y in slot order, epilogue
# 6), not the expert-FFN calls the traffic line is per
LAYER_ONLY_KERNELS = ("_kernel<6,",)


# the sources of what one moe_mxfp4_ffn call runs at decode (the weight-streaming kernels, or for
# one token the one-launch FFN and its per-block sum) and at prefill (the gather and the grouped
# GEMM): kernels, their headers and the host code that picks and launches them
FFN_SOURCES = {
    "stream": ("ffn_stream.hip", "ffn_small.hip", "combine.hip", "common.h", "kernels.h", "moe_abi.cpp"),
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
    names = sorted(k for k in f if any(t in k for t in FFN_KERNELS)
                   and not any(t in k.replace(" ", "") for t in LAYER_ONLY_KERNELS))
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


def host_description():
    """The host the oracle baseline runs on: the CPU model name (the field lscpu shows, read
    from /proc/cpuinfo) and NumPy's BLAS backend."""
    import platform
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    if model is None:
        model = platform.processor() or platform.machine()
    blas = None
    try:
        dep = np.__config__.CONFIG["Build Dependencies"]["blas"]
        blas = f"{dep.get('name')} {dep.get('version')}"
    except Exception:
        pass
    return model, blas


def event_time(torch, fn, min_ms=100.0, warm_ms=100.0, max_calls=50000):
    """Average device time of fn(i) over back-to-back calls between one pair of HIP events on
    the current stream (the one the library launches on): calls for at least warm_ms of wall
    time first (clocks settle), then at least min_ms of timed calls, whatever --steps is."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        fn(n)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= warm_ms:
                break
    per_call = (time.perf_counter() - t0) / n
    calls = int(min(max_calls, max(20, np.ceil(min_ms * 1e-3 / per_call))))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(calls):
        fn(n + i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / calls, calls


class LayerBench:
    """One workload's weights (L rotated device copies) and the timing of layer steps and of
    the expert FFN at any batch size."""

    def __init__(self, args, torch, synth, moe, dev, cfg, T0, log):
        self.args, self.torch, self.synth, self.moe, self.dev, self.cfg, self.log = args, torch, synth, moe, dev, cfg, log
        self.L = args.layers or (24 if cfg.E <= 32 else 36)
        t0 = time.time()
        self.inp = synth.make_inputs(cfg, T0)
        log(f"generated {cfg.name} T={T0} in {time.time() - t0:.1f}s")
        inp = self.inp
        base_w1 = moe.MXFP4Weight(self.u8(inp.w1_codes), self.u8(inp.w1_scales), self.bf16(inp.w1_bias))
        base_w2 = moe.MXFP4Weight(self.u8(inp.w2_codes), self.u8(inp.w2_scales), self.bf16(inp.w2_bias))
        if args.layout == "tiled":  # one-time load-time conversion, outside the timed region
            base_w1, base_w2 = moe.moe_mxfp4_pack(base_w1), moe.moe_mxfp4_pack(base_w2)
        self.base_rt = moe.Router(torch.from_numpy(inp.router_w).to(dev), torch.from_numpy(inp.router_b).to(dev))
        self.layers = [(self.base_rt, base_w1, base_w2)]

        def clone(w):
            return moe.MXFP4Weight(w.codes.clone(), w.scales.clone(), w.bias.clone(), w.layout, w.shape_nk)
        for _ in range(self.L - 1):  # device-side copies at distinct addresses
            self.layers.append((moe.Router(self.base_rt.weight.clone(), self.base_rt.bias.clone()), clone(base_w1),
                                clone(base_w2)))
        gb = self.L * sum(t.numel() for t in (base_w1.codes, base_w1.scales, base_w2.codes, base_w2.scales)) / 1e9
        log(f"{self.L} layer copies resident ({gb:.1f} GB)")
        H, I = cfg.H, cfg.I
        self.expert_bytes = 2 * I * EXPERT_BYTES_PER_ROW(H) + H * EXPERT_BYTES_PER_ROW(I)

    def u8(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)

    def bf16(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.dev).view(self.torch.bfloat16)

    def batch(self, T, x_np=None, block=False, norm_scale=None):
        """Device buffers of one batch of T tokens (x from the workload's generator unless given)."""
        torch, moe, cfg, dev = self.torch, self.moe, self.cfg, self.dev
        H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k
        x = self.bf16(self.synth.make_x(cfg, T) if x_np is None else x_np)
        b = {"T": T, "x": x, "ws": moe.workspace(T, E, k, H, I, self.args.path, device=dev),
             "out": torch.empty((T, H), dtype=torch.bfloat16, device=dev), "block": block,
             "norm_scale": norm_scale}
        # the realised routing (same for every copy); the block routes the normalised rows
        b["x_layer"] = moe.moe_rmsnorm(x, norm_scale, NORM_EPS) if block else x
        idx, tw = moe.moe_route(b["x_layer"], self.base_rt, k)
        b["counts"] = np.bincount(idx.cpu().numpy().ravel(), minlength=E)
        b["touched"] = int((b["counts"] > 0).sum())
        b["offsets"], b["sorted_slot"], b["slot_row"] = moe.moe_permute(idx, E)
        b["y"] = torch.empty((T * k, H), dtype=torch.float32, device=dev)
        return b

    def step(self, b, i):
        rt, w1, w2 = self.layers[i % self.L]
        opts = self.moe.Options(path=self.args.path)
        if b["block"]:
            self.moe.moe_block_forward_ex(b["x"], b["norm_scale"], NORM_EPS, rt, w1, w2, self.cfg.k, opts,
                                          out=b["out"], ws=b["ws"])
        else:
            self.moe.moe_forward_ex(b["x"], rt, w1, w2, self.cfg.k, opts, out=b["out"], ws=b["ws"])

    def time_steps(self, b, steps, warmup):
        """Exactly `warmup` untimed steps, then exactly `steps` timed steps between two events."""
        torch = self.torch
        for i in range(warmup):
            self.step(b, i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(steps):
            self.step(b, i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps

    def ffn_roofline(self, b):
        """The dominant step, the expert FFN (moe_mxfp4_ffn: gate_up + down, plus the gather on
        the grouped-GEMM paths), timed with events around back-to-back calls over the rotated
        copies (the routing is the same for every copy, so it is computed once)."""
        cfg, moe, T = self.cfg, self.moe, b["T"]
        H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k
        opts = moe.Options(path=self.args.path)

        def call(i):
            _, w1, w2 = self.layers[i % self.L]
            moe.moe_mxfp4_ffn(b["x_layer"], k, E, b["offsets"], b["sorted_slot"], w1, w2, opts, y=b["y"], ws=b["ws"])
        ffn_ms, calls = event_time(self.torch, call)
        ffn_bytes = b["touched"] * self.expert_bytes + T * H * 2
        ffn_flops = 2.0 * T * k * (2 * I * H + H * I)
        if cfg.name.startswith("decode"):
            achieved = ffn_bytes / (ffn_ms * 1e-3) / 1e9
            r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(cfg.name, T)}
        else:
            # The metric's prefill figure is the fraction of the MXFP4 MFMA peak (10.1 PFLOP/s dense).
            # The bf16 MFMA peak (2.5 PFLOP/s) is the ceiling of exact bf16 activations and is
            # reported alongside, as is the two-term activation path's own ceiling.
            achieved = ffn_flops / (ffn_ms * 1e-3) / 1e12
            r = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MXFP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(achieved / MXFP4_PEAK_TFLOPS, 4), "traffic": stored_traffic(cfg.name, T),
                 "frac_of_bf16_peak": round(achieved / BF16_PEAK_TFLOPS, 4),
                 "path_ceiling": path_ceiling(self.args.path, I)}
        r.update({"kernel": "moe_mxfp4_ffn (gate_up + down)", "ms_per_launch": round(ffn_ms, 5),
                  "timed_calls": calls, "algorithmic_bytes": int(ffn_bytes), "algorithmic_flops": ffn_flops})
        self.log(f"{cfg.name} T={T} ffn: {ffn_ms * 1e3:.1f} us over {calls} calls, {r['achieved']} {r['unit']} "
                 f"({r['frac']:.1%})")
        return r

    def layer_bytes(self, b):
        cfg = self.cfg
        T, H, E, k = b["T"], cfg.H, cfg.E, cfg.k
        return b["touched"] * self.expert_bytes + E * H * 4 + E * 4 + T * H * 4 + T * k * 8

    def free(self):
        self.layers = []
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def path_ceiling(path, I):
    """The MFMA ceiling of the prefill kernel family, in algorithmic flops (AUTO's grouped GEMM
    takes the MXFP6 down input from 1024 activations on)."""
    if path == 0:
        path = 4 if I >= 1024 else 3
    if path == 3:
        return {"tflops": 2500.0, "basis": "FP8xFP4 scaled MFMA 5.0 PFLOP/s / 2 (two exact E4M3 terms per bf16 "
                                           "activation)"}
    if path == 4:
        # gate_up (2/3 of the flops) on FP8xFP4 at 2.5 PFLOP/s algorithmic, down (1/3) on FP6xFP4 at
        # 10.1 / 2 PFLOP/s: the harmonic combination
        return {"tflops": round(1.0 / ((2.0 / 3.0) / 2500.0 + (1.0 / 3.0) / 5050.0), 1),
                "basis": "gate_up FP8xFP4 5.0 PFLOP/s / 2, down FP6xFP4 10.1 PFLOP/s / 2 (two E2M3 terms), "
                         "weighted 2:1 by their flops"}
    return {"tflops": BF16_PEAK_TFLOPS, "basis": "bf16 MFMA 2.5 PFLOP/s"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "one GPU only: the layer runs on a single device, so --gpus must be 1"}), flush=True)
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

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    cfg = synth.get_config(args.workload)
    T = args.T or cfg.T_list[-1]
    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k
    lb = LayerBench(args, torch, synth, moe, dev, cfg, T, log)
    if args.chain:
        chain_main(args, torch, synth, moe, dev, cfg, T, lb, log)
        return
    inp = lb.inp
    norm_scale_np = None
    if args.block:  # the block's input: the residual stream, normalised inside the timed step
        inp.x = synth.make_block_x(cfg, T)
        norm_scale_np = synth.make_norm_scale(cfg)
        b = lb.batch(T, inp.x, block=True, norm_scale=torch.from_numpy(norm_scale_np).to(dev))
    else:
        b = lb.batch(T, inp.x)
    # the FFN roofline first: its >= 100 ms of warm-up and timed calls leave the clocks settled
    # for the layer steps (their own W warm-up steps then K timed steps follow unchanged)
    roofline = lb.ffn_roofline(b)
    ms = lb.time_steps(b, args.steps, args.warmup)
    tok_s = T / (ms * 1e-3)
    log(f"T={T}: {ms * 1e3:.1f} us/step, {tok_s:.0f} tok/s, touched {b['touched']}/{E}")
    decode_like = cfg.name.startswith("decode")

    sweep = []
    if not args.no_sweep and decode_like and not args.block:
        for Ts in cfg.T_list:
            if Ts == T:
                continue
            bs = lb.batch(Ts)
            rs = lb.ffn_roofline(bs)
            ms_s = lb.time_steps(bs, args.steps, args.warmup)
            gbps = lb.layer_bytes(bs) / (ms_s * 1e-3) / 1e9
            sweep.append({"T": Ts, "ms_per_step": round(ms_s, 5), "tokens_per_s": round(Ts / (ms_s * 1e-3), 1),
                          "touched_experts": bs["touched"], "layer_GBps": round(gbps, 1),
                          "layer_frac_of_hbm_peak": round(gbps / HBM_PEAK_GBS, 4),
                          "ffn_ms_per_launch": rs["ms_per_launch"], "ffn_GBps": rs["achieved"],
                          "ffn_frac_of_hbm_peak": rs["frac"]})
            log(f"sweep T={Ts}: {ms_s * 1e3:.1f} us/step, touched {bs['touched']}, layer {gbps:.0f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, inp, T, log, norm_scale_np)

    layer_bytes = lb.layer_bytes(b)
    counts = b["counts"]
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
                   "layers_rotated": lb.L, "path": args.path,
                   "touched_experts": b["touched"], "per_expert_slots_min_max": [int(counts.min()), int(counts.max())],
                   "layer_GBps": round(layer_bytes / (ms * 1e-3) / 1e9, 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if args.block:
        line["config"]["block"] = f"x + layer(RMSNorm(x)), eps {NORM_EPS:g}"
    if sweep:
        line["sweep"] = sweep
    # the metric's other half: the 4096-token prefill of the 20b-shaped layer, % of the MXFP4 peak
    if not args.no_prefill and decode_like and not args.block:
        lb.free()
        del lb, b
        pcfg = synth.get_config("prefill20b")
        pT = pcfg.T_list[-1]
        plb = LayerBench(args, torch, synth, moe, dev, pcfg, pT, log)
        pb = plb.batch(pT, plb.inp.x)
        proof = plb.ffn_roofline(pb)
        pms = plb.time_steps(pb, args.steps, args.warmup)
        log(f"prefill20b T={pT}: {pms * 1e3:.1f} us/step, {pT / (pms * 1e-3):.0f} tok/s")
        pc = pb["counts"]
        line["prefill"] = {"workload": pcfg.name, "T": pT, "E": pcfg.E, "k": pcfg.k, "path": args.path,
                           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(pms, 5),
                           "tokens_per_s": round(pT / (pms * 1e-3), 1), "layers_rotated": plb.L,
                           "per_expert_slots_min_max": [int(pc.min()), int(pc.max())],
                           "roofline": proof}
    print(json.dumps(line), flush=True)


def chain_main(args, torch, synth, moe, dev, cfg, T, lb, log):
    """L chained blocks per step: x_{l+1} = x_l + layer_l(bf16(RMSNorm_l(x_l))) (moe_block_forward_ex)
    over L distinct layer copies, so each layer's router reads the previous layer's output and
    its experts are streamed from HBM (L copies exceed the last-level cache). With
    --prefetch-hot N, each block first records an event; a side stream waits for it and reads
    that layer's N most popular experts (counts of the previous step through the same layer)
    while the block routes, as a test of warming the last-level cache for the expert stream."""
    L, H, E, k = args.chain, cfg.H, cfg.E, cfg.k
    if L > lb.L:
        raise SystemExit(f"--chain {L} needs --layers >= {L}")
    x0 = lb.bf16(synth.make_block_x(cfg, T))
    norms = [torch.from_numpy(synth.make_norm_scale(cfg)).to(dev) for _ in range(L)]
    ws = moe.workspace(T, E, k, H, cfg.I, args.path, device=dev)
    bufs = [torch.empty_like(x0), torch.empty_like(x0)]
    opts = moe.Options(path=args.path)
    side = torch.cuda.Stream()
    nb = len(lb.layers)

    # the routing each layer sees in the chain (same every step: same inputs), for the hot sets
    hot, touched = [], []
    x = x0
    for l in range(L):
        rt, w1, w2 = lb.layers[l % nb]
        xn = moe.moe_rmsnorm(x, norms[l], NORM_EPS)
        idx, _ = moe.moe_route(xn, rt, k)
        counts = np.bincount(idx.cpu().numpy().ravel(), minlength=E)
        touched.append(int((counts > 0).sum()))
        hot.append([int(e) for e in np.argsort(-counts, kind="stable")[:args.prefetch_hot] if counts[e] > 0])
        x = moe.moe_block_forward_ex(x, norms[l], NORM_EPS, rt, w1, w2, k, opts, ws=ws)
    per_e1 = lb.layers[0][1].codes.numel() // E  # tiled gate_up codes per expert (contiguous)
    per_e2 = lb.layers[0][2].codes.numel() // E
    sink = torch.zeros(1, dtype=torch.int64, device=dev)

    def prefetch(l):
        _, w1, w2 = lb.layers[l % nb]
        with torch.cuda.stream(side):
            for e in hot[l]:
                sink.add_(w1.codes[e * per_e1:(e + 1) * per_e1].view(torch.int32).sum(dtype=torch.int64))
                sink.add_(w2.codes[e * per_e2:(e + 1) * per_e2].view(torch.int32).sum(dtype=torch.int64))

    def step(_):
        x = x0
        for l in range(L):
            rt, w1, w2 = lb.layers[l % nb]
            if args.prefetch_hot:
                ev = torch.cuda.Event()
                ev.record()
                side.wait_event(ev)
                prefetch(l)
            out = bufs[l % 2]
            moe.moe_block_forward_ex(x, norms[l], NORM_EPS, rt, w1, w2, k, opts, out=out, ws=ws)
            x = out
        if args.prefetch_hot:
            torch.cuda.current_stream().wait_stream(side)

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
    per_layer = ms / L
    log(f"chain of {L} blocks, T={T}, prefetch {args.prefetch_hot}: {ms * 1e3:.1f} us/step, "
        f"{per_layer * 1e3:.1f} us per layer")
    line = {"metric": "chained MoE blocks tokens/s (one decode step through L layers)",
            "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": cfg.name, "T": T, "E": E, "k": k, "chain_layers": L, "path": args.path,
                       "prefetch_hot_experts": args.prefetch_hot, "ms_per_layer": round(per_layer, 5),
                       "layer_tokens_per_s": round(T / (per_layer * 1e-3), 1),
                       "touched_per_layer": touched},
            "roofline": None, "cpu_baseline": None}
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
        model, blas = host_description()
        cpu = {"value": round(reps * n / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "cpu_model": model, "blas": blas, "sample": f"first {n} of the {B} sequences, {reps} repetitions, fp64 numpy decode attention; {dt:.1f} s"}
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
    model, blas = host_description()
    return {"value": round(reps * n / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "blas": blas,
            "sample": f"first {n} of the {T} tokens, {reps} repetitions, full {'block' if norm_scale is not None else 'layer'} in fp64 numpy (router, "
                      f"top-{cfg.k}, per-expert MXFP4 decode, FFN, combine); {dt:.1f} s"}


if __name__ == "__main__":
    main()
