"""Benchmark of the quantized top-k MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME|all]

A step is one qmoe_forward (router, top-k, dispatch, grouped gate/up GEMM,
grouped down GEMM, combine) over one batch of seeded synthetic tokens whose
inputs are already resident in HBM. The headline workload is the
Mixtral-shaped prefill layer (T=4096, d=4096, 8 experts top-2, d_ff=14336,
INT4 asymmetric group-128 weights): W untimed warm-up steps, then exactly K
steps bracketed by device synchronisations give `value` and `ms_per_step`.

With --config all (the default) every other workload is measured in the same
run and reported under "workloads": per workload the median and minimum of 50
event-timed calls (200 for the tiny and decode-shaped layers), tokens/s at the
median, the per-kernel split, the dominant kernel's roofline fraction (MFMA for
the prefill shapes, HBM for the decode shapes, whose calls each follow a 1 GiB
read that evicts the 256 MB MALL), the HBM counter traffic where committed
counters cover the current kernel code, the sampled GPU clock, and the fp64
oracle timed on a bounded token sample on the host cores. Decode shapes also
report the same forward recorded once into a HIP graph and replayed
(`step_us_graph`). Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "MoE-layer tokens/s (1 GPU) + % of MFMA peak (prefill) / % HBM BW (decode)"
HEADLINE = "mixtral_prefill"
ALL = ("mixtral_prefill", "qwen3_prefill", "dsv2lite_prefill", "qwen3_decode", "qwen3_decode_fp8",
       "qwen3_prefill_mixed", "qwen3_decode_mixed", "tiny")


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def algorithmic_work(cfg):
    """FLOPs of the whole layer and of one launch of each grouped GEMM."""
    P = cfg.T * cfg.k
    fl13 = 2.0 * P * cfg.d * 2 * cfg.F + 2.0 * cfg.T * cfg.S * cfg.d * 2 * cfg.Fs
    fl2 = 2.0 * P * cfg.F * cfg.d + 2.0 * cfg.T * cfg.S * cfg.Fs * cfg.d
    return dict(layer=cfg.expert_flops(), gemm_gate_up=fl13, gemm_down=fl2)


def packed_bytes(cfg, f, fmt, matrix):
    """Packed bytes (codes + scales (+ zeros)) of one expert's W13 (matrix 13)
    or W2 (matrix 2) in format fmt."""
    n = (2 if matrix == 13 else 1) * cfg.d * f
    rows = 2 * f if matrix == 13 else cfg.d
    if fmt in ("int4_asym_g128", "int4_sym_g128", "int3_sym_g128"):
        return n // 2 + (n // 128) * 2 * (2 if fmt == "int4_asym_g128" else 1)
    return n + 4 * rows


def kernel_code_digest(path: str) -> str:
    """SHA-256 of a C++/HIP source with its comments and whitespace removed, so
    that only a change to the code itself retires counters taken on it."""
    import hashlib
    import re
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    copy-calibrated FETCH_SIZE + WRITE_SIZE counter runs, or None when no run
    covers it or the kernel code has changed since the counters were taken."""
    rec_path = os.path.join(ROOT, "profiles", "traffic.json")
    src = os.path.join(ROOT, "quantized_mixture_experts_qmoe_amd", "csrc", "qmoe_kernels.hip")
    try:
        rec = json.load(open(rec_path))
        digest = kernel_code_digest(src)
    except OSError:
        return None
    if rec.get("kernel_code_digest") != digest:
        return None
    return rec.get("kernels", {}).get(kernel, {}).get(workload)


class ClockProbe:
    """Shader clock during a timed region: the library's probe wavefront runs on
    a second stream (default priority) beside the region and samples the
    shader-cycle and real-time counters; clock = cycles / ticks * tick rate."""

    def __init__(self):
        import ctypes as C
        import torch
        import quantized_mixture_experts_qmoe_amd as Q
        self.Q, self.C, self.torch = Q, C, torch
        self.stream = torch.cuda.Stream()
        self.n = 2048
        self.buf = torch.zeros((self.n, 2), dtype=torch.int64, device="cuda")
        self.khz = C.c_int64(0)
        self._call(1, 1)
        torch.cuda.synchronize()
        self.last = None

    def _call(self, dur, period):
        rc = self.Q.qmoe_clock_probe(self.stream.cuda_stream, int(dur), int(period), self.n, self.buf.data_ptr(),
                                     self.C.byref(self.khz))
        if rc != 0:
            raise RuntimeError(f"qmoe_clock_probe: {self.Q.qmoe_last_error()}")

    def window(self, seconds: float):
        probe = self

        class _W:
            def __enter__(self):
                probe.buf.zero_()
                probe.torch.cuda.synchronize()
                ticks = max(1, int(seconds * probe.khz.value * 1e3))
                probe._call(ticks, max(1, ticks // (probe.n - 1)))
                return self

            def __exit__(self, *a):
                probe.torch.cuda.synchronize()
                s = probe.buf.cpu().numpy()
                s = s[s[:, 1] > 0].astype(np.float64)
                probe.last = None
                if len(s) >= 3:
                    hz = probe.khz.value * 1e3
                    dc, dr = np.diff(s[:, 0]), np.diff(s[:, 1])
                    mhz = dc / np.maximum(dr, 1) * hz / 1e6
                    probe.last = {"mean_mhz": float((s[-1, 0] - s[0, 0]) / (s[-1, 1] - s[0, 1]) * hz / 1e6),
                                  "median_mhz": float(np.median(mhz)), "p10_mhz": float(np.percentile(mhz, 10)),
                                  "p90_mhz": float(np.percentile(mhz, 90)), "samples": int(len(s)),
                                  "window_s": float((s[-1, 1] - s[0, 1]) / hz)}
        return _W()

    def summary(self):
        return self.last


def cpu_baseline(inp, target_s: float):
    """The fp64 oracle on a token sample of the same layer: 8 and 16 tokens are
    timed first to separate the per-call cost (the oracle dequantizes each
    expert it uses on every call) from the per-token cost, which sizes the
    sample for about `target_s` seconds; the rate is taken over the final,
    sized run."""
    from oracle import oracle as O
    cfg = inp.cfg
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    layer = O.OracleLayer(inp)
    rng = np.random.default_rng(123)
    order = rng.permutation(cfg.T).astype(np.int32)
    times = []
    for n in (8, 16):
        probe = np.sort(order[:min(n, cfg.T)])
        t0 = time.perf_counter()
        layer.forward(inp.x, tokens=probe)
        times.append(time.perf_counter() - t0)
    per_token = max((times[1] - times[0]) / 8.0, 1e-9)
    per_call = max(times[0] - 8 * per_token, 0.0)
    n_tokens = int(min(cfg.T, max(16, (target_s - per_call) / per_token)))
    toks = np.sort(order[:n_tokens])
    t0 = time.perf_counter()
    layer.forward(inp.x, tokens=toks)
    dt = time.perf_counter() - t0
    layer.close()
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(toks)} of {cfg.T} tokens of the same layer (fp64 forward incl. per-expert "
                      f"dequantization; quantization setup untimed), {dt:.1f} s"}


def bench_workload(name, steps, warmup, contract_steps, clock, cpu_s, flush_mb):
    """Measures one workload; returns its result object. contract_steps > 0:
    also time exactly that many steps between device synchronisations (the
    headline's value)."""
    import torch
    import quantized_mixture_experts_qmoe_amd as Q
    from quantized_mixture_experts_qmoe_amd.inputs import CONFIGS, make_inputs

    cfg = CONFIGS[name]
    decode = cfg.T <= 64
    log(f"workload {name}: generating seeded inputs")
    inp = make_inputs(cfg, seed=0)
    log(f"workload {name}: packing experts (host quantizer -> device arena)")
    layer = Q.QMoE(inp, max_tokens=cfg.T, device=0)
    x = torch.from_numpy(inp.x.view(np.int16)).view(torch.bfloat16).cuda()
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    fl = flush_mb if (decode and flush_mb > 0) else 0
    # The flush reads (never writes) a buffer larger than the MALL, as the
    # other layers' weight reads would between two decode steps of this layer:
    # the evicted lines are clean, so the timed step pays no write-back.
    scratch = torch.ones(fl * 1024 * 1024 // 4, dtype=torch.float32, device="cuda") if fl else None
    sink = torch.empty((), dtype=torch.float32, device="cuda") if fl else None

    def flush():
        if scratch is not None:
            torch.sum(scratch, dim=0, out=sink)

    flush()
    layer.forward(x, y=y, stream=stream)   # first call: code loading, not timed
    torch.cuda.synchronize()
    tw = time.perf_counter()
    for _ in range(max(warmup - 1, 1)):
        flush()
        layer.forward(x, y=y, stream=stream)
    torch.cuda.synchronize()
    per_call_s = (time.perf_counter() - tw) / max(warmup - 1, 1)   # for the clock probe's window
    res = {"config": {"T": cfg.T, "d_model": cfg.d, "experts": cfg.E, "top_k": cfg.k, "d_ff": cfg.F,
                      "shared": cfg.S, "d_ff_shared": cfg.Fs, "weights": cfg.wformat,
                      "per_expert_formats": cfg.expert_formats is not None, "router_bias": cfg.bias}}

    # 1. the contract's K steps, bracketed by device-wide synchronisations
    #    (headline only), with no events inside and nothing else on the GPU:
    #    the clock probe runs beside the per-call timing below instead (a
    #    device-wide synchronisation would wait for the probe's window)
    if contract_steps:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(contract_steps):
            layer.forward(x, y=y, stream=stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        res["contract"] = {"steps": contract_steps, "elapsed_s": elapsed}

    # 2. per-call event timing: median and min over `steps` calls
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    with clock.window(1.1 * steps * per_call_s):
        for a, b in ev:
            flush()
            a.record(stream)
            layer.forward(x, y=y, stream=stream)
            b.record(stream)
        torch.cuda.synchronize()
    call_us = np.array([1e3 * a.elapsed_time(b) for a, b in ev])
    res["step_us"] = {"median": float(np.median(call_us)), "min": float(call_us.min()),
                      "mean": float(call_us.mean()), "calls": steps,
                      "mall_flushed": bool(fl)}
    res["tokens_per_s"] = cfg.T / (np.median(call_us) * 1e-6)
    res["gpu_clock"] = clock.summary()
    if decode and fl:
        # warm: the same calls without the flush (weights partly MALL-resident)
        warm = []
        for _ in range(min(steps, 50)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            layer.forward(x, y=y, stream=stream)
            b.record(stream)
            warm.append((a, b))
        torch.cuda.synchronize()
        res["step_us_warm_mall_aside"] = float(np.median([1e3 * a.elapsed_time(b) for a, b in warm]))
    if decode:
        # the same forward recorded once into a HIP graph and replayed (a
        # serving loop's form: no per-launch host cost between the kernels);
        # same flush before each replay
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            layer.forward(x, y=y, stream=side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            layer.forward(x, y=y, stream=torch.cuda.current_stream())
        torch.cuda.synchronize()
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in gev:
            flush()
            a.record(stream)
            graph.replay()
            b.record(stream)
        torch.cuda.synchronize()
        g_us = np.array([1e3 * a.elapsed_time(b) for a, b in gev])
        res["step_us_graph"] = {"median": float(np.median(g_us)), "min": float(g_us.min()), "calls": steps,
                                "mall_flushed": bool(fl), "what": "one HIP graph replay of the forward"}
        del graph

    # 3. kernel durations: every kernel launch of n_dom more calls between its
    #    own pair of events on the launch stream (with events on every kernel,
    #    each start event follows the previous kernel's end event); the
    #    dominant kernel's average gives the roofline, all of them the split
    n_dom = min(steps, 50)
    layer.profile_enable(True)
    with clock.window(1.1 * n_dom * per_call_s):
        for _ in range(n_dom):
            flush()
            layer.forward(x, y=y, stream=stream)
        prof = layer.profile_read()
    layer.profile_enable(False)
    res["kernel_clock"] = clock.summary()
    dom = prof["gemm_gate_up"]
    # per step (a layer with per-expert formats launches each GEMM once per format)
    res["kernels_us"] = {k: round(1e3 * v[0] / n_dom, 2) for k, v in prof.items() if v[1]}
    res["kernel_timing"] = f"HIP events around every kernel of {n_dom} calls on the launch stream"

    work = algorithmic_work(cfg)
    ms13, n13 = dom
    per_step = max(1, round(n13 / n_dom))   # per-expert formats: one launch per format
    k13_us = 1e3 * ms13 / n_dom
    kname = "gemm_gate_up" if per_step == 1 else f"gemm_gate_up ({per_step} launches per step, one per format)"
    if not decode:
        achieved = work["gemm_gate_up"] / (k13_us * 1e-6) / 1e12
        res["roofline"] = {"bound": "mfma", "kernel": kname, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                           "traffic": measured_traffic("gemm_gate_up", name), "traffic_unit": "bytes/launch",
                           "per_launch": f"{work['gemm_gate_up']:.4e} FLOP", "avg_us": k13_us}
        res["layer_tflops"] = work["layer"] / (res["step_us"]["median"] * 1e-6) / 1e12
    else:
        # bytes of the packed weights of the distinct experts this batch selects
        route = Q.QMoE.route_buffers(cfg.T, cfg.E, cfg.k)
        layer.forward(x, y=y, route=route)
        torch.cuda.synchronize()
        used = np.unique(route["topk_idx"].cpu().numpy())
        b13 = sum(packed_bytes(cfg, cfg.F, cfg.expert_format(int(e)), 13) for e in used) + cfg.T * cfg.d * 2
        b2 = sum(packed_bytes(cfg, cfg.F, cfg.expert_format(int(e)), 2) for e in used)
        step_bytes = b13 + b2 + cfg.E * cfg.d * 2 + cfg.T * cfg.d * 2
        achieved = b13 / (k13_us * 1e-6) / 1e9
        res["roofline"] = {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                           "traffic": measured_traffic("gemm_gate_up", name), "traffic_unit": "bytes/launch",
                           "per_launch": f"{b13} B ({len(used)} distinct experts)", "avg_us": k13_us}
        step_gbs = step_bytes / (res["step_us"]["median"] * 1e-6) / 1e9
        res["step_hbm"] = {"bytes": step_bytes, "achieved": step_gbs, "unit": "GB/s",
                           "frac": step_gbs / PEAK_HBM_GBS,
                           "what": "packed weights of the selected experts + router weight + x + y"}
    if "step_us_graph" in res:
        log(f"{name}: graph replay median {res['step_us_graph']['median']:.1f} us "
            f"(min {res['step_us_graph']['min']:.1f})")
    log(f"{name}: median {res['step_us']['median']:.1f} us (min {res['step_us']['min']:.1f}), "
        f"{res['tokens_per_s']:.4g} tokens/s, {res['roofline']['kernel']} {res['roofline']['frac']:.3f} of "
        f"{res['roofline']['bound']} peak; clock {res['gpu_clock']}; kernels "
        + ", ".join(f"{k}={v}" for k, v in res["kernels_us"].items()))
    layer.close()
    del layer, scratch
    torch.cuda.empty_cache()
    if cpu_s > 0:
        log(f"{name}: cpu baseline (oracle on a token sample, about {cpu_s:.0f} s)")
        res["cpu_baseline"] = cpu_baseline(inp, cpu_s)
        log(f"{name}: cpu baseline {res['cpu_baseline']['value']:.4g} tokens/s "
            f"on {res['cpu_baseline']['cores']} threads")
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="headline: steps timed between synchronisations")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="all", help="a workload name, or 'all' (headline plus every workload)")
    ap.add_argument("--calls", type=int, default=0,
                    help="event-timed calls per workload (0: 50, or 200 for the tiny and decode-shaped layers)")
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="oracle sample size per workload in seconds of host time (headline: 4x)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-mb", type=int, default=1024,
                    help="MiB read before every timed decode call to evict the 256 MB MALL (0: none)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (3 times), the "
                         "reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.copy_calibration_mb:
        import torch
        n = args.copy_calibration_mb * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 3}))
        return 0
    if args.gpus != 1:
        print(f"bench.py: the layer runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(the experts are not sharded across GPUs).", file=sys.stderr)
        return 2

    from quantized_mixture_experts_qmoe_amd.inputs import CONFIGS
    head = HEADLINE if args.config == "all" else args.config
    if head not in CONFIGS:
        print(f"bench.py: unknown workload {head}", file=sys.stderr)
        return 2
    others = [n for n in ALL if n != head] if args.config == "all" else []
    clock = ClockProbe()

    def calls_for(n):
        return args.calls or (200 if CONFIGS[n].T <= 64 else 50)

    cpu_s = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    hres = bench_workload(head, calls_for(head), args.warmup, args.steps, clock, 4 * cpu_s, args.flush_mb)
    workloads = {}
    for n in others:
        workloads[n] = bench_workload(n, calls_for(n), args.warmup, 0, clock, cpu_s, args.flush_mb)

    cfg = CONFIGS[head]
    c = hres["contract"]
    ms_per_step = 1e3 * c["elapsed_s"] / args.steps
    value = cfg.T * args.steps / c["elapsed_s"]
    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": head, "T": cfg.T, "d_model": cfg.d, "experts": cfg.E, "top_k": cfg.k,
                   "d_ff": cfg.F, "shared": cfg.S, "weights": cfg.wformat, "parallelism": "none (1 GPU)"},
        "layer_tflops": algorithmic_work(cfg)["layer"] / (ms_per_step * 1e-3) / 1e12,
        "step_us": hres["step_us"],
        "gpu_clock": hres["gpu_clock"],
        "kernels_us": hres["kernels_us"],
        "roofline": hres["roofline"],
        "cpu_baseline": hres.get("cpu_baseline"),
        "workloads": workloads,
    }
    out["layer_mfma_frac"] = out["layer_tflops"] / PEAK_BF16_TFLOPS
    for key in ("step_us_graph", "step_us_warm_mall_aside", "step_hbm"):
        if key in hres:
            out[key] = hres[key]
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
