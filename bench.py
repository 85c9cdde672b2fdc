"""Benchmark of the quantized top-k MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one qmoe_forward (router, top-k, dispatch, grouped gate/up GEMM,
grouped down GEMM, combine) over one batch of seeded synthetic tokens whose
inputs are already resident in HBM. The default workload is the Mixtral-shaped
prefill layer (T=4096, d=4096, 8 experts top-2, d_ff=14336, INT4 asymmetric
group-128 weights). Prints ONE JSON line on stdout; progress goes to stderr.

The roofline object is for the dominant kernel (grouped gate/up GEMM for the
prefill workloads, the same kernel's weight stream for decode): algorithmic
FLOPs (or bytes) per launch divided by its average duration, measured with HIP
events recorded on the launch stream around every launch inside the timed
region. The CPU baseline times the fp64 oracle on a bounded token sample of the
same workload on the host cores.
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


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def algorithmic_work(cfg):
    """FLOPs of the whole layer and of one launch of each grouped GEMM, and the
    bytes of packed weights (all experts) for reference."""
    P = cfg.T * cfg.k
    fl13 = 2.0 * P * cfg.d * 2 * cfg.F + 2.0 * cfg.T * cfg.S * cfg.d * 2 * cfg.Fs
    fl2 = 2.0 * P * cfg.F * cfg.d + 2.0 * cfg.T * cfg.S * cfg.Fs * cfg.d
    return dict(layer=cfg.expert_flops(), gemm_gate_up=fl13, gemm_down=fl2)


def packed_bytes_per_expert(cfg, f, fmt=None):
    fmt = cfg.wformat if fmt is None else fmt
    n = 3 * cfg.d * f
    if fmt in ("int4_asym_g128", "int4_sym_g128", "int3_sym_g128"):
        groups = n // 128
        return n // 2 + groups * 2 * (2 if fmt == "int4_asym_g128" else 1)
    return n + 4 * (2 * f + cfg.d)


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


def cpu_baseline(inp, n_tokens: int = 0, target_s: float = 15.0):
    """The fp64 oracle on a token sample of the same layer: 16 and 32 tokens are
    timed first to separate the per-call cost (the oracle dequantizes each
    expert it uses on every call) from the per-token cost, which sizes the
    sample for about `target_s` seconds (or `n_tokens` when given); the rate is
    taken over the final, sized run."""
    from oracle import oracle as O
    cfg = inp.cfg
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    log(f"cpu baseline: quantizing the oracle's copy of the layer ({threads} threads)")
    layer = O.OracleLayer(inp)
    rng = np.random.default_rng(123)
    order = rng.permutation(cfg.T).astype(np.int32)
    if not n_tokens:
        times = []
        for n in (16, 32):
            probe = np.sort(order[:min(n, cfg.T)])
            t0 = time.perf_counter()
            layer.forward(inp.x, tokens=probe)
            times.append(time.perf_counter() - t0)
        per_token = max((times[1] - times[0]) / 16.0, 1e-9)
        per_call = max(times[0] - 16 * per_token, 0.0)
        n_tokens = int(min(cfg.T, max(32, (target_s - per_call) / per_token)))
    toks = np.sort(order[:min(n_tokens, cfg.T)])
    log(f"cpu baseline: oracle forward on {len(toks)} sampled tokens")
    t0 = time.perf_counter()
    layer.forward(inp.x, tokens=toks)
    dt = time.perf_counter() - t0
    layer.close()
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(toks)} of {cfg.T} tokens of the same layer (fp64 forward incl. per-expert "
                      f"dequantization; quantization setup untimed), {dt:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral_prefill")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0: sized for about 15 s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-mb", type=int, default=-1,
                    help="read this many MiB between timed decode steps to evict the 256 MB MALL "
                         "(default: 1024 for decode workloads, 0 otherwise)")
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

    import torch
    import quantized_mixture_experts_qmoe_amd as Q
    from quantized_mixture_experts_qmoe_amd.inputs import CONFIGS, make_inputs

    cfg = CONFIGS[args.config]
    decode = cfg.T <= 64
    log(f"workload {cfg.name}: generating seeded inputs")
    inp = make_inputs(cfg, seed=0)
    log("packing experts (host quantizer -> device arena)")
    layer = Q.QMoE(inp, max_tokens=cfg.T, device=0)
    x = torch.from_numpy(inp.x.view(np.int16)).view(torch.bfloat16).cuda()
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    flush_mb = args.flush_mb if args.flush_mb >= 0 else (1024 if decode else 0)
    # The flush reads (never writes) a buffer larger than the MALL, as the other
    # layers' weight reads would between two decode steps of this layer: the
    # evicted lines are clean, so the timed step pays no write-back for them.
    scratch = torch.ones(flush_mb * 1024 * 1024 // 4, dtype=torch.float32, device="cuda") if flush_mb else None
    flush_sink = torch.empty((), dtype=torch.float32, device="cuda") if flush_mb else None

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        layer.forward(x, y=y, stream=stream)
    torch.cuda.synchronize()

    def run_steps(n):
        """n steps; returns the summed step time in seconds. Decode steps are
        timed one by one with events (the MALL flush between them is not)."""
        if scratch is None:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                layer.forward(x, y=y, stream=stream)
            torch.cuda.synchronize()
            return time.perf_counter() - t0
        total = 0.0
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        for _ in range(n):
            torch.sum(scratch, dim=0, out=flush_sink)
            ev0.record(stream)
            layer.forward(x, y=y, stream=stream)
            ev1.record(stream)
            ev1.synchronize()
            total += ev0.elapsed_time(ev1) / 1e3
        return total

    # Timed region: only the dominant kernel carries events (each event record
    # idles the GPU for a few microseconds, which would inflate short steps).
    log(f"timing {args.steps} steps")
    layer.profile_enable(["gemm_gate_up"])
    elapsed = run_steps(args.steps)
    prof_timed = layer.profile_read()
    layer.profile_enable(False)
    # Per-kernel split from a separate pass with every kernel timed.
    split_steps = min(args.steps, 10)
    log(f"per-kernel split over {split_steps} more steps")
    layer.profile_enable(True)
    run_steps(split_steps)
    prof = layer.profile_read()
    layer.profile_enable(False)

    ms_per_step = 1e3 * elapsed / args.steps
    value = cfg.T * args.steps / elapsed
    work = algorithmic_work(cfg)
    kernels = {k: {"avg_us": 1e3 * v[0] / max(v[1], 1), "launches": v[1]} for k, v in prof.items() if v[1]}
    ms13, n13 = prof_timed["gemm_gate_up"]
    # per step: a layer with per-expert formats launches each GEMM once per format
    per_step = max(1, round(n13 / args.steps))
    k13 = 1e3 * ms13 / args.steps   # the gate/up GEMM's time per step (us) over the timed region
    kname = "gemm_gate_up" if per_step == 1 else f"gemm_gate_up ({per_step} launches per step, one per format)"
    if not decode:
        achieved = work["gemm_gate_up"] / (k13 * 1e-6) / 1e12
        roof = {"bound": "mfma", "kernel": kname, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic("gemm_gate_up", cfg.name), "traffic_unit": "bytes/launch",
                "per_launch": f"{work['gemm_gate_up']:.4e} FLOP"}
    else:
        # bytes of the gate/up weights of the distinct experts this batch selects
        route = Q.QMoE.route_buffers(cfg.T, cfg.E, cfg.k)
        layer.forward(x, y=y, route=route)
        torch.cuda.synchronize()
        used = np.unique(route["topk_idx"].cpu().numpy())
        b13 = sum(packed_bytes_per_expert(cfg, cfg.F, cfg.expert_format(int(e))) * 2 // 3 for e in used)
        b13 += cfg.T * cfg.d * 2
        achieved = b13 / (k13 * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                "traffic": measured_traffic("gemm_gate_up", cfg.name), "traffic_unit": "bytes/launch",
                "per_launch": f"{b13} B ({len(used)} distinct experts)"}
    layer_tflops = work["layer"] / (ms_per_step * 1e-3) / 1e12
    log(f"{value:.4g} tokens/s, {ms_per_step:.3f} ms/step, layer {layer_tflops:.1f} TFLOP/s; kernels: "
        + ", ".join(f"{k}={v['avg_us']:.1f}us" for k, v in kernels.items()))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_tokens)
        log(f"cpu baseline {cpu['value']:.3g} tokens/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d, "experts": cfg.E, "top_k": cfg.k,
                   "d_ff": cfg.F, "shared": cfg.S, "weights": cfg.wformat, "parallelism": "none (1 GPU)"},
        "layer_tflops": layer_tflops,
        "layer_mfma_frac": layer_tflops / PEAK_BF16_TFLOPS,
        "kernels_us": {k: round(v["avg_us"], 2) for k, v in kernels.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    layer.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
