"""Benchmark of the MI355X mixture-of-experts layer (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME ...]

A step is one pass of the whole layer (route, group, grouped SwiGLU experts, combine)
over one batch of seeded synthetic inputs already resident in HBM.  The headline
workload is the Inkling-shaped prefill batch (T = 8,192), where the layer is bound by
bf16 MFMA throughput; the Inkling-shaped decode batch (T = 32), bound by streaming the
active experts' weights from HBM, is measured in the same run and reported in the same
JSON line under "decode", and the same decode batch with MXFP4 routed-expert weights
under "decode_mxfp4".  Rank 0 prints one JSON line.

Per-stage durations come from HIP events recorded on the launch stream between the
C-ABI calls of every timed step.  The dominant kernel work is the grouped SwiGLU step
(m-tile plan + gate/up GEMM + down GEMM); its roofline is reported against the bf16
MFMA peak (prefill) or the HBM peak (decode).  The CPU oracle is timed on a bounded
token sample of the prefill workload on the host's cores as a reported baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = ("MoE-layer tokens/s + % bf16 MFMA peak (prefill), % HBM BW (decode), 1 GPU")
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4,096 flop/clk x 2.4 GHz (dense; 2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0       # HBM3E, 8 TB/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


GROUPED_SOURCES = ["grouped_gemm.hip", "moe_device.h", "moe_launch.h"]


def grouped_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GROUPED_SOURCES:
        with open(os.path.join(ROOT, "sparse_mixture_experts_fp32_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic(workload: str):
    """HBM bytes per launch of the grouped SwiGLU step from the committed rocprofv3 counter
    summary of this workload, or None when the kernel sources changed since it was taken
    (or no summary exists)."""
    path = os.path.join(ROOT, "profiles", f"grouped_swiglu_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                fields[k.strip("`")] = v.strip().strip("`")
    if fields.get("sources_sha256") != grouped_sources_sha256():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", nargs="*",
                   default=["inkling_prefill", "inkling_decode", "inkling_decode_mxfp4"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=1024,
                   help="tokens of the prefill batch the oracle is timed on")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="first run one plain device-to-device copy of BYTES bytes, the "
                        "reference kernel for scaling hardware byte counters")
    return p.parse_args()


def layer_flops(c):
    router = 2 * c.T * c.d * (c.E + c.S)
    experts = 2 * c.T * (c.k + c.S) * 3 * c.d * c.I
    return router, experts


def run(c, steps, warmup, torch):
    import numpy as np

    from gpu_util import StagedRunner, device_inputs
    from moe_inputs import make_inputs

    t0 = time.perf_counter()
    inp = make_inputs(c)
    log(f"[{c.name}] inputs generated in {time.perf_counter() - t0:.1f} s")
    dev = device_inputs(inp, torch)
    torch.cuda.synchronize()
    log(f"[{c.name}] inputs resident in HBM")
    runner = StagedRunner(c, dev, torch)
    T, A = c.T, c.k + c.S
    R = T * A
    counts = runner.counts
    stream = torch.cuda.current_stream()

    def step(ev=None):
        runner.step(stream, ev)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    stage = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evs])  # ms
    step_ms = np.array([e[0].elapsed_time(e[4]) for e in evs])
    cnt = counts.cpu().numpy()
    touched = int((cnt[:c.E] > 0).sum())
    esize = 2 if c.dtype == "bf16" else 4
    f_router, f_experts = layer_flops(c)
    if c.weight_format == "mxfp4":   # routed: 4-bit codes + one scale byte per 32
        w_bytes = touched * 3 * c.d * c.I * (0.5 + 1 / 32) + c.S * 3 * c.d * c.I * esize
    else:
        w_bytes = (touched + c.S) * 3 * c.d * c.I * esize
    alg_bytes = (w_bytes + (c.E + c.S) * c.d * esize + T * c.d * esize + T * c.d * 4)
    grouped_bytes = w_bytes + T * c.d * esize + R * c.d * 4
    ms = wall * 1e3 / steps
    grouped_ms = float(stage[:, 2].mean())
    res = {
        "T": T, "ms_per_step": ms, "tokens_per_s": T * steps / wall,
        "event_ms_per_step_median": float(np.median(step_ms)),
        "event_ms_per_step_p10": float(np.percentile(step_ms, 10)),
        "event_ms_per_step_p90": float(np.percentile(step_ms, 90)),
        "stage_ms": {"route": float(stage[:, 0].mean()), "permute": float(stage[:, 1].mean()),
                     "grouped_swiglu": grouped_ms, "combine": float(stage[:, 3].mean())},
        "layer_tflops": (f_router + f_experts) / (ms * 1e-3) / 1e12,
        "layer_alg_gbs": alg_bytes / (ms * 1e-3) / 1e9,
        "touched_routed_experts": touched, "max_rows_per_expert": int(cnt[:c.E].max()),
        "grouped_flops": f_experts, "grouped_alg_bytes": grouped_bytes,
        "grouped_tflops": f_experts / (grouped_ms * 1e-3) / 1e12,
        "grouped_gbs": grouped_bytes / (grouped_ms * 1e-3) / 1e9,
    }
    del dev, runner
    torch.cuda.empty_cache()
    return res, inp


def cpu_baseline(c, inp, n_tokens):
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O
    tokens = np.arange(min(n_tokens, c.T))
    t0 = time.perf_counter()
    O.moe_forward(c, inp, mode="bf16_flow", tokens=tokens)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f
                          if ln.startswith("model name")), model)
    except OSError:
        pass
    return {"value": len(tokens) / dt, "unit": "tokens/s", "cores": int(threads),
            "usable_cores": len(os.sched_getaffinity(0)), "cpu_model": model,
            "kind": "oracle", "seconds": dt,
            "sample": f"first {len(tokens)} tokens of the {c.name} batch (T={c.T}), "
                      f"float64 NumPy oracle in bf16-flow mode, one call incl. routing "
                      f"and per-expert float64 promotion"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer is built and measured on a "
              "single MI355X (no sharding, no collectives); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from moe_inputs import CONFIGS
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calibration} bytes")
        del src, dst
    results = {}
    prefill_inputs = None
    for name in args.workload:
        c = CONFIGS[name]
        # The line's own workload times exactly --steps steps; the decode blocks beside a
        # prefill line take at least 50 (each step is ~1 ms or less).
        steps = args.steps if (name == args.workload[0] or c.T >= 1024) else max(args.steps, 50)
        res, inp = run(c, steps, args.warmup, torch)
        res["steps"] = steps
        results[name] = res
        log(f"[{name}] {json.dumps(res)}")
        if name == "inkling_prefill":
            prefill_inputs = inp
        else:
            del inp
    head = args.workload[0]
    c = CONFIGS[head]
    r = results[head]
    # The grouped step's bound: MFMA when its algorithmic intensity (FLOPs per byte of
    # weights, x and Y_rows) is above the ridge of the two peaks, HBM below it.
    intensity = r["grouped_tflops"] * 1e3 / r["grouped_gbs"]
    if intensity >= PEAK_BF16_TFLOPS * 1e3 / PEAK_HBM_GBS:
        roof = {"bound": "mfma", "achieved": r["grouped_tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": r["grouped_tflops"] / PEAK_BF16_TFLOPS,
                "traffic": profiled_traffic(head),
                "kernel": "grouped SwiGLU (gate/up + down GEMMs)"}
    else:
        roof = {"bound": "hbm", "achieved": r["grouped_gbs"], "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": r["grouped_gbs"] / PEAK_HBM_GBS,
                "traffic": profiled_traffic(head),
                "kernel": "grouped SwiGLU (gate/up + down GEMMs)"}
    line = {
        "metric": METRIC, "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head, "T": c.T, "d": c.d, "E": c.E, "S": c.S, "I": c.I,
                   "k": c.k, "router": c.router},
        "roofline": roof,
        "layer_tflops": r["layer_tflops"],
        "layer_frac_bf16_mfma": r["layer_tflops"] / PEAK_BF16_TFLOPS,
        "step_ms_p10_p50_p90": [r["event_ms_per_step_p10"], r["event_ms_per_step_median"],
                                r["event_ms_per_step_p90"]],
        "stage_ms": r["stage_ms"],
        "touched_routed_experts": r["touched_routed_experts"],
    }
    for key, name in (("decode", "inkling_decode"), ("decode_mxfp4", "inkling_decode_mxfp4")):
        if name not in results or head == name:
            continue
        d = results[name]
        line[key] = {
            "workload": name, "T": d["T"], "steps": d["steps"], "tokens_per_s": d["tokens_per_s"],
            "ms_per_step": d["ms_per_step"],
            "step_ms_p10_p50_p90": [d["event_ms_per_step_p10"], d["event_ms_per_step_median"],
                                    d["event_ms_per_step_p90"]],
            "stage_ms": d["stage_ms"],
            "touched_routed_experts": d["touched_routed_experts"],
            "roofline": {"bound": "hbm", "achieved": d["grouped_gbs"], "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": d["grouped_gbs"] / PEAK_HBM_GBS,
                         "traffic": profiled_traffic(name)},
            "layer_alg_gbs": d["layer_alg_gbs"],
            "layer_frac_hbm": d["layer_alg_gbs"] / PEAK_HBM_GBS,
        }
    if not args.no_cpu_baseline and prefill_inputs is not None:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(CONFIGS["inkling_prefill"], prefill_inputs,
                                            args.cpu_sample)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
