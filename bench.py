"""Benchmark of the MI355X mixture-of-experts layer (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME ...]

A step is one pass of the whole layer (route, group, grouped SwiGLU experts, combine)
over one batch of seeded synthetic inputs already resident in HBM.  The headline
workload is the Inkling-shaped prefill batch (T = 8,192), where the layer is bound by
bf16 MFMA throughput; it heads the JSON line.  The same run measures the other
workloads and reports each in the line's "configs" map: the Inkling-shaped decode batch
(T = 32, bound by streaming the active experts' weights from HBM) in bf16 and with MXFP4
routed-expert weights, the tiny fp32 layer, the Qwen3.8-shaped layer and the skewed
(Zipf-offset) Inkling batch.  Rank 0 prints one JSON line.

Per-stage durations come from HIP events recorded on the launch stream between the
C-ABI calls of every timed step.  The dominant kernel work is the grouped SwiGLU step
(m-tile plan + gate/up GEMM + down GEMM); its roofline is reported against the MFMA peak
of the layer's dtype or the HBM peak, whichever side of the ridge its algorithmic
intensity falls on.  The CPU leg runs the oracle on the host's cores: its routing of
every batch (which gives the count of near-tie tokens the parity rule excludes) and, as
the reported baseline, the whole prefill batch timed.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE-layer tokens/s + % bf16 MFMA peak (prefill), % HBM BW (decode), 1 GPU")
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4,096 flop/clk x 2.4 GHz (dense; 2.5 PFLOP/s)
PEAK_F32_TFLOPS = 157.3     # dense fp32 MFMA
PEAK_HBM_GBS = 8000.0       # HBM3E, 8 TB/s
DEFAULT_WORKLOADS = ["inkling_prefill", "inkling_decode", "inkling_decode_mxfp4",
                     "tiny_fp32", "qwen38", "inkling_skewed"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


GROUPED_SOURCES = ["grouped_gemm.hip", "moe_device.h", "moe_launch.h"]


def grouped_sources_sha256() -> str:
    """sha256 of the grouped GEMM's sources with their comments and blank lines removed:
    it changes when the compiled kernels can, not when only their comments do."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in GROUPED_SOURCES:
        with open(os.path.join(ROOT, "sparse_mixture_experts_fp32_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln).encode())
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
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", nargs="*", default=DEFAULT_WORKLOADS)
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the CPU leg (oracle routing counts and the oracle timing)")
    p.add_argument("--cpu-sample", type=int, default=0,
                   help="tokens of the prefill batch the oracle is timed on (0: all)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="first run one plain device-to-device copy of BYTES bytes, the "
                        "reference kernel for scaling hardware byte counters")
    return p.parse_args()


def layer_flops(c):
    router = 2 * c.T * c.d * (c.E + c.S)
    experts = 2 * c.T * (c.k + c.S) * 3 * c.d * c.I
    return router, experts


def run(c, steps, warmup, torch, warm_s=0.0):
    """Time `steps` steps of workload c after `warmup` untimed ones (and, when warm_s > 0,
    further untimed steps until warm_s seconds of them have run: a decode step lasts
    ~0.5-1.3 ms, and the GPU's clocks settle only after some hundred of them)."""
    import numpy as np

    from moe_inputs import make_inputs
    from sparse_mixture_experts_fp32_amd.staged import StagedRunner, device_inputs

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
    warm_steps, tw = warmup, time.perf_counter()
    while time.perf_counter() - tw < warm_s:
        for _ in range(10):
            step()
        warm_steps += 10
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
        "T": T, "warmup_steps": warm_steps, "ms_per_step": ms, "tokens_per_s": T * steps / wall,
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


def cpu_gap_excluded(c, inp):
    """CPU leg: the oracle's routing of the whole batch (float64), and the number of
    tokens whose k-th / (k+1)-th selection-score gap is below the parity rule's
    threshold (1e-6; 1e-4 for pre-norm layers), which the bit-exact index rule skips."""
    import numpy as np

    from oracle import moe_oracle as O
    x = inp["x"]
    if c.prenorm:
        x = O.prenorm_input(c, inp["x"], inp["norm_gain"], c.norm_eps,
                            1.0 if c.norm_zero_centred else 0.0)
    r = O.route(c, x, inp["w_router"], inp.get("sel_bias"), inp.get("logit_offset"))
    return int(np.sum(r.gap < (1e-4 if c.prenorm else 1e-6)))


def cpu_baseline(c, inp, n_tokens):
    """CPU leg: the oracle as it stands, timed on the host's cores over the first
    n_tokens tokens of the batch (all of them when n_tokens is 0)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O
    n = c.T if n_tokens <= 0 else min(n_tokens, c.T)
    tokens = np.arange(n)
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
    what = (f"the whole {c.name} batch ({c.T} tokens)" if n == c.T else
            f"the first {n} of the {c.T} tokens of the {c.name} batch (a sample)")
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads),
            "usable_cores": len(os.sched_getaffinity(0)), "cpu_model": model,
            "kind": "oracle", "seconds": dt,
            "sample": f"{what}: one float64 NumPy oracle call in bf16-flow mode, routing "
                      f"and the per-expert float64 promotion of every touched expert's "
                      f"weights included, input generation excluded"}


def grouped_roofline(c, r, workload):
    """Roofline of the grouped SwiGLU step: the MFMA peak of the layer's dtype when the
    step's algorithmic intensity (FLOPs per byte of weights, x and Y_rows) lies above the
    ridge of that peak and the HBM peak, the HBM peak below it."""
    peak = PEAK_BF16_TFLOPS if c.dtype == "bf16" else PEAK_F32_TFLOPS
    intensity = r["grouped_tflops"] * 1e3 / r["grouped_gbs"]
    kernel = "grouped SwiGLU (gate/up + down GEMMs)"
    if intensity >= peak * 1e3 / PEAK_HBM_GBS:
        return {"bound": "mfma", "achieved": r["grouped_tflops"], "peak": peak,
                "unit": "TFLOP/s", "frac": r["grouped_tflops"] / peak,
                "traffic": profiled_traffic(workload), "kernel": kernel}
    return {"bound": "hbm", "achieved": r["grouped_gbs"], "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": r["grouped_gbs"] / PEAK_HBM_GBS,
            "traffic": profiled_traffic(workload), "kernel": kernel}


def zipf_scale(c):
    """The calibrated Zipf offset scale a* of a skewed workload (stored beside the input
    generator), or None."""
    if c.zipf_s == 0.0:
        return None
    path = os.path.join(ROOT, "moe_inputs", "zipf_calibration.json")
    with open(path) as f:
        rec = json.load(f).get(c.name)
    return None if rec is None else {"a": rec["a"], "hot8_share": rec["hot8_share"]}


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
    head = args.workload[0]
    for name in args.workload:
        c = CONFIGS[name]
        # The line's own workload times exactly --steps steps after exactly --warmup
        # untimed ones; a small batch beside it times at least 50 (each of its steps is
        # ~1 ms or less), and every workload beside it warms up for at least 0.5 s.
        steps = args.steps if (name == head or c.T >= 1024) else max(args.steps, 50)
        res, inp = run(c, steps, args.warmup, torch, 0.0 if name == head else 0.5)
        res["steps"] = steps
        if not args.no_cpu_baseline:
            t0 = time.perf_counter()
            res["gap_excluded_tokens"] = cpu_gap_excluded(c, inp)
            log(f"[{name}] oracle routing on the host: "
                f"{res['gap_excluded_tokens']} near-tie tokens "
                f"({time.perf_counter() - t0:.1f} s)")
        results[name] = res
        log(f"[{name}] {json.dumps(res)}")
        if name == "inkling_prefill":
            prefill_inputs = inp
        del inp
    c = CONFIGS[head]
    r = results[head]
    line = {
        "metric": METRIC, "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if c.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": head, "T": c.T, "d": c.d, "E": c.E, "S": c.S, "I": c.I,
                   "k": c.k, "router": c.router},
        "roofline": grouped_roofline(c, r, head),
        "layer_tflops": r["layer_tflops"],
        "layer_frac_bf16_mfma": r["layer_tflops"] / PEAK_BF16_TFLOPS,
        "step_ms_p10_p50_p90": [r["event_ms_per_step_p10"], r["event_ms_per_step_median"],
                                r["event_ms_per_step_p90"]],
        "stage_ms": r["stage_ms"],
        "touched_routed_experts": r["touched_routed_experts"],
        "gap_excluded_tokens": r.get("gap_excluded_tokens"),
        "configs": {},
    }
    for name in args.workload:
        if name == head:
            continue
        d, cc = results[name], CONFIGS[name]
        peak = PEAK_BF16_TFLOPS if cc.dtype == "bf16" else PEAK_F32_TFLOPS
        block = {
            "workload": name, "T": d["T"], "d": cc.d, "E": cc.E, "S": cc.S, "I": cc.I,
            "k": cc.k, "router": cc.router, "dtype": cc.dtype,
            "weights": cc.weight_format, "steps": d["steps"], "warmup_steps": d["warmup_steps"],
            "tokens_per_s": d["tokens_per_s"], "ms_per_step": d["ms_per_step"],
            "step_ms_p10_p50_p90": [d["event_ms_per_step_p10"], d["event_ms_per_step_median"],
                                    d["event_ms_per_step_p90"]],
            "stage_ms": d["stage_ms"],
            "layer_tflops": d["layer_tflops"], "layer_frac_mfma": d["layer_tflops"] / peak,
            "layer_alg_gbs": d["layer_alg_gbs"],
            "layer_frac_hbm": d["layer_alg_gbs"] / PEAK_HBM_GBS,
            "roofline": grouped_roofline(cc, d, name),
            "touched_routed_experts": d["touched_routed_experts"],
            "max_rows_per_expert": d["max_rows_per_expert"],
            "gap_excluded_tokens": d.get("gap_excluded_tokens"),
        }
        if cc.zipf_s:
            block["zipf"] = zipf_scale(cc)
        line["configs"][name] = block
    if not args.no_cpu_baseline and prefill_inputs is not None:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(CONFIGS["inkling_prefill"], prefill_inputs,
                                            args.cpu_sample)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
