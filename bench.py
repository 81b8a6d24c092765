#!/usr/bin/env python3
"""Throughput of the MI355X GEMM / fully-connected hot path on one GPU.

A step is one call of the hot path on one batch of synthetic input already
resident in HBM: by default the 4096x4096x4096 FP32 GEMM (C = A*B, alpha 1,
beta 0), i.e. one gemm_f32 launch. ``--workload`` selects another of the
workloads in linear_layer_amd/workloads.py for ad-hoc measurement.

Prints ONE JSON line with the metric (TFLOPS = 2*M*N*K*batch / time per step),
a ``roofline`` object for the GEMM kernel (achieved = algorithmic FLOPs per
launch / average launch duration, from a second pass of K steps each between
its own pair of HIP events on the launch stream; peak = MI355X's published
dense matrix peak for the dtype; for the workloads with a few rows of A,
which HBM bounds, compulsory bytes per launch over the same duration against
the 8 TB/s HBM peak) and a ``cpu_baseline``
object: the float64 CPU oracle timed on a bounded sample of the same workload
(a block of whole output rows, or of whole batch items) on this host's cores.

The default run also measures the other configurations of the same family --
256^3, 1024^3 with alpha 1.5 and beta 0.5, the fused layer ReLU(X*W + b) at
2047x4096x11008 and the FP16-input 8192^3 product -- before the headline, and
reports each under ``configs``: time per step, TFLOP/s and fraction of its
dtype's matrix peak (back to back and per launch), its plan and an oracle
sample. All oracle samples run after all GPU timing.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

COPY_BYTES = 256 << 20

# Published MI355X HBM bandwidth (GB/s), the peak of the memory-bound workloads.
PEAK_HBM_GBS = 8000.0
# Published MI355X dense matrix peaks (TFLOP/s).
PEAK_TFLOPS = {"gemm_f32": 157.3, "linear": 157.3, "linear_nt": 157.3, "gemm_f32_batched": 157.3,
               "gemm_f16f32": 2516.6, "gemm_bf16f32": 2516.6, "gemm_f16f32_nt": 2516.6}
KERNEL_SOURCES = {   # the kernels, and the planner that picks which one runs
    "gemm_f32": ["gemm_f32.hip", "gemm_f32_nt.hip", "common.hpp", "api.hip"],
    "linear": ["gemm_f32.hip", "gemm_f32_nt.hip", "common.hpp", "api.hip"],
    "gemm_f16f32": ["gemm_f16.hip", "common.hpp", "api.hip"],
    "gemm_bf16f32": ["gemm_f16.hip", "common.hpp", "api.hip"],
    "linear_nt": ["gemm_f32.hip", "gemm_f32_nt.hip", "common.hpp", "api.hip"],
    "gemm_f32_batched": ["gemm_f32.hip", "gemm_f32_nt.hip", "common.hpp", "api.hip"],
    "gemm_f16f32_nt": ["gemm_f16.hip", "common.hpp", "api.hip"],
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gemm_f32_4096")
    ap.add_argument("--tile", type=int, default=-1, help="force a tile shape (-1: automatic)")
    ap.add_argument("--split-k", type=int, default=-1, help="force the K-split count (-1: automatic)")
    ap.add_argument("--stream-k", type=int, default=-1,
                    help="stream-K for leftover tiles: -1 automatic, 0 never, 1 whenever possible")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample (0 disables it)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations (256^3, 1024^3 alpha/beta, the fused layer, "
                         "FP16 8192^3) that the default run measures after the headline one")
    ap.add_argument("--config-cpu-seconds", type=float, default=4.0,
                    help="target CPU time of each other configuration's oracle sample")
    ap.add_argument("--workspace", action="store_true",
                    help="fused-layer workloads: run linear_bias_act_ws with a workspace "
                         "(stream-K in one launch) instead of linear_bias_act")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the GEMM, run a plain device-to-device copy of 256 MiB "
                         "--steps times (the reference kernel for scaling HBM byte counters)")
    return ap.parse_args()


def copy_calibration(steps: int):
    """A plain copy of known size: each launch reads and writes COPY_BYTES."""
    import torch
    n = COPY_BYTES // 4
    src = torch.ones(n, device="cuda:0", dtype=torch.float32)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES,
                      "steps": steps, "ms_per_copy": round(ms, 5),
                      "GB_per_s": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1)}), flush=True)


def code_text(src: str) -> str:
    """C++ source without its comments and blank lines or trailing spaces, so
    that the hash below follows the code, not its commentary. String and
    character literals are kept as they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            while i < n and src[i] != "\n":
                i += 1
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(l.rstrip() for l in "".join(out).splitlines() if l.strip())


def kernel_hash(kind: str) -> str:
    """Hash of the code (comments aside) of the kernels and planner of a kind."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "linear_layer_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kind: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    s = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or not s or s.group(1) != kernel_hash(kind):
        return None
    return float(m.group(1))


def cpu_baseline_batched(w, A, B, C, target_s: float):
    """Time the oracle on the first items of a batched workload."""
    import oracle

    def run(items):
        t0 = time.perf_counter()
        oracle.gemm_batched(A[:items], B[:items], w.alpha, w.beta, None if C is None else C[:items])
        return time.perf_counter() - t0

    items = 1
    dt = run(items)
    items = int(max(1, min(w.batch, items * target_s / max(dt, 1e-6))))
    dt = run(items)
    flops = 2.0 * items * w.M * w.N * w.K
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOPS",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": f"first {items} of {w.batch} batch items ({w.M}x{w.N}x{w.K} each, float64, "
                  f"{dt:.2f} s)",
        "seconds": dt,
    }


def cpu_baseline(w, x, target_s: float):
    """Time the float64 oracle on whole output rows of the same workload."""
    import numpy as np
    import oracle
    from linear_layer_amd import workloads as wl

    A = x["A"]
    B = x["B"]
    if w.kind in wl.HALF_KINDS:
        A, B = wl.half_bits(A), wl.half_bits(B)
    else:
        A, B = A.numpy(), B.numpy()
    bt = w.kind in wl.B_TRANSPOSED_KINDS
    C = x["C"].numpy() if "C" in x else None
    bias = x["bias"].numpy() if "bias" in x else None

    if w.kind in wl.BATCHED_KINDS:
        return cpu_baseline_batched(w, A, B, C, target_s)

    def run(rows):
        t0 = time.perf_counter()
        if w.kind in ("linear", "linear_nt"):
            oracle.linear(A[:rows], B, bias, w.act, w_trans=bt)
        else:
            oracle.gemm(A[:rows], B, w.alpha, w.beta, None if C is None else C[:rows],
                        bf16=w.kind == "gemm_bf16f32", b_trans=bt)
        return time.perf_counter() - t0

    rows = min(8, w.M)
    dt = run(rows)
    rows = int(max(1, min(w.M, rows * target_s / max(dt, 1e-6))))
    dt = run(rows)
    flops = 2.0 * rows * w.N * w.K
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOPS",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": f"first {rows} of {w.M} output rows ({rows}x{w.N}x{w.K}, float64, "
                  f"{dt:.2f} s)",
        "seconds": dt,
    }


def prepare(w, args, dev, workspace=False):
    """Device inputs of workload w, the step callable and the plan it runs.
    workspace: the fused layer through linear_bias_act_ws, with a workspace
    allocated (zero-filled) here, outside any timing."""
    import torch
    import linear_layer_amd as ll
    from linear_layer_amd import workloads as wl

    x = wl.make_inputs(w)
    A = x["A"].to(dev)
    B = x["B"].to(dev)
    batched = w.kind in wl.BATCHED_KINDS
    C = torch.empty(((w.batch,) if batched else ()) + (w.M, w.N), device=dev, dtype=torch.float32)
    if "C" in x:
        C.copy_(x["C"].to(dev))
    bias = x["bias"].to(dev) if "bias" in x else None
    dtype_id = ll.DTYPE_F16 if w.kind in wl.HALF_KINDS else ll.DTYPE_F32
    props = torch.cuda.get_device_properties(dev)
    # the plan the step runs: the fused layer with ReLU pays for its extra
    # pass; B given N-by-K is planned on its own
    plan_id = dtype_id
    if w.kind.startswith("linear") and w.act == 1:
        plan_id |= ll.PLAN_RELU
    if w.kind in wl.B_TRANSPOSED_KINDS:
        plan_id |= ll.PLAN_B_NK
    cus = props.multi_processor_count
    plan = {
        "tile": ll.tile_name(dtype_id, ll.chosen_tile(plan_id, w.M, w.N, w.K, cus, w.batch)),
        "split_k": ll.chosen_split_k(plan_id, w.M, w.N, w.K, cus, w.batch),
        "stream_k_tiles": ll.chosen_stream_k(plan_id, w.M, w.N, w.K, cus, w.batch),
    }

    ws = None
    if workspace:
        nbytes = ll.linear_workspace_size(w.M, w.N, w.K, w.kind == "linear_nt", w.act, cus)
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=dev)
        plan["workspace_bytes"] = nbytes

    def step():
        if ws is not None:
            ll.linear_bias_act_ws(A, B, bias, w.act, C, ws, w_trans=w.kind == "linear_nt")
        elif w.kind == "gemm_f32":
            ll.gemm_f32(A, B, C, w.alpha, w.beta)
        elif w.kind == "gemm_f16f32":
            ll.gemm_f16f32(A, B, C, w.alpha, w.beta)
        elif w.kind == "gemm_bf16f32":
            ll.gemm_bf16f32(A, B, C, w.alpha, w.beta)
        elif w.kind == "gemm_f16f32_nt":
            ll.gemm_f16f32_nt(A, B, C, w.alpha, w.beta)
        elif w.kind == "linear_nt":
            ll.linear_bias_act_nt(A, B, bias, w.act, C)
        elif w.kind == "gemm_f32_batched":
            ll.gemm_f32_batched(A, B, C, w.alpha, w.beta)
        else:
            ll.linear_bias_act(A, B, bias, w.act, C)

    return x, step, plan


def time_steps(step, steps: int, warmup: int, dev, min_warm_ms: float = 0.0):
    """W untimed steps (continued, when min_warm_ms > 0, until that much GPU
    time has passed, so that short kernels run at a settled clock), then K
    steps back to back between two events on the launch stream (device
    synchronisation on both sides); then a second pass of K steps, each
    between its own pair of events, for per-launch times. Returns
    (ms per step, per-launch ms, warm-up steps run)."""
    import torch
    t_warm = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    done = warmup
    while min_warm_ms > 0 and (time.perf_counter() - t_warm) * 1e3 < min_warm_ms:
        for _ in range(max(warmup, 8)):
            step()
        done += max(warmup, 8)
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)  # the stream the library launches on
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    return ms_per_step, launch_ms, done


# The other configurations of the headline metric's workload family (the
# 256^3 and 1024^3 alpha/beta products, the fused layer and the FP16-input
# product), measured after the headline one in the default run.
OTHER_CONFIGS = ["gemm_f32_256", "gemm_f32_1024_ab", "linear_relu_2047x4096x11008", "gemm_f16f32_8192"]
# The fused layer is also timed through the workspace entry point, which keeps
# the epilogue fused into every tile of its stream-K plan (one launch instead
# of three), reported under this key.
WS_CONFIG = "linear_relu_2047x4096x11008"


# Warm-up of each other configuration: the driver's W steps, continued until
# this much GPU time has passed (a few steps of a 20-us kernel would be timed
# while the clock still ramps up).
CONFIG_WARM_MS = 50.0


def config_record(w, step, plan, args, dev):
    """One configuration's GPU figures: time per step, TFLOP/s and fraction of
    the dtype's matrix peak (from the back-to-back pass and from the per-launch
    pass) and the plan; the oracle sample is added later."""
    ms_per_step, launch_ms, warm = time_steps(step, args.steps, args.warmup, dev, CONFIG_WARM_MS)
    flops = float(w.flops)
    peak = PEAK_TFLOPS[w.kind]
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    avg = sum(launch_ms) / len(launch_ms)
    rec = {
        "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha, "beta": w.beta, **plan,
        "steps": args.steps, "warmup_steps": warm,
        "ms_per_step": round(ms_per_step, 5),
        "tflops": round(tflops, 3),
        "frac_of_peak": round(tflops / peak, 4),
        "kernel_avg_ms": round(avg, 5),
        "kernel_median_ms": round(sorted(launch_ms)[len(launch_ms) // 2], 5),
        "kernel_frac_of_peak": round(flops / (avg * 1e-3) / 1e12 / peak, 4),
        "peak_tflops": peak,
    }
    return rec


def roofline(w, achieved_tflops, avg_ms, launch_ms, peak_tflops, args):
    """The roofline object: against the dtype's matrix peak in TFLOP/s, or,
    for the workloads HBM bounds (a few rows of A), algorithmic bytes per call
    over the average call against the HBM peak in GB/s."""
    traffic = measured_traffic(w.name + ("_workspace" if args.workspace else ""), w.kind)
    times = {"kernel_avg_ms": round(avg_ms, 5), "kernel_min_ms": round(min(launch_ms), 5),
             "kernel_median_ms": round(sorted(launch_ms)[len(launch_ms) // 2], 5)}
    if w.bound == "hbm":
        gbs = w.hbm_bytes / (avg_ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic, **times,
                "bytes_per_launch": w.hbm_bytes}
    return {"bound": "mfma", "achieved": round(achieved_tflops, 3), "peak": peak_tflops,
            "unit": "TFLOP/s", "frac": round(achieved_tflops / peak_tflops, 4), "traffic": traffic,
            **times, "flops_per_launch": float(w.flops)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has "
              f"no multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    import torch
    import linear_layer_amd as ll
    from linear_layer_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ll.load()  # fails loudly if the HIP library is missing
    w = wl.WORKLOADS[args.workload]
    if args.workspace and w.kind not in ("linear", "linear_nt"):
        print("--workspace applies to the fused-layer workloads only", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dtype_id = ll.DTYPE_F16 if w.kind in wl.HALF_KINDS else ll.DTYPE_F32
    if args.tile >= 0:
        ll.set_tile(dtype_id, args.tile)
    if args.split_k >= 1:
        ll.set_split_k(args.split_k)
    if args.stream_k != -1:
        ll.set_stream_k(args.stream_k)
    props = torch.cuda.get_device_properties(dev)
    # the headline's inputs, made and uploaded before any timing
    x, step, plan = prepare(w, args, dev, workspace=args.workspace)

    # The other configurations (default run only, with the automatic plan)
    # are timed first and the headline right after them, and every oracle
    # sample runs after all GPU timing: while the host works the GPU idles
    # and its clock drops.
    configs, config_inputs = None, {}
    if (args.workload == "gemm_f32_4096" and not args.no_configs and args.tile < 0 and not args.workspace
            and args.split_k < 1 and args.stream_k == -1):
        configs = {}
        for name in OTHER_CONFIGS + [WS_CONFIG + "_workspace"]:
            wsv = name.endswith("_workspace")
            wo = wl.WORKLOADS[WS_CONFIG if wsv else name]
            xo, so, po = prepare(wo, args, dev, workspace=wsv)
            configs[name] = config_record(wo, so, po, args, dev)
            if not wsv:
                config_inputs[name] = (wo, xo)
            del so
            torch.cuda.empty_cache()

    # the headline: exactly W warm-up steps, then K timed steps
    ms_per_step, launch_ms, _ = time_steps(step, args.steps, args.warmup, dev)
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    flops = float(w.flops)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.kind]
    del step
    torch.cuda.empty_cache()

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, x, args.cpu_seconds)
    if configs is not None and args.config_cpu_seconds > 0:
        for name, (wo, xo) in config_inputs.items():
            configs[name]["cpu_baseline"] = cpu_baseline(wo, xo, args.config_cpu_seconds)

    batched = w.kind in wl.BATCHED_KINDS
    dtype = {"gemm_f32": "f32", "linear": "f32", "linear_nt": "f32", "gemm_f32_batched": "f32",
             "gemm_f16f32": "f16 in, f32 accumulate", "gemm_f16f32_nt": "f16 in, f32 accumulate",
             "gemm_bf16f32": "bf16 in, f32 accumulate"}[w.kind]
    out = {
        "metric": "TFLOPS (2MNK/t) for 4096^3 FP32 GEMM on 1 MI355X; % of matrix peak"
        if w.name == "gemm_f32_4096" else f"TFLOPS (2MNK/t), {w.name}"
        + (" through linear_bias_act_ws" if args.workspace else ""),
        "value": round(value, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded uniform inputs, resident in HBM)",
        "config": {
            "workload": w.name, "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha, "beta": w.beta,
            **({"act": "relu" if w.act == 1 else "none", "bias": True}
               if w.kind in ("linear", "linear_nt") else {}),
            **({"b_layout": "N-by-K"} if w.kind in wl.B_TRANSPOSED_KINDS else {}),
            **({"batch": w.batch} if batched else {}),
            **plan,
            "device": props.name, "cus": props.multi_processor_count, "hip": torch.version.hip,
        },
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": roofline(w, achieved, avg_launch_ms, launch_ms, peak, args),
        "cpu_baseline": cpu,
    }
    if configs is not None:
        out["configs"] = configs
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
