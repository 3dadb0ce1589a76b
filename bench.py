#!/usr/bin/env python3
"""Throughput of the bounded-decay chunked GLA forward pass on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input that
is already resident in HBM: the gate + chunk-local cumulative log-decay kernel,
the segment pre-pass (when the plan has several segments) and the fused chunk
output kernel, enqueued through the C ABI on the current stream.

Prints one JSON line.  `value` is tokens/s (batch * sequence tokens, all heads) of
the whole step; `roofline` is the fused output kernel (the dominant kernel): its
algorithmic HBM bytes per launch over its average launch time, measured with HIP
events on the stream it runs on, against the 8 TB/s HBM3E peak; `cpu_baseline` is
the fp64 CPU oracle timed on a bounded sample of the same workload on this host.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload bf16_64k_strong]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s and MFMA TFLOP/s (% bf16 peak), chunked GLA fwd at T=64K, d=128"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
KERNEL_SOURCES = ["chunked_linear_attention_gla_amd/csrc/chunk_kernels.hip",
                  "chunked_linear_attention_gla_amd/csrc/gla_device.h"]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes_per_token_head(dk: int, dv: int, es: int) -> int:
    # q, k (dk each) and v (dv) in storage precision, the per-token decay input (4 B),
    # and o (dv fp32) written once
    return (2 * dk + dv) * es + 4 + 4 * dv


def algorithmic_flops_per_token_head(dk: int, dv: int) -> int:
    # q.S and the k^T v state update (2 dk dv each), plus the intra-chunk q k^T and A v
    # over the causal 16x16 tiles of a 64-token chunk: 10 of 16 tiles, i.e. on average
    # (64 + 16) / 2 = 40 keys per query
    return 4 * dk * dv + 2 * 40 * (dk + dv)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bf16_64k_strong")
    ap.add_argument("--path", default=None, help="unified (default) or diag_branch")
    ap.add_argument("--plan", default=None, help="segments,dv_split (default: the library's plan)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration) and exit")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 3}))


def cpu_baseline(w, target_s: float):
    """Time the fp64 oracle on a bounded sample of the workload (all heads, a prefix of
    the sequence sized to take about target_s seconds on this host)."""
    import numpy as np
    import oracle
    from chunked_linear_attention_gla_amd import inputs as gin
    lib_threads = oracle.max_threads()

    def run(T):
        inp = gin.make_inputs(w, "cuda:0", T=T)
        flat = lambda t: t.reshape(w.B * w.H, *t.shape[2:])
        args = [gin.to_numpy_bits(flat(inp[n])) for n in ("q", "k", "v", "x")]
        s0 = None if inp["S0"] is None else flat(inp["S0"]).cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        oracle.forward(*args, s0, gate=w.gate)
        return time.perf_counter() - t0

    T0 = 256
    dt0 = run(T0)
    T = int(min(w.T, max(T0, target_s / max(dt0, 1e-6) * T0)))
    T = max(64, T // 64 * 64)
    dt = run(T)
    return {"value": w.B * T / dt, "unit": "tokens/s", "cores": lib_threads, "kind": "oracle",
            "sample": f"all {w.B * w.H} heads of {w.name}, first {T} of {w.T} tokens (seed {w.seed}); "
                      f"fp64 sequential recurrence, OpenMP over heads x 16-column blocks; {dt:.1f} s"}


def load_traffic(workload: str, plan, path: str):
    """HBM traffic of the output kernel from committed rocprofv3 counter runs, only if
    they were taken on the kernel source and plan in use now."""
    fn = os.path.join(ROOT, "profiles", f"chunk_output_kernel_{workload}_traffic.json")
    if not os.path.exists(fn):
        return None
    with open(fn) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_sha() or rec.get("plan") != list(plan) \
            or rec.get("path", "unified") != path:
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this build has no "
              f"multi-GPU path; heads shard across GPUs with no communication, see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    import chunked_linear_attention_gla_amd as gla
    from chunked_linear_attention_gla_amd import inputs as gin

    w = gin.WORKLOADS[args.workload]
    path = args.path or "unified"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = gin.make_inputs(w, dev)
    q, k, v, x, S0 = inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"]
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt_code = gla.GLA_BF16 if q.dtype == torch.bfloat16 else gla.GLA_F32
    if args.plan:
        plan = gla.Plan(*(int(s) for s in args.plan.split(",")))
    else:
        plan = gla.plan_default(B, H, T, dk, dv, dt_code, path)
    o = torch.empty(B, H, T, dv, device=dev, dtype=torch.float32)
    ST = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32)
    b = torch.empty(B, H, T, device=dev, dtype=torch.float32)
    seg_bytes = gla.segment_workspace_size(B, H, T, dk, dv, plan)
    seg = torch.empty(max(seg_bytes, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    n_ev = 4
    def step(evs=None):
        if evs is not None:
            evs[0].record()
        gla.gate_cumsum(x, gate=w.gate, out=b)
        if evs is not None:
            evs[1].record()
        if plan.segments > 1:
            gla.segment_states(k, v, b, plan, seg)
        if evs is not None:
            evs[2].record()
        gla.chunk_output(q, k, v, b, S0, plan, seg if plan.segments > 1 else None, o, ST, path=path)
        if evs is not None:
            evs[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()

    stage_ms = [[e[j].elapsed_time(e[j + 1]) for e in events] for j in range(n_ev - 1)]
    avg = lambda xs: sum(xs) / len(xs)
    ms_gate, ms_seg, ms_out = (avg(s) for s in stage_ms)
    ms_step = elapsed * 1e3 / args.steps
    tokens = B * T
    value = tokens / (ms_step / 1e3)
    es = q.element_size()
    bh = B * H
    bytes_out = bh * T * algorithmic_bytes_per_token_head(dk, dv, es) + bh * dk * dv * 4 * (2 if S0 is not None else 1)
    flops = bh * T * algorithmic_flops_per_token_head(dk, dv)
    achieved = bytes_out / (ms_out / 1e3) / 1e9
    traffic = load_traffic(w.name, plan, path)
    tflops = flops / (ms_step / 1e3) / 1e12

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if es == 2 else "f32",
        "data": "synthetic (seeded; inputs resident in HBM before timing)",
        "config": {"workload": w.name, "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "gate": w.gate,
                   "x": f"N({w.x_mean},{w.x_std})", "path": path,
                   "plan": {"segments": plan.segments, "dv_split": plan.dv_split}},
        "tflops": round(tflops, 2),
        "tflops_frac_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
        "stage_ms": {"gate_cumsum": round(ms_gate, 4), "segment_states": round(ms_seg, 4),
                     "chunk_output": round(ms_out, 4)},
        "roofline": {
            "kernel": "chunk_output_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_out,
            "avg_launch_ms": round(ms_out, 4),
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
