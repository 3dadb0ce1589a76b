#!/usr/bin/env python3
"""Throughput of the bounded-decay chunked GLA forward pass on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input that
is already resident in HBM: the segment pre-pass (when the plan has several
segments) and the fused chunk output kernel, both forming the gate and the
chunk-local cumulative log-decay from x themselves, enqueued through the C ABI on
the current stream.

The device is brought to steady clocks before the warm-up steps (the settle phase:
the step repeated for --settle-s seconds): from process start the output kernel
runs ~14 % slower over its first ~25 ms of load while the clocks ramp up, and a
short warm-up would time that ramp instead of the steady state.

Prints one JSON line.  `value` is tokens/s (batch * sequence tokens, all heads) of
the whole step; `roofline` is the fused output kernel (the dominant kernel): its
algorithmic HBM bytes per launch over its average launch time, measured with HIP
events on the stream it runs on, against the 8 TB/s HBM3E peak; `ablation` times the
diagonal-branch variant (negative-softplus gate, diagonal tiles by position pairs)
on its own strong-decay inputs beside the unified path on the same inputs;
`cpu_baseline` is the fp64 CPU oracle timed on a bounded sample of the same workload
on this host.

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
                  "chunked_linear_attention_gla_amd/csrc/ws_kernels.hip",
                  "chunked_linear_attention_gla_amd/csrc/chunk_common.h",
                  "chunked_linear_attention_gla_amd/csrc/gla_device.h"]
ABLATION_WORKLOAD = "bf16_64k_strong_softplus"


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


def backward_bytes_per_token_head(dk: int, dv: int, es: int) -> int:
    # reads q, k (dk each), v and dO (dv each) in storage precision and x; writes dq, dk
    # (dk fp32 each), dv (dv fp32) and dx
    return (2 * dk + 2 * dv) * es + 4 + 4 * (2 * dk + dv) + 4


def backward_flops_per_token_head(dk: int, dv: int) -> int:
    # three forward-shaped passes (dq, dk, dv) and, for dx, q.k and dO.v on the causal
    # tiles plus S dO and D v against the states before and after each chunk
    return 3 * algorithmic_flops_per_token_head(dk, dv) + 2 * 40 * (dk + dv) + 4 * dk * dv


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bf16_64k_strong")
    ap.add_argument("--x-mean", type=float, default=None,
                    help="override the workload's gate-input mean (e.g. -6 for the weak-decay regime; profiling)")
    ap.add_argument("--path", default=None, help="unified (default) or diag_branch")
    ap.add_argument("--plan", default=None, help="segments,dv_split (default: the library's plan)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle sample")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of repeated steps before the warm-up, so that timing starts at steady clocks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ablation", action="store_true", help="skip the diagonal-branch comparison")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--backward-only", action="store_true", help="time only the backward pass (profiling)")
    ap.add_argument("--no-per-channel", action="store_true", help="skip the per-channel-decay measurement")
    ap.add_argument("--no-serving", action="store_true", help="skip the decode and packed-sequence measurements")
    ap.add_argument("--no-delta", action="store_true", help="skip the gated-delta-rule measurement")
    ap.add_argument("--delta-only", action="store_true", help="time only the gated delta rule")
    ap.add_argument("--serving-only", action="store_true", help="time only decode and packed sequences")
    ap.add_argument("--per-channel-only", action="store_true", help="time only the per-channel forward")
    ap.add_argument("--ramp", type=int, default=0, metavar="N",
                    help="only time the first N steps from process start, one by one (no settle, no warm-up), "
                         "and print the output kernel's time per group of 10 launches: the clock ramp")
    ap.add_argument("--ramp-stream", type=int, default=0, metavar="N",
                    help="only time the first N launches of the flat stream of the step's byte mix "
                         "(gla_bench_stream) from process start, per group of 10 launches")
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


def device_copy_rate(torch, nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """Plain device-to-device copy on the same GPU (torch's copy kernel), for context: what
    a flat stream of reads and writes reaches here, beside the 8 TB/s published peak."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    gbs = 2 * nbytes / (ms / 1e3) / 1e9
    del src, dst
    return {"what": "device-to-device copy of 1 GiB (bytes read + written per second)", "ms": round(ms, 4),
            "GB_per_s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def settle(torch, fn, seconds: float) -> float:
    """Repeat fn (enqueueing GPU work) for about `seconds` of wall time, synchronising every
    few calls, so that the device's clocks have ramped up before anything is timed.
    Returns the seconds spent."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    return round(time.perf_counter() - t0, 3)


def stream_ceiling(gla, torch, nbytes: int, reps: int = 10) -> dict:
    """The forward's byte mix (3 x nbytes read, 2 x nbytes written: q, k, v and o of the
    headline step) as one flat grid-stride stream (gla_bench_stream, a HIP kernel of this
    library): the practical streaming rate of this device for that mix."""
    dev = torch.device("cuda:0")
    a = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    b, c = torch.ones_like(a), torch.ones_like(a)
    out = torch.empty(2 * nbytes, dtype=torch.uint8, device=dev)
    fn = lambda: gla.bench_stream(a, b, c, out)
    settle(torch, fn, 0.1)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        fn()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    gbs = 5 * nbytes / (ms / 1e3) / 1e9
    del a, b, c, out
    return {"what": f"flat grid-stride stream of the step's byte mix (3 x {nbytes >> 20} MiB read, "
                    f"{2 * nbytes >> 20} MiB written; gla_bench_stream, 8192 workgroups)",
            "ms": round(ms, 4), "GB_per_s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def chunk_stream_ceiling(gla, torch, BH: int, T: int, segments: int, reps: int = 10) -> dict:
    """The output pass's access pattern without its arithmetic (gla_bench_chunk_stream):
    BH * segments workgroups, at most one per compute unit, each streaming its run of
    64-token chunks in order (q, k, v in bf16 and o in fp32 at d = 128) with the next
    chunk's loads in flight.  The ceiling of that pattern, below the flat stream's."""
    dev = torch.device("cuda:0")
    nb = BH * T * 256
    q = torch.ones(nb, dtype=torch.uint8, device=dev)
    k, v = torch.ones_like(q), torch.ones_like(q)
    o = torch.empty(2 * nb, dtype=torch.uint8, device=dev)
    fn = lambda: gla.bench_chunk_stream(q, k, v, o, BH, T, segments)
    settle(torch, fn, 0.1)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        fn()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    gbs = 5 * nb / (ms / 1e3) / 1e9
    del q, k, v, o
    return {"what": f"the output pass's loads and stores without its arithmetic ({BH} heads x {segments} segments, "
                    f"one workgroup per compute unit, 64-token chunks in order; gla_bench_chunk_stream)",
            "ms": round(ms, 4), "GB_per_s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def cpu_baseline(w, target_s: float, per_channel: bool = False):
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
        (oracle.forward_pc if per_channel else oracle.forward)(*args, s0, gate=w.gate)
        return time.perf_counter() - t0

    T0 = 256
    dt0 = run(T0)
    T = int(min(w.T, max(T0, target_s / max(dt0, 1e-6) * T0)))
    T = max(64, T // 64 * 64)
    dt = run(T)
    return {"value": w.B * T / dt, "unit": "tokens/s", "cores": lib_threads, "kind": "oracle",
            "sample": f"all {w.B * w.H} heads of {w.name}, first {T} of {w.T} tokens (seed {w.seed}); "
                      f"fp64 sequential {'per-channel ' if per_channel else ''}recurrence, OpenMP over heads x "
                      f"16-column blocks; {dt:.1f} s"}


def cpu_baseline_backward(w, target_s: float):
    """Time the fp64 backward oracle on a bounded sample of the workload, like cpu_baseline."""
    import numpy as np
    import torch
    import oracle
    from chunked_linear_attention_gla_amd import inputs as gin
    lib_threads = oracle.max_threads()

    def run(T):
        inp = gin.make_inputs(w, "cuda:0", T=T)
        flat = lambda t: t.reshape(w.B * w.H, *t.shape[2:])
        args = [gin.to_numpy_bits(flat(inp[n])) for n in ("q", "k", "v", "x")]
        s0 = None if inp["S0"] is None else flat(inp["S0"]).cpu().numpy().astype(np.float64)
        gen = torch.Generator(device="cuda:0").manual_seed(w.seed + 500)
        dO = torch.randn(w.B * w.H, T, w.dv, device="cuda:0", generator=gen).to(inp["q"].dtype)
        dST = torch.randn(w.B * w.H, w.dk, w.dv, device="cuda:0", generator=gen) * 0.1
        dO64 = dO.double().cpu().numpy()
        dST64 = dST.double().cpu().numpy()
        t0 = time.perf_counter()
        oracle.backward(*args, dO64, s0, dST64, gate=w.gate)
        return time.perf_counter() - t0

    T0 = 128
    dt0 = run(T0)
    T = int(min(w.T, max(T0, target_s / max(dt0, 1e-6) * T0)))
    T = max(64, T // 64 * 64)
    dt = run(T)
    return {"value": w.B * T / dt, "unit": "tokens/s", "cores": lib_threads, "kind": "oracle",
            "sample": f"backward, all {w.B * w.H} heads of {w.name}, first {T} of {w.T} tokens (seed {w.seed}); "
                      f"fp64 recurrence with 64-token checkpoints, OpenMP over heads; {dt:.1f} s"}


def output_kernel_name(dtype_bytes: int, dk: int, slice_cols: int) -> str:
    # the library runs the wave-specialised output pass for bf16 with dk in {64, 128}
    # and slices of 32, 64 or 128 value columns, the plain one otherwise
    if dtype_bytes == 2 and dk in (64, 128) and slice_cols in (32, 64, 128):
        return "chunk_output_ws_kernel"
    return "chunk_output_kernel"


def load_traffic(kernel: str, workload: str, plan, path: str):
    """HBM traffic of the output kernel from committed rocprofv3 counter runs, only if
    they were taken on the kernel source and plan in use now."""
    fn = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(fn):
        return None
    with open(fn) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_sha() or rec.get("plan") != list(plan) \
            or rec.get("path", "unified") != path:
        return None
    return rec.get("bytes_per_launch")


class StepTimer:
    """One workload, one path: inputs, outputs and workspace on the device, and a step
    that enqueues the segment pre-pass and the output pass (both forming the gate and
    the chunk-local cumulative log-decay from x), with optional HIP events between them
    on the current stream."""

    def __init__(self, gla, gin, torch, w, path, plan=None):
        dev = torch.device("cuda:0")
        self.gla, self.torch, self.w, self.path = gla, torch, w, path
        inp = gin.make_inputs(w, dev)
        self.q, self.k, self.v, self.x, self.S0 = inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"]
        B, H, T, dk = self.q.shape
        dv = self.v.shape[-1]
        self.shape = (B, H, T, dk, dv)
        dt_code = gla.GLA_BF16 if self.q.dtype == torch.bfloat16 else gla.GLA_F32
        self.plan = plan or gla.plan_default(B, H, T, dk, dv, dt_code, path)
        self.o = torch.empty(B, H, T, dv, device=dev, dtype=torch.float32)
        self.ST = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32)
        seg_bytes = gla.segment_workspace_size(B, H, T, dk, dv, self.plan)
        self.seg = torch.empty(max(seg_bytes, 256), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def step(self, evs=None):
        gla, plan = self.gla, self.plan
        if evs is not None:
            evs[0].record()
        if plan.segments > 1:
            gla.segment_states(self.k, self.v, self.x, plan, self.seg, gate=self.w.gate)
        if evs is not None:
            evs[1].record()
        gla.chunk_output(self.q, self.k, self.v, self.x, self.S0, plan, self.seg if plan.segments > 1 else None,
                         self.o, self.ST, gate=self.w.gate, path=self.path)
        if evs is not None:
            evs[2].record()

    def run(self, steps, warmup, settle_s=0.0):
        """Returns (ms per step from the host clock, [pre-pass, output] ms from events)."""
        torch = self.torch
        if settle_s > 0:
            settle(torch, self.step, settle_s)
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(events[i])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        stage = [sum(e[j].elapsed_time(e[j + 1]) for e in events) / steps for j in range(2)]
        return elapsed * 1e3 / steps, stage


class BackwardTimer:
    """The backward pass (gla_chunk_bwd) of one workload with a given dO and dS_T, outputs
    and workspace preallocated, timed with HIP events on the current stream around each
    call."""

    def __init__(self, gla, gin, torch, w, path):
        dev = torch.device("cuda:0")
        self.gla, self.torch, self.w, self.path = gla, torch, w, path
        inp = gin.make_inputs(w, dev)
        self.q, self.k, self.v, self.x, self.S0 = inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"]
        B, H, T, dk = self.q.shape
        dv = self.v.shape[-1]
        self.shape = (B, H, T, dk, dv)
        gen = torch.Generator(device=dev).manual_seed(w.seed + 500)
        self.dO = torch.randn(B, H, T, dv, device=dev, generator=gen).to(self.q.dtype)
        self.dST = torch.randn(B, H, dk, dv, device=dev, generator=gen) * 0.1
        f32 = dict(device=dev, dtype=torch.float32)
        self.out = (torch.empty(B, H, T, dk, **f32), torch.empty(B, H, T, dk, **f32),
                    torch.empty(B, H, T, dv, **f32), torch.empty(B, H, T, **f32), torch.empty(B, H, dk, dv, **f32))
        dt_code = gla.GLA_BF16 if self.q.dtype == torch.bfloat16 else gla.GLA_F32
        need = gla.backward_workspace_size(B, H, T, dk, dv, dt_code, w.gate, path)
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def step(self):
        self.gla.chunk_bwd(self.q, self.k, self.v, self.x, self.dO, self.S0, self.dST, gate=self.w.gate,
                           path=self.path, workspace=self.ws, out=self.out)

    def run(self, steps, warmup, settle_s=0.0):
        """Returns (ms per call from the host clock, ms per call from events)."""
        torch = self.torch
        if settle_s > 0:
            settle(torch, self.step, settle_s)
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(steps):
            self.step()
            ev[i + 1].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        return elapsed * 1e3 / steps, ev[0].elapsed_time(ev[steps]) / steps


def time_calls(torch, fn, steps, warmup, settle_s=0.3):
    """(ms per call from the host clock, ms per call from HIP events on the current stream),
    after settle_s seconds of repeated calls (steady clocks) and `warmup` calls."""
    if settle_s > 0:
        settle(torch, fn, settle_s)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(steps):
        fn()
    ev[1].record()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps, ev[0].elapsed_time(ev[1]) / steps


def per_channel_bytes_per_token_head(dk: int, dv: int, es: int) -> int:
    # q, k, v in storage precision, x (one fp32 per key channel) and o (fp32)
    return (2 * dk + dv) * es + 4 * dk + 4 * dv


def per_channel_result(gla, gin, torch, steps, warmup, cpu_seconds, settle_s=0.3):
    """The per-channel-decay forward (gla_chunk_fwd_pc: segment pre-pass + output pass)
    on its own 64K workload, timed per call."""
    w = gin.WORKLOADS["bf16_64k_pc"]
    dev = torch.device("cuda:0")
    inp = gin.make_inputs(w, dev)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    o = torch.empty(B, H, T, dv, device=dev)
    ST = torch.empty(B, H, dk, dv, device=dev)
    plan = gla.plan_default_pc(B, H, T, dk, dv)
    ws = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    fn = lambda: gla.chunk_fwd_pc(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"], gate=w.gate, plan=plan,
                                  o=o, S_T=ST, workspace=ws)
    ms_host, ms_ev = time_calls(torch, fn, steps, warmup, settle_s)
    es = inp["q"].element_size()
    del inp, o, ws
    nbytes = B * H * T * per_channel_bytes_per_token_head(dk, dv, es) + B * H * dk * dv * 4
    achieved = nbytes / (ms_ev / 1e3) / 1e9
    res = {
        "what": "gla_chunk_fwd_pc: per-channel decay forward, all kernels of the call",
        "workload": w.name, "x": f"N({w.x_mean},{w.x_std}) per (token, key channel)",
        "plan": {"segments": plan.segments, "dv_split": plan.dv_split}, "steps": steps,
        "ms_per_call": round(ms_host, 4), "ms_per_call_events": round(ms_ev, 4),
        "tokens_per_s": round(B * T / (ms_ev / 1e3), 1),
        "tflops": round(B * H * T * algorithmic_flops_per_token_head(dk, dv) / (ms_ev / 1e3) / 1e12, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_call": nbytes},
    }
    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(w, cpu_seconds, per_channel=True)
    return res


def decode_result(gla, gin, torch, steps, warmup, cpu_seconds, sets: int = 6, settle_s=0.3):
    """One decode step for every (sequence, head) of a serving batch (gla_decode_step),
    the state updated in place.  The timed steps rotate over `sets` independent batches
    (inputs and states), 128 MiB of state each, so that the 768 MiB they span exceed the
    256 MB Infinity Cache and every step streams its state from HBM; the same step
    repeated on one batch (its state then stays cache-resident) is reported beside it."""
    import numpy as np
    w = gin.WORKLOADS["bf16_decode"]
    dev = torch.device("cuda:0")
    batches = [gin.make_decode_inputs(w, dev, seed=w.seed + 1000 * i) for i in range(sets)]
    inp = batches[0]
    o = torch.empty(w.B, w.H, w.dv, device=dev)
    step = lambda b_: gla.decode_step(b_["q"], b_["k"], b_["v"], b_["x"], b_["S"], gate=w.gate, o=o)
    it = [0]

    def rotating():
        step(batches[it[0] % sets])
        it[0] += 1
    n_steps = steps * 10 // sets * sets
    ms_host, ms_ev = time_calls(torch, rotating, n_steps, warmup, settle_s)
    _, ms_res = time_calls(torch, lambda: step(inp), steps * 10, warmup, min(settle_s, 0.05))
    es = inp["q"].element_size()
    bh = w.B * w.H
    per_head = 2 * w.dk * w.dv * 4 + (2 * w.dk + w.dv) * es + 4 + 4 * w.dv
    achieved = bh * per_head / (ms_ev / 1e3) / 1e9
    res = {"what": "gla_decode_step: one token per (sequence, head), fp32 state read and written in place",
           "workload": w.name, "B": w.B, "H": w.H, "dk": w.dk, "dv": w.dv, "steps": n_steps,
           "state_sets": sets, "state_MiB_total": sets * bh * w.dk * w.dv * 4 >> 20,
           "ms_per_step": round(ms_host, 5), "ms_per_step_events": round(ms_ev, 5),
           "tokens_per_s": round(w.B / (ms_ev / 1e3), 1),
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_step": bh * per_head},
           "cache_resident": {
               "what": "the same step repeated on one batch: its 128 MiB state stays in the Infinity Cache, "
                       "so this rate is not an HBM figure",
               "ms_per_step_events": round(ms_res, 5),
               "GB_per_s": round(bh * per_head / (ms_res / 1e3) / 1e9, 1)}}
    if cpu_seconds > 0:
        import oracle
        flat = lambda t: t.reshape(bh, 1, *t.shape[2:])
        args = [gin.to_numpy_bits(flat(inp[n])) for n in ("q", "k", "v")] + \
               [gin.to_numpy_bits(inp["x"].reshape(bh, 1))]
        S0 = inp["S"].reshape(bh, w.dk, w.dv).cpu().numpy().astype(np.float64)
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < cpu_seconds:
            oracle.forward(*args, S0, gate=w.gate)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": w.B / dt, "unit": "tokens/s", "cores": oracle.max_threads(),
                               "kind": "oracle", "sample": f"the whole step ({bh} heads), {reps} repetitions"}
    return res


def varlen_result(gla, gin, torch, steps, warmup, cpu_seconds, settle_s=0.3):
    """Forward over a packed batch of sequences of mixed lengths (gla_chunk_fwd_varlen)."""
    import numpy as np
    w = gin.WORKLOADS["bf16_varlen_256k"]
    dev = torch.device("cuda:0")
    lengths = gin.varlen_lengths(64, w.T, w.seed)
    inp = gin.make_varlen_inputs(w, lengths, dev)
    N, H, T = len(lengths), w.H, w.T
    o = torch.empty(H, T, w.dv, device=dev)
    ST = torch.empty(N, H, w.dk, w.dv, device=dev)
    ws = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
    fn = lambda: gla.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["x"], inp["cu_seqlens"], max(lengths),
                                      inp["S0"], gate=w.gate, o=o, S_T=ST, workspace=ws)
    ms_host, ms_ev = time_calls(torch, fn, steps, warmup, settle_s)
    es = inp["q"].element_size()
    nbytes = H * T * algorithmic_bytes_per_token_head(w.dk, w.dv, es) + N * H * w.dk * w.dv * 4
    achieved = nbytes / (ms_ev / 1e3) / 1e9
    res = {"what": "gla_chunk_fwd_varlen: packed sequences, all kernels of the call", "workload": w.name,
           "sequences": N, "min_len": min(lengths), "max_len": max(lengths), "H": H, "total_tokens": T,
           "steps": steps, "ms_per_call": round(ms_host, 4), "ms_per_call_events": round(ms_ev, 4),
           "tokens_per_s": round(T / (ms_ev / 1e3), 1),
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_call": nbytes}}
    if cpu_seconds > 0:
        import oracle
        cu = [0] + list(np.cumsum(lengths))
        done, t0 = 0, time.perf_counter()
        for n in range(N):
            a, b = int(cu[n]), int(cu[n + 1])
            oracle.forward(*(gin.to_numpy_bits(inp[t][:, a:b]) for t in ("q", "k", "v", "x")), None, gate=w.gate)
            done += b - a
            if time.perf_counter() - t0 > cpu_seconds:
                break
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": done / dt, "unit": "tokens/s", "cores": oracle.max_threads(),
                               "kind": "oracle", "sample": f"the first {n + 1} of {N} sequences ({done} tokens, "
                                                           f"all {H} heads), one oracle call per sequence"}
    return res


def delta_result(gla, gin, torch, steps, warmup, cpu_seconds, settle_s=0.3):
    """The chunked gated delta rule (gla_chunk_fwd_delta: gate + cumsum, the parallel
    per-chunk solve, the serial output pass) on its 64K workload."""
    import numpy as np
    w = gin.WORKLOADS["bf16_64k_delta"]
    dev = torch.device("cuda:0")
    inp = gin.make_inputs(w, dev)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    o = torch.empty(B, H, T, dv, device=dev)
    ST = torch.empty(B, H, dk, dv, device=dev)
    plan = gla.plan_default_delta(B, H, T, dk, dv)
    ws = torch.empty(B * H * (T * (4 + 2 * (dk + dv)) + plan.segments * dk * (dk + dv) * 4) + (1 << 20),
                     dtype=torch.uint8, device=dev)
    fn = lambda: gla.chunk_fwd_delta(inp["q"], inp["k"], inp["v"], inp["x"], inp["beta"], inp["S0"], gate=w.gate,
                                     plan=plan, o=o, S_T=ST, workspace=ws)
    ms_host, ms_ev = time_calls(torch, fn, steps, warmup, settle_s)
    es = inp["q"].element_size()
    # q, k, v, x, beta in; o out (the per-chunk W and U are implementation traffic)
    per_th = (2 * dk + dv) * es + 8 + 4 * dv
    nbytes = B * H * T * per_th + B * H * dk * dv * 4
    achieved = nbytes / (ms_ev / 1e3) / 1e9
    res = {"what": "gla_chunk_fwd_delta: gated delta rule forward, all kernels of the call", "workload": w.name,
           "x": f"N({w.x_mean},{w.x_std})", "beta": "U(0,1)", "steps": steps,
           "plan": {"segments": plan.segments, "dv_split": plan.dv_split},
           "ms_per_call": round(ms_host, 4), "ms_per_call_events": round(ms_ev, 4),
           "tokens_per_s": round(B * T / (ms_ev / 1e3), 1),
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_call": nbytes}}
    if cpu_seconds > 0:
        import oracle
        flat = lambda t: t.reshape(B * H, *t.shape[2:])

        def run(Tn):
            args = [gin.to_numpy_bits(flat(inp[n])[:, :Tn]) for n in ("q", "k", "v", "x", "beta")]
            t0 = time.perf_counter()
            oracle.forward_delta(*args, None, gate=w.gate)
            return time.perf_counter() - t0
        dt0 = run(256)
        Tn = int(min(T, max(256, cpu_seconds / max(dt0, 1e-6) * 256))) // 64 * 64
        dt = run(Tn)
        res["cpu_baseline"] = {"value": B * Tn / dt, "unit": "tokens/s", "cores": oracle.max_threads(),
                               "kind": "oracle", "sample": f"all {B * H} heads, first {Tn} of {T} tokens; "
                                                           f"fp64 token-by-token delta rule; {dt:.1f} s"}
    return res


def backward_result(gla, gin, torch, w, path, steps, warmup, settle_s=0.3, weak=False):
    t = BackwardTimer(gla, gin, torch, w, path)
    ms_host, ms_ev = t.run(steps, warmup, settle_s)
    B, H, T, dk, dv = t.shape
    es = t.q.element_size()
    del t
    bh = B * H
    nbytes = bh * T * backward_bytes_per_token_head(dk, dv, es) + bh * dk * dv * 4 * 3
    flops = bh * T * backward_flops_per_token_head(dk, dv)
    achieved = nbytes / (ms_ev / 1e3) / 1e9
    res = {
        "what": "gla_chunk_bwd: dq, dk, dv, dx, dS0 from dO and dS_T (all kernels of the call)",
        "steps": steps,
        "ms_per_call": round(ms_host, 4),
        "ms_per_call_events": round(ms_ev, 4),
        "tokens_per_s": round(B * T / (ms_ev / 1e3), 1),
        "tflops": round(flops / (ms_ev / 1e3) / 1e12, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_call": nbytes},
    }
    if weak:
        # the same call where no chunk's crossing factor a e^gamma is exactly 0: the dq pass
        # then stores, and the dk pass reads, the state of every chunk
        ww = w.with_(x_mean=-6.0, x_std=1.0)
        tw = BackwardTimer(gla, gin, torch, ww, path)
        steps_w = max(steps // 2, 5)
        _, ms_w = tw.run(steps_w, warmup, 0.0)
        del tw
        res["weak_decay"] = {
            "what": "same shapes, x ~ N(-6,1): every chunk's state is stored by the dq pass and read by the dk pass",
            "x": f"N({ww.x_mean},{ww.x_std})", "steps": steps_w, "ms_per_call_events": round(ms_w, 4),
            "tokens_per_s": round(B * T / (ms_w / 1e3), 1)}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (there is no "
              f"multi-GPU path; (batch, head) pairs are independent, so heads would shard across "
              f"GPUs with no communication)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    import chunked_linear_attention_gla_amd as gla
    from chunked_linear_attention_gla_amd import inputs as gin

    w = gin.WORKLOADS[args.workload]
    if args.x_mean is not None:
        w = w.with_(x_mean=args.x_mean)
    path = args.path or "unified"
    torch.cuda.set_device(torch.device("cuda:0"))
    plan = gla.Plan(*(int(s) for s in args.plan.split(","))) if args.plan else None
    if args.ramp_stream:
        # the flat stream of the headline step's bytes, launch by launch from the first one
        B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
        nbytes = B * H * T * dk * 2  # one bf16 operand tensor; o (fp32) is twice that
        a = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
        b_, c_ = torch.ones_like(a), torch.ones_like(a)
        out = torch.empty(2 * nbytes, dtype=torch.uint8, device="cuda:0")
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.ramp_stream)]
        for e in evs:
            e[0].record()
            gla.bench_stream(a, b_, c_, out)
            e[1].record()
        torch.cuda.synchronize()
        us = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
        groups = [{"launches": f"{i}-{min(i + 9, len(us) - 1)}", "gpu_ms_before": round(sum(us[:i]) / 1e3, 1),
                   "stream_us_mean": round(sum(us[i:i + 10]) / len(us[i:i + 10]), 1)} for i in range(0, len(us), 10)]
        print(json.dumps({"workload": w.name, "bytes_per_launch": 5 * nbytes, "ramp_stream": groups}), flush=True)
        return
    if args.delta_only:
        print(json.dumps({"delta": delta_result(gla, gin, torch, args.steps, args.warmup, 0.0, args.settle_s)}),
              flush=True)
        return
    if args.serving_only:
        print(json.dumps({"decode": decode_result(gla, gin, torch, args.steps, args.warmup, 0.0,
                                                  settle_s=args.settle_s),
                          "varlen": varlen_result(gla, gin, torch, args.steps, args.warmup, 0.0, args.settle_s)}),
              flush=True)
        return
    if args.per_channel_only:
        print(json.dumps({"per_channel": per_channel_result(gla, gin, torch, args.steps, args.warmup, 0.0,
                                                            args.settle_s)}), flush=True)
        return
    if args.backward_only:
        print(json.dumps({"workload": w.name, "x": f"N({w.x_mean},{w.x_std})",
                          "backward": backward_result(gla, gin, torch, w, path, args.steps, args.warmup,
                                                      args.settle_s)}), flush=True)
        return
    timer = StepTimer(gla, gin, torch, w, path, plan)
    plan = timer.plan
    if args.ramp:
        # the output kernel launch by launch from the first step of the process on
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.ramp)]
        for e in evs:
            timer.step(e)
        torch.cuda.synchronize()
        out_us = [e[1].elapsed_time(e[2]) * 1e3 for e in evs]
        groups = [{"launches": f"{i}-{min(i + 9, len(out_us) - 1)}",
                   "gpu_ms_before": round(sum(e_[0].elapsed_time(e_[2]) for e_ in evs[:i]), 1),
                   "output_kernel_us_mean": round(sum(out_us[i:i + 10]) / len(out_us[i:i + 10]), 1)}
                  for i in range(0, len(out_us), 10)]
        print(json.dumps({"workload": w.name, "ramp": groups}), flush=True)
        return
    ms_step, (ms_seg, ms_out) = timer.run(args.steps, args.warmup, args.settle_s)
    B, H, T, dk, dv = timer.shape
    es = timer.q.element_size()
    S0 = timer.S0
    del timer

    tokens = B * T
    value = tokens / (ms_step / 1e3)
    bh = B * H
    bytes_out = bh * T * algorithmic_bytes_per_token_head(dk, dv, es) + bh * dk * dv * 4 * (2 if S0 is not None else 1)
    flops = bh * T * algorithmic_flops_per_token_head(dk, dv)
    achieved = bytes_out / (ms_out / 1e3) / 1e9
    kname = output_kernel_name(es, dk, dv // plan.dv_split)
    traffic = load_traffic(kname, w.name, plan, path)
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
        "settle_s": args.settle_s,
        "stage_ms": {"segment_states": round(ms_seg, 4), "chunk_output": round(ms_out, 4)},
        "roofline": {
            "kernel": kname,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_out,
            "avg_launch_ms": round(ms_out, 4),
        },
        "context": {"device_copy": device_copy_rate(torch),
                    "stream_ceiling": stream_ceiling(gla, torch, B * H * T * dk * es)},
    }
    if dk == 128 and dv == 128 and es == 2 and T % (64 * plan.segments) == 0:
        result["context"]["chunk_stream_ceiling"] = chunk_stream_ceiling(gla, torch, B * H, T, plan.segments)
    if w.name == gin.HEADLINE and path == "unified" and not args.plan and not args.no_ablation:
        # the pages' comparison: conventional gate + diagonal branch against the unified
        # path, both on the ablation's own inputs (same shapes, strong decay)
        wa = gin.WORKLOADS[ABLATION_WORKLOAD]
        steps_a = min(args.steps, 20)
        abl = {"workload": wa.name, "gate": wa.gate, "x": f"N({wa.x_mean},{wa.x_std})", "steps": steps_a}
        for p_ in ("diag_branch", "unified"):
            t = StepTimer(gla, gin, torch, wa, p_)
            ms_a, st_a = t.run(steps_a, min(args.warmup, 5), args.settle_s)
            abl[p_] = {"ms_per_step": round(ms_a, 4), "chunk_output_ms": round(st_a[1], 4),
                       "tokens_per_s": round(wa.B * wa.T / (ms_a / 1e3), 1)}
            del t
        abl["unified_speedup_step"] = round(abl["diag_branch"]["ms_per_step"] / abl["unified"]["ms_per_step"], 3)
        abl["unified_speedup_output_kernel"] = round(
            abl["diag_branch"]["chunk_output_ms"] / abl["unified"]["chunk_output_ms"], 3)
        result["ablation"] = abl
    if w.name == gin.HEADLINE and path == "unified" and not args.plan and not args.no_ablation:
        # the same shapes with weakly decaying gates: no chunk's decay factor underflows,
        # so the segment pre-pass runs every chunk of its segments (nothing truncated)
        ww = w.with_(x_mean=-6.0, x_std=1.0)
        steps_w = min(args.steps, 20)
        t = StepTimer(gla, gin, torch, ww, path)
        ms_w, st_w = t.run(steps_w, min(args.warmup, 5), args.settle_s)
        del t
        result["weak_decay"] = {
            "what": "same shapes, x ~ N(-6,1): the segment pre-pass runs every chunk (no exact truncation)",
            "x": f"N({ww.x_mean},{ww.x_std})", "steps": steps_w, "ms_per_step": round(ms_w, 4),
            "stage_ms": {"segment_states": round(st_w[0], 4), "chunk_output": round(st_w[1], 4)},
            "tokens_per_s": round(ww.B * ww.T / (ms_w / 1e3), 1)}
    if not args.no_backward and not args.plan:
        result["backward"] = backward_result(gla, gin, torch, w, path, min(args.steps, 20), min(args.warmup, 5),
                                             args.settle_s, weak=True)
        if not args.no_cpu_baseline:
            result["backward"]["cpu_baseline"] = cpu_baseline_backward(w, args.cpu_seconds / 2)
    if not args.no_per_channel and not args.plan and w.name == gin.HEADLINE:
        result["per_channel"] = per_channel_result(gla, gin, torch, min(args.steps, 20), min(args.warmup, 5),
                                                   0.0 if args.no_cpu_baseline else args.cpu_seconds / 2,
                                                   args.settle_s)
    if not args.no_serving and not args.plan and w.name == gin.HEADLINE:
        cs = 0.0 if args.no_cpu_baseline else args.cpu_seconds / 4
        result["decode"] = decode_result(gla, gin, torch, min(args.steps, 20), min(args.warmup, 5), cs,
                                         settle_s=args.settle_s)
        result["varlen"] = varlen_result(gla, gin, torch, min(args.steps, 20), min(args.warmup, 5), cs,
                                         args.settle_s)
    if not args.no_delta and not args.plan and w.name == gin.HEADLINE:
        result["delta"] = delta_result(gla, gin, torch, min(args.steps, 10), min(args.warmup, 3),
                                       0.0 if args.no_cpu_baseline else args.cpu_seconds / 4, args.settle_s)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
