"""gla_chunk_fwd_noalloc (the forward without a workspace argument, its segment
workspace taken from a device array inside the library) against gla_chunk_fwd with a
caller-allocated workspace, both through the C ABI, on two calls in a row: the second
with a smaller input, so it runs on an array that still holds the first call's states.
Same plan and kernels, so the outputs must be identical bit for bit."""
import ctypes

import pytest
import torch

from chunked_linear_attention_gla_amd import _lib
from chunked_linear_attention_gla_amd import inputs as gin
from gpu_util import device

pytestmark = pytest.mark.gpu

BF16, F32 = 0, 1
GATES = {"bounded": 0, "neg_softplus": 1}


def run_both(lib, w, inp):
    dev = device()
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    dt = BF16 if w.qkv_dtype == "bf16" else F32
    gate = GATES[w.gate]
    ptr = lambda t: None if t is None else t.data_ptr()
    st = torch.cuda.current_stream().cuda_stream
    args = [ptr(inp[n]) for n in ("q", "k", "v", "x", "S0")]
    # existing entry point, workspace sized from its own query
    o_ref = torch.full((B, H, T, dv), float("nan"), device=dev)
    s_ref = torch.full((B, H, dk, dv), float("nan"), device=dev)
    need = ctypes.c_size_t(0)
    assert lib.gla_chunk_fwd(*args, ptr(o_ref), ptr(s_ref), B, H, T, dk, dv, dt, gate, 0, None,
                             ctypes.byref(need), st) == 0
    ws = torch.empty(need.value, dtype=torch.uint8, device=dev)
    have = ctypes.c_size_t(need.value)
    assert lib.gla_chunk_fwd(*args, ptr(o_ref), ptr(s_ref), B, H, T, dk, dv, dt, gate, 0, ptr(ws),
                             ctypes.byref(have), st) == 0
    # the new entry point
    o = torch.full_like(o_ref, float("nan"))
    s = torch.full_like(s_ref, float("nan"))
    assert lib.gla_chunk_fwd_noalloc(*args, ptr(o), ptr(s), B, H, T, dk, dv, dt, gate, 0, st) == 0
    torch.cuda.synchronize()
    return o, s, o_ref, s_ref


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    lib = _lib.load()
    base = gin.WORKLOADS["bf16_8k"]
    # weak decay, so the segment states carry the whole history into later segments
    w1 = base.with_(B=1, H=8, T=64 * 40 + 17, x_mean=-6.0, seed=71)
    w2 = base.with_(B=1, H=4, T=64 * 20 + 5, x_mean=-6.0, seed=72)
    for w in (w1, w2):
        inp = gin.make_inputs(w, device())
        B, H = w.B, w.H
        plan = _lib.plan_default(B, H, w.T, w.dk, w.dv)
        assert plan.segments > 1  # the scratch array is in use
        o, s, o_ref, s_ref = run_both(lib, w, inp)
        assert torch.isfinite(o_ref).all() and torch.isfinite(s_ref).all()
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref), w


def test_noalloc_rejects_bad_arguments_before_any_launch():
    lib = _lib.load()
    dev = device()
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device=dev)
    x = torch.zeros(1, 2, 64, device=dev)
    o = torch.zeros(1, 2, 64, 64, device=dev)
    s = torch.zeros(1, 2, 64, 64, device=dev)
    p = lambda t: t.data_ptr()
    st = torch.cuda.current_stream().cuda_stream
    assert lib.gla_chunk_fwd_noalloc(p(q), p(q), p(q), p(x), None, p(o), p(s), 1, 2, 64, 64, 96, BF16, 0, 0, st) == 2
    assert lib.gla_chunk_fwd_noalloc(p(q), p(q), p(q), p(x), None, p(o), None, 1, 2, 64, 64, 64, BF16, 0, 0, st) == 1
    assert lib.gla_chunk_fwd_noalloc(p(q), p(q), p(q), p(x), None, p(q), p(s), 1, 2, 64, 64, 64, BF16, 0, 0, st) == 4
