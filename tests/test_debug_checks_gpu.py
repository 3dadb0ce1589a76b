"""The LDS-checked debug build (libgla_debug.so: the same sources compiled with
-DGLA_DEBUG) on the GPU.  Its self-test raises both flag bits without any invalid
access, so the checks can fire; every entry point run through it -- ragged and
segmented plans, both paths and gates, fp32, 16-column slices, per-channel decay,
the delta rule, the backward pass, packed sequences and decode -- must leave every
flag clear and give the release build's results (max |debug - release| within 1e-6
of the release output's scale: the two builds run the same arithmetic)."""
import ctypes

import pytest
import torch

import chunked_linear_attention_gla_amd as gla
from chunked_linear_attention_gla_amd import inputs as gin
from gpu_util import device

pytestmark = pytest.mark.gpu


def small(name, **kw):
    w = gin.WORKLOADS[name].with_(**kw)
    return w, gin.make_inputs(w, device())


def same(a, b):
    for x, y in zip(a, b):
        x, y = x.double(), y.double()
        scale = max(y.abs().max().item(), 1e-30) if y.numel() else 1.0
        assert torch.isfinite(x).all()
        assert (x - y).abs().max().item() <= 1e-6 * scale if y.numel() else True


def through_debug_build(fn):
    """fn() with the release library, then with the debug build; the debug build's
    flags must stay clear."""
    ref = fn()
    with gla.use_library() as dbg:
        gla.debug_flags(dbg)
        got = fn()
        torch.cuda.synchronize()
        flags = gla.debug_flags(dbg)
    assert flags == 0, f"LDS check flags {flags:#x}"
    same(got, ref)


def test_selftest_raises_both_bits_and_reading_clears():
    dev = device()
    probe = torch.zeros(64, device=dev)
    out = torch.empty(64, device=dev)
    with gla.use_library() as dbg:
        gla.debug_flags(dbg)
        rc = dbg.gla_debug_selftest(probe.data_ptr(), out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        assert gla.debug_flags(dbg) == 3
        assert gla.debug_flags(dbg) == 0
    assert torch.equal(out.cpu(), torch.arange(63, -1, -1, dtype=torch.float32))


@pytest.mark.parametrize("path,gate,plan", [("unified", "bounded", (3, 1)), ("unified", "bounded", (2, 8)),
                                            ("diag_branch", "neg_softplus", (2, 1))])
def test_forward(path, gate, plan):
    w, inp = small("bf16_8k", B=1, H=3, T=64 * 9 + 13, x_mean=-2.0 if gate == "neg_softplus" else 0.0, gate=gate)
    through_debug_build(lambda: gla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"], gate=gate,
                                              path=path, plan=gla.Plan(*plan)))


def test_forward_fp32():
    w, inp = small("fp32_small", B=1, H=2, T=64 * 4 + 3, dk=64, dv=64)
    through_debug_build(lambda: gla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["x"], None, plan=gla.Plan(2, 1)))


def test_per_channel():
    w, inp = small("bf16_64k_pc", B=1, H=2, T=64 * 5 + 7, x_mean=0.0)
    through_debug_build(lambda: gla.chunk_fwd_pc(inp["q"], inp["k"], inp["v"], inp["x"], None, plan=gla.Plan(2, 1)))


@pytest.mark.parametrize("qkv,d", [("bf16", 128), ("f32", 64)])
def test_delta_rule(qkv, d):
    w, inp = small("bf16_64k_delta", B=1, H=2, T=64 * 6 + 5, dk=d, dv=d, qkv_dtype=qkv, x_mean=-3.0)
    through_debug_build(lambda: gla.chunk_fwd_delta(inp["q"], inp["k"], inp["v"], inp["x"], inp["beta"], None,
                                                    plan=gla.Plan(3, 1)))


@pytest.mark.parametrize("qkv,d,T", [("bf16", 128, 64 * 5 + 3), ("bf16", 64, 64 * 4 + 9), ("f32", 128, 64 * 3 + 1)])
def test_backward(qkv, d, T):
    w, inp = small("bf16_8k", B=1, H=2, T=T, dk=d, dv=d, qkv_dtype=qkv)
    gen = torch.Generator(device=device()).manual_seed(77)
    dO = torch.randn(1, 2, T, d, device=device(), generator=gen).to(inp["q"].dtype)
    dST = torch.randn(1, 2, d, d, device=device(), generator=gen) * 0.1
    through_debug_build(lambda: gla.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["x"], dO, inp["S0"], dST))


def test_packed_sequences_and_decode():
    dev = device()
    lens = [70, 1, 200, 64]
    w = gin.WORKLOADS["bf16_varlen_256k"].with_(H=2)
    inp = gin.make_varlen_inputs(w, lens, dev)
    through_debug_build(lambda: gla.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["x"], inp["cu_seqlens"],
                                                     max(lens), inp["S0"]))
    for per_channel in (False, True):
        wd = gin.WORKLOADS["bf16_decode"].with_(B=2, H=3, per_channel=per_channel)
        dec = gin.make_decode_inputs(wd, dev)

        def step():
            s = dec["S"].clone()
            o = gla.decode_step(dec["q"], dec["k"], dec["v"], dec["x"], s)
            return o, s
        through_debug_build(step)
