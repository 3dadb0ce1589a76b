"""GPU parity of the rows beyond the dense forward at their full workload sizes, in the
default launch plans bench.py times: the fp64 oracles run on sampled heads (whole
sequence) or sampled sequences.  Bar: max |gpu - ref| / max |ref| <= 2e-2 (bf16
operands) per output tensor."""
import numpy as np
import pytest
import torch

import oracle
import chunked_linear_attention_gla_amd as gla
from chunked_linear_attention_gla_amd import inputs as gin
from gpu_util import TOL, device, rel

pytestmark = pytest.mark.gpu

TOLB = TOL["bf16"]


def heads_np(t, heads):
    """[B, H, ...] device tensor -> the sampled flat heads as oracle input (bf16 bits / fp32)."""
    flat = t.reshape(t.shape[0] * t.shape[1], *t.shape[2:])
    return gin.to_numpy_bits(flat[list(heads)])


def heads_f64(t, heads):
    flat = t.reshape(t.shape[0] * t.shape[1], *t.shape[2:])
    return flat[list(heads)].detach().cpu().double().numpy()


def test_backward_64k_sampled_heads():
    """gla_chunk_bwd at B=1, H=32, T=65536 (the bench's backward leg): all five gradients
    of two heads against the fp64 backward oracle."""
    w = gin.WORKLOADS["bf16_64k_strong"]
    dev = device()
    inp = gin.make_inputs(w, dev)
    gen = torch.Generator(device=dev).manual_seed(w.seed + 500)
    dO = torch.randn(w.B, w.H, w.T, w.dv, device=dev, generator=gen).to(inp["q"].dtype)
    dST = torch.randn(w.B, w.H, w.dk, w.dv, device=dev, generator=gen) * 0.1
    got = gla.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["x"], dO, inp["S0"], dST, gate=w.gate)
    torch.cuda.synchronize()
    heads = [3, 30]
    ref = oracle.backward(*(heads_np(inp[n], heads) for n in ("q", "k", "v", "x")), heads_f64(dO, heads), None,
                          heads_f64(dST, heads), gate=w.gate)
    for name, g_, r_ in zip(("dq", "dk", "dv", "dx", "dS0"), got, ref):
        gg = heads_f64(g_, heads)
        assert np.isfinite(gg).all(), name
        assert rel(gg, r_) <= TOLB, (name, rel(gg, r_))


def test_per_channel_64k_sampled_heads():
    w = gin.WORKLOADS["bf16_64k_pc"]
    inp = gin.make_inputs(w, device())
    o, ST = gla.chunk_fwd_pc(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"], gate=w.gate)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(ST).all()
    heads = [0, 17]
    o_ref, S_ref = oracle.forward_pc(*(heads_np(inp[n], heads) for n in ("q", "k", "v", "x")), None, gate=w.gate)
    assert rel(heads_f64(o, heads), o_ref) <= TOLB
    assert rel(heads_f64(ST, heads), S_ref) <= TOLB


def test_delta_64k_sampled_heads():
    w = gin.WORKLOADS["bf16_64k_delta"]
    inp = gin.make_inputs(w, device())
    o, ST = gla.chunk_fwd_delta(inp["q"], inp["k"], inp["v"], inp["x"], inp["beta"], inp["S0"], gate=w.gate)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(ST).all()
    heads = [1, 22]
    o_ref, S_ref = oracle.forward_delta(*(heads_np(inp[n], heads) for n in ("q", "k", "v", "x", "beta")), None,
                                        gate=w.gate)
    assert rel(heads_f64(o, heads), o_ref) <= TOLB
    assert rel(heads_f64(ST, heads), S_ref) <= TOLB


def test_decode_full_batch():
    """One decode step for all 64 x 32 heads of the serving batch."""
    w = gin.WORKLOADS["bf16_decode"]
    inp = gin.make_decode_inputs(w, device())
    S_in = inp["S"].clone()
    o = gla.decode_step(inp["q"], inp["k"], inp["v"], inp["x"], inp["S"], gate=w.gate)
    torch.cuda.synchronize()
    BH = w.B * w.H
    one = lambda t: gin.to_numpy_bits(t.reshape(BH, 1, *t.shape[2:]))
    o_ref, S_ref = oracle.forward(one(inp["q"]), one(inp["k"]), one(inp["v"]),
                                  gin.to_numpy_bits(inp["x"].reshape(BH, 1)),
                                  S_in.reshape(BH, w.dk, w.dv).cpu().numpy().astype(np.float64), gate=w.gate)
    assert rel(o.reshape(BH, 1, w.dv).cpu().double().numpy(), o_ref) <= TOLB
    assert rel(inp["S"].reshape(BH, w.dk, w.dv).cpu().double().numpy(), S_ref) <= TOLB


def test_varlen_256k_sampled_sequences():
    """The 64-sequence packed batch of the bench; the longest, the shortest and one
    middle sequence (all 16 heads) against the oracle."""
    w = gin.WORKLOADS["bf16_varlen_256k"]
    lengths = gin.varlen_lengths(64, w.T, w.seed)
    inp = gin.make_varlen_inputs(w, lengths, device())
    o, ST = gla.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["x"], inp["cu_seqlens"], max(lengths), None,
                                 gate=w.gate)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(ST).all()
    cu = [0] + list(np.cumsum(lengths))
    picks = [int(np.argmax(lengths)), int(np.argmin(lengths)), 31]
    for n in picks:
        a, b = int(cu[n]), int(cu[n + 1])
        o_ref, S_ref = oracle.forward(*(gin.to_numpy_bits(inp[t][:, a:b]) for t in ("q", "k", "v", "x")), None,
                                      gate=w.gate)
        assert rel(o[:, a:b].cpu().double().numpy(), o_ref) <= TOLB, n
        assert rel(ST[n].cpu().double().numpy(), S_ref) <= TOLB, n
