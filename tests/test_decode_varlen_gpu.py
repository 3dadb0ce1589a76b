"""GPU parity of the decode step (gla_decode_step) and of packed variable-length
sequences (gla_chunk_fwd_varlen) against the fp64 oracle on the same seeded inputs.
Bar: max |gpu - ref| / max |ref| <= 2e-2 with bf16 operands, <= 1e-4 on the fp32 path.

The decode step is the recurrence over one token with the carried state as S0, so its
oracle is the forward oracle at T = 1 (per-channel oracle for a per-channel decay); a
packed batch is, sequence by sequence, the forward over that sequence with its own S0."""
import numpy as np
import pytest
import torch

import oracle
import chunked_linear_attention_gla_amd as gla
from chunked_linear_attention_gla_amd import inputs as gin
from gpu_util import TOL, device, rel

pytestmark = pytest.mark.gpu

DEC = gin.WORKLOADS["bf16_decode"]
VAR = gin.WORKLOADS["bf16_varlen_256k"]


def np_bits(t):
    return gin.to_numpy_bits(t)


# ------------------------------------------------------------------------------ decode

@pytest.mark.parametrize("qkv,dk,dv", [("bf16", 128, 128), ("bf16", 64, 128), ("bf16", 128, 64), ("f32", 64, 64)])
@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("gate", ["bounded", "neg_softplus"])
def test_decode_step_matches_oracle(qkv, dk, dv, per_channel, gate):
    w = DEC.with_(B=3, H=5, dk=dk, dv=dv, qkv_dtype=qkv, per_channel=per_channel, gate=gate)
    inp = gin.make_decode_inputs(w, device())
    S_in = inp["S"].clone()
    o = gla.decode_step(inp["q"], inp["k"], inp["v"], inp["x"], inp["S"], gate=gate)
    torch.cuda.synchronize()
    BH = 15
    flat = lambda t: t.reshape(BH, 1, *t.shape[2:])
    q, k, v = (np_bits(flat(inp[n])) for n in ("q", "k", "v"))
    x = np_bits(inp["x"].reshape(BH, 1, *inp["x"].shape[2:]))
    S0 = S_in.reshape(BH, dk, dv).cpu().numpy().astype(np.float64)
    fwd = oracle.forward_pc if per_channel else oracle.forward
    o_ref, S_ref = fwd(q, k, v, x, S0, gate=gate)
    tol = TOL[qkv]
    assert rel(o.reshape(BH, 1, dv).cpu().double().numpy(), o_ref) <= tol
    assert rel(inp["S"].reshape(BH, dk, dv).cpu().double().numpy(), S_ref) <= tol


@pytest.mark.parametrize("per_channel", [False, True])
def test_decode_chain_matches_chunked_forward(per_channel):
    """70 decode steps from S0 equal one chunked forward over the 70 tokens."""
    w = gin.WORKLOADS["bf16_8k"].with_(B=2, H=3, T=70, s0_std=0.1, per_channel=per_channel, x_mean=-3.0)
    inp = gin.make_inputs(w, device())
    S = inp["S0"].clone()
    outs = []
    for t in range(70):
        outs.append(gla.decode_step(inp["q"][:, :, t].contiguous(), inp["k"][:, :, t].contiguous(),
                                    inp["v"][:, :, t].contiguous(), inp["x"][:, :, t].contiguous(), S))
    o_dec = torch.stack(outs, dim=2)
    fwd = gla.chunk_fwd_pc if per_channel else gla.chunk_fwd
    o, ST = fwd(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"])
    torch.cuda.synchronize()
    flat = lambda t: t.reshape(6, *t.shape[2:])
    ofn = oracle.forward_pc if per_channel else oracle.forward
    o_ref, S_ref = ofn(*(np_bits(flat(inp[n])) for n in ("q", "k", "v", "x")),
                       flat(inp["S0"]).cpu().numpy().astype(np.float64))
    assert rel(flat(o_dec).cpu().double().numpy(), o_ref) <= TOL["bf16"]
    assert rel(flat(S).cpu().double().numpy(), S_ref) <= TOL["bf16"]
    assert rel(o_dec.cpu().double().numpy(), o.cpu().double().numpy()) <= TOL["bf16"]


# ------------------------------------------------------------------------------ packed sequences

def varlen_check(w, lengths, gate="bounded", path="unified", tol=None, seed=None, plan=None, edit_x=None):
    dev = device()
    inp = gin.make_varlen_inputs(w, lengths, dev, seed=seed)
    if edit_x is not None:
        edit_x(inp["x"], [0] + list(np.cumsum(lengths)))
    max_len = max(lengths) if lengths else 0
    o, ST = gla.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["x"], inp["cu_seqlens"], max_len, inp["S0"],
                                 gate=gate, path=path, plan=plan)
    torch.cuda.synchronize()
    tol = TOL[w.qkv_dtype] if tol is None else tol
    cu = [0] + list(np.cumsum(lengths))
    worst = 0.0
    for n, L in enumerate(lengths):
        a, b = int(cu[n]), int(cu[n + 1])
        s0 = None if inp["S0"] is None else inp["S0"][n].cpu().numpy().astype(np.float64)
        o_ref, S_ref = oracle.forward(*(np_bits(inp[t][:, a:b]) for t in ("q", "k", "v", "x")), s0, gate=gate)
        got_s = ST[n].cpu().double().numpy()
        if L:
            e = rel(o[:, a:b].cpu().double().numpy(), o_ref)
            assert e <= tol, (n, L, e)
            worst = max(worst, e)
        assert rel(got_s, S_ref) <= tol, (n, L)
    return worst


def test_varlen_mixed_lengths():
    w = VAR.with_(H=3, s0_std=0.1)
    varlen_check(w, [1, 63, 64, 65, 0, 300, 17, 1000, 129])


def test_varlen_long_sequences_use_segments():
    """Long enough for the default plan to cut every sequence into segments."""
    w = VAR.with_(H=2, x_mean=-5.0)
    varlen_check(w, [4100, 37, 2500, 0, 64 * 40])


@pytest.mark.parametrize("segments", [2, 4, 7])
def test_varlen_explicit_segments(segments):
    """Every sequence cut into the same number of segments, including sequences shorter
    than that many chunks (empty segments) and empty sequences."""
    w = VAR.with_(H=2, s0_std=0.1, x_mean=-5.0)
    varlen_check(w, [64 * 9 + 5, 3, 0, 64 * 2, 1000], plan=gla.Plan(segments, 1))


@pytest.mark.parametrize("segments", [3, 5])
def test_varlen_segments_with_decay_bursts(segments):
    """Weak decay with whole chunks of strong decay (x = +8) just before each segment
    end of every sequence: the segment pre-pass of each sequence starts at such a chunk."""
    lengths = [64 * 11 + 5, 3, 0, 64 * 4, 1300]

    def bursts(x, cu):
        for n, L in enumerate(lengths):
            nc = (L + 63) // 64
            for p in range(segments - 1):
                c = (p + 1) * nc // segments - 1
                if c >= 0 and (c + 1) * 64 <= L:
                    x[:, cu[n] + c * 64: cu[n] + (c + 1) * 64] = 8.0

    w = VAR.with_(H=2, s0_std=0.1, x_mean=-5.0)
    varlen_check(w, lengths, plan=gla.Plan(segments, 1), edit_x=bursts)


def test_varlen_length_mix_sample():
    w = VAR.with_(H=2, s0_std=0.1)
    varlen_check(w, gin.varlen_lengths(12, 6000, seed=5))


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_varlen_head_dims(dk, dv):
    w = VAR.with_(H=2, dk=dk, dv=dv, s0_std=0.1)
    varlen_check(w, [70, 5, 200])


def test_varlen_diag_branch_ablation():
    w = VAR.with_(H=2, gate="neg_softplus", x_mean=-4.0)
    varlen_check(w, [90, 1, 333], gate="neg_softplus", path="diag_branch")


def test_varlen_fp32():
    w = VAR.with_(H=2, dk=64, dv=64, qkv_dtype="f32", s0_std=0.1)
    varlen_check(w, [70, 5, 200, 64])


def test_varlen_matches_dense_calls():
    """A packed batch equals one dense call per sequence (both on the GPU)."""
    w = VAR.with_(H=2, s0_std=0.1)
    lengths = [200, 64, 333]
    inp = gin.make_varlen_inputs(w, lengths, device())
    o, ST = gla.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["x"], inp["cu_seqlens"], 333, inp["S0"])
    cu = [0, 200, 264, 597]
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        sl = lambda t: t[:, a:b].unsqueeze(0).contiguous()
        od, Sd = gla.chunk_fwd(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["x"]),
                               inp["S0"][n:n + 1].contiguous())
        torch.cuda.synchronize()
        assert rel(o[:, a:b].cpu().double().numpy(), od[0].cpu().double().numpy()) <= 1e-3
        assert rel(ST[n].cpu().double().numpy(), Sd[0].cpu().double().numpy()) <= 1e-3


def test_varlen_all_empty_returns_initial_states():
    w = VAR.with_(H=2, s0_std=0.1)
    inp = gin.make_varlen_inputs(w, [0, 0, 0], device())
    o, ST = gla.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["x"], inp["cu_seqlens"], 0, inp["S0"])
    torch.cuda.synchronize()
    assert torch.equal(ST, inp["S0"])
