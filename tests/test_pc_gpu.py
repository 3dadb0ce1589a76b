"""GPU parity of the per-channel-decay forward (gla_chunk_fwd_pc through the C ABI)
against the fp64 per-channel oracle on the same seeded inputs.  Bar: max |gpu - ref| /
max |ref| <= 2e-2 with bf16 operands, <= 1e-4 on the fp32 path, for o and S_T."""
import numpy as np
import pytest
import torch

import oracle
import chunked_linear_attention_gla_amd as gla
from chunked_linear_attention_gla_amd import inputs as gin
from gpu_util import CHAIN_TOL, CHAIN_TOL_STATE, TOL, device, rel

pytestmark = pytest.mark.gpu

BASE = gin.WORKLOADS["bf16_64k_pc"]


def make(T, H=3, B=1, dk=128, dv=128, qkv="bf16", x_mean=0.0, x_std=1.0, s0=0.1, seed=9):
    w = BASE.with_(B=B, H=H, T=T, dk=dk, dv=dv, qkv_dtype=qkv, x_mean=x_mean, x_std=x_std, s0_std=s0, seed=seed)
    return w, gin.make_inputs(w, device())


def oracle_pc(inp, gate="bounded", S0="inp"):
    q, k, v, x = inp["q"], inp["k"], inp["v"], inp["x"]
    B, H = q.shape[:2]
    flat = lambda t: t.reshape(B * H, *t.shape[2:])
    s0 = inp["S0"] if isinstance(S0, str) else S0
    s0n = None if s0 is None else flat(s0).cpu().numpy().astype(np.float64)
    return oracle.forward_pc(*(gin.to_numpy_bits(flat(t)) for t in (q, k, v, x)), s0n, gate=gate)


def check(w, inp, plan=None, gate="bounded", tol=None):
    o, ST = gla.chunk_fwd_pc(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"], gate=gate, plan=plan)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_pc(inp, gate)
    B, H, T, dv = o.shape
    got_o = o.reshape(B * H, T, dv).cpu().double().numpy()
    got_s = ST.reshape(B * H, *ST.shape[2:]).cpu().double().numpy()
    assert np.isfinite(got_o).all() and np.isfinite(got_s).all()
    tol = TOL[w.qkv_dtype] if tol is None else tol
    eo, es = rel(got_o, o_ref), rel(got_s, S_ref)
    assert eo <= tol and es <= tol, (eo, es)
    return eo, es


@pytest.mark.parametrize("T", [1, 15, 16, 17, 64, 65, 64 * 9 + 13])
def test_short_and_ragged(T):
    w, inp = make(T)
    check(w, inp)


@pytest.mark.parametrize("regime,x_mean,x_std", [("weak", -6.0, 1.0), ("mixed", 0.0, 3.0), ("strong", 4.0, 1.0)])
def test_decay_regimes(regime, x_mean, x_std):
    """weak decay carries the state across many chunks; mixed spreads channels from
    a ~ 1 to the -5 bound within one head."""
    w, inp = make(64 * 20 + 5, H=2, x_mean=x_mean, x_std=x_std)
    check(w, inp)


@pytest.mark.parametrize("qkv,segments,partial", [("bf16", 4, False), ("bf16", 6, True), ("f32", 3, False)])
def test_decay_bursts_segmented(qkv, segments, partial):
    """Weak decay with whole chunks of strong decay (x = +8 in every channel) at the
    ends of segments, where the segment pre-pass may start its recurrence.  partial:
    in one of those chunks a single channel keeps its weak decay, so that chunk does
    not cut the state and the pass must run further back."""
    dk = dv = 64 if qkv == "f32" else 128
    w, inp = make(64 * 26 + 9, H=2, qkv=qkv, dk=dk, dv=dv, x_mean=-6.0, seed=31)
    nc = (w.T + 63) // 64
    ends = [(p + 1) * nc // segments - 1 for p in range(segments - 1)]
    for ch in ends + [e - 1 for e in ends]:
        inp["x"][:, :, ch * 64:(ch + 1) * 64, :] = 8.0
    if partial:
        inp["x"][:, :, ends[0] * 64:(ends[0] + 1) * 64, 5] = -6.0
    check(w, inp, plan=gla.Plan(segments, 1))


def test_extreme_channels():
    """Some channels with x = +inf (g = -5 exactly: the bound) and some with x = -inf
    (a = 1), mixed with ordinary values in the same tiles."""
    w, inp = make(64 * 6 + 7, H=2)
    x = inp["x"]
    x[..., 0::5] = float("inf")
    x[..., 1::7] = float("-inf")
    check(w, inp)


@pytest.mark.parametrize("dk,dv,split", [(64, 64, 1), (64, 128, 1), (128, 64, 1), (128, 128, 2), (64, 128, 2)])
def test_head_dims_and_slices(dk, dv, split):
    w, inp = make(64 * 5 + 9, dk=dk, dv=dv)
    check(w, inp, plan=gla.Plan(1, split))


@pytest.mark.parametrize("segments", [2, 3, 8])
def test_segmented_plans(segments):
    w, inp = make(64 * 24 + 11, H=2, x_mean=-5.0)
    check(w, inp, plan=gla.Plan(segments, 1))


def test_default_plan_long_sequence():
    w, inp = make(64 * 64 + 31, H=2, x_mean=-4.0, s0=0.0)
    inp["S0"] = None
    check(w, inp)


def test_fp32_path():
    w, inp = make(64 * 4 + 3, H=2, dk=64, dv=64, qkv="f32")
    check(w, inp)
    check(w, inp, plan=gla.Plan(3, 1))


def test_fp32_dk128_is_rejected():
    w, inp = make(64, H=1, dk=128, dv=64, qkv="f32")
    with pytest.raises(gla.GLAError):
        gla.chunk_fwd_pc(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"])


def test_shared_decay_matches_the_scalar_path():
    """x equal across channels: the per-channel kernels and the scalar kernels compute
    the same recurrence."""
    w, inp = make(64 * 7 + 5, H=2)
    xs = inp["x"][..., 0].contiguous()
    inp["x"] = xs[..., None].expand(-1, -1, -1, 128).contiguous()
    o1, S1 = gla.chunk_fwd_pc(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"])
    o2, S2 = gla.chunk_fwd(inp["q"], inp["k"], inp["v"], xs, inp["S0"])
    torch.cuda.synchronize()
    o_ref, _ = oracle.forward(*(gin.to_numpy_bits(t.reshape(2, *t.shape[2:])) for t in (inp["q"], inp["k"],
                                                                                           inp["v"], xs)),
                              inp["S0"].reshape(2, 128, 128).cpu().numpy().astype(np.float64))
    assert rel(o1.reshape(2, -1, 128).cpu().double().numpy(), o_ref) <= TOL["bf16"]
    assert rel(o1.cpu().double().numpy(), o2.cpu().double().numpy()) <= TOL["bf16"]


def test_chaining_matches_single_call():
    w, inp = make(64 * 10, H=2, x_mean=-5.0)
    q, k, v, x, S0 = inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"]
    o, ST = gla.chunk_fwd_pc(q, k, v, x, S0)
    s = 64 * 4
    oa, Sa = gla.chunk_fwd_pc(q[:, :, :s].contiguous(), k[:, :, :s].contiguous(), v[:, :, :s].contiguous(),
                              x[:, :, :s].contiguous(), S0)
    ob, Sb = gla.chunk_fwd_pc(q[:, :, s:].contiguous(), k[:, :, s:].contiguous(), v[:, :, s:].contiguous(),
                              x[:, :, s:].contiguous(), Sa)
    torch.cuda.synchronize()
    o_cat = torch.cat([oa, ob], dim=2)
    assert rel(o_cat.cpu().double().numpy(), o.cpu().double().numpy()) <= CHAIN_TOL
    assert rel(Sb.cpu().double().numpy(), ST.cpu().double().numpy()) <= CHAIN_TOL_STATE


def test_chaining_weak_decay_state_handover():
    """Weak per-channel decay and a two-chunk second call: the chained S_T depends
    strongly on the handed-over state (from zero it is far off) and still matches the
    single segmented call to fp32 summation order."""
    w, inp = make(64 * 12, H=2, x_mean=-7.0, seed=33)
    q, k, v, x, S0 = inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"]
    o, ST = gla.chunk_fwd_pc(q, k, v, x, S0, plan=gla.Plan(4, 1))
    s = 64 * 10
    cut = lambda t, a, b: t[:, :, a:b].contiguous()
    oa, Sa = gla.chunk_fwd_pc(*(cut(t, 0, s) for t in (q, k, v, x)), S0, plan=gla.Plan(1, 1))
    ob, Sb = gla.chunk_fwd_pc(*(cut(t, s, None) for t in (q, k, v, x)), Sa, plan=gla.Plan(1, 1))
    _, Sz = gla.chunk_fwd_pc(*(cut(t, s, None) for t in (q, k, v, x)), None, plan=gla.Plan(1, 1))
    torch.cuda.synchronize()
    assert rel(Sb.cpu().double().numpy(), ST.cpu().double().numpy()) <= CHAIN_TOL_STATE
    assert rel(Sz.cpu().double().numpy(), ST.cpu().double().numpy()) > 0.1
    assert rel(torch.cat([oa, ob], 2).cpu().double().numpy(), o.cpu().double().numpy()) <= CHAIN_TOL


def test_empty_sequence_returns_initial_state():
    w, inp = make(0, H=2)
    o, ST = gla.chunk_fwd_pc(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"])
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(ST, inp["S0"])


def test_repeat_calls_are_bitwise_identical():
    w, inp = make(64 * 8 + 1, H=2)
    o1, S1 = gla.chunk_fwd_pc(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"], plan=gla.Plan(4, 1))
    o2, S2 = gla.chunk_fwd_pc(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"], plan=gla.Plan(4, 1))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_largest_head_extent():
    """The largest sequence the ABI accepts for one head at dk = dv = 128: x (fp32 per
    channel) and o span 0xFFFF0000 bytes, so their byte offsets pass 2^31 at token
    4194304.  Whole chunks with x = +8 in every channel (chunk decay about e^-320,
    exactly 0 in fp32) are planted before the checked windows, so the fp64 oracle
    restarted from a zero state at such a chunk yields the outputs after it.  Checked:
    the first 192 tokens (with S0), four chunks across the 2^31-byte offset, the last
    two chunks and S_T."""
    t_max = 0xFFFF0000 // (128 * 4)
    w, inp = make(t_max, H=1, seed=4243)
    mid = (1 << 31) // (128 * 4) // 64
    last = t_max // 64
    for ch in (mid - 3, last - 3):
        inp["x"][:, :, ch * 64:(ch + 1) * 64, :] = 8.0
    o, ST = gla.chunk_fwd_pc(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"])
    torch.cuda.synchronize()
    head = {n: inp[n][:, :, :192].contiguous() for n in ("q", "k", "v", "x")}
    head["S0"] = inp["S0"]
    o_ref, _ = oracle_pc(head)
    assert rel(o[0, 0, :192].cpu().double().numpy(), o_ref[0]) <= TOL["bf16"]
    zero = torch.zeros(1, 1, 128, 128, device=device())
    for a, c, b in ((mid - 3, mid - 2, mid + 2), (last - 3, last - 2, last)):
        sub = {n: inp[n][:, :, a * 64:b * 64].contiguous() for n in ("q", "k", "v", "x")}
        o_ref, S_ref = oracle_pc(sub, S0=zero)
        got = o[0, 0, c * 64:b * 64].cpu().double().numpy()
        assert np.isfinite(got).all()
        assert rel(got, o_ref[0, (c - a) * 64:]) <= TOL["bf16"], (a, b)
        if b == last:
            assert rel(ST[0, 0].cpu().double().numpy(), S_ref[0]) <= TOL["bf16"]
