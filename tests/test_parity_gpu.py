"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on the
same seeded inputs.  Bar: max |gpu - ref| / max |ref| <= 2e-2 with bf16 operands,
<= 1e-4 on the fp32 path, separately for o and the final state S_T."""
import numpy as np
import pytest
import torch

import oracle
import chunked_linear_attention_gla_amd as gla
from chunked_linear_attention_gla_amd import inputs as gin
from gpu_util import CHAIN_TOL, CHAIN_TOL_STATE, TOL, device, gpu_heads, oracle_heads, rel

pytestmark = pytest.mark.gpu

SMALL = gin.WORKLOADS["bf16_8k"]


def small(T, H=3, B=1, dk=128, dv=128, qkv="bf16", x_mean=0.0, x_std=1.0, s0=0.1, seed=7, x_const=None,
          gate="bounded"):
    w = SMALL.with_(B=B, H=H, T=T, dk=dk, dv=dv, qkv_dtype=qkv, x_mean=x_mean, x_std=x_std, s0_std=s0,
                    seed=seed, gate=gate)
    return w, gin.make_inputs(w, device(), x_const=x_const)


def check(inp, w, plan=None, path="unified", gate="bounded", tol=None):
    o, ST = gla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"], gate=gate, path=path, plan=plan)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_heads(inp, gate=gate)
    B, H, T, dv = o.shape
    got_o = o.reshape(B * H, T, dv).cpu().double().numpy()
    got_s = ST.reshape(B * H, *ST.shape[2:]).cpu().double().numpy()
    tol = TOL[w.qkv_dtype] if tol is None else tol
    eo, es = rel(got_o, o_ref), rel(got_s, S_ref)
    assert np.isfinite(got_o).all() and np.isfinite(got_s).all()
    assert eo <= tol and es <= tol, (eo, es)
    return eo, es


# ------------------------------------------------------------------------------ gate + cumsum

@pytest.mark.parametrize("gate", ["bounded", "neg_softplus"])
@pytest.mark.parametrize("T", [1, 64, 100, 1000])
def test_gate_cumsum_matches_fp64(gate, T):
    dev = device()
    g = torch.Generator(device=dev).manual_seed(3)
    x = torch.randn(2, 3, T, device=dev, generator=g) * 3.0
    x[0, 0, 0] = float("inf")
    x[1, 2, -1] = float("-inf")
    x[1, 1, T // 2] = 50.0
    b = gla.gate_cumsum(x, gate=gate)
    torch.cuda.synchronize()
    xn = x.cpu().numpy()
    gref = oracle.gate(xn, gate)
    if gate == "neg_softplus":
        gref = np.maximum(gref, -128.0)  # the stage's documented floor (e^-128 is 0 in fp32)
    ref = oracle.chunk_local_cumsum(np.pad(gref, [(0, 0), (0, 0), (0, (-T) % 64)]))[..., :T]
    got = b.cpu().double().numpy()
    assert np.all(np.abs(got - ref) <= 1e-6 * np.abs(ref) + 1e-6)


@pytest.mark.parametrize("qkv,segments,bursts", [("f32", 3, "none"), ("f32", 11, "none"), ("bf16", 11, "none"),
                                                 ("f32", 3, "bursts"), ("bf16", 5, "bursts"),
                                                 ("f32", 20, "front"), ("bf16", 20, "front")])
def test_segment_states_are_prefix_states(qkv, segments, bursts):
    """Stage entry point gla_segment_states: for every segment p but the last, the
    workspace holds the segment's total log-decay and the state at the end of segment
    p reached from a zero state at the start of the head (the pre-pass's local states
    combined in order).  11 segments exercise the prefix scan's batches of 8.  With
    bursts, a few whole chunks have x = +8 (chunk log-decay about -320, whose e^ is
    zero in fp32) inside weak-decay segments: the pre-pass then starts at the last such
    chunk of each segment, and the states must still match the fp64 recurrence.
    front: x = +8 over the first 12 of 24 chunks, so segments 0-9 of 20 have a zero
    decay factor: the scan's first batch (segments 1-8) has nothing to combine, and the
    next batch carries segment 9's state (its own local state) into segment 10."""
    w, inp = small(64 * 23 + 7, H=2, qkv=qkv, dk=64, dv=64, s0=0.0, x_mean=-6.0, seed=21)
    if bursts == "bursts":
        for ch in (1, 5, 6, 13, 17):
            inp["x"][:, :, ch * 64:(ch + 1) * 64] = 8.0
    elif bursts == "front":
        inp["x"][:, :, :12 * 64] = 8.0
    plan = gla.Plan(segments, 1)
    B, H, T = w.B, w.H, w.T
    ws = torch.zeros(gla.segment_workspace_size(B, H, T, w.dk, w.dv, plan), dtype=torch.uint8, device=device())
    gla.segment_states(inp["k"], inp["v"], inp["x"], plan, ws)
    torch.cuda.synchronize()
    nst = B * H * (segments - 1) * w.dk * w.dv
    states = ws[: nst * 4].view(torch.float32).reshape(B * H, segments - 1, w.dk, w.dv).cpu().double().numpy()
    decays = ws[nst * 4: nst * 4 + B * H * segments * 4].view(torch.float32).reshape(B * H, segments)
    decays = decays.cpu().double().numpy()
    nc = (T + 63) // 64
    g = oracle.gate(inp["x"].reshape(B * H, T).cpu().numpy().astype(np.float64))
    for p in range(segments - 1):
        t_beg = min(T, p * nc // segments * 64)
        t_end = min(T, (p + 1) * nc // segments * 64)
        _, S_ref = oracle_heads(inp, T=t_end)
        assert rel(states[:, p], S_ref) <= TOL[qkv], p
        ref_g = g[:, t_beg:t_end].sum(axis=1)
        assert np.all(np.abs(decays[:, p] - ref_g) <= 1e-5 * np.abs(ref_g) + 1e-4), p


def test_bounded_gate_tile_sums_above_minus_80():
    dev = device()
    g = torch.Generator(device=dev).manual_seed(4)
    x = torch.randn(1, 4, 4096, device=dev, generator=g) + 4.0  # strong decay
    b = gla.gate_cumsum(x).cpu().double().numpy().reshape(4, -1, 4, 16)
    prev = np.concatenate([np.zeros_like(b[..., :1, -1:]), b[..., :-1, -1:]], axis=-2)
    tile_sums = b[..., -1:] - prev  # chunk-local: each tile's own sum
    assert np.all(tile_sums > -80.0)


# ------------------------------------------------------------------------------ forward parity

@pytest.mark.parametrize("qkv,segments", [("bf16", 5), ("bf16", 16), ("f32", 4)])
def test_decay_bursts_segmented(qkv, segments):
    """Weak decay with whole chunks of strong decay (x = +8) at and around segment
    boundaries: the segment pre-pass starts at each segment's last such chunk; o and
    S_T against the fp64 oracle, with S0 carried through the first segment."""
    w, inp = small(64 * 37 + 21, H=2, qkv=qkv, dk=64, dv=64, x_mean=-6.0, seed=23)
    nc = (w.T + 63) // 64
    for ch in sorted({1, 2, nc // segments, nc // segments - 1, 2 * nc // segments, nc - 2}):
        inp["x"][:, :, ch * 64:(ch + 1) * 64] = 8.0
    check(inp, w, plan=gla.Plan(segments, 1))


@pytest.mark.parametrize("qkv,dk", [("bf16", 128), ("f32", 64)])
def test_strong_front_weak_tail_segmented(qkv, dk):
    """x = +8 over the first half of the sequence and weak decay after it, with 24
    segments: the prefix scan skips its first batch (every factor zero), combines the
    rest, and the output pass starts each segment from those states (S0 given)."""
    w, inp = small(64 * 48 + 5, H=2, qkv=qkv, dk=dk, dv=dk, x_mean=-6.0, seed=29)
    inp["x"][:, :, :24 * 64] = 8.0
    check(inp, w, plan=gla.Plan(24, 1))


@pytest.mark.parametrize("T", [64, 200, 640, 1000])
def test_bf16_default_plan(T):
    w, inp = small(T)
    check(inp, w)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_bf16_other_head_dims(dk, dv):
    w, inp = small(300, dk=dk, dv=dv)
    check(inp, w)


@pytest.mark.parametrize("plan", [(1, 1), (1, 2), (1, 4), (1, 8), (2, 1), (3, 2), (4, 4), (7, 8), (16, 2)])
def test_bf16_every_plan(plan):
    w, inp = small(16 * 64 + 17, H=2)
    check(inp, w, plan=gla.Plan(*plan))


def test_fp32_path_small_workload():
    w = gin.WORKLOADS["fp32_small"]
    inp = gin.make_inputs(w, device())
    check(inp, w)


@pytest.mark.parametrize("plan", [(1, 1), (2, 2), (4, 4)])
@pytest.mark.parametrize("dk", [64, 128])
def test_fp32_path_plans(plan, dk):
    w, inp = small(64 * 7 + 9, H=2, dk=dk, dv=64, qkv="f32")
    check(inp, w, plan=gla.Plan(*plan))


@pytest.mark.parametrize("regime", ["weak", "unit", "strong"])
def test_decay_regimes(regime):
    # weak decay (a ~ 0.99) and unit decay (a = 1) make the carried state dominate o,
    # so a broken inter-chunk path or segment hand-over cannot hide under the tolerance
    kw = dict(weak=dict(x_mean=-6.0), unit=dict(x_const=float("-inf")), strong=dict(x_mean=4.0))[regime]
    w, inp = small(2048 + 64 * 3, H=4, **kw)
    check(inp, w)
    check(inp, w, plan=gla.Plan(8, 2))


def test_zero_initial_state():
    w, inp = small(500, s0=0.0)
    assert inp["S0"] is None
    check(inp, w)


def test_empty_sequence_returns_initial_state():
    w, inp = small(0)
    o, ST = gla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"])
    torch.cuda.synchronize()
    assert o.shape[2] == 0
    assert torch.equal(ST, inp["S0"])
    w, inp = small(0, s0=0.0)
    o, ST = gla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["x"], None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ST).item() == 0


@pytest.mark.parametrize("T", [1, 15, 63, 65])
def test_short_and_ragged(T):
    w, inp = small(T, H=2)
    check(inp, w)


def test_many_heads_batch():
    w, inp = small(256, B=5, H=7)
    check(inp, w)


def test_default_plan_many_heads_dk64_dv128():
    """Enough heads that the default plan keeps full 128-column slices of dk = 64 heads
    (built only as wave-specialised kernels)."""
    w, inp = small(130, B=4, H=16, dk=64, dv=128)
    check(inp, w)


def test_chaining_matches_single_call():
    w, inp = small(64 * 20, H=2, x_mean=-5.0)
    o, ST = gla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"])
    T1 = 64 * 7
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    o1, S1 = gla.chunk_fwd(*(sl(inp[n], 0, T1) for n in "qkvx"), inp["S0"])
    o2, S2 = gla.chunk_fwd(*(sl(inp[n], T1, None) for n in "qkvx"), S1)
    torch.cuda.synchronize()
    assert rel(torch.cat([o1, o2], 2).cpu().numpy(), o.cpu().numpy()) <= CHAIN_TOL
    assert rel(S2.cpu().numpy(), ST.cpu().numpy()) <= CHAIN_TOL_STATE


@pytest.mark.parametrize("qkv", ["bf16", "f32"])
def test_chaining_weak_decay_state_handover(qkv):
    """Weak decay (x ~ N(-7,1): a ~ 0.995 per token) and a short second call (two
    chunks), so the chained S_T depends strongly on the handed-over state: starting
    the second call from zero instead moves S_T by far more than the bound.  The
    single call runs a segmented plan (4 segments), the chained calls one segment each,
    so the two sum the state in different orders."""
    d = 128 if qkv == "bf16" else 64  # the fp32 kernels take slices of at most 64 columns
    w, inp = small(64 * 12, H=2, x_mean=-7.0, qkv=qkv, seed=31, dk=d, dv=d)
    o, ST = gla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"], plan=gla.Plan(4, 1))
    T1 = 64 * 10
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    o1, S1 = gla.chunk_fwd(*(sl(inp[n], 0, T1) for n in "qkvx"), inp["S0"], plan=gla.Plan(1, 1))
    o2, S2 = gla.chunk_fwd(*(sl(inp[n], T1, None) for n in "qkvx"), S1, plan=gla.Plan(1, 1))
    _, Sz = gla.chunk_fwd(*(sl(inp[n], T1, None) for n in "qkvx"), None, plan=gla.Plan(1, 1))
    torch.cuda.synchronize()
    es = rel(S2.cpu().double().numpy(), ST.cpu().double().numpy())
    assert es <= CHAIN_TOL_STATE, es
    assert rel(Sz.cpu().double().numpy(), ST.cpu().double().numpy()) > 0.1  # S_T does depend on S1
    tol_o = CHAIN_TOL if qkv == "bf16" else CHAIN_TOL_STATE
    assert rel(torch.cat([o1, o2], 2).cpu().double().numpy(), o.cpu().double().numpy()) <= tol_o
    # and the single call against the fp64 oracle
    o_ref, S_ref = oracle_heads(inp)
    assert rel(ST.reshape(2, d, d).cpu().double().numpy(), S_ref) <= TOL[qkv]


def test_empty_sequence_through_the_c_abi_with_queried_workspace():
    """T = 0 through gla_chunk_fwd itself: the workspace is sized from the library's
    own query and the call must write S_T = S0 (a 0-byte query would make a caller pass
    a NULL workspace, which the library reads as another size query)."""
    import ctypes
    from chunked_linear_attention_gla_amd import _lib
    lib = _lib.load()
    dev = device()
    B, H, d = 2, 3, 128
    S0 = torch.randn(B, H, d, d, device=dev)
    ST = torch.full_like(S0, float("nan"))
    need = ctypes.c_size_t(0)
    rc = lib.gla_chunk_fwd(None, None, None, None, S0.data_ptr(), None, ST.data_ptr(), B, H, 0, d, d, 0, 0, 0,
                           None, ctypes.byref(need), None)
    assert rc == 0 and need.value > 0
    ws = torch.empty(need.value, dtype=torch.uint8, device=dev)
    n = ctypes.c_size_t(need.value)
    rc = lib.gla_chunk_fwd(None, None, None, None, S0.data_ptr(), None, ST.data_ptr(), B, H, 0, d, d, 0, 0, 0,
                           ws.data_ptr(), ctypes.byref(n), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0 and torch.equal(ST, S0)


def test_repeat_calls_are_bitwise_identical():
    w, inp = small(64 * 33, H=4)
    plan = gla.Plan(4, 4)
    o1, S1 = gla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"], plan=plan)
    o2, S2 = gla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"], plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


# ------------------------------------------------------------------------------ ablation path

@pytest.mark.parametrize("gate,x_mean", [("neg_softplus", -4.0), ("neg_softplus", 0.0), ("bounded", 4.0)])
def test_diag_branch_matches_oracle(gate, x_mean):
    w, inp = small(64 * 9 + 5, H=3, x_mean=x_mean, gate=gate)
    check(inp, w, path="diag_branch", gate=gate)
    check(inp, w, path="diag_branch", gate=gate, plan=gla.Plan(3, 4))


@pytest.mark.parametrize("dk,dv,plan,path", [
    (64, 64, (2, 2), "unified"), (64, 128, (3, 4), "diag_branch"), (128, 128, (5, 1), "diag_branch"),
    (64, 64, (1, 1), "diag_branch"), (128, 64, (2, 2), "diag_branch"), (128, 128, (17, 1), "unified")])
def test_wave_specialised_shapes(dk, dv, plan, path):
    """Head dims, slice widths (32, 64, 128 columns: 1, 2 or 4 compute waves) and
    segment lengths (odd, even, single chunk) of the wave-specialised kernels, both
    paths; 17 chunks of 64 plus a ragged tail."""
    gate = "neg_softplus" if path == "diag_branch" else "bounded"
    w, inp = small(17 * 64 + 9, H=2, dk=dk, dv=dv, x_mean=-2.0 if path == "diag_branch" else 0.0, gate=gate)
    check(inp, w, plan=gla.Plan(*plan), path=path, gate=gate)


def test_diag_branch_fp32():
    w, inp = small(64 * 4 + 3, H=2, dk=64, dv=64, qkv="f32", x_mean=-4.0, gate="neg_softplus")
    check(inp, w, path="diag_branch", gate="neg_softplus")


def test_forced_overflow_breaks_only_the_unified_factorisation():
    """x = -6 under the softplus gate gives g ~ -6.0025, a tile sum near -96, and a
    reciprocal e^96 beyond fp32: the unified factorisation overflows, the
    diagonal-branch path (all factors <= 1) still matches the oracle."""
    w, inp = small(256, H=2, x_const=-6.0, gate="neg_softplus")
    o_u, S_u = gla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["x"], inp["S0"], gate="neg_softplus",
                             path="unified")
    torch.cuda.synchronize()
    assert not torch.isfinite(o_u).all()
    check(inp, w, path="diag_branch", gate="neg_softplus")


@pytest.mark.parametrize("qkv,dk", [("bf16", 128), ("f32", 64)])
def test_softplus_gate_at_minus_infinity(qkv, dk):
    """x = -inf under the softplus gate is a zero decay (a = 0) in the oracle.  The
    kernels floor that gate at g = -128, whose exponential is already exactly 0 in fp32,
    so cumulative log-decays stay finite: isolated tokens, a pair, and a whole chunk at
    -inf, through the diagonal-branch path (the path built for that gate), against the
    fp64 oracle with its exact a = 0."""
    w, inp = small(64 * 5 + 9, H=2, dk=dk, dv=64, qkv=qkv, x_mean=-2.0, gate="neg_softplus", seed=41)
    inp["x"][0, 0, [3, 70, 71, 150, 320]] = float("-inf")
    inp["x"][0, 1, 64:128] = float("-inf")
    check(inp, w, path="diag_branch", gate="neg_softplus")
    check(inp, w, path="diag_branch", gate="neg_softplus", plan=gla.Plan(3, 1))


def test_softplus_gate_at_minus_infinity_backward_and_decode():
    """The same zero decays through the backward pass (diagonal-branch path, all five
    gradients) and the decode step, against the fp64 oracles."""
    dev = device()
    w, inp = small(64 * 3 + 5, H=2, dk=64, dv=64, x_mean=-2.0, gate="neg_softplus", seed=43)
    inp["x"][0, 0, [0, 5, 64, 65, 100]] = float("-inf")
    inp["x"][0, 1, 128:192] = float("-inf")
    gen = torch.Generator(device=dev).manual_seed(44)
    dO = torch.randn(1, 2, w.T, 64, device=dev, generator=gen).to(torch.bfloat16)
    dST = torch.randn(1, 2, 64, 64, device=dev, generator=gen) * 0.1
    got = gla.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["x"], dO, inp["S0"], dST, gate="neg_softplus",
                        path="diag_branch")
    torch.cuda.synchronize()
    flat = lambda t: t.reshape(2, *t.shape[2:])
    ref = oracle.backward(*(gin.to_numpy_bits(flat(inp[n])) for n in ("q", "k", "v", "x")),
                          flat(dO).cpu().double().numpy(), flat(inp["S0"]).cpu().double().numpy(),
                          flat(dST).cpu().double().numpy(), gate="neg_softplus")
    for name, g_, r_ in zip(("dq", "dk", "dv", "dx", "dS0"), got, ref):
        g_ = g_.reshape(r_.shape).cpu().double().numpy()
        assert np.isfinite(g_).all() and rel(g_, r_) <= TOL["bf16"], name
    # decode: one token at x = -inf replaces the state by k v^T
    wd = gin.WORKLOADS["bf16_decode"].with_(B=2, H=3, dk=64, dv=64, gate="neg_softplus")
    dinp = gin.make_decode_inputs(wd, dev)
    dinp["x"][0, 1] = float("-inf")
    S_in = dinp["S"].clone()
    od = gla.decode_step(dinp["q"], dinp["k"], dinp["v"], dinp["x"], dinp["S"], gate="neg_softplus")
    torch.cuda.synchronize()
    f1 = lambda t: t.reshape(6, 1, *t.shape[2:])
    o_ref, S_ref = oracle.forward(*(gin.to_numpy_bits(f1(dinp[n])) for n in ("q", "k", "v")),
                                  gin.to_numpy_bits(dinp["x"].reshape(6, 1)),
                                  S_in.reshape(6, 64, 64).cpu().numpy().astype(np.float64), gate="neg_softplus")
    assert rel(od.reshape(6, 1, 64).cpu().double().numpy(), o_ref) <= TOL["bf16"]
    assert rel(dinp["S"].reshape(6, 64, 64).cpu().double().numpy(), S_ref) <= TOL["bf16"]
