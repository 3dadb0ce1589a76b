"""GPU parity of the chunked gated delta rule (gla_chunk_fwd_delta through the C ABI)
against the fp64 token-by-token oracle on the same seeded inputs.  Bar: max |gpu - ref|
/ max |ref| <= 2e-2 with bf16 operands, <= 1e-4 on the fp32 path, for o and S_T."""
import numpy as np
import pytest
import torch

import oracle
import chunked_linear_attention_gla_amd as gla
from chunked_linear_attention_gla_amd import inputs as gin
from gpu_util import CHAIN_TOL, CHAIN_TOL_DELTA, TOL, device, rel

pytestmark = pytest.mark.gpu

BASE = gin.WORKLOADS["bf16_64k_delta"]


def make(T, H=3, B=1, dk=128, dv=128, qkv="bf16", x_mean=0.0, x_std=1.0, s0=0.1, seed=13):
    w = BASE.with_(B=B, H=H, T=T, dk=dk, dv=dv, qkv_dtype=qkv, x_mean=x_mean, x_std=x_std, s0_std=s0, seed=seed)
    return w, gin.make_inputs(w, device())


def oracle_delta(inp, gate="bounded"):
    q = inp["q"]
    B, H = q.shape[:2]
    flat = lambda t: t.reshape(B * H, *t.shape[2:])
    s0 = None if inp["S0"] is None else flat(inp["S0"]).cpu().numpy().astype(np.float64)
    return oracle.forward_delta(*(gin.to_numpy_bits(flat(inp[n])) for n in ("q", "k", "v", "x", "beta")), s0,
                                gate=gate)


def check(w, inp, plan=None, gate="bounded", tol=None):
    o, ST = gla.chunk_fwd_delta(inp["q"], inp["k"], inp["v"], inp["x"], inp["beta"], inp["S0"], gate=gate,
                                plan=plan)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_delta(inp, gate)
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


@pytest.mark.parametrize("regime,x_mean", [("weak", -6.0), ("mid", 0.0), ("strong", 4.0)])
def test_decay_regimes(regime, x_mean):
    """weak decay: the erase-and-write memory carries across many chunks."""
    w, inp = make(64 * 20 + 5, H=2, x_mean=x_mean)
    check(w, inp)


def test_full_write_strength_unit_decay():
    """beta = 1 and a = 1 (x = -inf): pure delta rule, each write replaces what the key
    retrieves; the hardest case for the triangular solve (M has unit scale)."""
    w, inp = make(64 * 6 + 3, H=2)
    inp["beta"].fill_(1.0)
    inp["x"].fill_(float("-inf"))
    check(w, inp)


def test_zero_write_strength_only_decays():
    # weak decay, so that the decayed initial state is still far above fp32 underflow
    w, inp = make(64 * 3 + 7, H=2, x_mean=-6.0)
    inp["beta"].zero_()
    check(w, inp)


@pytest.mark.parametrize("dk,dv,split", [(64, 64, 1), (64, 128, 2), (128, 64, 2), (128, 128, 1), (128, 128, 4),
                                         (64, 64, 2)])
def test_head_dims_and_slices(dk, dv, split):
    w, inp = make(64 * 5 + 9, dk=dk, dv=dv)
    check(w, inp, plan=gla.Plan(1, split))


@pytest.mark.parametrize("segments,split", [(2, 1), (3, 2), (8, 1), (5, 4)])
def test_segmented_plans(segments, split):
    """Segments after the first start from S0 folded with the earlier segments'
    affine maps; weak decay so the carried state matters."""
    w, inp = make(64 * 24 + 11, H=2, x_mean=-5.0)
    check(w, inp, plan=gla.Plan(segments, split))


def test_segmented_pure_delta_rule():
    """beta = 1, a = 1: the segment transitions are products of projections."""
    w, inp = make(64 * 16 + 3, H=2)
    inp["beta"].fill_(1.0)
    inp["x"].fill_(float("-inf"))
    check(w, inp, plan=gla.Plan(4, 1))


def test_default_plan_long_sequence():
    w, inp = make(64 * 64 + 31, H=2, x_mean=-4.0, s0=0.0)
    inp["S0"] = None
    check(w, inp)


def test_fp32_path():
    w, inp = make(64 * 4 + 3, H=2, dk=64, dv=64, qkv="f32")
    check(w, inp)
    check(w, inp, plan=gla.Plan(1, 2))
    check(w, inp, plan=gla.Plan(3, 1))


def test_without_initial_state_and_softplus_gate():
    w, inp = make(64 * 4 + 1, H=2, s0=0.0, x_mean=-4.0)
    inp["S0"] = None
    check(w, inp, gate="neg_softplus")


def test_chaining_matches_single_call():
    w, inp = make(64 * 10, H=2, x_mean=-5.0)
    q, k, v, x, be, S0 = inp["q"], inp["k"], inp["v"], inp["x"], inp["beta"], inp["S0"]
    o, ST = gla.chunk_fwd_delta(q, k, v, x, be, S0)
    s = 64 * 4
    cut = lambda t, a, b: t[:, :, a:b].contiguous()
    oa, Sa = gla.chunk_fwd_delta(*(cut(t, 0, s) for t in (q, k, v, x, be)), S0)
    ob, Sb = gla.chunk_fwd_delta(*(cut(t, s, 640) for t in (q, k, v, x, be)), Sa)
    torch.cuda.synchronize()
    assert rel(torch.cat([oa, ob], 2).cpu().double().numpy(), o.cpu().double().numpy()) <= CHAIN_TOL
    assert rel(Sb.cpu().double().numpy(), ST.cpu().double().numpy()) <= CHAIN_TOL_DELTA


def test_empty_sequence_returns_initial_state():
    w, inp = make(0, H=2)
    o, ST = gla.chunk_fwd_delta(inp["q"], inp["k"], inp["v"], inp["x"], inp["beta"], inp["S0"])
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(ST, inp["S0"])


def test_largest_head_extent():
    """The largest sequence the ABI accepts for one head at dk = dv = 128 (o spans
    0xFFFF0000 bytes; its byte offsets pass 2^31 at token 4194304).  Whole chunks with
    x = +8 are planted before the checked windows: the state's transition over such a
    chunk, e^gamma I - K~^T W, is of order e^-320, so the fp64 oracle restarted from a
    zero state there yields the outputs after it.  Checked: the first 192 tokens (with
    S0), four chunks across the 2^31-byte offset of o, the last two chunks and S_T."""
    t_max = 0xFFFF0000 // (128 * 4)
    w, inp = make(t_max, H=1, seed=4244)
    mid = (1 << 31) // (128 * 4) // 64
    last = t_max // 64
    for ch in (mid - 3, last - 3):
        inp["x"][:, :, ch * 64:(ch + 1) * 64] = 8.0
    o, ST = gla.chunk_fwd_delta(inp["q"], inp["k"], inp["v"], inp["x"], inp["beta"], inp["S0"])
    torch.cuda.synchronize()
    names = ("q", "k", "v", "x", "beta")
    head = {n: inp[n][:, :, :192].contiguous() for n in names}
    head["S0"] = inp["S0"]
    o_ref, _ = oracle_delta(head)
    assert rel(o[0, 0, :192].cpu().double().numpy(), o_ref[0]) <= TOL["bf16"]
    for a, c, b in ((mid - 3, mid - 2, mid + 2), (last - 3, last - 2, last)):
        sub = {n: inp[n][:, :, a * 64:b * 64].contiguous() for n in names}
        sub["S0"] = None
        o_ref, S_ref = oracle_delta(sub)
        got = o[0, 0, c * 64:b * 64].cpu().double().numpy()
        assert np.isfinite(got).all()
        assert rel(got, o_ref[0, (c - a) * 64:]) <= TOL["bf16"], (a, b)
        if b == last:
            assert rel(ST[0, 0].cpu().double().numpy(), S_ref[0]) <= TOL["bf16"]


@pytest.mark.parametrize("qkv,beta_one", [("bf16", False), ("bf16", True), ("f32", False)])
def test_reset_chunks_inside_segments(qkv, beta_one):
    """Weak decay (the state carries across whole segments) with a few strong-decay
    chunks (x = +8: chunk log-decay about -320) planted inside the segments.  Their
    transition e^gamma I - (k e^{gamma-b})^T W is below 2^-114 in size, so the local-state
    half of the segment pre-pass starts at the last such chunk of each segment instead
    of the segment start: segment 0 at chunk 7, segment 1 at chunk 19 (two planted in a
    row), segment 2 at none (no planted chunk: all of its chunks run).  The whole call
    must still match the fp64 oracle, with beta ~ U(0,1) and with beta = 1."""
    d = 128 if qkv == "bf16" else 64
    w, inp = make(64 * 40 + 11, H=2, dk=d, dv=d, qkv=qkv, x_mean=-6.0, seed=23)
    for ch in (7, 18, 19, 33):
        inp["x"][:, :, ch * 64:(ch + 1) * 64] = 8.0
    if beta_one:
        inp["beta"].fill_(1.0)
    check(w, inp, plan=gla.Plan(4, 1))


def test_repeat_calls_are_bitwise_identical():
    """Same inputs, same o and S_T bit for bit, with segments (pre-pass with reset
    flags, folds of the segment maps)."""
    w, inp = make(64 * 24 + 5, H=2, x_mean=-3.0)
    args = (inp["q"], inp["k"], inp["v"], inp["x"], inp["beta"], inp["S0"])
    o1, S1 = gla.chunk_fwd_delta(*args, plan=gla.Plan(4, 1))
    o2, S2 = gla.chunk_fwd_delta(*args, plan=gla.Plan(4, 1))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("beta_one", [False, True])
def test_reset_flags_mark_only_negligible_transitions(beta_one):
    """The per-chunk pass's reset flags, read from the workspace (b, the Tinv of every
    chunk, the segment maps, then one int32 flag per chunk): every planted strong-decay
    chunk (x = +8) is flagged and no weakly decaying chunk is; and for each flagged chunk
    the fp64 oracle's transition over it -- the delta rule run over the chunk alone with
    v = 0 from S_0 = I, i.e. the state map S_start -> S_end -- has entries below 2^-114."""
    w, inp = make(64 * 40 + 11, H=2, x_mean=-6.0, seed=23)
    planted = (7, 18, 19, 33)
    for ch in planted:
        inp["x"][:, :, ch * 64:(ch + 1) * 64] = 8.0
    if beta_one:
        inp["beta"].fill_(1.0)
    BH, T, d, P, es = 2, w.T, 128, 4, 2
    nc = (T + 63) // 64
    al = lambda n: (n + 255) // 256 * 256
    off = al(BH * T * 4) + al(BH * nc * 64 * 64 * es) + al(BH * (P - 1) * d * d * 4) * 2
    ws = torch.zeros(off + al(BH * nc * 4), dtype=torch.uint8, device=device())
    gla.chunk_fwd_delta(inp["q"], inp["k"], inp["v"], inp["x"], inp["beta"], inp["S0"], plan=gla.Plan(P, 1),
                        workspace=ws)
    torch.cuda.synchronize()
    flags = ws[off:off + BH * nc * 4].view(torch.int32).reshape(BH, nc).cpu().numpy()
    expect = np.zeros((BH, nc), dtype=np.int32)
    expect[:, list(planted)] = 1
    assert (flags == expect).all(), np.argwhere(flags != expect)
    for h in range(BH):
        for c in planted:
            sl = slice(c * 64, (c + 1) * 64)
            kc = gin.to_numpy_bits(inp["k"][0, h, sl])
            zero = np.zeros_like(kc)
            _, trans = oracle.forward_delta(zero, kc, zero, inp["x"][0, h, sl].cpu().numpy(),
                                            inp["beta"][0, h, sl].cpu().numpy(), np.eye(d))
            assert np.abs(trans).max() < 2.0 ** -114, (h, c)
