"""Seeded randomized parity sweep through the C ABI: sequence length, batch and head
counts, head sizes, launch plans, gates, paths, decay regimes and the optional states
are drawn from fixed seeds, and each call is checked against the fp64 oracles at the
same bars as the targeted tests (2e-2 with bf16 operands, 1e-4 on the fp32 path).
Entry points: forward, backward, per-channel forward, delta rule, packed sequences and
the decode step.

The negative-softplus gate runs on the diagonal-branch path, and on the unified path
only where its decays stay mild (x >= 0): that gate has no lower bound, so strong decays
can take a 16-token tile past the range the unified path relies on."""
import numpy as np
import pytest
import torch

import oracle
import chunked_linear_attention_gla_amd as gla
from chunked_linear_attention_gla_amd import inputs as gin
from gpu_util import TOL, rel
import test_backward_gpu as bw
import test_decode_varlen_gpu as dv_
import test_delta_gpu as dl
import test_parity_gpu as fw
import test_pc_gpu as pcm

pytestmark = pytest.mark.gpu

CASES = 24


def common(r):
    T = int(r.integers(1, 1300))
    return dict(T=T, H=int(r.integers(1, 4)), B=int(r.integers(1, 3)), dk=int(r.choice([64, 128])),
                dv=int(r.choice([64, 128])), x_mean=float(r.choice([-6.0, -2.0, 0.0, 2.0, 4.0])),
                x_std=float(r.choice([0.5, 1.0, 3.0])), s0=float(r.choice([0.0, 0.1])))


def gate_path(r, x_mean):
    gate = str(r.choice(["bounded", "neg_softplus"]))
    if gate == "bounded" or x_mean >= 0.0:
        return gate, str(r.choice(["unified", "diag_branch"]))
    return gate, "diag_branch"


def plan(r, T, dv, max_split=2):
    nc = max(1, -(-T // 64))
    segments = int(r.integers(1, min(6, nc) + 1))
    split = int(r.choice([s for s in (1, 2, 4) if s <= max_split and dv // s >= 64]))
    return gla.Plan(segments, split) if r.random() < 0.7 else None


@pytest.mark.parametrize("case", range(CASES))
def test_forward(case):
    r = np.random.default_rng(9000 + case)
    c = common(r)
    gate, path = gate_path(r, c["x_mean"])
    qkv = "f32" if (c["dk"] == 64 and c["dv"] == 64 and path == "unified" and r.random() < 0.4) else "bf16"
    w, inp = fw.small(c["T"], H=c["H"], B=c["B"], dk=c["dk"], dv=c["dv"], qkv=qkv, x_mean=c["x_mean"],
                      x_std=c["x_std"], s0=c["s0"], seed=100 + case, gate=gate)
    fw.check(inp, w, plan=plan(r, c["T"], c["dv"], 1 if qkv == "f32" else 2), path=path, gate=gate)


@pytest.mark.parametrize("case", range(CASES))
def test_backward(case):
    r = np.random.default_rng(9100 + case)
    c = common(r)
    gate, path = gate_path(r, c["x_mean"])
    w, inp, dO, dST = bw.make(c["T"], H=c["H"], B=c["B"], dk=c["dk"], dv=c["dv"], x_mean=c["x_mean"],
                              x_std=c["x_std"], s0=c["s0"], dst=bool(r.random() < 0.6), seed=200 + case, gate=gate)
    bw.check(w, inp, dO, dST, gate=gate, path=path)


@pytest.mark.parametrize("case", range(CASES))
def test_per_channel(case):
    r = np.random.default_rng(9200 + case)
    c = common(r)
    w, inp = pcm.make(c["T"], H=c["H"], B=c["B"], dk=c["dk"], dv=c["dv"], x_mean=c["x_mean"], x_std=c["x_std"],
                      s0=c["s0"], seed=300 + case)
    pcm.check(w, inp, plan=plan(r, c["T"], c["dv"]))


@pytest.mark.parametrize("case", range(CASES))
def test_delta_rule(case):
    r = np.random.default_rng(9300 + case)
    c = common(r)
    w, inp = dl.make(c["T"], H=c["H"], B=c["B"], dk=c["dk"], dv=c["dv"], x_mean=c["x_mean"], x_std=c["x_std"],
                     s0=c["s0"], seed=400 + case)
    dl.check(w, inp, plan=plan(r, c["T"], c["dv"]))


@pytest.mark.parametrize("case", range(CASES))
def test_packed_sequences(case):
    r = np.random.default_rng(9400 + case)
    c = common(r)
    n = int(r.integers(1, 9))
    lengths = [int(L) for L in r.choice([0, 1, 17, 63, 64, 65, 200, 700, 1500], size=n)]
    if sum(lengths) == 0:
        lengths.append(33)
    gate, path = gate_path(r, c["x_mean"])
    w = dv_.VAR.with_(H=c["H"], dk=c["dk"], dv=c["dv"], x_mean=c["x_mean"], x_std=c["x_std"], s0_std=c["s0"],
                      gate=gate)
    nc = max(1, -(-max(lengths) // 64))
    segs = int(r.integers(1, min(4, nc) + 1))
    dv_.varlen_check(w, lengths, gate=gate, path=path, seed=500 + case,
                     plan=gla.Plan(segs, 1) if r.random() < 0.5 else None)


@pytest.mark.parametrize("case", range(CASES))
def test_decode_step(case):
    r = np.random.default_rng(9500 + case)
    c = common(r)
    gate = str(r.choice(["bounded", "neg_softplus"]))
    per_channel = bool(r.random() < 0.5)
    qkv = "f32" if (c["dk"] == 64 and c["dv"] == 64 and r.random() < 0.3) else "bf16"
    B, H, dk, dv = int(r.integers(1, 9)), int(r.integers(1, 9)), c["dk"], c["dv"]
    w = dv_.DEC.with_(B=B, H=H, dk=dk, dv=dv, qkv_dtype=qkv, per_channel=per_channel, gate=gate,
                      x_mean=c["x_mean"], x_std=c["x_std"])
    inp = gin.make_decode_inputs(w, fw.device(), seed=600 + case)
    S_in = inp["S"].clone()
    o = gla.decode_step(inp["q"], inp["k"], inp["v"], inp["x"], inp["S"], gate=gate)
    torch.cuda.synchronize()
    BH = B * H
    flat = lambda t: t.reshape(BH, 1, *t.shape[2:])
    q, k, v = (gin.to_numpy_bits(flat(inp[n])) for n in ("q", "k", "v"))
    x = gin.to_numpy_bits(inp["x"].reshape(BH, 1, *inp["x"].shape[2:]))
    fwd = oracle.forward_pc if per_channel else oracle.forward
    o_ref, S_ref = fwd(q, k, v, x, S_in.reshape(BH, dk, dv).cpu().numpy().astype(np.float64), gate=gate)
    tol = TOL[qkv]
    assert rel(o.reshape(BH, 1, dv).cpu().double().numpy(), o_ref) <= tol
    assert rel(inp["S"].reshape(BH, dk, dv).cpu().double().numpy(), S_ref) <= tol
