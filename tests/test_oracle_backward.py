"""Pins of the fp64 backward oracle (oracle.backward) to things other than itself:

* reverse-mode autodiff of an independent PyTorch implementation of the same
  recurrence (fp64, CPU), written out here;
* central finite differences of the numpy closed form (oracle.closed_form, itself
  pinned to the recurrence in test_oracle.py) along random directions;
* a ≡ 1 (x = -inf under the bounded gate): the gradients of causal linear
  attention o = tril(QK^T)V + Q S0, S_T = S0 + K^T V, written with numpy matmuls;
* the log-decay gradient identity dL/dg_t = sum_{t' >= t} (q_t'.dq_t' - k_t'.dk_t')
  + <dS_T, S_T>, checked on the oracle's outputs (it ties dx to dq and dk);
* planted mistakes in the backward must make the autodiff pin fail.

The recurrence (the plainest reading of the chunked linear attention with a
per-position decay of "Engineering Long-Context Training for Trillion-Parameter
MoE Models: Three Key Breakthroughs", §3.1-§3.2): S_t = a_t S_{t-1} + k_t v_t^T,
o_t = S_t^T q_t, a_t = exp(g(x_t)).
"""
import os
import tempfile

import numpy as np
import pytest
import torch

import oracle

FD_H = 1e-5


def rel(a, b):
    return oracle.max_rel_err(a, b)


def case(rng, BH, T, dk, dv, s0=True, dst=True, x_shift=0.0, x_scale=1.5):
    q = rng.standard_normal((BH, T, dk)).astype(np.float32)
    k = rng.standard_normal((BH, T, dk)).astype(np.float32)
    v = rng.standard_normal((BH, T, dv)).astype(np.float32)
    x = (x_shift + x_scale * rng.standard_normal((BH, T))).astype(np.float32)
    S0 = rng.standard_normal((BH, dk, dv)) if s0 else None
    dO = rng.standard_normal((BH, T, dv))
    dST = rng.standard_normal((BH, dk, dv)) if dst else None
    return q, k, v, x, S0, dO, dST


def torch_gate(x, gate):
    if gate == "bounded":
        return -5.0 * torch.sigmoid(x)
    return torch.nn.functional.logsigmoid(x)  # -softplus(-x)


def torch_reference_grads(q, k, v, x, S0, dO, dST, gate):
    """Autograd of a plain fp64 PyTorch loop over tokens."""
    t64 = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    Q, K, V, X = t64(q), t64(k), t64(v), t64(x)
    BH, T, dk = Q.shape
    dv = V.shape[-1]
    S0t = t64(S0) if S0 is not None else t64(np.zeros((BH, dk, dv)))
    a = torch.exp(torch_gate(X, gate))
    S = S0t
    outs = []
    for t in range(T):
        S = a[:, t, None, None] * S + K[:, t, :, None] * V[:, t, None, :]
        outs.append((Q[:, t, :, None] * S).sum(dim=1))
    o = torch.stack(outs, dim=1) if T else torch.zeros(BH, 0, dv, dtype=torch.float64)
    L = (o * torch.tensor(dO)).sum()
    if dST is not None:
        L = L + (S * torch.tensor(dST)).sum()
    L.backward()
    g = lambda t: t.grad.numpy() if t.grad is not None else np.zeros(t.shape)
    return g(Q), g(K), g(V), g(X), g(S0t)


NAMES = ("dq", "dk", "dv", "dx", "dS0")


@pytest.mark.parametrize("gate", ["bounded", "neg_softplus"])
@pytest.mark.parametrize("T,dk,dv", [(1, 4, 4), (5, 4, 3), (64, 4, 4), (70, 8, 6), (130, 3, 5)])
@pytest.mark.parametrize("states", [(True, True), (False, False), (True, False)])
def test_backward_matches_torch_autograd(gate, T, dk, dv, states):
    rng = np.random.default_rng(T * 100 + dk * 10 + dv)
    q, k, v, x, S0, dO, dST = case(rng, 2, T, dk, dv, *states)
    got = oracle.backward(q, k, v, x, dO, S0, dST, gate=gate)
    ref = torch_reference_grads(q, k, v, x, S0, dO, dST, gate)
    for name, g_, r_ in zip(NAMES, got, ref):
        assert rel(g_, r_) <= 1e-10, (name, rel(g_, r_))


def _loss_closed_form(q, k, v, x, S0, dO, dST, gate):
    o, ST = oracle.closed_form(q, k, v, x, S0, gate=gate)
    return float(np.sum(o * dO) + (np.sum(ST * dST) if dST is not None else 0.0))


@pytest.mark.parametrize("gate", ["bounded", "neg_softplus"])
def test_backward_directional_finite_differences(gate):
    """<grad, delta> against (L(theta + h delta) - L(theta - h delta)) / 2h, in fp64,
    with L = <dO, o> + <dS_T, S_T> evaluated by the quadratic closed form."""
    rng = np.random.default_rng(5)
    q, k, v, x, S0, dO, dST = case(rng, 2, 23, 4, 3)
    args = {"q": q.astype(np.float64), "k": k.astype(np.float64), "v": v.astype(np.float64),
            "x": x.astype(np.float64), "S0": S0}
    grads = dict(zip(("q", "k", "v", "x", "S0"), oracle.backward(q, k, v, x, dO, S0, dST, gate=gate)))
    for name in args:
        delta = rng.standard_normal(args[name].shape)
        plus = dict(args); plus[name] = args[name] + FD_H * delta
        minus = dict(args); minus[name] = args[name] - FD_H * delta
        fd = (_loss_closed_form(plus["q"], plus["k"], plus["v"], plus["x"], plus["S0"], dO, dST, gate)
              - _loss_closed_form(minus["q"], minus["k"], minus["v"], minus["x"], minus["S0"], dO, dST, gate)) \
            / (2 * FD_H)
        an = float(np.sum(grads[name] * delta))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_unit_decay_gradients_are_causal_linear_attention():
    """x = -inf under the bounded gate gives a = 1: o = tril(QK^T)V + Q S0 and
    S_T = S0 + K^T V, whose gradients are written here with numpy matmuls."""
    rng = np.random.default_rng(9)
    q, k, v, _, S0, dO, dST = case(rng, 1, 40, 5, 4)
    x = np.full((1, 40), -np.inf, dtype=np.float32)
    dq, dk, dv, dx, dS0 = oracle.backward(q, k, v, x, dO, S0, dST, gate="bounded")
    Q, K, V, G, S, DS = (a[0].astype(np.float64) for a in (q, k, v, dO, S0, dST))
    M = np.tril(np.ones((40, 40)))
    P = M * (G @ V.T)                     # [t, s] = dO_t . v_s for s <= t
    A = M * (Q @ K.T)                     # [t, s] = q_t . k_s for s <= t
    assert rel(dq[0], P @ K + G @ S.T) <= 1e-12
    assert rel(dk[0], P.T @ Q + V @ DS.T) <= 1e-12
    assert rel(dv[0], A.T @ G + K @ DS) <= 1e-12
    assert rel(dS0[0], Q.T @ G + DS) <= 1e-12
    assert np.all(dx == 0.0)              # the bounded gate is flat at x = -inf


@pytest.mark.parametrize("gate", ["bounded", "neg_softplus"])
def test_log_decay_gradient_identity(gate):
    """dL/dg_t = sum_{t'>=t} (q_t'.dq_t' - k_t'.dk_t') + <dS_T, S_T>; dx = g'(x) dL/dg."""
    rng = np.random.default_rng(13)
    q, k, v, x, S0, dO, dST = case(rng, 3, 150, 6, 5)
    dq, dk, dv, dx, dS0 = oracle.backward(q, k, v, x, dO, S0, dST, gate=gate)
    _, ST = oracle.forward(q, k, v, x, S0.astype(np.float64), gate=gate)
    s = np.sum(q.astype(np.float64) * dq, axis=-1) - np.sum(k.astype(np.float64) * dk, axis=-1)
    dg = np.flip(np.cumsum(np.flip(s, -1), -1), -1) + np.sum(dST * ST, axis=(-2, -1))[:, None]
    xs = x.astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(-xs))
    slope = -5.0 * sig * (1.0 - sig) if gate == "bounded" else 1.0 / (1.0 + np.exp(xs))
    assert rel(dg * slope, dx) <= 1e-10


def test_empty_sequence_gradient_is_dst():
    rng = np.random.default_rng(3)
    q, k, v, x, S0, dO, dST = case(rng, 2, 0, 4, 4)
    dq, dk, dv, dx, dS0 = oracle.backward(q, k, v, x, dO, S0, dST)
    assert dq.shape == (2, 0, 4) and dx.shape == (2, 0)
    np.testing.assert_array_equal(dS0, dST)


def test_bf16_storage_is_read_as_widened_values():
    """bf16 bit patterns give the same gradients as their fp32 widenings."""
    rng = np.random.default_rng(17)
    q, k, v, x, S0, dO, dST = case(rng, 2, 33, 4, 4)
    to_bf16 = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 values do
    qb, kb, vb = to_bf16(q), to_bf16(k), to_bf16(v)
    widen = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    g1 = oracle.backward(qb, kb, vb, x, dO, S0, dST)
    g2 = oracle.backward(widen(qb), widen(kb), widen(vb), x, dO, S0, dST)
    for a, b in zip(g1, g2):
        np.testing.assert_array_equal(a, b)


def _backward_pin_passes(lib_path):
    rng = np.random.default_rng(31)
    ok = True
    for gate in ("bounded", "neg_softplus"):
        q, k, v, x, S0, dO, dST = case(rng, 2, 70, 4, 3)
        got = oracle.backward(q, k, v, x, dO, S0, dST, gate=gate, lib_path=lib_path)
        ref = torch_reference_grads(q, k, v, x, S0, dO, dST, gate)
        ok &= all(rel(g_, r_) <= 1e-10 for g_, r_ in zip(got, ref))
    return bool(ok)


@pytest.mark.parametrize("mutant", [7, 8, 9, 10])
def test_planted_backward_mistakes_are_caught(mutant):
    """Planted mistakes in the backward (state gradient not decayed when carried to
    the previous token; a_t missing from the gate gradient; dq from the state
    before the token's update; dv from q instead of k) must fail the autodiff pin."""
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, f"libgla_oracle_m{mutant}.so")
        oracle.build(path, mutant=mutant)
        assert not _backward_pin_passes(path)
    assert _backward_pin_passes(oracle.LIB_PATH)
