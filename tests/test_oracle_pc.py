"""Pins of the per-channel-decay oracle (oracle.forward_pc) to things other than itself.

The recurrence (per-channel reading of the per-position decay of "Engineering
Long-Context Training for Trillion-Parameter MoE Models: Three Key Breakthroughs",
§3.1, with the gates of §3.2): S_t[d, :] = a_t[d] S_{t-1}[d, :] + k_t[d] v_t,
o_t = S_t^T q_t, a_t[d] = exp(g(x_t[d])).

* the numpy closed form with explicit per-channel decay products (closed_form_pc);
* x equal across channels reduces to the scalar recurrence (oracle.forward, itself
  pinned in test_oracle.py);
* a = 1 (x = -inf, bounded gate): causal linear attention written with matmuls;
* channel separability: channels where q and k are zero do not influence o;
* chaining over a split of the sequence; the single-token closed form;
* planted mistakes (decay by value column, channel 0's decay for every row, decay
  index shifted by one token) must fail these pins.
"""
import os
import tempfile

import numpy as np
import pytest

import oracle

rel = oracle.max_rel_err


def case(rng, BH, T, dk, dv, s0=True, x_shift=0.0, x_scale=1.5, infs=False):
    q = rng.standard_normal((BH, T, dk)).astype(np.float32)
    k = rng.standard_normal((BH, T, dk)).astype(np.float32)
    v = rng.standard_normal((BH, T, dv)).astype(np.float32)
    x = (x_shift + x_scale * rng.standard_normal((BH, T, dk))).astype(np.float32)
    if infs and x.size >= 4:
        flat = x.reshape(-1)
        flat[::7] = np.inf
        flat[3::11] = -np.inf
    S0 = rng.standard_normal((BH, dk, dv)) if s0 else None
    return q, k, v, x, S0


@pytest.mark.parametrize("gate", ["bounded", "neg_softplus"])
@pytest.mark.parametrize("T,dk,dv", [(1, 1, 1), (5, 4, 3), (17, 3, 5), (40, 8, 8), (70, 6, 4)])
@pytest.mark.parametrize("s0", [True, False])
def test_recurrence_matches_closed_form(gate, T, dk, dv, s0):
    rng = np.random.default_rng(T * 31 + dk * 7 + dv)
    q, k, v, x, S0 = case(rng, 2, T, dk, dv, s0=s0, infs=True)
    o, ST = oracle.forward_pc(q, k, v, x, S0, gate=gate)
    o2, ST2 = oracle.closed_form_pc(q, k, v, x, S0, gate=gate)
    assert rel(o, o2) <= 1e-12 and rel(ST, ST2) <= 1e-12


@pytest.mark.parametrize("gate", ["bounded", "neg_softplus"])
def test_shared_decay_is_the_scalar_recurrence(gate):
    rng = np.random.default_rng(2)
    q, k, v, x, S0 = case(rng, 3, 150, 8, 5)
    xs = x[..., 0].copy()
    xb = np.repeat(xs[..., None], 8, axis=-1)
    o, ST = oracle.forward_pc(q, k, v, xb, S0, gate=gate)
    o2, ST2 = oracle.forward(q, k, v, xs, S0, gate=gate)
    assert rel(o, o2) <= 1e-13 and rel(ST, ST2) <= 1e-13


def test_unit_decay_is_causal_linear_attention():
    rng = np.random.default_rng(4)
    q, k, v, _, S0 = case(rng, 1, 33, 5, 4)
    x = np.full((1, 33, 5), -np.inf, dtype=np.float32)
    o, ST = oracle.forward_pc(q, k, v, x, S0, gate="bounded")
    Q, K, V, S = (a[0].astype(np.float64) for a in (q, k, v, S0))
    assert rel(o[0], np.tril(Q @ K.T) @ V + Q @ S) <= 1e-12
    assert rel(ST[0], S + K.T @ V) <= 1e-12


def test_channels_without_q_and_k_do_not_matter():
    rng = np.random.default_rng(6)
    q, k, v, x, _ = case(rng, 2, 90, 6, 3, s0=False)
    q[..., 3:] = 0.0
    k[..., 3:] = 0.0
    o1, ST1 = oracle.forward_pc(q, k, v, x, None)
    x2 = x.copy()
    x2[..., 3:] = rng.standard_normal(x2[..., 3:].shape).astype(np.float32) * 4
    o2, ST2 = oracle.forward_pc(q, k, v, x2, None)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(ST1[:, :3], ST2[:, :3])
    # and they do matter when k is nonzero there
    k[..., 3:] = 1.0
    q[..., 3:] = 1.0
    assert rel(oracle.forward_pc(q, k, v, x, None)[0], oracle.forward_pc(q, k, v, x2, None)[0]) > 1e-3


@pytest.mark.parametrize("split", [1, 37, 64, 99])
def test_chaining(split):
    rng = np.random.default_rng(8)
    q, k, v, x, S0 = case(rng, 2, 100, 4, 6)
    o, ST = oracle.forward_pc(q, k, v, x, S0)
    oa, Sa = oracle.forward_pc(q[:, :split], k[:, :split], v[:, :split], x[:, :split], S0)
    ob, Sb = oracle.forward_pc(q[:, split:], k[:, split:], v[:, split:], x[:, split:], Sa)
    assert rel(np.concatenate([oa, ob], axis=1), o) <= 1e-13 and rel(Sb, ST) <= 1e-13


def test_single_token():
    rng = np.random.default_rng(10)
    q, k, v, x, S0 = case(rng, 1, 1, 5, 3)
    o, ST = oracle.forward_pc(q, k, v, x, S0, gate="bounded")
    a = np.exp(-5.0 / (1.0 + np.exp(-x[0, 0].astype(np.float64))))
    S1 = a[:, None] * S0[0] + np.outer(k[0, 0].astype(np.float64), v[0, 0].astype(np.float64))
    assert rel(ST[0], S1) <= 1e-14
    assert rel(o[0, 0], S1.T @ q[0, 0].astype(np.float64)) <= 1e-14


def test_empty_sequence():
    rng = np.random.default_rng(12)
    q, k, v, x, S0 = case(rng, 2, 0, 4, 4)
    o, ST = oracle.forward_pc(q, k, v, x, S0)
    assert o.shape == (2, 0, 4)
    np.testing.assert_array_equal(ST, S0)


def _pins_pass(lib_path):
    rng = np.random.default_rng(21)
    ok = True
    q, k, v, x, S0 = case(rng, 2, 40, 4, 6)
    o, ST = oracle.forward_pc(q, k, v, x, S0, lib_path=lib_path)
    o2, ST2 = oracle.closed_form_pc(q, k, v, x, S0)
    ok &= rel(o, o2) <= 1e-12 and rel(ST, ST2) <= 1e-12
    return bool(ok)


@pytest.mark.parametrize("mutant", [11, 12, 13])
def test_planted_mistakes_are_caught(mutant):
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, f"libgla_oracle_m{mutant}.so")
        oracle.build(path, mutant=mutant)
        assert not _pins_pass(path)
    assert _pins_pass(oracle.LIB_PATH)
