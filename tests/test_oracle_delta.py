"""Pins of the gated-delta-rule oracle (oracle.forward_delta) to things other than itself.

The recurrence (the gated delta rule read for the Delta-Net-style structures of
"Engineering Long-Context Training for Trillion-Parameter MoE Models: Three Key
Breakthroughs", §3.1 and §3.3, with the decay gate of §3.2):
    S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t.

* the whole sequence as one triangular solve with explicit decay products
  (oracle.closed_form_delta), which shares no step with the token loop;
* beta = 0: the state only decays;
* a = 1, beta = 1, one-hot keys: every write replaces one row of the state;
* a = 1, beta = 1, unit keys: reading with the key just written returns its value;
* chaining over a split; the single-token form;
* planted mistakes (erase term not decayed, write not scaled by beta) must fail.
"""
import os
import tempfile

import numpy as np
import pytest

import oracle

rel = oracle.max_rel_err


def case(rng, BH, T, dk, dv, s0=True, x_shift=0.0, x_scale=1.5, unit_keys=True):
    q = rng.standard_normal((BH, T, dk)).astype(np.float32)
    k = rng.standard_normal((BH, T, dk)).astype(np.float32)
    if unit_keys and dk > 0:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((BH, T, dv)).astype(np.float32)
    x = (x_shift + x_scale * rng.standard_normal((BH, T))).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (BH, T)).astype(np.float32)
    S0 = rng.standard_normal((BH, dk, dv)) if s0 else None
    return q, k, v, x, beta, S0


@pytest.mark.parametrize("gate", ["bounded", "neg_softplus"])
@pytest.mark.parametrize("T,dk,dv", [(1, 3, 2), (6, 4, 3), (33, 5, 4), (64, 8, 8), (90, 6, 5)])
@pytest.mark.parametrize("s0", [True, False])
def test_recurrence_matches_triangular_solve(gate, T, dk, dv, s0):
    rng = np.random.default_rng(T * 13 + dk + 7 * dv)
    q, k, v, x, beta, S0 = case(rng, 2, T, dk, dv, s0=s0)
    beta.reshape(-1)[::5] = 1.0
    beta.reshape(-1)[2::7] = 0.0
    x.reshape(-1)[3::9] = np.inf
    x.reshape(-1)[4::11] = -np.inf
    o, ST = oracle.forward_delta(q, k, v, x, beta, S0, gate=gate)
    o2, ST2 = oracle.closed_form_delta(q, k, v, x, beta, S0, gate=gate)
    assert rel(o, o2) <= 1e-10 and rel(ST, ST2) <= 1e-10


def test_zero_write_strength_only_decays():
    rng = np.random.default_rng(3)
    q, k, v, x, beta, S0 = case(rng, 2, 40, 4, 3)
    beta[:] = 0.0
    o, ST = oracle.forward_delta(q, k, v, x, beta, S0)
    a = np.exp(-5.0 / (1.0 + np.exp(-x.astype(np.float64))))
    D = np.cumprod(a, axis=-1)
    o_ref = D[..., None] * np.einsum("btd,bdn->btn", q.astype(np.float64), S0)
    assert rel(o, o_ref) <= 1e-13
    assert rel(ST, D[:, -1, None, None] * S0) <= 1e-13


def test_one_hot_keys_replace_rows():
    rng = np.random.default_rng(5)
    dk, dv, T = 6, 4, 10
    q, _, v, _, beta, S0 = case(rng, 1, T, dk, dv)
    rows = rng.integers(0, dk, T)
    k = np.zeros((1, T, dk), dtype=np.float32)
    k[0, np.arange(T), rows] = 1.0
    x = np.full((1, T), -np.inf, dtype=np.float32)   # a = 1
    beta[:] = 1.0
    _, ST = oracle.forward_delta(q, k, v, x, beta, S0)
    expect = S0[0].copy()
    for t in range(T):
        expect[rows[t]] = v[0, t]
    np.testing.assert_allclose(ST[0], expect, rtol=0, atol=1e-15)


def test_reading_the_key_just_written_returns_its_value():
    rng = np.random.default_rng(7)
    q, k, v, x, beta, S0 = case(rng, 2, 30, 8, 5)
    x[:] = -np.inf
    beta[:] = 1.0
    o, _ = oracle.forward_delta(k, k, v, x, beta, S0)     # q_t = k_t
    assert rel(o, v.astype(np.float64)) <= 1e-6          # k is unit length only to fp32 rounding


@pytest.mark.parametrize("split", [1, 29, 64])
def test_chaining(split):
    rng = np.random.default_rng(9)
    q, k, v, x, beta, S0 = case(rng, 2, 80, 4, 6)
    o, ST = oracle.forward_delta(q, k, v, x, beta, S0)
    sl = lambda a, lo, hi: a[:, lo:hi]
    oa, Sa = oracle.forward_delta(*(sl(a, 0, split) for a in (q, k, v, x, beta)), S0)
    ob, Sb = oracle.forward_delta(*(sl(a, split, 80) for a in (q, k, v, x, beta)), Sa)
    assert rel(np.concatenate([oa, ob], 1), o) <= 1e-13 and rel(Sb, ST) <= 1e-13


def test_single_token():
    rng = np.random.default_rng(11)
    q, k, v, x, beta, S0 = case(rng, 1, 1, 5, 3)
    o, ST = oracle.forward_delta(q, k, v, x, beta, S0)
    a = np.exp(-5.0 / (1.0 + np.exp(-float(x[0, 0]))))
    kk, vv, b = k[0, 0].astype(np.float64), v[0, 0].astype(np.float64), float(beta[0, 0])
    S1 = a * (np.eye(5) - b * np.outer(kk, kk)) @ S0[0] + b * np.outer(kk, vv)
    assert rel(ST[0], S1) <= 1e-14
    assert rel(o[0, 0], S1.T @ q[0, 0].astype(np.float64)) <= 1e-14


def test_empty_sequence():
    rng = np.random.default_rng(12)
    q, k, v, x, beta, S0 = case(rng, 2, 0, 4, 4)
    o, ST = oracle.forward_delta(q, k, v, x, beta, S0)
    assert o.shape == (2, 0, 4)
    np.testing.assert_array_equal(ST, S0)


def _pin_passes(lib_path):
    rng = np.random.default_rng(23)
    q, k, v, x, beta, S0 = case(rng, 2, 40, 4, 6)
    o, ST = oracle.forward_delta(q, k, v, x, beta, S0, lib_path=lib_path)
    o2, ST2 = oracle.closed_form_delta(q, k, v, x, beta, S0)
    return rel(o, o2) <= 1e-10 and rel(ST, ST2) <= 1e-10


@pytest.mark.parametrize("mutant", [14, 15])
def test_planted_mistakes_are_caught(mutant):
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, f"libgla_oracle_m{mutant}.so")
        oracle.build(path, mutant=mutant)
        assert not _pin_passes(path)
    assert _pin_passes(oracle.LIB_PATH)
