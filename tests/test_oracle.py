"""Pins for the CPU oracle, against what the pages and the mathematics fix.

The oracle (oracle.forward, a sequential fp64 recurrence in C) is checked against:
  * the quadratic closed form with decay weights as explicit products (numpy);
  * decay exactly 1 -> plain causal linear attention (numpy matmul);
  * decay exactly e^-5 -> a Toeplitz closed form;
  * a single token, and a three-token example whose values are written out by hand;
  * chaining, linearity in (v, S0), independence of value columns;
  * the gate's printed constants and ranges ("Engineering Long-Context Training for
    Trillion-Parameter MoE Models: Three Key Breakthroughs", §3.2);
and the numpy closed form is checked against the same special cases, so neither
side is only checked against itself.  test_planted_mistakes_are_caught builds
variants of the C oracle with known mistakes and checks that these pins fail.
"""
import json
import math
import os
import tempfile
import zlib

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
FLT_MAX = float(np.finfo(np.float32).max)
FLT_MIN_NORMAL = float(np.finfo(np.float32).tiny)


def rand_case(rng, BH, T, dk, dv, s0=True, kind="f32", x_scale=2.0, x_shift=0.0):
    q = rng.standard_normal((BH, T, dk)).astype(np.float32)
    k = rng.standard_normal((BH, T, dk)).astype(np.float32)
    v = rng.standard_normal((BH, T, dv)).astype(np.float32)
    x = (x_shift + x_scale * rng.standard_normal((BH, T))).astype(np.float32)
    S0 = rng.standard_normal((BH, dk, dv)).astype(np.float32) if s0 else None
    if kind == "bf16":
        # round-to-nearest-even fp32 -> bf16 bit patterns, written out here in the test
        def to_bf16(a):
            u = a.view(np.uint32).astype(np.uint64)
            r = ((u >> 16) & 1) + 0x7FFF
            return ((u + r) >> 16).astype(np.uint16)
        q, k, v = to_bf16(q), to_bf16(k), to_bf16(v)
    return q, k, v, x, S0


def rel(a, b):
    return oracle.max_rel_err(a, b)


# ----------------------------------------------------------------------------- gate

def test_page_constants_fixture():
    with open(os.path.join(HERE, "golden", "page_constants.json")) as f:
        g = json.load(f)
    assert g["g_min"] == -5.0 and g["safe_tile_tokens"] == 16
    # printed lower bound: the bounded gate tends to g_min as x -> +inf, to 0 as x -> -inf
    assert oracle.gate(np.inf, "bounded") == g["g_min"]
    assert oracle.gate(-np.inf, "bounded") == 0.0
    lib = oracle.load()
    assert lib.gla_oracle_gate(math.inf, 0) == g["g_min"]
    assert lib.gla_oracle_gate(-math.inf, 0) == 0.0


def test_bounded_gate_values_and_range():
    lib = oracle.load()
    assert oracle.gate(0.0, "bounded") == -2.5          # -5 * 1/2
    assert lib.gla_oracle_gate(0.0, 0) == -2.5
    xs = np.linspace(-30, 30, 2001)
    g = oracle.gate(xs, "bounded")
    assert np.all(g > -5.0) and np.all(g < 0.0)         # open range (g_min, 0) for finite x
    # sigmoid(x) + sigmoid(-x) = 1  =>  g(x) + g(-x) = g_min
    np.testing.assert_allclose(g + g[::-1], -5.0, rtol=0, atol=1e-13)
    # monotone decreasing
    assert np.all(np.diff(g) < 0)
    # C and numpy implementations agree
    for xv in [-50.0, -3.0, -1e-3, 0.5, 7.0, 80.0]:
        assert abs(lib.gla_oracle_gate(xv, 0) - float(oracle.gate(xv, "bounded"))) <= 1e-15
        ref = -5.0 / (1.0 + math.exp(-xv)) if xv > -700 else 0.0
        assert abs(float(oracle.gate(xv, "bounded")) - ref) <= 1e-14


def test_softplus_gate_values():
    lib = oracle.load()
    assert abs(float(oracle.gate(0.0, "neg_softplus")) + math.log(2.0)) < 1e-15
    for xv in [-20.0, -4.0, -0.3, 0.0, 1.7, 6.0, 30.0]:
        ref = math.log(1.0 / (1.0 + math.exp(-xv)))    # log sigmoid(x)
        assert abs(float(oracle.gate(xv, "neg_softplus")) - ref) <= 1e-13 * max(1.0, abs(ref))
        assert abs(lib.gla_oracle_gate(xv, 1) - ref) <= 1e-13 * max(1.0, abs(ref))
    # unbounded below: behaves like x for very negative x
    assert abs(float(oracle.gate(-1e6, "neg_softplus")) + 1e6) < 1e-6
    assert float(oracle.gate(np.inf, "neg_softplus")) == 0.0
    assert float(oracle.gate(-np.inf, "neg_softplus")) == -np.inf


def test_sixteen_token_tile_stays_in_fp32_range():
    """[LCT §3.2]: with g >= -5 the reciprocal decay over any 16-token tile stays
    representable.  16 * 5 = 80 and e^80 < FLT_MAX, e^-80 > smallest normal fp32;
    a 32-token tile (e^160) would not be."""
    rng = np.random.default_rng(0)
    x = rng.normal(4.0, 1.0, size=(64, 16))             # strong-decay regime
    tile_sums = oracle.gate(x, "bounded").sum(axis=1)
    assert np.all(tile_sums > -80.0)
    assert math.exp(80.0) < FLT_MAX and math.exp(-80.0) > FLT_MIN_NORMAL
    assert math.exp(160.0) > FLT_MAX
    # the unbounded gate breaks it: x = -6 gives g ~ -6.0025, tile sum ~ -96.04
    s = 16 * float(oracle.gate(-6.0, "neg_softplus"))
    assert s < -96.0 and math.exp(-s) > FLT_MAX


def test_chunk_local_cumsum_definition():
    g = np.arange(1, 129, dtype=np.float64) * -0.01
    b = oracle.chunk_local_cumsum(g, 64)
    for c in range(2):
        acc = 0.0
        for j in range(64):
            acc += g[64 * c + j]
            assert b[64 * c + j] == pytest.approx(acc, abs=1e-15)
    gc = np.full(128, -2.0)
    np.testing.assert_array_equal(oracle.chunk_local_cumsum(gc)[:64], -2.0 * np.arange(1, 65))
    with pytest.raises(ValueError):
        oracle.chunk_local_cumsum(np.zeros(65))


# ----------------------------------------------------------------------------- recurrence

@pytest.mark.parametrize("gate", ["bounded", "neg_softplus"])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (2, 7, 4, 8), (1, 64, 8, 4), (3, 65, 5, 3), (1, 33, 16, 16)])
@pytest.mark.parametrize("s0", [False, True])
def test_recurrence_matches_closed_form(gate, shape, s0):
    BH, T, dk, dv = shape
    rng = np.random.default_rng(zlib.crc32(repr((gate, shape, s0)).encode()))
    q, k, v, x, S0 = rand_case(rng, BH, T, dk, dv, s0=s0)
    if T > 3:
        x[0, 1] = np.inf
        x[-1, 2] = -np.inf
    o, ST = oracle.forward(q, k, v, x, S0, gate=gate)
    o2, ST2 = oracle.closed_form(q, k, v, x, S0, gate=gate)
    assert rel(o, o2) <= 1e-12
    assert rel(ST, ST2) <= 1e-12


def test_recurrence_matches_closed_form_bf16_storage():
    rng = np.random.default_rng(5)
    q, k, v, x, S0 = rand_case(rng, 2, 40, 8, 8, kind="bf16")
    o, ST = oracle.forward(q, k, v, x, S0)
    o2, ST2 = oracle.closed_form(q, k, v, x, S0)
    assert rel(o, o2) <= 1e-12 and rel(ST, ST2) <= 1e-12


@pytest.mark.parametrize("gate,xval", [("bounded", -np.inf), ("neg_softplus", np.inf)])
def test_unit_decay_is_causal_linear_attention(gate, xval):
    """a_t = 1: o = tril(Q K^T) V + Q S0,  S_T = S0 + K^T V."""
    rng = np.random.default_rng(11)
    q, k, v, _, S0 = rand_case(rng, 2, 50, 6, 5)
    x = np.full((2, 50), xval, dtype=np.float32)
    Q, K, V, S = (a.astype(np.float64) for a in (q, k, v, S0))
    o_ref = np.tril(Q @ K.transpose(0, 2, 1)) @ V + Q @ S
    ST_ref = S + K.transpose(0, 2, 1) @ V
    o, ST = oracle.forward(q, k, v, x, S0, gate=gate)
    o2, ST2 = oracle.closed_form(q, k, v, x, S0, gate=gate)
    for got_o, got_s in ((o, ST), (o2, ST2)):
        assert rel(got_o, o_ref) <= 1e-12 and rel(got_s, ST_ref) <= 1e-12


def test_min_decay_is_toeplitz():
    """x = +inf under the bounded gate: a_t = e^-5 exactly, so the weight of s in t is
    e^{-5 (t - s)} and the initial state is weighted e^{-5 (t + 1)}."""
    rng = np.random.default_rng(12)
    T = 20
    q, k, v, _, S0 = rand_case(rng, 1, T, 3, 4)
    x = np.full((1, T), np.inf, dtype=np.float32)
    Q, K, V, S = q[0].astype(np.float64), k[0].astype(np.float64), v[0].astype(np.float64), S0[0].astype(np.float64)
    t = np.arange(T)
    D = np.where(t[:, None] >= t[None, :], np.exp(-5.0 * (t[:, None] - t[None, :])), 0.0)
    o_ref = ((Q @ K.T) * D) @ V + np.exp(-5.0 * (t + 1))[:, None] * (Q @ S)
    ST_ref = math.exp(-5.0 * T) * S + K.T @ (np.exp(-5.0 * (T - 1 - t))[:, None] * V)
    o, ST = oracle.forward(q, k, v, x, S0)
    o2, ST2 = oracle.closed_form(q, k, v, x, S0)
    for got_o, got_s in ((o[0], ST[0]), (o2[0], ST2[0])):
        assert rel(got_o, o_ref) <= 1e-12 and rel(got_s, ST_ref) <= 1e-12


def test_single_token():
    """T = 1: o_0 = e^{g_0} S0^T q_0 + (q_0 . k_0) v_0 and S_T = e^{g_0} S0 + k_0 v_0^T."""
    rng = np.random.default_rng(13)
    q, k, v, x, S0 = rand_case(rng, 1, 1, 4, 3)
    a = math.exp(-5.0 / (1.0 + math.exp(-float(x[0, 0]))))
    Q, K, V, S = q[0, 0].astype(np.float64), k[0, 0].astype(np.float64), v[0, 0].astype(np.float64), S0[0].astype(np.float64)
    o_ref = a * (S.T @ Q) + float(Q @ K) * V
    ST_ref = a * S + np.outer(K, V)
    o, ST = oracle.forward(q, k, v, x, S0)
    o2, ST2 = oracle.closed_form(q, k, v, x, S0)
    for got_o, got_s in ((o[0, 0], ST[0]), (o2[0, 0], ST2[0])):
        np.testing.assert_allclose(got_o, o_ref, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(got_s, ST_ref, rtol=1e-13, atol=1e-13)


def test_three_token_hand_example():
    """dk = dv = 1, x = 0 (a = e^-2.5), S0 = 0.5, q = (1, 2, 3), k = (1, 1, 2), v = (1, -1, 0.5).
    By hand:  S_0 = 0.5a + 1,  S_1 = a S_0 - 1,  S_2 = a S_1 + 1,  o_t = q_t S_t."""
    a = math.exp(-2.5)
    S_0 = 0.5 * a + 1.0
    S_1 = 0.5 * a * a + a - 1.0
    S_2 = 0.5 * a ** 3 + a * a - a + 1.0
    o_ref = np.array([S_0, 2.0 * S_1, 3.0 * S_2])
    q = np.array([[[1.0], [2.0], [3.0]]], dtype=np.float32)
    k = np.array([[[1.0], [1.0], [2.0]]], dtype=np.float32)
    v = np.array([[[1.0], [-1.0], [0.5]]], dtype=np.float32)
    x = np.zeros((1, 3), dtype=np.float32)
    S0 = np.array([[[0.5]]], dtype=np.float32)
    for fn in (oracle.forward, oracle.closed_form):
        o, ST = fn(q, k, v, x, S0)
        np.testing.assert_allclose(o[0, :, 0], o_ref, rtol=1e-14, atol=1e-15)
        assert ST[0, 0, 0] == pytest.approx(S_2, rel=1e-14)


@pytest.mark.parametrize("split", [1, 37, 64, 99])
def test_chaining(split):
    rng = np.random.default_rng(14)
    q, k, v, x, S0 = rand_case(rng, 2, 100, 8, 6, x_shift=-3.0)
    o, ST = oracle.forward(q, k, v, x, S0)
    oa, Sa = oracle.forward(q[:, :split], k[:, :split], v[:, :split], x[:, :split], S0)
    ob, Sb = oracle.forward(q[:, split:], k[:, split:], v[:, split:], x[:, split:], Sa)
    assert rel(np.concatenate([oa, ob], axis=1), o) <= 1e-13
    assert rel(Sb, ST) <= 1e-13


def test_linearity_and_column_separability():
    rng = np.random.default_rng(15)
    q, k, v, x, S0 = rand_case(rng, 1, 30, 5, 4)
    o, ST = oracle.forward(q, k, v, x, S0)
    # o and S_T are jointly linear in (v, S0)
    o2, ST2 = oracle.forward(q, k, (2.0 * v).astype(np.float32), x, 2.0 * S0)
    assert rel(o2, 2.0 * o) <= 1e-14 and rel(ST2, 2.0 * ST) <= 1e-14
    # o is linear in q; S_T does not depend on q
    o3, ST3 = oracle.forward((-4.0 * q).astype(np.float32), k, v, x, S0)  # exact in fp32
    assert rel(o3, -4.0 * o) <= 1e-14
    np.testing.assert_array_equal(ST3, ST)
    # column j of o and S_T depends only on column j of v and S0 (one-hot tests)
    for j in range(4):
        vj = np.zeros_like(v)
        vj[..., j] = v[..., j]
        Sj = np.zeros_like(S0)
        Sj[..., j] = S0[..., j]
        oj, STj = oracle.forward(q, k, vj, x, Sj)
        np.testing.assert_allclose(oj[..., j], o[..., j], rtol=1e-13, atol=1e-13)
        assert np.all(np.delete(oj, j, axis=-1) == 0.0)
        np.testing.assert_allclose(STj[..., j], ST[..., j], rtol=1e-13, atol=1e-13)


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(16)
    q, k, v, x, S0 = rand_case(rng, 2, 0, 3, 2)
    o, ST = oracle.forward(q, k, v, x, S0)
    assert o.shape == (2, 0, 2)
    np.testing.assert_array_equal(ST, S0.astype(np.float64))


def test_threads_and_column_blocks_do_not_change_result():
    rng = np.random.default_rng(17)
    q, k, v, x, S0 = rand_case(rng, 3, 70, 8, 20)
    o1, S1 = oracle.forward(q, k, v, x, S0, nthreads=1, col_block=20)
    o2, S2 = oracle.forward(q, k, v, x, S0, nthreads=4, col_block=3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


# ----------------------------------------------------------------------------- pin sensitivity

def _pins_pass(lib_path):
    """Run the core pins against an oracle build; True when all hold."""
    rng = np.random.default_rng(21)
    ok = True
    for gate in ("bounded", "neg_softplus"):
        q, k, v, x, S0 = rand_case(rng, 2, 9, 4, 3)
        o, ST = oracle.forward(q, k, v, x, S0, gate=gate, lib_path=lib_path)
        o2, ST2 = oracle.closed_form(q, k, v, x, S0, gate=gate)
        ok &= rel(o, o2) <= 1e-12 and rel(ST, ST2) <= 1e-12
    return bool(ok)


@pytest.mark.parametrize("mutant", [1, 2, 3, 4, 5, 6])
def test_planted_mistakes_are_caught(mutant):
    """Each planted mistake (token t dropped from o_t; decay applied to the new outer
    product; q/k roles swapped; gate sign flipped; decay index shifted; initial state
    not decayed) must make the closed-form pin fail."""
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, f"libgla_oracle_m{mutant}.so")
        oracle.build(path, mutant=mutant)
        assert not _pins_pass(path)
    assert _pins_pass(oracle.LIB_PATH)
