"""Helpers shared by the GPU parity tests: run the HIP path and the CPU oracle on the
same seeded inputs and compare them."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from chunked_linear_attention_gla_amd import inputs as gin

# Tolerances of the comparison, max |gpu - ref| / max |ref| over each whole tensor:
# 2e-2 for bf16 operands and 1e-4 for the fp32 path, on o and on the final state.
TOL = {"bf16": 2e-2, "f32": 1e-4}

# One call over a sequence vs the same sequence split into chained calls (S_T of
# one call is S0 of the next).  Both hand over an fp32 state at a chunk boundary,
# but the plans differ, so the state is summed in a different order.
# o: the q.S product rounds that state to bf16, where an fp32 difference of ~1e-7 can
#   move one element by one bf16 ulp (2^-8 relative); one element of a 128-term dot
#   product then moves o by at most ~2^-8 / sqrt(128) ~ 4e-4 of its scale.
CHAIN_TOL = 2e-3
# S_T of the scalar and per-channel paths: the carried state stays fp32 end to end
# and the bf16 operands of every state update (k e^{gamma-b}, v) are the same in both
# computations (chunk boundaries coincide), so the two differ only in the order of
# fp32 sums: a few fp32 ulps (1.2e-7 each) of the state's scale.
CHAIN_TOL_STATE = 1e-5
# S_T of the gated delta rule: the carried state enters the effective writes
# U = U~ - W S through a bf16 product, so S_T inherits the bf16 rounding of the
# handed-over state exactly as o does (same bound as CHAIN_TOL).
CHAIN_TOL_DELTA = 2e-3


def device():
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def oracle_heads(inp, heads=None, gate="bounded", T=None, S0=None):
    """fp64 oracle on flat head indices `heads` (default all) and the first T tokens."""
    q, k, v, x = inp["q"], inp["k"], inp["v"], inp["x"]
    B, H, Tfull, dk = q.shape
    dv = v.shape[-1]
    T = Tfull if T is None else T
    idx = list(range(B * H)) if heads is None else list(heads)
    sel = lambda t: t.reshape(B * H, *t.shape[2:])[idx]
    s0 = inp["S0"] if S0 is None else S0
    s0n = None if s0 is None else sel(s0).detach().cpu().numpy().astype(np.float64)
    o, ST = oracle.forward(gin.to_numpy_bits(sel(q)[:, :T]), gin.to_numpy_bits(sel(k)[:, :T]),
                           gin.to_numpy_bits(sel(v)[:, :T]), gin.to_numpy_bits(sel(x)[:, :T]),
                           s0n, gate=gate)
    return o, ST


def gpu_heads(t, heads, T=None):
    B, H = t.shape[:2]
    flat = t.reshape(B * H, *t.shape[2:])[list(heads)]
    if T is not None:
        flat = flat[:, :T]
    return flat.detach().cpu().double().numpy()


def rel(got, ref):
    return oracle.max_rel_err(got, ref)


def gpu_rel(got: torch.Tensor, ref: torch.Tensor) -> float:
    """max |got - ref| / max |ref| computed on the device, one head slice at a time."""
    g = got.reshape(-1, *got.shape[-2:])
    r = ref.reshape(-1, *ref.shape[-2:])
    scale = max(r[i].abs().max().item() for i in range(r.shape[0]))
    diff = max((g[i] - r[i]).abs().max().item() for i in range(g.shape[0]))
    return diff / scale if scale else diff
