"""fp64 CPU oracle for the chunked gated-linear-attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU product path
(``chunked_linear_attention_gla_amd``) never imports, links or calls it, and the
two share no code: no kernels, headers, helpers, constants or pre/post-processing.

Sources (web pages; cited by title and section):
  [LCT] "Engineering Long-Context Training for Trillion-Parameter MoE Models:
         Three Key Breakthroughs"
  [STM] "Scaling Trillion-Parameter MoE and Long-Context LLMs: Architecture and
         Engineering in Practice"
  [ESU] "Engineering Stability in Ultra-Long Context and Trillion-Parameter
         Sparse Models"

Independent formulations of the forward pass live here, and the backward
pass of the recurrence:

* :func:`forward` -- the sequential recurrence, one token at a time, in C (fp64,
  OpenMP over heads and value-column blocks).  This is the oracle proper.
* :func:`closed_form` -- the quadratic form, numpy fp64, with every decay weight
  formed as an explicit product of per-token decays (no cumulative sums, no
  exponent differences).  Used to pin :func:`forward` on tiny inputs.
* :func:`forward_pc` / :func:`closed_form_pc` -- the same two formulations for a
  decay with one value per key channel (the state's row d decays by a_t[d]).
* :func:`forward_delta` / :func:`closed_form_delta` -- the gated delta rule, token by
  token and as one triangular solve over the sequence.
* :func:`backward` -- the reverse-mode chain rule of the same recurrence, one token
  at a time, in C (fp64): dq, dk, dv, dx and dS0 from dO and dS_T.
* :func:`gate` / :func:`chunk_local_cumsum` -- the log-decay of [LCT §3.2] and the
  chunk-local inclusive cumulative sum of it, the per-position cumulative decay
  Gamma of [LCT §3.1] in log form, restarted at each chunk.

The recurrence (the plainest reading of [LCT §3.1] / [ESU §2.1]; the pages do not
write it out):  S_t = a_t S_{t-1} + k_t v_t^T,  o_t = S_t^T q_t,  a_t = exp(g(x_t)).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
# GLA_ORACLE_LIB points the tests at another build of the same source (the host
# sanitizer run builds one with clang's address and undefined-behaviour checks)
LIB_PATH = os.environ.get("GLA_ORACLE_LIB") or os.path.join(_HERE, "libgla_oracle.so")

GATE_BOUNDED_SIGMOID = 0  # g = -5 * sigmoid(x)          [LCT §3.2] improved form
GATE_NEG_SOFTPLUS = 1     # g = -softplus(-x) = log sigmoid(x)  conventional, unbounded
_GATES = {"bounded": GATE_BOUNDED_SIGMOID, "bounded_sigmoid": GATE_BOUNDED_SIGMOID,
          "neg_softplus": GATE_NEG_SOFTPLUS, "softplus": GATE_NEG_SOFTPLUS}


def gate_id(gate) -> int:
    if isinstance(gate, str):
        return _GATES[gate]
    if gate in (GATE_BOUNDED_SIGMOID, GATE_NEG_SOFTPLUS):
        return int(gate)
    raise ValueError(f"unknown gate {gate!r}")


def compile_command(out_path: str = LIB_PATH, mutant: int = 0) -> list:
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", _SRC, "-o", out_path, "-lm"]
    if mutant:
        cmd.insert(1, f"-DGLA_ORACLE_MUTANT={int(mutant)}")
    return cmd


def build(out_path: str = LIB_PATH, mutant: int = 0) -> str:
    """Compile the C oracle (gcc, OpenMP).  ``mutant`` plants a known mistake (tests only)."""
    subprocess.run(compile_command(out_path, mutant), check=True)
    return out_path


_lib_cache = {}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        if path != LIB_PATH:
            raise FileNotFoundError(path)
        build(path)
    lib = ctypes.CDLL(path)
    lib.gla_oracle_forward.restype = ctypes.c_int
    lib.gla_oracle_forward.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_longlong, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int]
    lib.gla_oracle_forward_pc.restype = ctypes.c_int
    lib.gla_oracle_forward_pc.argtypes = lib.gla_oracle_forward.argtypes
    lib.gla_oracle_forward_delta.restype = ctypes.c_int
    lib.gla_oracle_forward_delta.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_longlong, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int]
    lib.gla_oracle_backward.restype = ctypes.c_int
    lib.gla_oracle_backward.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_longlong, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.gla_oracle_gate.restype = ctypes.c_double
    lib.gla_oracle_gate.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.gla_oracle_max_threads.restype = ctypes.c_int
    lib.gla_oracle_max_threads.argtypes = []
    _lib_cache[path] = lib
    return lib


def max_threads() -> int:
    return int(load().gla_oracle_max_threads())


def _qkv_kind(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 1  # bf16 bit patterns
    if a.dtype == np.float32:
        return 0
    raise TypeError(f"q/k/v must be uint16 (bf16 bits) or float32, got {a.dtype}")


def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, x: np.ndarray,
            S0: Optional[np.ndarray] = None, gate="bounded", nthreads: int = 0,
            col_block: int = 16, lib_path: str = LIB_PATH) -> Tuple[np.ndarray, np.ndarray]:
    """Sequential fp64 recurrence (the oracle proper).

    q, k: [..., T, dk]; v: [..., T, dv]; all three uint16 (bf16 bits) or float32 and
    of the same kind.  x: [..., T] float32.  S0: [..., dk, dv] float32 or float64, or None
    (zero state).  Leading dims are flattened into independent heads.
    Returns (o [..., T, dv], S_T [..., dk, dv]) as float64.
    """
    kind = _qkv_kind(q)
    if _qkv_kind(k) != kind or _qkv_kind(v) != kind:
        raise TypeError("q, k, v must share a storage kind")
    lead = q.shape[:-2]
    T, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1] or x.shape != lead + (T,):
        raise ValueError("shape mismatch")
    BH = int(np.prod(lead)) if lead else 1
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if S0 is not None:
        S0 = np.ascontiguousarray(S0, dtype=np.float64)  # fp32 widens exactly
        if S0.shape != lead + (dk, dv):
            raise ValueError("S0 shape mismatch")
    o = np.empty(lead + (T, dv), dtype=np.float64)
    ST = np.empty(lead + (dk, dv), dtype=np.float64)
    lib = load(lib_path)
    rc = lib.gla_oracle_forward(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, kind,
        x.ctypes.data, None if S0 is None else S0.ctypes.data,
        o.ctypes.data, ST.ctypes.data, BH, T, dk, dv, gate_id(gate), col_block, nthreads)
    if rc != 0:
        raise ValueError(f"gla_oracle_forward rejected its arguments (rc={rc})")
    return o, ST


def forward_pc(q: np.ndarray, k: np.ndarray, v: np.ndarray, x: np.ndarray,
               S0: Optional[np.ndarray] = None, gate="bounded", nthreads: int = 0,
               col_block: int = 16, lib_path: str = LIB_PATH):
    """Per-channel-decay recurrence (fp64, one token at a time, in C):

        S_t[d, :] = a_t[d] S_{t-1}[d, :] + k_t[d] v_t,  a_t[d] = exp(g(x_t[d])),  o_t = S_t^T q_t

    q, k [..., T, dk], v [..., T, dv] as for :func:`forward`; x [..., T, dk] fp32.
    Returns (o [..., T, dv], S_T [..., dk, dv]) in float64.
    """
    kind = _qkv_kind(q)
    if _qkv_kind(k) != kind or _qkv_kind(v) != kind:
        raise TypeError("q, k, v must share a storage kind")
    lead = q.shape[:-2]
    T, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1] or x.shape != q.shape:
        raise ValueError("shape mismatch")
    BH = int(np.prod(lead)) if lead else 1
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    x = np.ascontiguousarray(x, dtype=np.float32)
    if S0 is not None:
        S0 = np.ascontiguousarray(S0, dtype=np.float64)
        if S0.shape != lead + (dk, dv):
            raise ValueError("S0 shape mismatch")
    o = np.empty(lead + (T, dv))
    ST = np.empty(lead + (dk, dv))
    rc = load(lib_path).gla_oracle_forward_pc(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, kind, x.ctypes.data,
        None if S0 is None else S0.ctypes.data, o.ctypes.data, ST.ctypes.data,
        BH, T, dk, dv, gate_id(gate), col_block, nthreads)
    if rc != 0:
        raise ValueError(f"gla_oracle_forward_pc rejected its arguments (rc={rc})")
    return o, ST


def forward_delta(q: np.ndarray, k: np.ndarray, v: np.ndarray, x: np.ndarray, beta: np.ndarray,
                  S0: Optional[np.ndarray] = None, gate="bounded", nthreads: int = 0,
                  col_block: int = 16, lib_path: str = LIB_PATH):
    """Gated delta rule, one token at a time (fp64, in C):

        S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t,  a_t = exp(g(x_t))

    q, k [..., T, dk], v [..., T, dv] as for :func:`forward`; x, beta [..., T] fp32.
    Returns (o [..., T, dv], S_T [..., dk, dv]) in float64.
    """
    kind = _qkv_kind(q)
    if _qkv_kind(k) != kind or _qkv_kind(v) != kind:
        raise TypeError("q, k, v must share a storage kind")
    lead = q.shape[:-2]
    T, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1] or x.shape != lead + (T,) or beta.shape != x.shape:
        raise ValueError("shape mismatch")
    BH = int(np.prod(lead)) if lead else 1
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    x = np.ascontiguousarray(x, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    if S0 is not None:
        S0 = np.ascontiguousarray(S0, dtype=np.float64)
        if S0.shape != lead + (dk, dv):
            raise ValueError("S0 shape mismatch")
    o = np.empty(lead + (T, dv))
    ST = np.empty(lead + (dk, dv))
    rc = load(lib_path).gla_oracle_forward_delta(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, kind, x.ctypes.data, beta.ctypes.data,
        None if S0 is None else S0.ctypes.data, o.ctypes.data, ST.ctypes.data,
        BH, T, dk, dv, gate_id(gate), col_block, nthreads)
    if rc != 0:
        raise ValueError(f"gla_oracle_forward_delta rejected its arguments (rc={rc})")
    return o, ST


def backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, x: np.ndarray, dO: np.ndarray,
             S0: Optional[np.ndarray] = None, dST: Optional[np.ndarray] = None, gate="bounded",
             nthreads: int = 0, lib_path: str = LIB_PATH):
    """Reverse-mode gradients of the recurrence (fp64, one token at a time, in C).

    Inputs as for :func:`forward`, plus dO = dL/do [..., T, dv] and dST = dL/dS_T
    [..., dk, dv] (None: zero), any float dtype (widened to float64).
    Returns (dq, dk [..., T, dk], dv [..., T, dv], dx [..., T], dS0 [..., dk, dv]),
    all float64, with L the scalar whose partials dO and dST are.
    """
    kind = _qkv_kind(q)
    if _qkv_kind(k) != kind or _qkv_kind(v) != kind:
        raise TypeError("q, k, v must share a storage kind")
    lead = q.shape[:-2]
    T, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1] or x.shape != lead + (T,) \
            or dO.shape != lead + (T, dv):
        raise ValueError("shape mismatch")
    BH = int(np.prod(lead)) if lead else 1
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    x = np.ascontiguousarray(x, dtype=np.float32)
    dO = np.ascontiguousarray(dO, dtype=np.float64)
    if S0 is not None:
        S0 = np.ascontiguousarray(S0, dtype=np.float64)
    if dST is not None:
        dST = np.ascontiguousarray(dST, dtype=np.float64)
    for a in (S0, dST):
        if a is not None and a.shape != lead + (dk, dv):
            raise ValueError("state shape mismatch")
    dq = np.empty(lead + (T, dk))
    dk_ = np.empty(lead + (T, dk))
    dv_ = np.empty(lead + (T, dv))
    dx = np.empty(lead + (T,))
    dS0 = np.empty(lead + (dk, dv))
    lib = load(lib_path)
    rc = lib.gla_oracle_backward(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, kind, x.ctypes.data,
        None if S0 is None else S0.ctypes.data, dO.ctypes.data, None if dST is None else dST.ctypes.data,
        dq.ctypes.data, dk_.ctypes.data, dv_.ctypes.data, dx.ctypes.data, dS0.ctypes.data,
        BH, T, dk, dv, gate_id(gate), nthreads)
    if rc != 0:
        raise ValueError(f"gla_oracle_backward failed (rc={rc})")
    return dq, dk_, dv_, dx, dS0


# --------------------------------------------------------------------------- numpy parts

def _sigmoid(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def gate(x, gate="bounded") -> np.ndarray:
    """Log-decay g(x) in fp64 [LCT §3.2].

    bounded:      g = g_min * sigmoid(x), g_min = -5, range (-5, 0) for finite x
    neg_softplus: g = -softplus(-x) = log(sigmoid(x)), range (-inf, 0)
    """
    x = np.asarray(x, dtype=np.float64)
    if gate_id(gate) == GATE_BOUNDED_SIGMOID:
        return -5.0 * _sigmoid(x)
    z = -x
    return -(np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z))))


def chunk_local_cumsum(g: np.ndarray, chunk: int = 64) -> np.ndarray:
    """b[t] = sum of g over the tokens of t's chunk up to and including t (fp64).

    This is log Gamma restarted at each chunk boundary [LCT §3.1]; T must be a
    multiple of ``chunk``.
    """
    g = np.asarray(g, dtype=np.float64)
    T = g.shape[-1]
    if T % chunk:
        raise ValueError("T must be a multiple of the chunk length")
    gc = g.reshape(g.shape[:-1] + (T // chunk, chunk))
    return np.cumsum(gc, axis=-1).reshape(g.shape)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _widen(a: np.ndarray) -> np.ndarray:
    return widen_bf16(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float64)


def decay_weights(a: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """From per-token decays a[T] form, by explicit products,
    W[t, s] = prod_{s < i <= t} a_i  for s <= t (0 above the diagonal), and
    D[t]    = prod_{i <= t} a_i     (the weight of the initial state in o_t).
    """
    T = a.shape[0]
    W = np.zeros((T, T), dtype=np.float64)
    D = np.empty(T, dtype=np.float64)
    for t in range(T):
        W[t, t] = 1.0
        acc = 1.0
        for s in range(t - 1, -1, -1):
            acc *= a[s + 1]
            W[t, s] = acc
        D[t] = acc * a[0]
    return W, D


def closed_form(q, k, v, x, S0=None, gate="bounded") -> Tuple[np.ndarray, np.ndarray]:
    """Quadratic closed form, fp64, one head at a time (tiny inputs only):

        o_t = D_t * S0^T q_t + sum_{s <= t} W[t, s] (q_t . k_s) v_s
        S_T = D_{T-1} * S0   + sum_s W[T-1, s] k_s v_s^T

    with W and D the explicit decay products of :func:`decay_weights`.
    """
    q = _widen(np.asarray(q))
    k = _widen(np.asarray(k))
    v = _widen(np.asarray(v))
    x = np.asarray(x, dtype=np.float64)
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    qf, kf, vf, xf = (q.reshape(BH, T, dk), k.reshape(BH, T, dk), v.reshape(BH, T, dv),
                      x.reshape(BH, T))
    S0f = None if S0 is None else np.asarray(S0, dtype=np.float64).reshape(BH, dk, dv)
    o = np.zeros((BH, T, dv))
    ST = np.zeros((BH, dk, dv))
    for h in range(BH):
        a = np.exp(gate_fn(xf[h], gate))
        if T == 0:
            ST[h] = 0.0 if S0f is None else S0f[h]
            continue
        W, D = decay_weights(a)
        scores = qf[h] @ kf[h].T                       # [t, s] = q_t . k_s
        o[h] = (W * scores) @ vf[h]
        ST[h] = kf[h].T @ (W[T - 1][:, None] * vf[h])
        if S0f is not None:
            o[h] += D[:, None] * (qf[h] @ S0f[h])
            ST[h] += D[T - 1] * S0f[h]
    return o.reshape(lead + (T, dv)), ST.reshape(lead + (dk, dv))


gate_fn = gate


def closed_form_delta(q, k, v, x, beta, S0=None, gate="bounded") -> Tuple[np.ndarray, np.ndarray]:
    """The gated delta rule over a whole (tiny) sequence as one triangular solve, fp64.

    Writing S_t = a_t S_{t-1} + k_t u_t^T with the effective write
    u_t = beta_t (v_t - a_t S_{t-1}^T k_t), every u_t is linear in the earlier ones:
        (I + diag(beta) L) U = diag(beta) (V - diag(D) K S0),
        L[t, s] = W[t, s] (k_t . k_s) for s < t,
    with W, D the explicit decay products of :func:`decay_weights`; then
        o_t = D_t S0^T q_t + sum_{s <= t} W[t, s] (q_t . k_s) u_s,
        S_T = D_{T-1} S0 + sum_s W[T-1, s] k_s u_s^T.
    Solved with numpy.linalg.solve; no token loop over the state.
    """
    q = _widen(np.asarray(q))
    k = _widen(np.asarray(k))
    v = _widen(np.asarray(v))
    x = np.asarray(x, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    qf, kf, vf = q.reshape(BH, T, dk), k.reshape(BH, T, dk), v.reshape(BH, T, dv)
    xf, bf = x.reshape(BH, T), beta.reshape(BH, T)
    S0f = np.zeros((BH, dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64).reshape(BH, dk, dv)
    o = np.zeros((BH, T, dv))
    ST = np.zeros((BH, dk, dv))
    for h in range(BH):
        if T == 0:
            ST[h] = S0f[h]
            continue
        W, D = decay_weights(np.exp(gate_fn(xf[h], gate)))
        L = np.tril(W * (kf[h] @ kf[h].T), -1)
        rhs = bf[h][:, None] * (vf[h] - D[:, None] * (kf[h] @ S0f[h]))
        U = np.linalg.solve(np.eye(T) + bf[h][:, None] * L, rhs)
        o[h] = D[:, None] * (qf[h] @ S0f[h]) + (W * (qf[h] @ kf[h].T)) @ U
        ST[h] = D[T - 1] * S0f[h] + kf[h].T @ (W[T - 1][:, None] * U)
    return o.reshape(lead + (T, dv)), ST.reshape(lead + (dk, dv))


def closed_form_pc(q, k, v, x, S0=None, gate="bounded") -> Tuple[np.ndarray, np.ndarray]:
    """Quadratic closed form of the per-channel recurrence, fp64 (tiny inputs only):

        o_t[n] = sum_d q_t[d] (D_t[d] S0[d, n] + sum_{s <= t} W_d[t, s] k_s[d] v_s[n])
        S_T    = diag(D_{T-1}) S0 + sum_s diag(W[T-1, s]) k_s v_s^T

    with W_d, D_d the explicit decay products of :func:`decay_weights` for channel d.
    """
    q = _widen(np.asarray(q))
    k = _widen(np.asarray(k))
    v = _widen(np.asarray(v))
    x = np.asarray(x, dtype=np.float64)
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    qf, kf, vf, xf = (q.reshape(BH, T, dk), k.reshape(BH, T, dk), v.reshape(BH, T, dv),
                      x.reshape(BH, T, dk))
    S0f = None if S0 is None else np.asarray(S0, dtype=np.float64).reshape(BH, dk, dv)
    o = np.zeros((BH, T, dv))
    ST = np.zeros((BH, dk, dv))
    for h in range(BH):
        if T == 0:
            ST[h] = 0.0 if S0f is None else S0f[h]
            continue
        W = np.empty((dk, T, T))
        D = np.empty((dk, T))
        for d in range(dk):
            W[d], D[d] = decay_weights(np.exp(gate_fn(xf[h, :, d], gate)))
        scores = np.einsum("td,dts,sd->ts", qf[h], W, kf[h])   # sum_d q_t[d] W_d[t,s] k_s[d]
        o[h] = scores @ vf[h]
        ST[h] = (W[:, T - 1, :] * kf[h].T) @ vf[h]             # [d, n] = sum_s W_d[T-1,s] k_s[d] v_s[n]
        if S0f is not None:
            o[h] += (qf[h] * D.T) @ S0f[h]
            ST[h] += D[:, T - 1][:, None] * S0f[h]
    return o.reshape(lead + (T, dv)), ST.reshape(lead + (dk, dv))


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| over the whole tensor (0 when both are all-zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    diff = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if scale == 0.0:
        return diff
    return diff / scale
