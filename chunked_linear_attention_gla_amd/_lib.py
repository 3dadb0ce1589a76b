"""ctypes binding of libgla.so (the C ABI in include/gla.h).

Argument marshalling only: shapes and dtypes are checked so that the sizes handed
to the library describe the tensors, outputs and workspace are allocated with
torch on the inputs' device, and the call goes to torch's current stream on that
device.  Every step of the computation runs in the library's HIP kernels; there is
no fallback: without the built library every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import NamedTuple, Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# GLA_LIB_PATH selects another build of the library (the tests' host sanitizer run)
LIB_PATH = os.environ.get("GLA_LIB_PATH") or os.path.join(_PKG, "libgla.so")

GLA_BF16, GLA_F32 = 0, 1
GATES = {"bounded": 0, "bounded_sigmoid": 0, "neg_softplus": 1, "softplus": 1}
PATHS = {"unified": 0, "diag_branch": 1, "diag": 1}
STATUS = {
    0: "GLA_OK", 1: "GLA_ERR_NULL", 2: "GLA_ERR_SHAPE", 3: "GLA_ERR_DTYPE", 4: "GLA_ERR_ALIAS",
    5: "GLA_ERR_WORKSPACE", 6: "GLA_ERR_HIP", 7: "GLA_ERR_PLAN", 8: "GLA_ERR_ALIGN", 9: "GLA_ERR_ARG",
    10: "GLA_ERR_UNSUPPORTED",
}
CHUNK = 64
MAX_SEGMENTS = 64


class GLAError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")


class Plan(NamedTuple):
    segments: int
    dv_split: int


class _CPlan(ctypes.Structure):
    _fields_ = [("segments", ctypes.c_int), ("dv_split", ctypes.c_int)]


_lib = None

_vp, _i, _ll, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_size_t
_pplan = ctypes.POINTER(_CPlan)
_psz = ctypes.POINTER(ctypes.c_size_t)
_SIGS = {
    "gla_status_string": (ctypes.c_char_p, [_i]),
    "gla_abi_version": (_i, []),
    "gla_plan_default": (_i, [_i, _i, _ll, _i, _i, _i, _i, _pplan]),
    "gla_plan_check": (_i, [_i, _i, _ll, _i, _i, _i, _i, _pplan]),
    "gla_segment_workspace_size": (_i, [_i, _i, _ll, _i, _i, _pplan, _psz]),
    "gla_workspace_size": (_i, [_i, _i, _ll, _i, _i, _i, _i, _pplan, _psz]),
    "gla_gate_cumsum": (_i, [_vp, _vp, _i, _i, _ll, _i, _vp]),
    "gla_segment_states": (_i, [_vp, _vp, _vp, _i, _i, _ll, _i, _i, _i, _i, _pplan, _vp, _sz, _vp]),
    "gla_chunk_output": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _ll, _i, _i, _i, _i, _i, _pplan,
                              _vp, _sz, _vp]),
    "gla_chunk_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _ll, _i, _i, _i, _i, _i,
                           _vp, _psz, _vp]),
    "gla_chunk_fwd_plan": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _ll, _i, _i, _i, _i, _i,
                                _pplan, _vp, _psz, _vp]),
    "gla_plan_default_pc": (_i, [_i, _i, _ll, _i, _i, _i, _pplan]),
    "gla_plan_check_pc": (_i, [_i, _i, _ll, _i, _i, _i, _pplan]),
    "gla_chunk_fwd_pc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _ll, _i, _i, _i, _i, _pplan,
                              _vp, _psz, _vp]),
    "gla_decode_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "gla_chunk_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _ll, _ll, _i, _i, _i, _i, _i,
                                  _pplan, _vp, _psz, _vp]),
    "gla_plan_default_delta": (_i, [_i, _i, _ll, _i, _i, _i, _pplan]),
    "gla_plan_check_delta": (_i, [_i, _i, _ll, _i, _i, _i, _pplan]),
    "gla_chunk_fwd_delta": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _ll, _i, _i, _i, _i, _pplan, _vp,
                                 _psz, _vp]),
    "gla_chunk_fwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _ll, _i, _i, _i, _i, _i, _vp]),
    "gla_bench_stream": (_i, [_vp, _vp, _vp, _vp, ctypes.c_ulonglong, _i, _vp]),
    "gla_bench_chunk_stream": (_i, [_vp, _vp, _vp, _vp, _i, ctypes.c_longlong, _i, _vp]),
    "gla_debug_flags": (_i, [ctypes.POINTER(ctypes.c_uint)]),
    "gla_debug_selftest": (_i, [_vp, _vp, _vp]),
    "gla_lane_selftest": (_i, [_vp, _vp, _vp]),
    "gla_chunk_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _ll, _i, _i,
                           _i, _i, _i, _vp, _psz, _vp]),
}


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m chunked_linear_attention_gla_amd._build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgla.so (raises when it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _open(path)
    return _lib


DEBUG_LIB_PATH = os.path.join(_PKG, "libgla_debug.so")


@contextlib.contextmanager
def use_library(path: str = DEBUG_LIB_PATH):
    """Route every call of this binding through another build of the library (the
    LDS-checked debug build by default) inside the block; yields that library."""
    global _lib
    prev = load()
    other = _open(path)
    _lib = other
    try:
        yield other
    finally:
        _lib = prev


def debug_flags(lib: Optional[ctypes.CDLL] = None) -> int:
    """Read and clear the LDS-check flags of a debug build (gla_debug_flags); raises
    GLAError (GLA_ERR_UNSUPPORTED) on a release build."""
    v = ctypes.c_uint(0)
    _check("gla_debug_flags", (lib or load()).gla_debug_flags(ctypes.byref(v)))
    return int(v.value)


def lane_selftest(values: torch.Tensor) -> torch.Tensor:
    """Run gla_lane_selftest on 64 fp32 values on a GPU; returns the 17 x 64 slots (see
    include/gla.h) as a tensor on the same device."""
    _need(values.is_cuda and values.dtype == torch.float32 and values.numel() == 64 and values.is_contiguous(),
          "values must be 64 contiguous fp32 values on a GPU")
    out = torch.empty(17, 64, device=values.device, dtype=torch.float32)
    _check("gla_lane_selftest", load().gla_lane_selftest(_ptr(values), _ptr(out), _stream(values.device)))
    return out


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise GLAError(fn, code)


def _cplan(plan: Optional[Plan]):
    return None if plan is None else ctypes.byref(_CPlan(int(plan.segments), int(plan.dv_split)))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GLA_BF16
    if t.dtype == torch.float32:
        return GLA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _gate(gate) -> int:
    return GATES[gate] if isinstance(gate, str) else int(gate)


def _path(path) -> int:
    return PATHS[path] if isinstance(path, str) else int(path)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_qkv(q, k, v, x=None, S0=None):
    _need(q.dim() == 4 and k.shape == q.shape, "q and k must be [B, H, T, dk] of one shape")
    B, H, T, dk = q.shape
    _need(v.dim() == 4 and tuple(v.shape[:3]) == (B, H, T), "v must be [B, H, T, dv]")
    dv = v.shape[3]
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous GPU tensor")
        _need(t.device == q.device, "all tensors must be on one device")
    if x is not None:
        _need(tuple(x.shape) == (B, H, T) and x.dtype == torch.float32 and x.is_cuda and x.is_contiguous()
              and x.device == q.device, "x must be a contiguous fp32 [B, H, T] tensor on q's device")
    if S0 is not None:
        _need(tuple(S0.shape) == (B, H, dk, dv) and S0.dtype == torch.float32 and S0.is_cuda
              and S0.is_contiguous() and S0.device == q.device,
              "S0 must be a contiguous fp32 [B, H, dk, dv] tensor on q's device")
    return B, H, T, dk, dv


# ------------------------------------------------------------------------------------ queries

def abi_version() -> int:
    return int(load().gla_abi_version())


def status_string(code: int) -> str:
    return load().gla_status_string(code).decode()


def plan_default(B: int, H: int, T: int, dk: int, dv: int, dtype=GLA_BF16, path="unified") -> Plan:
    cp = _CPlan()
    _check("gla_plan_default", load().gla_plan_default(B, H, T, dk, dv, dtype, _path(path), ctypes.byref(cp)))
    return Plan(cp.segments, cp.dv_split)


def plan_check(B: int, H: int, T: int, dk: int, dv: int, plan: Plan, dtype=GLA_BF16, path="unified") -> int:
    """Status code of gla_plan_check (0 = valid)."""
    return int(load().gla_plan_check(B, H, T, dk, dv, dtype, _path(path), _cplan(plan)))


def workspace_size(B: int, H: int, T: int, dk: int, dv: int, dtype=GLA_BF16, path="unified",
                   plan: Optional[Plan] = None) -> int:
    n = ctypes.c_size_t(0)
    _check("gla_workspace_size", load().gla_workspace_size(B, H, T, dk, dv, dtype, _path(path), _cplan(plan),
                                                           ctypes.byref(n)))
    return int(n.value)


def backward_workspace_size(B: int, H: int, T: int, dk: int, dv: int, dtype=GLA_BF16, gate="bounded",
                            path="unified") -> int:
    """Workspace bytes gla_chunk_bwd needs for these sizes (default plans of this device)."""
    n = ctypes.c_size_t(0)
    _check("gla_chunk_bwd", load().gla_chunk_bwd(None, None, None, None, None, None, None, None, None, None, None,
                                                 None, B, H, T, dk, dv, dtype, _gate(gate), _path(path), None,
                                                 ctypes.byref(n), None))
    return int(n.value)


def segment_workspace_size(B: int, H: int, T: int, dk: int, dv: int, plan: Plan) -> int:
    n = ctypes.c_size_t(0)
    _check("gla_segment_workspace_size",
           load().gla_segment_workspace_size(B, H, T, dk, dv, _cplan(plan), ctypes.byref(n)))
    return int(n.value)


# ------------------------------------------------------------------------------------ calls

def gate_cumsum(x: torch.Tensor, gate="bounded", out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Chunk-local cumulative log-decay b (fp32, same shape as x = [B, H, T])."""
    _need(x.dim() == 3 and x.dtype == torch.float32 and x.is_cuda and x.is_contiguous(),
          "x must be a contiguous fp32 [B, H, T] GPU tensor")
    B, H, T = x.shape
    if out is None:
        out = torch.empty_like(x)
    _need(out.shape == x.shape and out.dtype == torch.float32 and out.is_contiguous() and out.device == x.device,
          "out must match x")
    _check("gla_gate_cumsum", load().gla_gate_cumsum(_ptr(x), _ptr(out), B, H, T, _gate(gate), _stream(x.device)))
    return out


def segment_states(k: torch.Tensor, v: torch.Tensor, x: torch.Tensor, plan: Plan, seg_ws: torch.Tensor,
                   gate="bounded") -> None:
    """Segment pre-pass into seg_ws (uint8 tensor of segment_workspace_size bytes); x is the
    fp32 [B, H, T] gate pre-activation."""
    B, H, T, dk, dv = _check_qkv(k, k, v, x)
    _check("gla_segment_states", load().gla_segment_states(
        _ptr(k), _ptr(v), _ptr(x), B, H, T, dk, dv, _dtype_code(k), _gate(gate), _cplan(plan), _ptr(seg_ws),
        seg_ws.numel() * seg_ws.element_size(), _stream(k.device)))


def chunk_output(q, k, v, x, S0, plan: Plan, seg_ws: Optional[torch.Tensor], o: torch.Tensor,
                 S_T: torch.Tensor, gate="bounded", path="unified") -> None:
    """Fused output pass (o and S_T written in place); x is the fp32 [B, H, T] gate
    pre-activation."""
    B, H, T, dk, dv = _check_qkv(q, k, v, x, S0)
    _need(tuple(o.shape) == (B, H, T, dv) and o.dtype == torch.float32 and o.is_contiguous(), "o must be fp32 [B,H,T,dv]")
    _need(tuple(S_T.shape) == (B, H, dk, dv) and S_T.dtype == torch.float32 and S_T.is_contiguous(),
          "S_T must be fp32 [B,H,dk,dv]")
    nbytes = 0 if seg_ws is None else seg_ws.numel() * seg_ws.element_size()
    _check("gla_chunk_output", load().gla_chunk_output(
        _ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(S0), _ptr(o), _ptr(S_T), B, H, T, dk, dv, _dtype_code(q),
        _gate(gate), _path(path), _cplan(plan), _ptr(seg_ws), nbytes, _stream(q.device)))


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, x: torch.Tensor,
              S0: Optional[torch.Tensor] = None, gate="bounded", path="unified", plan: Optional[Plan] = None,
              o: Optional[torch.Tensor] = None, S_T: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunked gated-linear-attention forward: returns (o [B,H,T,dv] fp32, S_T [B,H,dk,dv] fp32).

    q, k: [B, H, T, dk] and v: [B, H, T, dv], all bfloat16 or all float32; x: [B, H, T] fp32 gate
    pre-activation; S0: [B, H, dk, dv] fp32 or None.  gate: "bounded" (g = -5 sigmoid(x)) or
    "neg_softplus"; path: "unified" or "diag_branch"; plan: None for the device default.
    """
    B, H, T, dk, dv = _check_qkv(q, k, v, x, S0)
    dev = q.device
    lib = load()
    dt = _dtype_code(q)
    if o is None:
        o = torch.empty(B, H, T, dv, device=dev, dtype=torch.float32)
    if S_T is None:
        S_T = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32)
    _need(tuple(o.shape) == (B, H, T, dv) and o.dtype == torch.float32 and o.is_contiguous() and o.device == dev,
          "o must be fp32 [B, H, T, dv] on q's device")
    _need(tuple(S_T.shape) == (B, H, dk, dv) and S_T.dtype == torch.float32 and S_T.is_contiguous()
          and S_T.device == dev, "S_T must be fp32 [B, H, dk, dv] on q's device")
    need = ctypes.c_size_t(0)
    cplan = _cplan(plan)
    _check("gla_chunk_fwd_plan", lib.gla_chunk_fwd_plan(
        _ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(S0), _ptr(o), _ptr(S_T), B, H, T, dk, dv, dt, _gate(gate),
        _path(path), cplan, None, ctypes.byref(need), _stream(dev)))
    if workspace is None or workspace.numel() * workspace.element_size() < need.value:
        workspace = torch.empty(max(int(need.value), 256), dtype=torch.uint8, device=dev)
    have = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    _check("gla_chunk_fwd_plan", lib.gla_chunk_fwd_plan(
        _ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(S0), _ptr(o), _ptr(S_T), B, H, T, dk, dv, dt, _gate(gate),
        _path(path), cplan, _ptr(workspace), ctypes.byref(have), _stream(dev)))
    return o, S_T


def plan_default_pc(B: int, H: int, T: int, dk: int, dv: int, dtype=GLA_BF16) -> Plan:
    cp = _CPlan()
    _check("gla_plan_default_pc", load().gla_plan_default_pc(B, H, T, dk, dv, dtype, ctypes.byref(cp)))
    return Plan(cp.segments, cp.dv_split)


def plan_default_delta(B: int, H: int, T: int, dk: int, dv: int, dtype=GLA_BF16) -> Plan:
    cp = _CPlan()
    _check("gla_plan_default_delta", load().gla_plan_default_delta(B, H, T, dk, dv, dtype, ctypes.byref(cp)))
    return Plan(cp.segments, cp.dv_split)


def plan_check_pc(B: int, H: int, T: int, dk: int, dv: int, plan: Plan, dtype=GLA_BF16) -> int:
    """Status code of gla_plan_check_pc (0 = valid)."""
    return int(load().gla_plan_check_pc(B, H, T, dk, dv, dtype, _cplan(plan)))


def chunk_fwd_pc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, x: torch.Tensor,
                 S0: Optional[torch.Tensor] = None, gate="bounded", plan: Optional[Plan] = None,
                 o: Optional[torch.Tensor] = None, S_T: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-channel-decay forward: returns (o [B,H,T,dv] fp32, S_T [B,H,dk,dv] fp32).

    As :func:`chunk_fwd`, except x: [B, H, T, dk] fp32, one gate pre-activation per key
    channel (row d of the state decays by exp(g(x[..., t, d]))).
    """
    B, H, T, dk, dv = _check_qkv(q, k, v, None, S0)
    dev = q.device
    _need(tuple(x.shape) == (B, H, T, dk) and x.dtype == torch.float32 and x.is_cuda and x.is_contiguous()
          and x.device == dev, "x must be a contiguous fp32 [B, H, T, dk] tensor on q's device")
    lib = load()
    dt = _dtype_code(q)
    if o is None:
        o = torch.empty(B, H, T, dv, device=dev, dtype=torch.float32)
    if S_T is None:
        S_T = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32)
    _need(tuple(o.shape) == (B, H, T, dv) and o.dtype == torch.float32 and o.is_contiguous() and o.device == dev,
          "o must be fp32 [B, H, T, dv] on q's device")
    _need(tuple(S_T.shape) == (B, H, dk, dv) and S_T.dtype == torch.float32 and S_T.is_contiguous()
          and S_T.device == dev, "S_T must be fp32 [B, H, dk, dv] on q's device")
    cplan = _cplan(plan)
    args = lambda ws: (_ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(S0), _ptr(o), _ptr(S_T), B, H, T, dk, dv, dt,
                       _gate(gate), cplan, ws)
    need = ctypes.c_size_t(0)
    _check("gla_chunk_fwd_pc", lib.gla_chunk_fwd_pc(*args(None), ctypes.byref(need), _stream(dev)))
    if workspace is None or workspace.numel() * workspace.element_size() < need.value:
        workspace = torch.empty(max(int(need.value), 256), dtype=torch.uint8, device=dev)
    have = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    _check("gla_chunk_fwd_pc", lib.gla_chunk_fwd_pc(*args(_ptr(workspace)), ctypes.byref(have), _stream(dev)))
    return o, S_T


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, x: torch.Tensor, S: torch.Tensor,
                gate="bounded", o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One recurrent step per head: S <- diag(a) S + k v^T (in place), returns o = S^T q.

    q, k: [B, H, dk], v: [B, H, dv] (bfloat16 or float32); x: fp32 [B, H] (one decay per head)
    or [B, H, dk] (one per key channel); S: fp32 [B, H, dk, dv], updated in place.
    """
    _need(q.dim() == 3 and k.shape == q.shape and v.dim() == 3 and v.shape[:2] == q.shape[:2],
          "q, k must be [B, H, dk] and v [B, H, dv]")
    B, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    for t in (q, k, v, x, S):
        _need(t.is_cuda and t.is_contiguous() and t.device == dev, "tensors must be contiguous on q's device")
    per_channel = x.dim() == 3
    _need(x.dtype == torch.float32 and tuple(x.shape) in ((B, H), (B, H, dk)), "x must be fp32 [B, H] or [B, H, dk]")
    _need(S.dtype == torch.float32 and tuple(S.shape) == (B, H, dk, dv), "S must be fp32 [B, H, dk, dv]")
    if o is None:
        o = torch.empty(B, H, dv, device=dev, dtype=torch.float32)
    _need(tuple(o.shape) == (B, H, dv) and o.dtype == torch.float32 and o.is_contiguous() and o.device == dev,
          "o must be fp32 [B, H, dv] on q's device")
    _check("gla_decode_step", load().gla_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(S), _ptr(o), B, H, dk,
                                                     dv, _dtype_code(q), _gate(gate), int(per_channel),
                                                     _stream(dev)))
    return o


def chunk_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, x: torch.Tensor, cu_seqlens: torch.Tensor,
                     max_seqlen: int, S0: Optional[torch.Tensor] = None, gate="bounded", path="unified",
                     plan: Optional[Plan] = None, o: Optional[torch.Tensor] = None, S_T: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward over packed sequences: returns (o [H, T, dv] fp32, S_T [N, H, dk, dv] fp32).

    q, k: [H, T, dk], v: [H, T, dv], x: fp32 [H, T] -- every head holds the N sequences back
    to back; cu_seqlens: int64 [N + 1] offsets on the device (sequence n is rows
    cu_seqlens[n]:cu_seqlens[n+1]); max_seqlen: the longest sequence (host int);
    S0: fp32 [N, H, dk, dv] or None; plan: (segments per sequence, dv_split) or None for the
    default.  Rows covered by no sequence are left unwritten in o.
    """
    _need(q.dim() == 3 and k.shape == q.shape and v.dim() == 3 and v.shape[:2] == q.shape[:2],
          "q, k must be [H, T, dk] and v [H, T, dv]")
    H, T, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    for t in (q, k, v, x, cu_seqlens):
        _need(t.is_cuda and t.is_contiguous() and t.device == dev, "tensors must be contiguous on q's device")
    _need(x.dtype == torch.float32 and tuple(x.shape) == (H, T), "x must be fp32 [H, T]")
    _need(cu_seqlens.dtype == torch.int64 and cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 2,
          "cu_seqlens must be int64 [N + 1]")
    N = cu_seqlens.numel() - 1
    if S0 is not None:
        _need(tuple(S0.shape) == (N, H, dk, dv) and S0.dtype == torch.float32 and S0.is_contiguous()
              and S0.device == dev, "S0 must be fp32 [N, H, dk, dv] on q's device")
    if o is None:
        o = torch.zeros(H, T, dv, device=dev, dtype=torch.float32)
    if S_T is None:
        S_T = torch.empty(N, H, dk, dv, device=dev, dtype=torch.float32)
    _need(tuple(o.shape) == (H, T, dv) and o.dtype == torch.float32 and o.is_contiguous() and o.device == dev,
          "o must be fp32 [H, T, dv] on q's device")
    _need(tuple(S_T.shape) == (N, H, dk, dv) and S_T.dtype == torch.float32 and S_T.is_contiguous()
          and S_T.device == dev, "S_T must be fp32 [N, H, dk, dv] on q's device")
    lib = load()
    cplan = _cplan(plan)
    args = lambda ws: (_ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(S0), _ptr(o), _ptr(S_T), _ptr(cu_seqlens), N, H,
                       T, int(max_seqlen), dk, dv, _dtype_code(q), _gate(gate), _path(path), cplan, ws)
    need = ctypes.c_size_t(0)
    _check("gla_chunk_fwd_varlen", lib.gla_chunk_fwd_varlen(*args(None), ctypes.byref(need), _stream(dev)))
    if workspace is None or workspace.numel() * workspace.element_size() < need.value:
        workspace = torch.empty(max(int(need.value), 256), dtype=torch.uint8, device=dev)
    have = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    _check("gla_chunk_fwd_varlen", lib.gla_chunk_fwd_varlen(*args(_ptr(workspace)), ctypes.byref(have),
                                                            _stream(dev)))
    return o, S_T


def chunk_fwd_delta(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, x: torch.Tensor, beta: torch.Tensor,
                    S0: Optional[torch.Tensor] = None, gate="bounded", plan: Optional[Plan] = None,
                    o: Optional[torch.Tensor] = None, S_T: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Gated delta rule forward: returns (o [B,H,T,dv] fp32, S_T [B,H,dk,dv] fp32) for
    S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t.

    As :func:`chunk_fwd`, plus beta: fp32 [B, H, T] write strengths; plan: (segments,
    dv_split) or None for the device default.
    """
    B, H, T, dk, dv = _check_qkv(q, k, v, x, S0)
    dev = q.device
    _need(tuple(beta.shape) == (B, H, T) and beta.dtype == torch.float32 and beta.is_cuda and beta.is_contiguous()
          and beta.device == dev, "beta must be a contiguous fp32 [B, H, T] tensor on q's device")
    if o is None:
        o = torch.empty(B, H, T, dv, device=dev, dtype=torch.float32)
    if S_T is None:
        S_T = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32)
    _need(tuple(o.shape) == (B, H, T, dv) and o.dtype == torch.float32 and o.is_contiguous() and o.device == dev,
          "o must be fp32 [B, H, T, dv] on q's device")
    _need(tuple(S_T.shape) == (B, H, dk, dv) and S_T.dtype == torch.float32 and S_T.is_contiguous()
          and S_T.device == dev, "S_T must be fp32 [B, H, dk, dv] on q's device")
    lib = load()
    cplan = _cplan(plan)
    args = lambda ws: (_ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T), B, H, T, dk,
                       dv, _dtype_code(q), _gate(gate), cplan, ws)
    need = ctypes.c_size_t(0)
    _check("gla_chunk_fwd_delta", lib.gla_chunk_fwd_delta(*args(None), ctypes.byref(need), _stream(dev)))
    if workspace is None or workspace.numel() * workspace.element_size() < need.value:
        workspace = torch.empty(max(int(need.value), 256), dtype=torch.uint8, device=dev)
    have = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    _check("gla_chunk_fwd_delta", lib.gla_chunk_fwd_delta(*args(_ptr(workspace)), ctypes.byref(have), _stream(dev)))
    return o, S_T


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, x: torch.Tensor, dO: torch.Tensor,
              S0: Optional[torch.Tensor] = None, dS_T: Optional[torch.Tensor] = None, gate="bounded",
              path="unified", workspace: Optional[torch.Tensor] = None, out=None):
    """Backward of :func:`chunk_fwd`: returns (dq, dk [B,H,T,dk], dv [B,H,T,dv], dx [B,H,T],
    dS0 [B,H,dk,dv]), all fp32, for a loss L with dL/do = dO and dL/dS_T = dS_T.

    dO: [B, H, T, dv] in q's dtype (the operand precision); dS_T: fp32 [B, H, dk, dv] or None.
    out: optional tuple of five preallocated output tensors of those shapes.
    """
    B, H, T, dk, dv = _check_qkv(q, k, v, x, S0)
    dev = q.device
    _need(tuple(dO.shape) == (B, H, T, dv) and dO.dtype == q.dtype and dO.is_cuda and dO.is_contiguous()
          and dO.device == dev, "dO must be a contiguous [B, H, T, dv] tensor of q's dtype on q's device")
    if dS_T is not None:
        _need(tuple(dS_T.shape) == (B, H, dk, dv) and dS_T.dtype == torch.float32 and dS_T.is_contiguous()
              and dS_T.device == dev, "dS_T must be a contiguous fp32 [B, H, dk, dv] tensor on q's device")
    lib = load()
    dt = _dtype_code(q)
    f32 = dict(device=dev, dtype=torch.float32)
    shapes = ((B, H, T, dk), (B, H, T, dk), (B, H, T, dv), (B, H, T), (B, H, dk, dv))
    if out is None:
        out = tuple(torch.empty(*sh, **f32) for sh in shapes)
    else:
        _need(len(out) == 5 and all(tuple(t.shape) == sh and t.dtype == torch.float32 and t.is_contiguous()
                                    and t.device == dev for t, sh in zip(out, shapes)),
              "out must be five contiguous fp32 tensors (dq, dk, dv, dx, dS0) on q's device")
    dq, dk_, dv_, dx, dS0 = out
    args = lambda ws: (_ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(S0), _ptr(dO), _ptr(dS_T), _ptr(dq), _ptr(dk_),
                       _ptr(dv_), _ptr(dx), _ptr(dS0), B, H, T, dk, dv, dt, _gate(gate), _path(path), ws)
    need = ctypes.c_size_t(0)
    _check("gla_chunk_bwd", lib.gla_chunk_bwd(*args(None), ctypes.byref(need), _stream(dev)))
    if workspace is None or workspace.numel() * workspace.element_size() < need.value:
        workspace = torch.empty(max(int(need.value), 256), dtype=torch.uint8, device=dev)
    have = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    _check("gla_chunk_bwd", lib.gla_chunk_bwd(*args(_ptr(workspace)), ctypes.byref(have), _stream(dev)))
    return dq, dk_, dv_, dx, dS0


def bench_stream(a: torch.Tensor, b: torch.Tensor, c: torch.Tensor, out: torch.Tensor, grid: int = 8192) -> None:
    """Measurement helper: the forward's byte mix as one flat stream (gla_bench_stream).
    a, b, c: tensors of n bytes (n a multiple of 16); out: 2n bytes; all on one GPU."""
    nb = a.numel() * a.element_size()
    _need(nb % 16 == 0 and all(t.numel() * t.element_size() == nb for t in (b, c)), "a, b, c must have n bytes")
    _need(out.numel() * out.element_size() == 2 * nb, "out must have 2n bytes")
    for t in (a, b, c, out):
        _need(t.is_cuda and t.is_contiguous() and t.device == a.device, "tensors must be contiguous on one GPU")
    _check("gla_bench_stream", load().gla_bench_stream(_ptr(a), _ptr(b), _ptr(c), _ptr(out), nb // 16, grid,
                                                       _stream(a.device)))


def bench_chunk_stream(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, BH: int, T: int,
                       segments: int) -> None:
    """Measurement helper: the output pass's access pattern without its arithmetic
    (gla_bench_chunk_stream).  q, k, v: BH * T * 256 bytes each; o: BH * T * 512 bytes;
    all contiguous on one GPU."""
    nb = BH * T * 256
    _need(all(t.numel() * t.element_size() >= nb for t in (q, k, v)), "q, k, v must hold BH * T * 256 bytes")
    _need(o.numel() * o.element_size() >= 2 * nb, "o must hold BH * T * 512 bytes")
    for t in (q, k, v, o):
        _need(t.is_cuda and t.is_contiguous() and t.device == q.device, "tensors must be contiguous on one GPU")
    _check("gla_bench_chunk_stream", load().gla_bench_chunk_stream(_ptr(q), _ptr(k), _ptr(v), _ptr(o), BH, T,
                                                                   segments, _stream(q.device)))
