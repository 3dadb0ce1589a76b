"""Seeded synthetic workloads for the bounded-decay chunked GLA forward pass.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic (no gate, no decay, no cumulative sums), so both the GPU
path and the CPU oracle may consume what it produces.

Workload recipe, shared by every named workload:
  q ~ N(0, 1) / sqrt(dk)                  (drawn in fp32, then stored)
  k ~ N(0, 1), L2-normalised per token    (normalised in fp32, then stored)
  v ~ N(0, 1)
  x ~ N(x_mean, x_std), one fp32 scalar per (batch, head, token), or per
      (batch, head, token, key channel) for the per-channel-decay workloads
  S0 ~ N(0, s0_std) fp32 when s0_std > 0, else absent (zero initial state)
  beta ~ U(0, 1) fp32 per (batch, head, token), delta-rule workloads only (drawn last)
q, k, v are stored in bf16 (round-to-nearest-even, torch's cast) or fp32; x, S0
always fp32.  N(m, s) means mean m and standard deviation s.  Draws happen in the
order q, k, v, x, S0 from one torch generator seeded with the workload's seed on
the target device, so a workload is reproducible per device.

The model-scale context lengths these sizes follow are the staged windows 8K,
64K, 256K and 1M of [LCT §2] ("Engineering Long-Context Training for
Trillion-Parameter MoE Models: Three Key Breakthroughs", §2).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    qkv_dtype: str          # "bf16" or "f32"
    x_mean: float
    x_std: float
    s0_std: float           # 0 -> no initial state
    gate: str               # "bounded" (g = -5 sigmoid(x)) or "neg_softplus"
    seed: int
    note: str = ""
    per_channel: bool = False  # x has one value per key channel: [B, H, T, dk]
    delta: bool = False        # also draw beta ~ U(0, 1) per (batch, head, token): delta-rule write strength

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "fp32_small": Workload("fp32_small", 1, 2, 256, 64, 64, "f32", 0.0, 1.0, 0.0,
                           "bounded", 1000, "fp32 path, correctness size"),
    "bf16_8k": Workload("bf16_8k", 4, 16, 8192, 128, 128, "bf16", 0.0, 1.0, 0.1,
                        "bounded", 1001, "bf16 q/k/v, fp32 x/S0/o/S_T"),
    "bf16_64k_strong": Workload("bf16_64k_strong", 1, 32, 65536, 128, 128, "bf16", 4.0, 1.0, 0.0,
                                "bounded", 1002,
                                "strong decay: g sits near the -5 bound, tile sums near -80"),
    "bf16_64k_strong_softplus": Workload("bf16_64k_strong_softplus", 1, 32, 65536, 128, 128, "bf16",
                                         -4.0, 1.0, 0.0, "neg_softplus", 1002,
                                         "ablation: g = -softplus(-x) in the same strong-decay regime"),
    "bf16_256k": Workload("bf16_256k", 1, 16, 262144, 128, 128, "bf16", 0.0, 2.0, 0.0,
                          "bounded", 1003, "long sequence; chained continuation of 65536 tokens"),
    "bf16_1m": Workload("bf16_1m", 1, 8, 1048576, 128, 128, "bf16", 0.0, 1.0, 0.0,
                        "bounded", 1004, "million-token head group"),
    "bf16_decode": Workload("bf16_decode", 64, 32, 1, 128, 128, "bf16", 0.0, 1.0, 0.0, "bounded", 1006,
                            "serving step: 64 sequences x 32 heads, one token each, fp32 state carried"),
    "bf16_varlen_256k": Workload("bf16_varlen_256k", 1, 16, 262144, 128, 128, "bf16", 0.0, 1.0, 0.0, "bounded",
                                 1007, "64 packed sequences, log-uniform length mix, 256K tokens in total"),
    "bf16_64k_delta": Workload("bf16_64k_delta", 1, 32, 65536, 128, 128, "bf16", 0.0, 1.0, 0.0, "bounded", 1008,
                               "gated delta rule: beta ~ U(0, 1) per token, unit-norm keys", delta=True),
    "bf16_64k_pc": Workload("bf16_64k_pc", 1, 32, 65536, 128, 128, "bf16", 4.0, 1.0, 0.0, "bounded", 1005,
                            "per-channel decay: x per (token, key channel), same shapes and regime",
                            per_channel=True),
}

# The 64K strong-decay workload is the one throughput is quoted on.
HEADLINE = "bf16_64k_strong"


def _dtype(name: str) -> torch.dtype:
    if name == "bf16":
        return torch.bfloat16
    if name == "f32":
        return torch.float32
    raise ValueError(name)


def make_inputs(w: Workload, device="cpu", *, T: Optional[int] = None, H: Optional[int] = None,
                B: Optional[int] = None, seed: Optional[int] = None,
                x_const: Optional[float] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Draw one seeded batch of workload ``w`` on ``device``.

    T, H, B, seed override the workload's values (smaller samples of the same
    recipe).  x_const replaces the gate pre-activation by a constant (for example
    -inf gives decay exactly 1 under the bounded gate).
    Returns dict(q, k, v, x, S0) with q/k [B,H,T,dk], v [B,H,T,dv], x [B,H,T]
    ([B,H,T,dk] for a per-channel workload), S0 [B,H,dk,dv] or None.
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    seed = w.seed if seed is None else seed
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    st = _dtype(w.qkv_dtype)
    f32 = dict(device=dev, dtype=torch.float32, generator=gen)

    q = torch.randn(B, H, T, w.dk, **f32)
    q.mul_(1.0 / math.sqrt(w.dk))
    q = q.to(st)
    k = torch.randn(B, H, T, w.dk, **f32)
    k.div_(torch.linalg.vector_norm(k, dim=-1, keepdim=True).clamp_min(1e-30))
    k = k.to(st)
    v = torch.randn(B, H, T, w.dv, **f32).to(st)
    x = torch.randn(B, H, T, *((w.dk,) if w.per_channel else ()), **f32)
    x.mul_(w.x_std).add_(w.x_mean)
    if x_const is not None:
        x.fill_(x_const)
    S0 = None
    if w.s0_std > 0:
        S0 = torch.randn(B, H, w.dk, w.dv, **f32).mul_(w.s0_std)
    out = dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), x=x.contiguous(), S0=S0)
    if w.delta:
        out["beta"] = torch.rand(B, H, T, **f32)
    return out


def varlen_lengths(n: int, total: int, seed: int, min_len: int = 1) -> list:
    """n sequence lengths summing to `total`, log-uniformly mixed (a packed batch of
    short and long documents), each at least min_len."""
    g = torch.Generator().manual_seed(seed)
    w = torch.exp(torch.rand(n, generator=g, dtype=torch.float64) * math.log(64.0))
    raw = (w / w.sum() * (total - n * min_len)).floor().long() + min_len
    raw[0] += total - int(raw.sum())
    return [int(r) for r in raw]


def make_varlen_inputs(w: Workload, lengths, device="cpu", seed: Optional[int] = None):
    """Packed sequences of the given lengths with workload w's recipe and head count:
    q, k [H, T, dk], v [H, T, dv], x [H, T] (every head holds the sequences back to back),
    cu_seqlens int64 [N + 1], S0 [N, H, dk, dv] or None; T = sum(lengths)."""
    T = int(sum(lengths))
    inp = make_inputs(w, device, B=1, T=T, seed=seed)
    inp = {k_: (None if v_ is None else v_[0]) for k_, v_ in inp.items() if k_ != "S0"}
    dev = torch.device(device)
    cu = torch.tensor([0] + list(lengths), dtype=torch.int64).cumsum(0).to(dev)
    S0 = None
    if w.s0_std > 0:
        gen = torch.Generator(device=dev).manual_seed((w.seed if seed is None else seed) + 77)
        S0 = torch.randn(len(lengths), w.H, w.dk, w.dv, device=dev, dtype=torch.float32,
                         generator=gen).mul_(w.s0_std)
    inp["cu_seqlens"] = cu
    inp["S0"] = S0
    return inp


def make_decode_inputs(w: Workload, device="cpu", seed: Optional[int] = None, B: Optional[int] = None):
    """One token per (batch, head) with workload w's recipe, plus a state S ~ N(0, 1)
    per head: q, k [B, H, dk], v [B, H, dv], x [B, H] (or [B, H, dk] per channel),
    S [B, H, dk, dv] fp32."""
    B = w.B if B is None else B
    inp = make_inputs(w, device, B=B, T=1, seed=seed)
    out = {k_: inp[k_][:, :, 0].contiguous() for k_ in ("q", "k", "v", "x")}
    dev = torch.device(device)
    gen = torch.Generator(device=dev).manual_seed((w.seed if seed is None else seed) + 99)
    out["S"] = torch.randn(B, w.H, w.dk, w.dv, device=dev, dtype=torch.float32, generator=gen)
    return out


def to_numpy_bits(t: torch.Tensor):
    """Host numpy view of a tensor for the oracle: bf16 -> uint16 bit patterns,
    fp32 -> float32 (values unchanged)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)
