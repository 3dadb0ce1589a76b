"""Compile the HIP sources of this package into libgla.so (gfx950).

Run as ``python -m chunked_linear_attention_gla_amd._build``.  The library is
built in-tree, next to this file, so it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgla.so")
SOURCES = ["gate_cumsum.hip", "chunk_kernels.hip", "ws_kernels.hip", "bwd_kernels.hip", "pc_kernels.hip",
           "decode.hip", "delta_kernels.hip", "api.hip"]
ARCH = os.environ.get("GLA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgla.so)")


def compile_command(out: str = LIB, extra=()) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep hipcc from forming packed fp32 arithmetic (v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # start every block that is only reached by a jump (loop heads among them) on a
        # 64-byte boundary; the padding is never executed.  Measured on the 64K-token
        # output pass: unaligned builds ran 0.545 or 0.58 ms depending on where an
        # unrelated code change left the loop heads; aligned builds run 0.545 ms
        "-mllvm", "-align-all-nofallthru-blocks=6",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out, *extra,
    ]


def build(out: str = LIB, verbose: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature; drop that noise
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
