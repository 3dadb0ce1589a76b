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
# the same sources with the kernels' LDS-bounds checks compiled in (see gla_debug_flags)
DEBUG_LIB = os.path.join(PKG, "libgla_debug.so")
SOURCES = ["gate_cumsum.hip", "chunk_kernels.hip", "ws_kernels.hip", "bwd_kernels.hip", "pc_kernels.hip",
           "decode.hip", "delta_kernels.hip", "bench_stream.hip", "api.hip"]
ARCH = os.environ.get("GLA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgla.so)")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # start every block that is only reached by a jump (loop heads among them) on a
    # 64-byte boundary; the padding is never executed.  Measured on the 64K-token
    # output pass: unaligned builds ran 0.545 or 0.58 ms depending on where an
    # unrelated code change left the loop heads; aligned builds run 0.545 ms
    "-mllvm", "-align-all-nofallthru-blocks=6",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def compile_command(out: str = LIB, extra=()) -> list:
    """One hipcc command that compiles every source and links libgla.so."""
    return [hipcc(), *FLAGS, "-shared", *[os.path.join(CSRC, s) for s in SOURCES], "-o", out, *extra]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature; drop that noise
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(out: str = LIB, verbose: bool = False, jobs: int = 0, defines=()) -> str:
    """Compiles each source to an object (in parallel) and links them into `out`.
    The kernels of a source are launched from that source, so no relocatable device
    code is needed.  `defines`: extra -D flags (the debug build)."""
    import concurrent.futures
    import tempfile
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    with tempfile.TemporaryDirectory(prefix="gla_build_") as tmpd:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmpd, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            cmds.append([hipcc(), *FLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj])
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            for cmd, err in zip(cmds, ex.map(_run, cmds)):
                if verbose:
                    print(" ".join(cmd), flush=True)
                    if err.strip():
                        print(err, file=sys.stderr)
        tmp = out + ".tmp"
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        _run(link)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list:
    """The release library and the debug-checked one, both in-tree."""
    import concurrent.futures
    with concurrent.futures.ThreadPoolExecutor(2) as ex:
        rel = ex.submit(build, LIB, verbose, 0)
        dbg = ex.submit(build, DEBUG_LIB, verbose, 0, ("GLA_DEBUG",))
        return [rel.result(), dbg.result()]


if __name__ == "__main__":
    print(build_all(verbose=True))
