"""Host-side address and undefined-behaviour checks (no GPU).

The C oracle and the library's host code (argument validation, plans, workspace
carving in api.hip) are rebuilt with clang's AddressSanitizer and
UndefinedBehaviorSanitizer -- host code only: device code is compiled as usual and
never runs here -- and the CPU suites that exercise them (the ABI validation tests and
the oracle pins) run again against those builds in a child process with the
sanitizer runtime preloaded.  Any report fails the run (UBSan halts on the first
error; ASan aborts on invalid accesses).  Leak checking is off: the Python
interpreter itself keeps allocations alive at exit."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def sanitized_builds(tmp_path_factory):
    rt = asan_runtime()
    if rt is None or not os.path.exists(CLANG):
        pytest.skip("clang sanitizer runtime not available")
    d = tmp_path_factory.mktemp("sanitized")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
    # the oracle: plain C, single-threaded here (its OpenMP pragmas are ignored without -fopenmp)
    ora = str(d / "libgla_oracle_san.so")
    subprocess.run([CLANG, "-O1", "-shared", "-fPIC", "-std=c99", "-Wno-unknown-pragmas", *san,
                    os.path.join(ROOT, "oracle", "gla_oracle.c"), "-o", ora, "-lm"], check=True)
    # the HIP library with the sanitizers on its host code only (-Xarch_host before each flag)
    sys.path.insert(0, ROOT)
    from chunked_linear_attention_gla_amd import _build
    lib = str(d / "libgla_san.so")
    host = []
    for f in san:
        host += ["-Xarch_host", f]
    cmd = _build.compile_command(lib, extra=host)
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return rt, ora, lib


def test_abi_and_oracle_suites_under_asan_and_ubsan(sanitized_builds):
    rt, ora, lib = sanitized_builds
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, GLA_LIB_PATH=lib, GLA_ORACLE_LIB=ora,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    suites = ["tests/test_abi.py", "tests/test_oracle.py", "tests/test_oracle_pc.py",
              "tests/test_oracle_delta.py", "tests/test_oracle_backward.py"]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                          *suites], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1800)
    out = res.stdout[-3000:] + res.stderr[-3000:]
    assert res.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out
