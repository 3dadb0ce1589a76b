"""C-ABI checks that need no GPU: the library loads, exports every entry point that
include/gla.h declares, and rejects bad arguments on the host before enqueueing
anything.  Pointers passed here are never dereferenced: every call below fails
validation (or only queries sizes) before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gla.h")

gla = pytest.importorskip("chunked_linear_attention_gla_amd")
from chunked_linear_attention_gla_amd import _lib  # noqa: E402

OK, NULL, SHAPE, DTYPE, ALIAS, WORKSPACE, HIP, PLAN, ALIGN, ARG, UNSUP = range(11)
BF16, F32 = 0, 1
BOUNDED, SOFTPLUS = 0, 1
UNIFIED, DIAG = 0, 1


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gla_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_forward_call():
    names = declared_functions()
    assert "gla_chunk_fwd" in names and "gla_gate_cumsum" in names and "gla_chunk_output" in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_debug_build_exports_the_same_entry_points():
    """The LDS-checked debug build is built beside the release library and exports
    every declared entry point too."""
    path = _lib.DEBUG_LIB_PATH
    assert os.path.exists(path), "libgla_debug.so is built by __graft_entry__.build()"
    dbg = ctypes.CDLL(path)
    missing = [n for n in declared_functions() if not hasattr(dbg, n)]
    assert not missing, missing


def test_debug_entry_points_on_the_release_build(lib):
    """The release build compiles the checks away: both debug calls say so, after
    rejecting NULL pointers, without any device call."""
    v = ctypes.c_uint(7)
    assert lib.gla_debug_flags(None) == NULL
    assert lib.gla_debug_flags(ctypes.byref(v)) == UNSUP and v.value == 7
    dummy = ctypes.c_void_p(16)
    assert lib.gla_debug_selftest(None, dummy, None) == NULL
    assert lib.gla_debug_selftest(dummy, dummy, None) == UNSUP


def test_lane_selftest_rejects_null_pointers(lib):
    dummy = ctypes.c_void_p(16)
    assert lib.gla_lane_selftest(None, dummy, None) == NULL
    assert lib.gla_lane_selftest(dummy, None, None) == NULL


def test_version_and_status_strings(lib):
    assert lib.gla_abi_version() == 2
    for code in range(11):
        s = lib.gla_status_string(code).decode()
        assert s.startswith("GLA_")
    assert "unknown" in lib.gla_status_string(99).decode()


def P(segments, dv_split):
    return ctypes.byref(_lib._CPlan(segments, dv_split))


def fwd(lib, q=0x1000, k=0x100000, v=0x200000, x=0x300000, S0=None, o=0x400000, ST=0x500000,
        B=1, H=2, T=256, dk=64, dv=64, dtype=BF16, gate=BOUNDED, path=UNIFIED, plan=(1, 1),
        ws=None, wsz=0):
    n = ctypes.c_size_t(wsz)
    pl = None if plan is None else P(*plan)
    rc = lib.gla_chunk_fwd_plan(q, k, v, x, S0, o, ST, B, H, T, dk, dv, dtype, gate, path, pl, ws,
                                ctypes.byref(n), None)
    return rc, n.value


def test_workspace_query_with_explicit_plan(lib):
    rc, n = fwd(lib, B=2, H=3, T=1000, dk=128, dv=128, plan=(4, 2))
    assert rc == OK
    bh = 6
    # the kernels form the cumulative log-decays from x: the workspace is the segment workspace
    seg = (bh * 3 * 128 * 128 * 4 + 255) // 256 * 256 + (bh * 4 * 4 + 255) // 256 * 256
    assert n == seg
    n2 = ctypes.c_size_t(0)
    assert lib.gla_workspace_size(2, 3, 1000, 128, 128, BF16, UNIFIED, P(4, 2), ctypes.byref(n2)) == OK
    assert n2.value == n
    n3 = ctypes.c_size_t(0)
    assert lib.gla_segment_workspace_size(2, 3, 1000, 128, 128, P(4, 2), ctypes.byref(n3)) == OK
    assert n3.value == seg
    assert lib.gla_segment_workspace_size(2, 3, 1000, 128, 128, P(1, 2), ctypes.byref(n3)) == OK
    assert n3.value == 0


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), SHAPE), (dict(H=-1), SHAPE), (dict(T=-5), SHAPE),
    (dict(dk=32), SHAPE), (dict(dk=96), SHAPE), (dict(dv=256), SHAPE), (dict(dv=48), SHAPE),
    (dict(dtype=7), DTYPE), (dict(gate=3), ARG), (dict(path=5), ARG),
    (dict(plan=(0, 1)), PLAN), (dict(plan=(65, 1)), PLAN), (dict(plan=(5, 1)), PLAN),  # 4 chunks < 5 segs
    (dict(plan=(1, 3)), PLAN), (dict(plan=(1, 16)), PLAN), (dict(plan=(1, 8)), PLAN),  # 64/8 = 8 cols
])
def test_bad_sizes_and_enums(lib, kw, code):
    rc, _ = fwd(lib, **kw)
    assert rc == code


def test_size_limits(lib):
    """One head's q, k, v and o are addressed through 32-bit buffer descriptors, so
    T * max(dk, dv) * 4 bytes may not exceed 0xFFFF0000; B * H is capped at 2^24.
    A workspace query exactly at the limit is accepted (no device work), one chunk
    past it is rejected before anything else."""
    t_max = 0xFFFF0000 // (128 * 4)  # 8388480 tokens, a multiple of 64
    rc, n = fwd(lib, B=1, H=1, T=t_max, dk=128, dv=128, plan=(1, 1))
    assert rc == OK and n == 256  # one segment: no segment workspace
    assert fwd(lib, B=1, H=1, T=t_max + 64, dk=128, dv=128, plan=(1, 1))[0] == SHAPE
    assert fwd(lib, B=1, H=1, T=2 * t_max, dk=64, dv=64, plan=(1, 1))[0] == OK
    assert fwd(lib, B=1, H=1, T=2 * t_max + 64, dk=64, dv=64, plan=(1, 1))[0] == SHAPE
    assert fwd(lib, B=1 << 12, H=1 << 12, T=64, plan=(1, 1))[0] == OK
    assert fwd(lib, B=1 << 13, H=1 << 12, T=64, plan=(1, 1))[0] == SHAPE


def test_fp32_diag_branch_needs_dk64(lib):
    rc, _ = fwd(lib, dtype=F32, path=DIAG, dk=128, dv=64, plan=(1, 1))
    assert rc == UNSUP
    rc, _ = fwd(lib, dtype=F32, path=DIAG, dk=64, dv=64, plan=(1, 1))
    assert rc == OK


def test_segments_at_most_chunks(lib):
    # segments split the chunks evenly; any count up to the number of chunks is valid
    assert fwd(lib, T=576, plan=(9, 1))[0] == OK
    assert fwd(lib, T=577, plan=(10, 1))[0] == OK
    assert fwd(lib, T=576, plan=(10, 1))[0] == PLAN


def test_ragged_and_empty_lengths_are_accepted(lib):
    for T in (0, 1, 63, 65, 200):
        rc, n = fwd(lib, T=T, plan=(1, 1))
        assert rc == OK
        assert n == 256  # one segment: no segment workspace, and never a 0-byte answer


def test_empty_sequence_workspace_query_is_never_zero(lib):
    """T = 0 still writes S_T, so the call must not be mistaken for a size query: a
    caller that allocates exactly what the query reports gets a non-NULL buffer only if
    the size is not 0.  Both queries report at least 256 bytes."""
    rc, n = fwd(lib, B=2, H=3, T=0, dk=128, dv=128, plan=(1, 1))
    assert rc == OK and n >= 256
    n2 = ctypes.c_size_t(0)
    assert lib.gla_workspace_size(2, 3, 0, 128, 128, BF16, UNIFIED, P(1, 1), ctypes.byref(n2)) == OK
    assert n2.value == n
    # one byte short of the reported size is rejected before any device call
    assert fwd(lib, B=2, H=3, T=0, dk=128, dv=128, plan=(1, 1), ws=0x10000000, wsz=n - 1)[0] == WORKSPACE


def test_workspace_too_small_and_misaligned(lib):
    rc, need = fwd(lib)
    assert rc == OK and need > 0
    rc, _ = fwd(lib, ws=0x10000000, wsz=need - 1)
    assert rc == WORKSPACE
    rc, _ = fwd(lib, ws=0x10000010, wsz=need)  # not 256-byte aligned
    assert rc == ALIGN


def test_null_pointers(lib):
    rc, need = fwd(lib)
    big = 0x10000000
    assert fwd(lib, q=None, ws=big, wsz=need)[0] == NULL
    assert fwd(lib, x=None, ws=big, wsz=need)[0] == NULL
    assert fwd(lib, ST=None, ws=big, wsz=need)[0] == NULL
    n = ctypes.c_size_t(0)
    assert lib.gla_chunk_fwd_plan(None, None, None, None, None, None, None, 1, 1, 64, 64, 64, 0, 0, 0,
                                  P(1, 1), None, None, None) == NULL


def test_aliasing_is_rejected(lib):
    rc, need = fwd(lib)
    ws = 0x10000000
    # B=1,H=2,T=256,dk=dv=64 bf16: q spans 64 KiB; put o inside q
    assert fwd(lib, o=0x1000 + 4096, ws=ws, wsz=need)[0] == ALIAS
    # S_T overlapping S0
    assert fwd(lib, S0=0x600000, ST=0x600000 + 16, ws=ws, wsz=need)[0] == ALIAS
    # workspace overlapping v
    assert fwd(lib, ws=0x200000, wsz=need)[0] == ALIAS
    # misaligned q
    assert fwd(lib, q=0x1008, ws=ws, wsz=need)[0] == ALIGN


def test_gate_cumsum_validation(lib):
    assert lib.gla_gate_cumsum(0x1000, 0x1000 + 4, 1, 1, 64, BOUNDED, None) == ALIAS
    assert lib.gla_gate_cumsum(None, 0x1000, 1, 1, 64, BOUNDED, None) == NULL
    assert lib.gla_gate_cumsum(0x1000, 0x100000, 1, 1, 64, 9, None) == ARG
    assert lib.gla_gate_cumsum(0x1000, 0x100000, 0, 1, 64, BOUNDED, None) == SHAPE
    assert lib.gla_gate_cumsum(0x1001, 0x100000, 1, 1, 64, BOUNDED, None) == ALIGN
    assert lib.gla_gate_cumsum(None, None, 1, 1, 0, BOUNDED, None) == OK  # T = 0: nothing to do


def test_stage_entry_points_validate(lib):
    # segment pre-pass: workspace too small, unknown gate, x misaligned
    assert lib.gla_segment_states(0x1000, 0x100000, 0x200000, 1, 2, 256, 64, 64, BF16, BOUNDED, P(2, 1),
                                  0x10000000, 8, None) == WORKSPACE
    assert lib.gla_segment_states(0x1000, 0x100000, 0x200000, 1, 2, 256, 64, 64, BF16, 7, P(2, 1),
                                  0x10000000, 1 << 20, None) == ARG
    assert lib.gla_segment_states(0x1000, 0x100000, 0x200001, 1, 2, 256, 64, 64, BF16, BOUNDED, P(2, 1),
                                  0x10000000, 1 << 20, None) == ALIGN
    # output pass: S_T overlapping x, no plan, x missing, unknown gate
    assert lib.gla_chunk_output(0x1000, 0x100000, 0x200000, 0x300000, None, 0x400000, 0x300000, 1, 2, 256, 64,
                                64, BF16, BOUNDED, UNIFIED, P(1, 1), None, 0, None) == ALIAS
    assert lib.gla_chunk_output(0x1000, 0x100000, 0x200000, 0x300000, None, 0x400000, 0x500000, 1, 2, 256, 64,
                                64, BF16, BOUNDED, UNIFIED, None, None, 0, None) == NULL
    assert lib.gla_chunk_output(0x1000, 0x100000, 0x200000, None, None, 0x400000, 0x500000, 1, 2, 256, 64,
                                64, BF16, BOUNDED, UNIFIED, P(1, 1), None, 0, None) == NULL
    assert lib.gla_chunk_output(0x1000, 0x100000, 0x200000, 0x300000, None, 0x400000, 0x500000, 1, 2, 256, 64,
                                64, BF16, 5, UNIFIED, P(1, 1), None, 0, None) == ARG
    assert lib.gla_plan_check(1, 2, 256, 64, 64, BF16, UNIFIED, P(2, 4)) == OK
    assert lib.gla_plan_check(1, 2, 256, 64, 64, BF16, UNIFIED, P(2, 8)) == PLAN


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    x = torch.zeros(1, 1, 64)
    with pytest.raises(ValueError):
        gla.chunk_fwd(q, q, q, x)


# ------------------------------------------------------------------------------ backward

def bwd(lib, B=1, H=2, T=0, dk=64, dv=64, dtype=BF16, gate=BOUNDED, path=UNIFIED, ws=None, wsz=0,
        q=0x1000, k=0x100000, v=0x200000, x=0x300000, S0=None, dO=0x400000, dST=None,
        dq=0x500000, dk_=0x600000, dv_=0x700000, dx=0x800000, dS0=0x900000, nbytes=True):
    n = ctypes.c_size_t(wsz)
    return lib.gla_chunk_bwd(q, k, v, x, S0, dO, dST, dq, dk_, dv_, dx, dS0, B, H, T, dk, dv, dtype, gate, path,
                             ws, ctypes.byref(n) if nbytes else None, None), n.value


def test_backward_validates_before_any_device_call(lib):
    assert bwd(lib, nbytes=False)[0] == NULL
    assert bwd(lib, dk=96)[0] == SHAPE
    assert bwd(lib, B=0)[0] == SHAPE
    assert bwd(lib, T=-1)[0] == SHAPE
    assert bwd(lib, dtype=7)[0] == DTYPE
    assert bwd(lib, gate=5)[0] == ARG
    assert bwd(lib, path=9)[0] == ARG


def test_backward_workspace_query_for_an_empty_sequence(lib):
    # T = 0 needs no plan (no device query): b, b', s and chunk arrays are empty,
    # the three state buffers remain
    rc, need = bwd(lib, B=2, H=3, T=0, dk=64, dv=128)
    assert rc == OK
    assert need == 3 * ((2 * 3 * 64 * 128 * 4 + 255) // 256 * 256)
    # with a workspace of that size, a missing dS0 is rejected before launching
    rc, _ = bwd(lib, B=2, H=3, T=0, dk=64, dv=128, ws=0x10000000, wsz=need, dS0=None)
    assert rc == NULL
    rc, _ = bwd(lib, B=2, H=3, T=0, dk=64, dv=128, ws=0x10000000, wsz=need - 1)
    assert rc == WORKSPACE


def test_plan_check_accepts_every_built_bf16_slice(lib):
    # full-width slices of dk = 64 heads exist only as wave-specialised kernels; the
    # check must accept them like the rest
    for dk in (64, 128):
        for split in (1, 2, 4):
            assert lib.gla_plan_check(4, 16, 1024, dk, 128, BF16, UNIFIED, P(1, split)) == OK, (dk, split)
            assert lib.gla_plan_check(4, 16, 1024, dk, 128, BF16, DIAG, P(1, split)) == OK, (dk, split)


def test_per_channel_plan_and_validation(lib):
    assert lib.gla_plan_check_pc(1, 2, 256, 64, 128, BF16, P(1, 1)) == OK
    assert lib.gla_plan_check_pc(1, 2, 256, 128, 128, BF16, P(4, 2)) == OK
    assert lib.gla_plan_check_pc(1, 2, 256, 128, 128, BF16, P(1, 4)) == PLAN
    assert lib.gla_plan_check_pc(1, 2, 256, 128, 64, F32, P(1, 1)) == UNSUP
    assert lib.gla_plan_check_pc(1, 2, 256, 64, 64, F32, P(1, 1)) == OK
    assert lib.gla_plan_check_pc(1, 2, 256, 64, 64, F32, P(5, 1)) == PLAN  # 4 chunks
    n = ctypes.c_size_t(0)
    fwd_pc = lambda **kw: lib.gla_chunk_fwd_pc(
        kw.get("q", 0x1000), 0x2000, 0x3000, 0x4000, None, 0x5000, 0x6000, 1, 2, kw.get("T", 256), 64, 64, BF16,
        kw.get("gate", BOUNDED), P(*kw.get("plan", (2, 1))), kw.get("ws", None), kw.get("nb", ctypes.byref(n)), None)
    assert fwd_pc(nb=None) == NULL
    assert fwd_pc(gate=4) == ARG
    assert fwd_pc(T=-2) == SHAPE
    assert fwd_pc() == OK and n.value >= 256  # size query with an explicit plan: no device call
    need = n.value
    n.value = need - 1
    assert fwd_pc(ws=0x10000000) == WORKSPACE
    n.value = need
    assert fwd_pc(ws=0x10000100, q=None) == NULL


def test_decode_step_validation(lib):
    def dec(**kw):
        return lib.gla_decode_step(kw.get("q", 0x1000), 0x2000, 0x3000, 0x4000, kw.get("S", 0x100000),
                                   kw.get("o", 0x200000), 2, 3, kw.get("dk", 64), 64, kw.get("dtype", BF16),
                                   kw.get("gate", BOUNDED), kw.get("pc", 0), None)
    assert dec(q=None) == NULL
    assert dec(dk=96) == SHAPE
    assert dec(dtype=3) == DTYPE
    assert dec(gate=2) == ARG
    assert dec(pc=2) == ARG
    assert dec(S=0x100004) == ALIGN
    assert dec(o=0x100000 + 4096) == ALIAS  # o inside S


def test_varlen_validation_before_any_device_call(lib):
    n = ctypes.c_size_t(0)

    def var(**kw):
        return lib.gla_chunk_fwd_varlen(0x1000, 0x2000, 0x3000, 0x4000, None, 0x5000, 0x6000, 0x7000,
                                        kw.get("N", 3), 2, kw.get("T", 500), kw.get("maxlen", 200), 64, 64,
                                        kw.get("dtype", BF16), kw.get("gate", BOUNDED), UNIFIED,
                                        P(*kw["plan"]) if "plan" in kw else None, None,
                                        kw.get("nb", ctypes.byref(n)), None)
    assert var(nb=None) == NULL
    assert var(N=0) == SHAPE
    assert var(maxlen=501) == SHAPE
    assert var(maxlen=-1) == SHAPE
    assert var(dtype=5) == DTYPE
    assert var(gate=3) == ARG
    assert var(plan=(5, 1)) == PLAN       # 200 tokens are 4 chunks
    assert var(plan=(4, 1)) == OK         # explicit plan: size query without a device
    align = lambda b: (b + 255) // 256 * 256
    # the local states and decays of 3 segments, the work order of the 3 sequences (the
    # kernels form the cumulative log-decays from x: no b buffer)
    assert n.value == align(3 * 2 * 3 * 64 * 64 * 4) + align(3 * 2 * 4 * 4) + align(3 * 4)


def test_delta_validation_and_workspace_query(lib):
    n = ctypes.c_size_t(0)

    def dl(**kw):
        return lib.gla_chunk_fwd_delta(kw.get("q", 0x1000), 0x2000, 0x3000, 0x4000, kw.get("beta", 0x5000), None,
                                       0x6000, 0x7000, 1, 2, kw.get("T", 100), kw.get("dk", 64), kw.get("dv", 64),
                                       kw.get("dtype", BF16), kw.get("gate", BOUNDED), P(*kw.get("plan", (1, 2))),
                                       kw.get("ws", None), kw.get("nb", ctypes.byref(n)), None)
    assert dl(nb=None) == NULL
    assert dl(dk=96) == SHAPE
    assert dl(dtype=4) == DTYPE
    assert dl(gate=7) == ARG
    assert dl(plan=(1, 3)) == PLAN
    assert dl(plan=(1, 4)) == PLAN          # 16-column slices are not built
    assert dl(plan=(3, 1)) == PLAN          # 100 tokens are 2 chunks
    assert dl(dtype=F32, dk=128, dv=64, plan=(1, 1)) == UNSUP
    assert lib.gla_plan_check_delta(1, 2, 1000, 128, 128, BF16, P(8, 1)) == OK
    assert dl() == OK                       # explicit plan: size query without a device
    es = 2
    align = lambda b: (b + 255) // 256 * 256
    # b per token, and one 64 x 64 Tinv per chunk (2 heads x 2 chunks)
    assert n.value == align(2 * 100 * 4) + align(2 * 2 * 64 * 64 * es)
    # two segments add one local state and one transition per head, and a reset flag per chunk
    assert dl(plan=(2, 1)) == OK
    assert n.value == (align(2 * 100 * 4) + align(2 * 2 * 64 * 64 * es) + align(2 * 64 * 64 * 4)
                       + align(2 * 64 * 64 * 4) + align(2 * 2 * 4))
    need = n.value
    assert dl(plan=(2, 1), ws=0x10000000, beta=None) == NULL
    n.value = need - 1
    assert dl(plan=(2, 1), ws=0x10000000) == WORKSPACE
