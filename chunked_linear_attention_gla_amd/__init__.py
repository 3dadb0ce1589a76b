"""Chunked gated linear attention with bounded decay, forward and backward passes, for MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/gla.h`` (``libgla.so``, built in-tree by ``_build.py``); this package
is the thin Python binding over it plus the seeded workload generators.
"""
from ._lib import (  # noqa: F401
    CHUNK, DEBUG_LIB_PATH, GATES, GLA_BF16, GLA_F32, MAX_SEGMENTS, PATHS, GLAError, LIB_PATH, Plan, abi_version,
    backward_workspace_size, bench_chunk_stream, bench_stream, chunk_bwd, chunk_fwd, chunk_fwd_delta, chunk_fwd_pc, chunk_fwd_varlen,
    chunk_output, debug_flags, decode_step, gate_cumsum, lane_selftest, load, plan_check, plan_check_pc, plan_default,
    plan_default_delta, plan_default_pc, segment_states, segment_workspace_size, status_string, use_library,
    workspace_size,
)
