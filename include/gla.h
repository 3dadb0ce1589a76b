/*
 * gla.h -- C ABI of the MI355X (gfx950) chunked gated-linear-attention forward pass.
 *
 * Sources (web pages; cited by title and section):
 *   [LCT] "Engineering Long-Context Training for Trillion-Parameter MoE Models:
 *          Three Key Breakthroughs"
 *   [STM] "Scaling Trillion-Parameter MoE and Long-Context LLMs: Architecture
 *          and Engineering in Practice"
 *   [ESU] "Engineering Stability in Ultra-Long Context and Trillion-Parameter
 *          Sparse Models"
 *
 * Operation.  Linear attention with a scalar per-(batch, head, token) decay,
 * computed chunk by chunk: matrix products inside each chunk and a state
 * carried from chunk to chunk [LCT §3.1], [ESU §2.1].  For each head,
 *     S_{-1} = S0,   S_t = a_t S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t,
 *     S_T = S_{T-1},  a_t = exp(g_t),
 * where the log-decay is g = -5 * sigmoid(x), the bounded "scaled sigmoid" of
 * [LCT §3.2] / [STM §II] / [ESU §2.2], or, for the ablation only, the
 * conventional unbounded negative softplus, g = -softplus(-x) = log sigmoid(x).
 * o_t includes token t itself; the initial state is decayed by a_0.  q is used
 * as given (no internal scale).
 *
 * The product path (GLA_GATE_BOUNDED_SIGMOID + GLA_PATH_UNIFIED) relies on the
 * bound: inside every 16-token tile the reciprocal cumulative decay stays below
 * e^80, so all causal tiles of a chunk, diagonal ones included, go through the
 * same dense matrix-core product [LCT §3.2, §3.3], [ESU §2.2].
 * GLA_PATH_DIAG_BRANCH is the conventional design of [LCT §3.1] / [ESU §2.1]:
 * diagonal tiles take an explicit element-wise position-pair path.  It exists
 * so the difference can be measured.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are device memory owned by the caller, row-major and
 *     contiguous:
 *       q, k [B][H][T][dk]      v [B][H][T][dv]     (dtype: bf16 or fp32)
 *       x, b [B][H][T]          fp32
 *       S0, S_T [B][H][dk][dv]  fp32                (S0 may be NULL: zero state)
 *       o [B][H][T][dv]         fp32
 *     q, k, v, o, S0, S_T must be 16-byte aligned; x and b 4-byte aligned.
 *   - The library allocates nothing and keeps no per-call state.  Work is
 *     enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 *     host is never synchronised: outputs are valid once the stream reaches
 *     that point.  Calls on different streams are safe when their output and
 *     workspace buffers are disjoint.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     rejected call enqueues nothing and writes nothing.  A HIP launch error
 *     is reported as GLA_ERR_HIP.  No C++ exception crosses this boundary.
 *   - T may be any value >= 0.  Sequences are processed in chunks of
 *     GLA_CHUNK tokens; a final partial chunk is handled in place (tokens past
 *     T are treated as absent).  T = 0 writes S_T = S0 (or zeros) and no o.
 *   - Supported sizes: dk in {64, 128}, dv in {64, 128}, B >= 1, H >= 1, and
 *     T * max(dk, dv) * 4 <= 0xFFFF0000 (one head's tensors are addressed
 *     through 32-bit buffer descriptors): T < 8M tokens at d = 128.
 *     The fp32 diagonal-branch path additionally needs dk == 64.
 */
#ifndef GLA_H_
#define GLA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GLA_ABI_VERSION 2

/* The enums below are int-sized.  C callers may pass any int value (a wrong one is
 * rejected with an error code); compiled as C++ they get int as their fixed
 * underlying type, so every int value is a valid value of the type and checking an
 * out-of-range argument is well defined. */
#ifdef __cplusplus
#define GLA_ENUM_INT : int
#else
#define GLA_ENUM_INT
#endif
#define GLA_CHUNK 64          /* tokens per chunk */
#define GLA_TILE 16           /* tokens per tile inside a chunk [LCT §3.2] */
#define GLA_MAX_SEGMENTS 64   /* upper bound on gla_plan_t.segments */

typedef enum GLA_ENUM_INT {
  GLA_OK = 0,
  GLA_ERR_NULL = 1,        /* a required pointer is NULL */
  GLA_ERR_SHAPE = 2,       /* B, H, T, dk or dv out of the supported range */
  GLA_ERR_DTYPE = 3,       /* unknown dtype */
  GLA_ERR_ALIAS = 4,       /* an output overlaps an input or another output */
  GLA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  GLA_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed */
  GLA_ERR_PLAN = 7,        /* plan fields invalid for these sizes */
  GLA_ERR_ALIGN = 8,       /* a pointer violates the alignment rule */
  GLA_ERR_ARG = 9,         /* unknown gate or path enum value */
  GLA_ERR_UNSUPPORTED = 10 /* valid enums, but this combination is not built */
} gla_status_t;

typedef enum GLA_ENUM_INT { GLA_BF16 = 0, GLA_F32 = 1 } gla_dtype_t;   /* storage of q, k, v */

/* Log-decay g(x) [LCT §3.2]. */
typedef enum GLA_ENUM_INT {
  GLA_GATE_BOUNDED_SIGMOID = 0, /* g = -5 * sigmoid(x), range (-5, 0) (the product) */
  GLA_GATE_NEG_SOFTPLUS = 1     /* g = -softplus(-x) = log sigmoid(x), range (-inf, 0);
                                   evaluated as max(g, -128): e^-128 is 0 in fp32 */
} gla_gate_t;

/* How the causal tiles of a chunk are computed. */
typedef enum GLA_ENUM_INT {
  GLA_PATH_UNIFIED = 0,     /* every causal 16x16 tile on MFMA: q*Gamma, k/Gamma (product) */
  GLA_PATH_DIAG_BRANCH = 1  /* off-diagonal tiles on MFMA, diagonal tiles element-wise (ablation) */
} gla_path_t;

/* Launch plan.  Each head's value columns are cut into dv_split slices and its
 * sequence into `segments` contiguous runs of chunks (segment p owns chunks
 * [p*nc/segments, (p+1)*nc/segments), nc = ceil(T/64)); every (head, slice,
 * segment) is one workgroup.  segments > 1 adds a pre-pass that computes the
 * state at the end of every segment but the last (gla_segment_states), so that
 * each segment can start from its own initial state.  Results do not depend on
 * the plan beyond floating-point summation order. */
typedef struct {
  int segments;  /* 1 .. GLA_MAX_SEGMENTS, and at most the number of chunks (>= 1 when T = 0) */
  int dv_split;  /* 1, 2, 4 or 8 with dv / dv_split in {16, 32, 64, 128} */
} gla_plan_t;

/* Human-readable name of a status code (static storage). */
const char* gla_status_string(gla_status_t status);

/* GLA_ABI_VERSION of the built library. */
int gla_abi_version(void);

/* Default plan for the current HIP device (queries its compute-unit count).
 * Returns GLA_ERR_HIP when no device is usable. */
gla_status_t gla_plan_default(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                              gla_path_t path, gla_plan_t* plan);

/* Validates a plan for these sizes without touching the device. */
gla_status_t gla_plan_check(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                            gla_path_t path, const gla_plan_t* plan);

/* Bytes of segment workspace that gla_segment_states writes and
 * gla_chunk_output reads for `plan` (0 when plan->segments == 1).  Host only. */
gla_status_t gla_segment_workspace_size(int B, int H, long long T, int dk, int dv,
                                        const gla_plan_t* plan, size_t* bytes);

/* Bytes of workspace gla_chunk_fwd needs: the segment workspace of `plan`, and at
 * least 256 (never 0, so a buffer allocated from the query is never NULL).
 * plan == NULL means the default plan of the current device (a HIP query).  Host
 * only, enqueues nothing. */
gla_status_t gla_workspace_size(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                                gla_path_t path, const gla_plan_t* plan, size_t* bytes);

/* Gate and chunk-local cumulative log-decay [LCT §3.1, §3.2].
 *   b[t] = sum over the tokens i of t's 64-token chunk with i <= t of g(x[i]),
 * i.e. log Gamma restarted at every chunk boundary, computed by one 64-lane
 * wavefront scan per chunk.  x and b: [B][H][T] fp32 (b may not overlap x).
 * The forward entry points form the same b inside their kernels (same scan, same
 * bits); this call exposes the stage on its own.
 * Non-finite x follows the gate's limits: x = +inf gives g = -5 (bounded) or
 * 0 (softplus); x = -inf gives g = 0 (bounded).  The softplus gate is floored at
 * g = -128 (x = -inf included), where a = e^g is already exactly 0 in fp32, so a
 * zero decay is kept while b stays finite.  NaN gives NaN. */
gla_status_t gla_gate_cumsum(const float* x, float* b, int B, int H, long long T,
                             gla_gate_t gate, void* stream);

/* Segment pre-pass (only meaningful when plan->segments > 1).  For every head
 * and every segment p but the last, runs the state recurrence over the
 * segment's chunks from a zero state (local final state H_p, total log-decay
 * Gamma_p), then combines the segments in order, so that `seg_ws`
 * (gla_segment_workspace_size bytes) receives Gamma_p and
 *   P_0 = H_0,  P_p = e^{Gamma_p} P_{p-1} + H_p,
 * the state at the end of segment p reached from a zero state at the start of
 * the head (gla_chunk_output adds the decayed S0).  Uses k, v and the gate input
 * x [B][H][T] fp32 (gate and chunk-local cumulative sum formed in the kernel, as
 * gla_gate_cumsum would).  Does nothing when segments == 1. */
gla_status_t gla_segment_states(const void* k, const void* v, const float* x,
                                int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                                gla_gate_t gate, const gla_plan_t* plan, void* seg_ws,
                                size_t seg_ws_bytes, void* stream);

/* Fused chunk output pass: for every chunk, the gate and chunk-local cumulative
 * log-decay of x, the intra-chunk causal product (q*Gamma)(k/Gamma)^T V, the
 * inter-chunk term (q*Gamma) S, and the decayed state update, o written once,
 * S_T written by the last segment [LCT §3.1-§3.3].  seg_ws from
 * gla_segment_states with the same plan and gate (ignored when
 * plan->segments == 1).  S0 may be NULL.  o and S_T must not overlap any input;
 * S_T must not overlap S0. */
gla_status_t gla_chunk_output(const void* q, const void* k, const void* v, const float* x,
                              const float* S0, float* o, float* S_T,
                              int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                              gla_gate_t gate, gla_path_t path, const gla_plan_t* plan,
                              const void* seg_ws, size_t seg_ws_bytes, void* stream);

/* The whole forward pass: gla_segment_states (when the plan has several
 * segments) and gla_chunk_output, enqueued in that order on `stream` with the
 * default plan of the current device; both form the gate and the chunk-local
 * cumulative log-decay from x in their kernels.
 *   workspace == NULL: *workspace_bytes receives the required size; nothing is
 *                      enqueued (this queries the device for the plan).
 *   otherwise:         *workspace_bytes is the caller's workspace size; a
 *                      smaller value than required returns GLA_ERR_WORKSPACE.
 * The workspace is device memory, 256-byte aligned, owned by the caller, and
 * must not overlap any argument. */
gla_status_t gla_chunk_fwd(const void* q, const void* k, const void* v, const float* x,
                           const float* S0, float* o, float* S_T,
                           int B, int H, long long T, int dk, int dv,
                           gla_dtype_t dtype, gla_gate_t gate, gla_path_t path,
                           void* workspace, size_t* workspace_bytes, void* stream);

/* gla_chunk_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The segment workspace comes from a 32 MiB device array inside
 * the library, one per GPU, held until the process ends; the call allocates nothing.  Same default plan, kernels and results
 * as gla_chunk_fwd.  A plan whose workspace exceeds the array returns
 * GLA_ERR_WORKSPACE before anything is enqueued (the default plans on a 256-CU
 * device need at most ~31 MB at dk = dv = 128).  Calls on one GPU share the array:
 * calls that can overlap on one GPU (different streams without ordering) race and
 * must be serialised by the caller.  Other errors as gla_chunk_fwd. */
gla_status_t gla_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* x,
                                   const float* S0, float* o, float* S_T,
                                   int B, int H, long long T, int dk, int dv,
                                   gla_dtype_t dtype, gla_gate_t gate, gla_path_t path, void* stream);

/* gla_chunk_fwd with an explicit plan (NULL = default plan). */
gla_status_t gla_chunk_fwd_plan(const void* q, const void* k, const void* v, const float* x,
                                const float* S0, float* o, float* S_T,
                                int B, int H, long long T, int dk, int dv,
                                gla_dtype_t dtype, gla_gate_t gate, gla_path_t path,
                                const gla_plan_t* plan,
                                void* workspace, size_t* workspace_bytes, void* stream);

/* Backward pass of gla_chunk_fwd: the gradients of a scalar loss L given
 * dO = dL/do and dS_T = dL/dS_T, for the same recurrence
 * S_t = a_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, a_t = e^{g(x_t)} [LCT §3.1, §3.2].
 *   q, k, v, x, S0, B..path: as passed to gla_chunk_fwd (S0 may be NULL: zero).
 *   dO   [B][H][T][dv] in `dtype` (the operand precision of q, k, v).
 *   dS_T [B][H][dk][dv] fp32, or NULL (zero).
 *   dq, dk [B][H][T][dk], dv [B][H][T][dv], dx [B][H][T], dS0 [B][H][dk][dv]: fp32
 *   outputs (dS0 is written even when S0 is NULL), device memory, none
 *   overlapping another argument or the workspace.
 * Method: dq is the forward pass with (q, k, v, S0) replaced by (dO, v, k, S0^T);
 * dk and dv are forward passes in reversed time over (v, dO, q, dS_T^T) and
 * (k, q, dO, dS_T), whose decays are those of the next token (the state gradient
 * D_t = q_t dO_t^T + a_{t+1} D_{t+1} is a forward recurrence run backwards); its
 * final state gives dS0 = a_0 D_0.  dL/dg_t is the sum over the (key token s,
 * output token j) pairs whose decay path spans t (s < t <= j, with j = "after the
 * end" for the final state), taken per chunk: pairs inside the chunk from q.k and
 * dO.v on the matrix cores, pairs that enter or leave the chunk from the states
 * before and after it, and pairs that cross it whole; dx = g'(x) dL/dg.  bf16
 * on the unified path: the dq pass forms the pairs inside and
 * entering each chunk (it holds the state before the chunk) and the dk pass the
 * pairs leaving and crossing it (it holds the state gradient after the chunk), the
 * dq pass handing over the state before each chunk whose crossing factor is not
 * exactly 0; both passes then run with one full-width slice.  Otherwise the dq and
 * dk passes store one state per pair of chunks (bf16 for bf16 operands) and a
 * separate dx kernel steps the other one across the neighbouring chunk.  Each pass
 * uses the device's default plan; the dq and dk passes need value slices of at
 * least 32 columns (GLA_ERR_UNSUPPORTED otherwise, which the default plans never
 * give).
 * workspace == NULL: *workspace_bytes receives the size and nothing is enqueued;
 * otherwise the workspace (256-byte aligned device memory) must be at least that
 * size.  Errors as gla_chunk_fwd; everything is validated before anything is
 * enqueued on `stream`. */
gla_status_t gla_chunk_bwd(const void* q, const void* k, const void* v, const float* x,
                           const float* S0, const void* dO, const float* dS_T,
                           float* dq, float* dk, float* dv, float* dx, float* dS0,
                           int B, int H, long long T, int dk_dim, int dv_dim,
                           gla_dtype_t dtype, gla_gate_t gate, gla_path_t path,
                           void* workspace, size_t* workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Gated delta rule.  [LCT §3.1, §3.3] name Delta-Net-style structures as the
 * other family with the same chunked diagonal-tile problem; the recurrence here
 * is the gated delta rule with the same decay gate:
 *     S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t,
 *     a_t = e^{g(x_t)}.
 * Chunked with an exact triangular solve per 64-token chunk: the effective writes
 * U = Tinv diag(beta) V - Tinv diag(beta e^b) K S_0 with Tinv = (I + diag(beta) L)^-1,
 * L the decay-weighted Gram matrix of the chunk's keys; both L and the attention
 * matrix come from the unified 16-token-tile product (no diagonal branch).
 *   beta [B][H][T] fp32 (a write strength, normally in [0, 1]); other arguments as
 *   for gla_chunk_fwd (S0 may be NULL).
 *   plan: NULL = gla_plan_default_delta; dv_split value-column slices (one
 *   workgroup per head, slice and segment; 16 columns per wave), segments as in
 *   gla_chunk_fwd.  Segments after the first start from S0 folded with the earlier
 *   segments' affine maps S_end = Phi S_start + H, computed by a pre-pass (Phi is the
 *   product of the chunk transitions e^gamma I - (k e^{gamma-b})^T W, dk x dk).
 * Built: bf16 with dk, dv in {64, 128} and slices of 32, 64 or 128 columns; fp32
 * with dk = dv = 64 and slices of 32 or 64.  Others: GLA_ERR_UNSUPPORTED or
 * GLA_ERR_PLAN.  The workspace holds b, each chunk's Tinv (64 x 64, operand dtype;
 * the passes after the solve form W and U~ from it and the chunk's k and v), the
 * segment maps and one reset flag per chunk; workspace == NULL returns its size.
 * Errors and validation as gla_chunk_fwd.
 * Segment pre-pass: a chunk whose transition scales any incoming state by less than
 * 2^-114 (a bound from the largest |k e^{gamma-b}| and |W| of each token, taken in
 * log2) is a reset point; a segment's local state is run from a zero state at its
 * last reset chunk instead of its first chunk.  Results then differ from running the
 * whole segment by less than 2^-114 of the state's scale. */
gla_status_t gla_plan_default_delta(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                                    gla_plan_t* plan);
gla_status_t gla_plan_check_delta(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                                  const gla_plan_t* plan);
gla_status_t gla_chunk_fwd_delta(const void* q, const void* k, const void* v, const float* x,
                                 const float* beta, const float* S0, float* o, float* S_T,
                                 int B, int H, long long T, int dk, int dv,
                                 gla_dtype_t dtype, gla_gate_t gate, const gla_plan_t* plan,
                                 void* workspace, size_t* workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode and packed sequences. */

/* One recurrent step for every head, for generating one token at a time with
 * the state carried between calls [LCT §3.1, §3.2]:
 *     S <- diag(a) S + k v^T   (in place),   o = S^T q,   a = e^{g(x)}.
 *   q, k [B][H][dk], v [B][H][dv] in `dtype`; x [B][H] fp32, or [B][H][dk] when
 *   per_channel = 1 (one decay per key channel, as gla_chunk_fwd_pc);
 *   S [B][H][dk][dv] fp32, read and overwritten (16-byte aligned); o [B][H][dv]
 *   fp32 (16-byte aligned).  dk, dv in {64, 128}.  S and o must not overlap each
 *   other or any input.  No workspace; errors as gla_chunk_fwd.  A step over S
 *   equals gla_chunk_fwd over one token with S0 = S (up to rounding). */
gla_status_t gla_decode_step(const void* q, const void* k, const void* v, const float* x,
                             float* S, float* o, int B, int H, int dk, int dv,
                             gla_dtype_t dtype, gla_gate_t gate, int per_channel, void* stream);

/* Forward over N packed sequences of different lengths (the scalar-decay
 * method of gla_chunk_fwd, chunks restarting at every sequence start).
 *   q, k [H][T][dk], v [H][T][dv], x [H][T], o [H][T][dv]: every head holds the
 *   N sequences back to back, sequence n in rows [cu_seqlens[n], cu_seqlens[n+1]);
 *   T = total rows.
 *   cu_seqlens: N+1 nondecreasing int64 offsets in device memory, cu_seqlens[0] >= 0,
 *   cu_seqlens[N] <= T, no sequence longer than max_seqlen (host value, <= T).  They
 *   are read on the device only: offsets outside [0, T] are clamped and longer
 *   sequences cut to max_seqlen, which yields wrong values but never an access
 *   outside the tensors.  Rows covered by no sequence are not written in o.
 *   S0, S_T [N][H][dk][dv] fp32 (S0 may be NULL), one state per sequence and head.
 * plan: NULL = the device default for N x H units of max_seqlen tokens; an explicit
 * plan is checked as for gla_chunk_fwd_plan with T = max_seqlen.  Every sequence is
 * cut into the plan's number of segments.  workspace == NULL returns the size.
 * Errors as gla_chunk_fwd. */
gla_status_t gla_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* x,
                                  const float* S0, float* o, float* S_T,
                                  const long long* cu_seqlens, int N, int H, long long T,
                                  long long max_seqlen, int dk, int dv,
                                  gla_dtype_t dtype, gla_gate_t gate, gla_path_t path,
                                  const gla_plan_t* plan,
                                  void* workspace, size_t* workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Per-channel decay.  The same chunked method with one decay per key channel
 * (the per-position decay of [LCT §3.1] read as a vector over the key
 * dimension):
 *     S_t[d][n] = a_t[d] S_{t-1}[d][n] + k_t[d] v_t[n],  a_t[d] = e^{g(x_t[d])},
 *     o_t = S_t^T q_t.
 * The decay cannot be factored out of the sum over d, so every causal 16x16
 * tile, diagonal or not, is one matrix product of q e^{b - r_u} with k
 * e^{r_u - b} referenced to the query tile's start; the bounded gate keeps the
 * reciprocal factor of a 16-token tile below e^80 [LCT §3.2-§3.3].  The gate and
 * the chunk-local cumulative sum run inside the kernels (no b buffer).
 *   x [B][H][T][dk] fp32 (one gate pre-activation per key channel, 16-byte
 *   aligned); other arguments as for gla_chunk_fwd (S0 may be NULL).
 * Built: bf16 with dk in {64, 128} and value slices of 64 or 128 columns
 * (dv_split 1 or 2); fp32 with dk = 64 and 64-column slices.  Other valid
 * shapes return GLA_ERR_PLAN or GLA_ERR_UNSUPPORTED.  The workspace holds the
 * segment states when the plan has several segments; workspace == NULL returns
 * its size (at least 256) in *workspace_bytes and enqueues nothing.  Errors and
 * validation as gla_chunk_fwd. */
gla_status_t gla_plan_default_pc(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                                 gla_plan_t* plan);
gla_status_t gla_plan_check_pc(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                               const gla_plan_t* plan);
gla_status_t gla_chunk_fwd_pc(const void* q, const void* k, const void* v, const float* x,
                              const float* S0, float* o, float* S_T,
                              int B, int H, long long T, int dk, int dv,
                              gla_dtype_t dtype, gla_gate_t gate, const gla_plan_t* plan,
                              void* workspace, size_t* workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Measurement helper (not part of the method).  A flat grid-stride stream with
 * the forward pass's byte mix: for every 16-byte unit j < units, one 16-byte load
 * from each of a, b, c at j and two 16-byte stores to out at 2j and 2j + 1 (48
 * bytes read for 32 written, the 768 : 512 of q, k, v in bf16 and o in fp32 per
 * token-head at d = 128).  Its rate is the device's practical streaming ceiling
 * for that mix, read beside the output pass's achieved bandwidth.  a, b, c: 16 *
 * units bytes each, out: 32 * units bytes, all device memory, 16-byte aligned, out
 * overlapping none of the inputs; grid = workgroups of 256 threads (8192 was the
 * fastest measured).  Enqueued on `stream`; errors as gla_chunk_fwd. */
gla_status_t gla_bench_stream(const void* a, const void* b, const void* c, void* out,
                              unsigned long long units, int grid, void* stream);

/* Measurement helper (not part of the method).  The output pass's access pattern
 * without its arithmetic: BH * segments workgroups of 512 threads, at most one per
 * compute unit (each reserves 96 KB of LDS), workgroup w taking head w / segments and
 * the (w % segments)-th run of (T / 64) / segments consecutive 64-token chunks, in
 * order, with the next chunk's loads in flight while the current chunk's output is
 * stored.  Per chunk it reads 16 KB from each of q, k, v (64 rows of 128 bf16) and
 * writes 32 KB of o (64 rows of 128 fp32): 16-byte unit j of a chunk's o is the xor of
 * unit j mod 1024 of q, k and v.  q, k, v: BH * T * 256 bytes each, o: BH * T * 512
 * bytes, device memory, 16-byte aligned, o overlapping none of the inputs.  BH or T
 * = 0: nothing is enqueued.  T not a multiple of 64, (T / 64) not a multiple of
 * segments, a negative size or segments < 1: GLA_ERR_SHAPE; other errors as
 * gla_bench_stream. */
gla_status_t gla_bench_chunk_stream(const void* q, const void* k, const void* v, void* o, int BH, long long T,
                                    int segments, void* stream);

/* Cross-lane self-test: one wavefront of 64 lanes runs each wavefront helper the
 * kernels build on -- DPP group maxima and sums over 8 and 16 lanes, the strided
 * exclusive scans over lane groups of 4, 8 and 16, the 64-lane inclusive scan, the
 * broadcast of each 16-lane row to the other three, the sum over the four rows, and
 * the gfx950 row-pair and half-wave swaps -- on in[0..63] (the swaps pair it with
 * in + 100) and writes 17 slots of 64 floats to out, in that order (slots 13/14: the
 * row-pair swap's two results, 15/16: the half-wave swap's).  A caller holds them
 * against the definitions to confirm the lane layouts on its device and compiler.
 * in, out: device memory (64 and 17 x 64 floats); enqueued on `stream`.  NULL
 * pointers: GLA_ERR_NULL; a failed launch: GLA_ERR_HIP. */
gla_status_t gla_lane_selftest(const float* in, float* out, void* stream);

/* ------------------------------------------------------------------------
 * Debug builds (the library compiled with -DGLA_DEBUG, libgla_debug.so next to
 * libgla.so): every LDS access made through the kernels' shared load/store
 * helpers is checked against the workgroup's static LDS allocation.  A failed
 * check never traps; it sets a bit in a per-device word, which this call reads
 * (ORed over the library's kernel units) into *flags and clears:
 *   bit 0: an access past the workgroup's LDS allocation,
 *   bit 1: an LDS helper handed a pointer that is not in LDS.
 * Synchronise the device before reading.  Acts on the current device.  Release
 * builds return GLA_ERR_UNSUPPORTED and leave *flags untouched; NULL flags:
 * GLA_ERR_NULL; a failed device copy: GLA_ERR_HIP. */
gla_status_t gla_debug_flags(unsigned int* flags);

/* Self-test of those checks (debug builds): one workgroup asks them about an
 * address one element past its own 256-byte LDS allocation and about the global
 * pointer `probe` (device memory, never dereferenced), accessing neither, so both
 * flag bits come up; `out` (64 floats of device memory) receives values the kernel
 * computes so that it is not optimised away.  Enqueued on `stream`.  Release
 * builds: GLA_ERR_UNSUPPORTED. */
gla_status_t gla_debug_selftest(const float* probe, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H_ */
