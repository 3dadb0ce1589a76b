// api.hip -- the C ABI declared in include/gla.h: argument validation, launch
// plans, workspace carving and launch sequencing.  No allocation, no host
// synchronisation; every launch goes to the caller's stream.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "gla.h"
#include "gla_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

bool valid_dtype(int d) { return d == GLA_BF16 || d == GLA_F32; }
bool valid_gate(int g) { return g == GLA_GATE_BOUNDED_SIGMOID || g == GLA_GATE_NEG_SOFTPLUS; }
bool valid_path(int p) { return p == GLA_PATH_UNIFIED || p == GLA_PATH_DIAG_BRANCH; }
size_t elem_size(gla_dtype_t d) { return d == GLA_BF16 ? 2 : 4; }

long long n_chunks(long long T) { return (T + GLA_CHUNK - 1) / GLA_CHUNK; }

gla_status_t check_sizes(int B, int H, long long T, int dk, int dv) {
  if (B < 1 || H < 1 || T < 0) return GLA_ERR_SHAPE;
  if (dk != 64 && dk != 128) return GLA_ERR_SHAPE;
  if (dv != 64 && dv != 128) return GLA_ERR_SHAPE;
  const long long BH = (long long)B * H;
  if (BH > (1LL << 24)) return GLA_ERR_SHAPE;
  // one head's q, k, v or o must fit a 32-bit buffer descriptor
  if ((unsigned long long)T * (unsigned long long)std::max(dk, dv) * 4ULL > 0xFFFF0000ULL) return GLA_ERR_SHAPE;
  return GLA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
  const void* p;
  size_t n;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

gla_status_t plan_check_impl(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype, gla_path_t path,
                             const gla_plan_t* plan) {
  gla_status_t st = check_sizes(B, H, T, dk, dv);
  if (st != GLA_OK) return st;
  if (!valid_dtype(dtype)) return GLA_ERR_DTYPE;
  if (!valid_path(path)) return GLA_ERR_ARG;
  if (!plan) return GLA_ERR_NULL;
  const long long nc = n_chunks(T);
  if (plan->segments < 1 || plan->segments > GLA_MAX_SEGMENTS) return GLA_ERR_PLAN;
  if (plan->segments > std::max(1LL, nc)) return GLA_ERR_PLAN;
  const int s = plan->dv_split;
  if (s != 1 && s != 2 && s != 4 && s != 8) return GLA_ERR_PLAN;
  if (dv % s) return GLA_ERR_PLAN;
  const int slice = dv / s;
  if (slice != 16 && slice != 32 && slice != 64 && slice != 128) return GLA_ERR_PLAN;
  if (!gla::chunk_config_built(dtype == GLA_BF16 ? 0 : 1, dk, slice, path == GLA_PATH_DIAG_BRANCH)) {
    // a valid plan shape that the library has no kernel for
    if (dtype == GLA_F32 && path == GLA_PATH_DIAG_BRANCH && dk != 64) return GLA_ERR_UNSUPPORTED;
    return GLA_ERR_PLAN;
  }
  return GLA_OK;
}

size_t seg_bytes(long long BH, int dk, int dv, int segments) {
  if (segments <= 1) return 0;
  return align_up((size_t)BH * (size_t)(segments - 1) * (size_t)dk * (size_t)dv * 4) +
         align_up((size_t)BH * (size_t)segments * 4);
}

// Workspace of the forward pass: the segment workspace (the kernels form the
// cumulative log-decays from x themselves).  Never 0: a caller that allocates what
// the query reports then holds a non-NULL buffer, which the call does not mistake
// for another size query (T = 0 still writes S_T).
size_t fwd_workspace_bytes(long long BH, int dk, int dv, int segments) {
  return std::max(seg_bytes(BH, dk, dv, segments), kAlign);
}

// Default plan.  Measured on MI355X (256 CUs): one workgroup per CU, each owning a
// full-width value slice, is fastest; segments are added until the grid covers the
// CUs (a segment costs one extra read of k and v, a narrower value slice costs a
// re-read of q and k and a repeated q.k^T).  The fp32 kernels are built for
// slices of at most 64 columns.
gla_status_t default_plan_for(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype, gla_path_t path,
                              int cus, gla_plan_t* plan) {
  const long long BH = (long long)B * H;
  const long long nc = n_chunks(T);
  int split = 1;
  if (dtype == GLA_F32) split = dv / 64;
  long long units = BH * split;
  // too few heads to fill the device even with segments: narrow the value slices
  while (units * GLA_MAX_SEGMENTS < cus && dv / (split * 2) >= 32 && dtype == GLA_BF16) {
    split *= 2;
    units *= 2;
  }
  int segs = 1;
  while (segs < GLA_MAX_SEGMENTS && units * segs < cus && nc / (2LL * segs) >= 4) segs *= 2;
  if (segs > std::max(1LL, nc)) segs = (int)std::max(1LL, nc);
  plan->segments = segs;
  plan->dv_split = split;
  return plan_check_impl(B, H, T, dk, dv, dtype, path, plan);
}

gla_status_t device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GLA_ERR_HIP;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return GLA_ERR_HIP;
  if (*cus <= 0) return GLA_ERR_HIP;
  return GLA_OK;
}

gla::ChunkParams make_params(const void* q, const void* k, const void* v, const float* b, const float* S0,
                             float* o, float* S_T, int B, int H, long long T, int dk, int dv,
                             const gla_plan_t& plan, const void* seg_ws) {
  gla::ChunkParams p;
  const long long BH = (long long)B * H;
  p.q = q;
  p.k = k;
  p.v = v;
  p.b = b;
  p.x = nullptr;
  p.gate = gla::kGateBoundedSigmoid;
  p.S0 = S0;
  p.o = o;
  p.ST = S_T;
  p.T = T;
  p.dk = dk;
  p.dv = dv;
  p.BH = (int)BH;
  p.nchunks = (int)n_chunks(T);
  p.segments = plan.segments;
  p.nslices = plan.dv_split;
  p.seg_state = nullptr;
  p.seg_decay = nullptr;
  if (plan.segments > 1 && seg_ws) {
    char* base = (char*)seg_ws;
    p.seg_state = (float*)base;
    p.seg_decay = (float*)(base + align_up((size_t)BH * (plan.segments - 1) * dk * dv * 4));
  }
  p.grid = 0;
  p.reverse = 0;
  p.pad = 0;
  p.Tl = T;
  p.s0_transposed = 0;
  p.seg_transposed = 0;
  p.state_out = nullptr;
  p.cu_seqlens = nullptr;
  p.H = H;
  p.unit_order = nullptr;
  p.gx_mode = 0;
  p.gx_op = nullptr;
  p.gx_b = nullptr;
  p.gx_x = nullptr;
  p.gx_out = nullptr;
  p.gx_states = nullptr;
  return p;
}

}  // namespace

extern "C" {

const char* gla_status_string(gla_status_t s) {
  switch (s) {
    case GLA_OK: return "GLA_OK";
    case GLA_ERR_NULL: return "GLA_ERR_NULL: a required pointer is NULL";
    case GLA_ERR_SHAPE: return "GLA_ERR_SHAPE: B, H, T, dk or dv out of the supported range";
    case GLA_ERR_DTYPE: return "GLA_ERR_DTYPE: unknown dtype";
    case GLA_ERR_ALIAS: return "GLA_ERR_ALIAS: an output overlaps an input or another output";
    case GLA_ERR_WORKSPACE: return "GLA_ERR_WORKSPACE: workspace missing or too small";
    case GLA_ERR_HIP: return "GLA_ERR_HIP: HIP runtime call or kernel launch failed";
    case GLA_ERR_PLAN: return "GLA_ERR_PLAN: plan invalid for these sizes";
    case GLA_ERR_ALIGN: return "GLA_ERR_ALIGN: pointer alignment violated";
    case GLA_ERR_ARG: return "GLA_ERR_ARG: unknown gate or path";
    case GLA_ERR_UNSUPPORTED: return "GLA_ERR_UNSUPPORTED: combination not built";
  }
  return "unknown gla_status_t";
}

int gla_abi_version(void) { return GLA_ABI_VERSION; }

gla_status_t gla_plan_check(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype, gla_path_t path,
                            const gla_plan_t* plan) {
  return plan_check_impl(B, H, T, dk, dv, dtype, path, plan);
}

gla_status_t gla_plan_default(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype, gla_path_t path,
                              gla_plan_t* plan) {
  if (!plan) return GLA_ERR_NULL;
  gla_status_t st = check_sizes(B, H, T, dk, dv);
  if (st != GLA_OK) return st;
  if (!valid_dtype(dtype)) return GLA_ERR_DTYPE;
  if (!valid_path(path)) return GLA_ERR_ARG;
  int cus = 0;
  st = device_cus(&cus);
  if (st != GLA_OK) return st;
  return default_plan_for(B, H, T, dk, dv, dtype, path, cus, plan);
}

gla_status_t gla_segment_workspace_size(int B, int H, long long T, int dk, int dv, const gla_plan_t* plan,
                                        size_t* bytes) {
  if (!plan || !bytes) return GLA_ERR_NULL;
  gla_status_t st = check_sizes(B, H, T, dk, dv);
  if (st != GLA_OK) return st;
  if (plan->segments < 1 || plan->segments > GLA_MAX_SEGMENTS) return GLA_ERR_PLAN;
  *bytes = seg_bytes((long long)B * H, dk, dv, plan->segments);
  return GLA_OK;
}

gla_status_t gla_workspace_size(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype, gla_path_t path,
                                const gla_plan_t* plan, size_t* bytes) {
  if (!bytes) return GLA_ERR_NULL;
  gla_plan_t pl;
  gla_status_t st;
  if (plan) {
    st = plan_check_impl(B, H, T, dk, dv, dtype, path, plan);
    if (st != GLA_OK) return st;
    pl = *plan;
  } else {
    st = gla_plan_default(B, H, T, dk, dv, dtype, path, &pl);
    if (st != GLA_OK) return st;
  }
  *bytes = fwd_workspace_bytes((long long)B * H, dk, dv, pl.segments);
  return GLA_OK;
}

gla_status_t gla_gate_cumsum(const float* x, float* b, int B, int H, long long T, gla_gate_t gate,
                             void* stream) {
  if (B < 1 || H < 1 || T < 0) return GLA_ERR_SHAPE;
  if (!valid_gate(gate)) return GLA_ERR_ARG;
  const long long BH = (long long)B * H;
  if (T == 0) return GLA_OK;
  if (!x || !b) return GLA_ERR_NULL;
  if (!aligned(x, 4) || !aligned(b, 4)) return GLA_ERR_ALIGN;
  const size_t n = (size_t)BH * (size_t)T * 4;
  if (overlap({x, n}, {b, n})) return GLA_ERR_ALIAS;
  hipError_t e = gla::launch_gate_cumsum(x, b, BH, T, gate == GLA_GATE_BOUNDED_SIGMOID ? gla::kGateBoundedSigmoid
                                                                                     : gla::kGateNegSoftplus,
                                         false, (hipStream_t)stream);
  return e == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

gla_status_t gla_segment_states(const void* k, const void* v, const float* x, int B, int H, long long T, int dk,
                                int dv, gla_dtype_t dtype, gla_gate_t gate, const gla_plan_t* plan, void* seg_ws,
                                size_t seg_ws_bytes, void* stream) {
  gla_status_t st = plan_check_impl(B, H, T, dk, dv, dtype, GLA_PATH_UNIFIED, plan);
  if (st != GLA_OK) return st;
  if (!valid_gate(gate)) return GLA_ERR_ARG;
  if (plan->segments <= 1 || T == 0) return GLA_OK;
  if (!k || !v || !x) return GLA_ERR_NULL;
  const long long BH = (long long)B * H;
  const size_t need = seg_bytes(BH, dk, dv, plan->segments);
  if (!seg_ws || seg_ws_bytes < need) return GLA_ERR_WORKSPACE;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(x, 4) || !aligned(seg_ws, kAlign)) return GLA_ERR_ALIGN;
  const size_t es = elem_size(dtype);
  const Range ws{seg_ws, need};
  if (overlap(ws, {k, (size_t)BH * T * dk * es}) || overlap(ws, {v, (size_t)BH * T * dv * es}) ||
      overlap(ws, {x, (size_t)BH * T * 4}))
    return GLA_ERR_ALIAS;
  gla::ChunkParams p = make_params(nullptr, k, v, nullptr, nullptr, nullptr, nullptr, B, H, T, dk, dv, *plan, seg_ws);
  p.x = x;
  p.gate = gate == GLA_GATE_BOUNDED_SIGMOID ? gla::kGateBoundedSigmoid : gla::kGateNegSoftplus;
  p.grid = (int)(BH * plan->dv_split * (plan->segments - 1));
  hipError_t e = gla::launch_segment_states(p, dtype == GLA_BF16 ? 0 : 1, (hipStream_t)stream);
  return e == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

gla_status_t gla_chunk_output(const void* q, const void* k, const void* v, const float* x, const float* S0,
                              float* o, float* S_T, int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                              gla_gate_t gate, gla_path_t path, const gla_plan_t* plan, const void* seg_ws,
                              size_t seg_ws_bytes, void* stream) {
  gla_status_t st = plan_check_impl(B, H, T, dk, dv, dtype, path, plan);
  if (st != GLA_OK) return st;
  if (!valid_gate(gate)) return GLA_ERR_ARG;
  if (!S_T) return GLA_ERR_NULL;
  if (T > 0 && (!q || !k || !v || !x || !o)) return GLA_ERR_NULL;
  const long long BH = (long long)B * H;
  const size_t es = elem_size(dtype);
  const size_t need = seg_bytes(BH, dk, dv, plan->segments);
  if (plan->segments > 1 && (!seg_ws || seg_ws_bytes < need)) return GLA_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(S_T, 16) ||
      !aligned(S0, 16) || !aligned(x, 4))
    return GLA_ERR_ALIGN;
  const Range rq{q, (size_t)BH * T * dk * es}, rk{k, (size_t)BH * T * dk * es}, rv{v, (size_t)BH * T * dv * es};
  const Range rx{x, (size_t)BH * T * 4}, rs0{S0, (size_t)BH * dk * dv * 4};
  const Range ro{o, (size_t)BH * T * dv * 4}, rst{S_T, (size_t)BH * dk * dv * 4};
  const Range rws{plan->segments > 1 ? seg_ws : nullptr, need};
  for (const Range& in : {rq, rk, rv, rx, rs0, rws})
    if (overlap(ro, in) || overlap(rst, in)) return GLA_ERR_ALIAS;
  if (overlap(ro, rst)) return GLA_ERR_ALIAS;
  gla::ChunkParams p = make_params(q, k, v, nullptr, S0, o, S_T, B, H, T, dk, dv, *plan, seg_ws);
  p.x = x;
  p.gate = gate == GLA_GATE_BOUNDED_SIGMOID ? gla::kGateBoundedSigmoid : gla::kGateNegSoftplus;
  p.grid = (int)(BH * plan->dv_split * plan->segments);
  hipError_t e = gla::launch_chunk_output(p, dtype == GLA_BF16 ? 0 : 1, path == GLA_PATH_DIAG_BRANCH,
                                          (hipStream_t)stream);
  return e == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

gla_status_t gla_chunk_fwd_plan(const void* q, const void* k, const void* v, const float* x, const float* S0,
                                float* o, float* S_T, int B, int H, long long T, int dk, int dv,
                                gla_dtype_t dtype, gla_gate_t gate, gla_path_t path, const gla_plan_t* plan,
                                void* workspace, size_t* workspace_bytes, void* stream) {
  if (!workspace_bytes) return GLA_ERR_NULL;
  gla_status_t st = check_sizes(B, H, T, dk, dv);
  if (st != GLA_OK) return st;
  if (!valid_dtype(dtype)) return GLA_ERR_DTYPE;
  if (!valid_gate(gate) || !valid_path(path)) return GLA_ERR_ARG;
  gla_plan_t pl;
  if (plan) {
    st = plan_check_impl(B, H, T, dk, dv, dtype, path, plan);
    if (st != GLA_OK) return st;
    pl = *plan;
  } else {
    st = gla_plan_default(B, H, T, dk, dv, dtype, path, &pl);
    if (st != GLA_OK) return st;
  }
  const long long BH = (long long)B * H;
  const size_t s_bytes = seg_bytes(BH, dk, dv, pl.segments);
  const size_t need = fwd_workspace_bytes(BH, dk, dv, pl.segments);
  if (!workspace) {
    *workspace_bytes = need;
    return GLA_OK;
  }
  if (*workspace_bytes < need) return GLA_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return GLA_ERR_ALIGN;
  if (!S_T) return GLA_ERR_NULL;
  if (T > 0 && (!q || !k || !v || !x || !o)) return GLA_ERR_NULL;
  if (!aligned(x, 4)) return GLA_ERR_ALIGN;
  const size_t es = elem_size(dtype);
  const Range rws{workspace, need};
  const Range ins[] = {{q, (size_t)BH * T * dk * es}, {k, (size_t)BH * T * dk * es}, {v, (size_t)BH * T * dv * es},
                       {x, (size_t)BH * T * 4},       {S0, (size_t)BH * dk * dv * 4}, {o, (size_t)BH * T * dv * 4},
                       {S_T, (size_t)BH * dk * dv * 4}};
  for (const Range& r : ins)
    if (overlap(rws, r)) return GLA_ERR_ALIAS;
  if (overlap(ins[5], ins[3]) || overlap(ins[6], ins[3])) return GLA_ERR_ALIAS;  // o, S_T vs x
  void* seg = workspace;
  // Validate the output pass fully before enqueueing anything.
  {
    const Range rq = ins[0], rk = ins[1], rv = ins[2], rs0 = ins[4], ro = ins[5], rst = ins[6];
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(S_T, 16) ||
        !aligned(S0, 16))
      return GLA_ERR_ALIGN;
    for (const Range& in : {rq, rk, rv, rs0})
      if (overlap(ro, in) || overlap(rst, in)) return GLA_ERR_ALIAS;
    if (overlap(ro, rst)) return GLA_ERR_ALIAS;
  }
  if (pl.segments > 1) {
    st = gla_segment_states(k, v, x, B, H, T, dk, dv, dtype, gate, &pl, seg, s_bytes, stream);
    if (st != GLA_OK) return st;
  }
  return gla_chunk_output(q, k, v, x, S0, o, S_T, B, H, T, dk, dv, dtype, gate, path, &pl, seg, s_bytes, stream);
}

gla_status_t gla_chunk_bwd(const void* q, const void* k, const void* v, const float* x, const float* S0,
                           const void* dO, const float* dS_T, float* dq, float* dk, float* dv, float* dx, float* dS0,
                           int B, int H, long long T, int dk_, int dv_, gla_dtype_t dtype, gla_gate_t gate,
                           gla_path_t path, void* workspace, size_t* workspace_bytes, void* stream) {
  if (!workspace_bytes) return GLA_ERR_NULL;
  gla_status_t st = check_sizes(B, H, T, dk_, dv_);
  if (st != GLA_OK) return st;
  if (!valid_dtype(dtype)) return GLA_ERR_DTYPE;
  if (!valid_gate(gate) || !valid_path(path)) return GLA_ERR_ARG;
  // plans of the three passes: dq and dk run with state dims (dv, dk), dv with (dk, dv)
  gla_plan_t pa, pc;
  // bf16 on the unified path: the gate gradient is formed inside the dq and dk passes (one
  // full-width slice each) instead of by the dx kernel
  const bool fused_dx = T > 0 && dtype == GLA_BF16 && path == GLA_PATH_UNIFIED;
  if (T > 0) {
    st = gla_plan_default(B, H, T, dv_, dk_, dtype, path, &pa);
    if (st != GLA_OK) return st;
    st = gla_plan_default(B, H, T, dk_, dv_, dtype, path, &pc);
    if (st != GLA_OK) return st;
    if (fused_dx && pa.dv_split != 1) {
      // one slice, segments doubled as the default plan does until the grid covers the CUs
      int cus = 0;
      st = device_cus(&cus);
      if (st != GLA_OK) return st;
      const long long units = (long long)B * H, nch = n_chunks(T);
      int segs = 1;
      while (segs < GLA_MAX_SEGMENTS && units * segs < cus && nch / (2LL * segs) >= 4) segs *= 2;
      if (segs > std::max(1LL, nch)) segs = (int)std::max(1LL, nch);
      pa.segments = segs;
      pa.dv_split = 1;
      pc = pa;
    }
  } else {
    pa.segments = pc.segments = 1;
    pa.dv_split = pc.dv_split = 1;
  }
  // the dq and dk passes store their state before / after every other chunk for dx; their
  // kernels do that for value slices of at least 32 columns
  if (T > 0 && (dk_ / pa.dv_split < 32)) return GLA_ERR_UNSUPPORTED;
  const long long BH = (long long)B * H;
  const long long nc = n_chunks(T);
  const size_t es = elem_size(dtype);
  const size_t tok = align_up((size_t)BH * (size_t)T * 4);
  const size_t tokr = align_up((size_t)BH * (size_t)nc * GLA_CHUNK * 4);
  // one stored state per pair of chunks (see store_chunk_state)
  const size_t chs = align_up((size_t)BH * (size_t)((nc + 1) / 2) * (size_t)dk_ * (size_t)dv_ * es);
  const size_t stt = align_up((size_t)BH * (size_t)dk_ * (size_t)dv_ * 4);
  const size_t segb = std::max(seg_bytes(BH, dv_, dk_, pa.segments), seg_bytes(BH, dk_, dv_, pc.segments));
  // b | b' (reversed, padded to whole chunks) | per-chunk states of the dq and dk passes |
  // final states of the three passes (the dv pass's is D_0) | segment states
  const size_t need = tok + tokr + 2 * chs + 3 * stt + segb;
  if (!workspace) {
    *workspace_bytes = need;
    return GLA_OK;
  }
  if (*workspace_bytes < need) return GLA_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return GLA_ERR_ALIGN;
  if (!dS0) return GLA_ERR_NULL;
  if (T > 0 && (!q || !k || !v || !x || !dO || !dq || !dk || !dv || !dx)) return GLA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dO, 16) || !aligned(S0, 16) ||
      !aligned(dS_T, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(dS0, 16) ||
      !aligned(x, 4) || !aligned(dx, 4))
    return GLA_ERR_ALIGN;
  const size_t nk = (size_t)BH * T * dk_, nv = (size_t)BH * T * dv_, ns = (size_t)BH * dk_ * dv_;
  const Range ins[] = {{q, nk * es}, {k, nk * es}, {v, nv * es}, {x, (size_t)BH * T * 4},
                       {S0, ns * 4}, {dO, nv * es}, {dS_T, ns * 4}};
  const Range outs[] = {{dq, nk * 4}, {dk, nk * 4}, {dv, nv * 4}, {dx, (size_t)BH * T * 4}, {dS0, ns * 4},
                        {workspace, need}};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const Range& in : ins)
      if (overlap(outs[i], in)) return GLA_ERR_ALIAS;
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlap(outs[i], outs[j])) return GLA_ERR_ALIAS;
  }
  char* w = (char*)workspace;
  float* b = (float*)w;
  float* br = (float*)(w + tok);
  void* Sfw = w + tok + tokr;
  void* Sbw = w + tok + tokr + chs;
  float* STt = (float*)(w + tok + tokr + 2 * chs);
  float* Sdk = (float*)(w + tok + tokr + 2 * chs + stt);
  float* D0 = (float*)(w + tok + tokr + 2 * chs + 2 * stt);
  void* seg = w + tok + tokr + 2 * chs + 3 * stt;
  hipStream_t s = (hipStream_t)stream;
  const int dt = dtype == GLA_BF16 ? 0 : 1;
  const int g = gate == GLA_GATE_BOUNDED_SIGMOID ? gla::kGateBoundedSigmoid : gla::kGateNegSoftplus;
  const bool diag = path == GLA_PATH_DIAG_BRANCH;
  const int pad = (int)(nc * GLA_CHUNK - T);
  hipError_t e = hipSuccess;
  if (T > 0) {
    e = gla::launch_gate_cumsum_pair(x, b, br, BH, T, g, s);
    // forward-shaped passes: segment pre-pass (when segmented) and output pass.  A
    // reversed pass reads its rows back to front behind `pad` zero rows, so that its
    // chunks are the forward chunks in reverse order.
    const auto make = [&](const void* pq, const void* pk, const void* pv, const float* pb, const float* ps0,
                          int s0t, int rev, float* po, float* pst, int sdk, int sdv, const gla_plan_t& pl) {
      gla::ChunkParams p = make_params(pq, pk, pv, pb, ps0, po, pst, B, H, T, sdk, sdv, pl, seg);
      p.reverse = rev;
      p.s0_transposed = s0t;
      if (rev) {
        p.pad = pad;
        p.Tl = T + pad;
      }
      return p;
    };
    const auto prepass = [&](gla::ChunkParams p, const gla_plan_t& pl) {
      if (pl.segments <= 1) return hipSuccess;
      p.grid = (int)(BH * pl.dv_split * (pl.segments - 1));
      return gla::launch_segment_states(p, dt, s);
    };
    const auto output = [&](gla::ChunkParams p, const gla_plan_t& pl, void* chunk_states) {
      p.state_out = chunk_states;
      p.grid = (int)(BH * pl.dv_split * pl.segments);
      return gla::launch_chunk_output(p, dt, diag, s);
    };
    // dq = forward(dO, v, k) from S0^T; stores S^T before every even chunk (fused_dx: forms
    // the pairs inside and entering each chunk into dx, and stores S^T before every chunk
    // whose crossing factor is not exactly 0)
    gla::ChunkParams pdq = make(dO, v, k, b, S0, 1, 0, dq, STt, dv_, dk_, pa);
    if (fused_dx) {
      pdq.gx_mode = 1;
      pdq.gx_op = q;
      pdq.gx_b = b;
      pdq.gx_out = dx;
      pdq.gx_states = Sfw;
    }
    if (e == hipSuccess) e = prepass(pdq, pa);
    if (e == hipSuccess) e = output(pdq, pa, fused_dx ? nullptr : Sfw);
    // dk = reversed forward(v, dO, q) from dS_T^T (stores D^T after every odd chunk; fused_dx:
    // adds the pairs leaving and crossing each chunk and finishes dx) and
    // dv = reversed forward(k, q, dO) from dS_T (final state D_0) carry the same state
    // gradient, transposed, under the same decays: with equal segment counts the dk
    // pass starts its segments from the dv pass's segment states, read transposed
    gla::ChunkParams pdk = make(v, dO, q, br, dS_T, 1, 1, dk, Sdk, dv_, dk_, pa);
    if (fused_dx) {
      pdk.gx_mode = 2;
      pdk.gx_op = k;
      pdk.gx_b = b;
      pdk.gx_x = x;
      pdk.gate = g;
      pdk.gx_out = dx;
      pdk.gx_states = Sfw;
    }
    void* const dk_states = fused_dx ? nullptr : Sbw;
    const gla::ChunkParams pdv = make(k, q, dO, br, dS_T, 0, 1, dv, D0, dk_, dv_, pc);
    if (pa.segments == pc.segments) {
      pdk.seg_transposed = 1;
      if (e == hipSuccess) e = prepass(pdv, pc);
      if (e == hipSuccess) e = output(pdk, pa, dk_states);
      if (e == hipSuccess) e = output(pdv, pc, nullptr);
    } else {
      if (e == hipSuccess) e = prepass(pdk, pa);
      if (e == hipSuccess) e = output(pdk, pa, dk_states);
      if (e == hipSuccess) e = prepass(pdv, pc);
      if (e == hipSuccess) e = output(pdv, pc, nullptr);
    }
    if (!fused_dx && e == hipSuccess)
      e = gla::launch_grad_dx(q, k, v, dO, b, x, Sfw, Sbw, dx, BH, T, dk_, dv_, dt, g, s);
  }
  if (e == hipSuccess) e = gla::launch_grad_ds0(D0, b, dS_T, dS0, BH, T, dk_, dv_, s);
  return e == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

gla_status_t gla_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* x, const float* S0,
                                  float* o, float* S_T, const long long* cu_seqlens, int N, int H, long long T,
                                  long long max_seqlen, int dk, int dv, gla_dtype_t dtype, gla_gate_t gate,
                                  gla_path_t path, const gla_plan_t* plan, void* workspace,
                                  size_t* workspace_bytes, void* stream) {
  if (!workspace_bytes) return GLA_ERR_NULL;
  if (N < 1) return GLA_ERR_SHAPE;
  gla_status_t st = check_sizes(N, H, T, dk, dv);
  if (st != GLA_OK) return st;
  if (max_seqlen < 0 || max_seqlen > T) return GLA_ERR_SHAPE;
  if (!valid_dtype(dtype)) return GLA_ERR_DTYPE;
  if (!valid_gate(gate) || !valid_path(path)) return GLA_ERR_ARG;
  // the plan is sized by the longest sequence; every sequence is cut into the same
  // number of segments
  gla_plan_t pl;
  if (plan) {
    st = plan_check_impl(N, H, max_seqlen, dk, dv, dtype, path, plan);
    if (st != GLA_OK) return st;
    pl = *plan;
  } else {
    int cus = 0;
    st = device_cus(&cus);
    if (st != GLA_OK) return st;
    st = default_plan_for(N, H, max_seqlen, dk, dv, dtype, path, cus, &pl);
    if (st != GLA_OK) return st;
  }
  const long long NH = (long long)N * H;
  const size_t s_bytes = seg_bytes(NH, dk, dv, pl.segments);
  const size_t o_bytes = align_up((size_t)N * 4);
  if (!workspace) {
    *workspace_bytes = s_bytes + o_bytes;
    return GLA_OK;
  }
  if (*workspace_bytes < s_bytes + o_bytes) return GLA_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return GLA_ERR_ALIGN;
  if (!S_T || !cu_seqlens) return GLA_ERR_NULL;
  if (T > 0 && (!q || !k || !v || !x || !o)) return GLA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(S_T, 16) ||
      !aligned(S0, 16) || !aligned(x, 4) || !aligned(cu_seqlens, 8))
    return GLA_ERR_ALIGN;
  const size_t es = elem_size(dtype);
  const Range ins[] = {{q, (size_t)H * T * dk * es},      {k, (size_t)H * T * dk * es},
                       {v, (size_t)H * T * dv * es},      {x, (size_t)H * T * 4},
                       {S0, (size_t)NH * dk * dv * 4},    {cu_seqlens, (size_t)(N + 1) * 8}};
  const Range outs[] = {{o, (size_t)H * T * dv * 4}, {S_T, (size_t)NH * dk * dv * 4},
                        {workspace, s_bytes + o_bytes}};
  for (size_t i = 0; i < 3; ++i) {
    for (const Range& in : ins)
      if (overlap(outs[i], in)) return GLA_ERR_ALIAS;
    for (size_t j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return GLA_ERR_ALIAS;
  }
  void* seg = workspace;
  hipStream_t s = (hipStream_t)stream;
  const int dt = dtype == GLA_BF16 ? 0 : 1;
  const long long max_chunks = n_chunks(max_seqlen);
  int* order = (int*)((char*)workspace + s_bytes);
  hipError_t e = gla::launch_varlen_order(cu_seqlens, N, T, max_chunks, order, s);
  gla::ChunkParams p = make_params(q, k, v, nullptr, S0, o, S_T, N, H, T, dk, dv, pl, seg);
  p.x = x;
  p.gate = gate == GLA_GATE_BOUNDED_SIGMOID ? gla::kGateBoundedSigmoid : gla::kGateNegSoftplus;
  p.cu_seqlens = cu_seqlens;
  p.nchunks = (int)max_chunks;
  p.unit_order = order;
  if (e == hipSuccess && pl.segments > 1) {
    p.grid = (int)(NH * pl.dv_split * (pl.segments - 1));
    e = gla::launch_segment_states(p, dt, s);
  }
  if (e == hipSuccess) {
    p.grid = (int)(NH * pl.dv_split * pl.segments);
    e = gla::launch_chunk_output(p, dt, path == GLA_PATH_DIAG_BRANCH, s);
  }
  return e == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

gla_status_t gla_decode_step(const void* q, const void* k, const void* v, const float* x, float* S, float* o,
                             int B, int H, int dk, int dv, gla_dtype_t dtype, gla_gate_t gate, int per_channel,
                             void* stream) {
  gla_status_t st = check_sizes(B, H, 1, dk, dv);
  if (st != GLA_OK) return st;
  if (!valid_dtype(dtype)) return GLA_ERR_DTYPE;
  if (!valid_gate(gate) || (per_channel != 0 && per_channel != 1)) return GLA_ERR_ARG;
  if (!q || !k || !v || !x || !S || !o) return GLA_ERR_NULL;
  if (!aligned(S, 16) || !aligned(o, 16) || !aligned(q, 4) || !aligned(k, 4) || !aligned(v, 4) || !aligned(x, 4))
    return GLA_ERR_ALIGN;
  const long long BH = (long long)B * H;
  const size_t es = elem_size(dtype);
  const Range ins[] = {{q, (size_t)BH * dk * es},
                       {k, (size_t)BH * dk * es},
                       {v, (size_t)BH * dv * es},
                       {x, (size_t)BH * (per_channel ? dk : 1) * 4}};
  const Range rs{S, (size_t)BH * dk * dv * 4}, ro{o, (size_t)BH * dv * 4};
  for (const Range& in : ins)
    if (overlap(rs, in) || overlap(ro, in)) return GLA_ERR_ALIAS;
  if (overlap(rs, ro)) return GLA_ERR_ALIAS;
  hipError_t e = gla::launch_decode_step(q, k, v, x, S, o, BH, dk, dv, dtype == GLA_BF16 ? 0 : 1,
                                         gate == GLA_GATE_BOUNDED_SIGMOID ? gla::kGateBoundedSigmoid
                                                                          : gla::kGateNegSoftplus,
                                         per_channel != 0, (hipStream_t)stream);
  return e == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

gla_status_t gla_plan_check_delta(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                                  const gla_plan_t* plan) {
  gla_status_t st = check_sizes(B, H, T, dk, dv);
  if (st != GLA_OK) return st;
  if (!valid_dtype(dtype)) return GLA_ERR_DTYPE;
  if (!plan) return GLA_ERR_NULL;
  const long long nc = n_chunks(T);
  if (plan->segments < 1 || plan->segments > GLA_MAX_SEGMENTS) return GLA_ERR_PLAN;
  if (plan->segments > std::max(1LL, nc)) return GLA_ERR_PLAN;
  const int sp = plan->dv_split;
  if (sp < 1 || dv % sp) return GLA_ERR_PLAN;
  if (!gla::delta_config_built(dtype == GLA_BF16 ? 0 : 1, dk, dv, dv / sp))
    return (dtype == GLA_F32 && (dk != 64 || dv != 64)) ? GLA_ERR_UNSUPPORTED : GLA_ERR_PLAN;
  return GLA_OK;
}

gla_status_t gla_plan_default_delta(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                                    gla_plan_t* plan) {
  if (!plan) return GLA_ERR_NULL;
  gla_status_t st = check_sizes(B, H, T, dk, dv);
  if (st != GLA_OK) return st;
  if (!valid_dtype(dtype)) return GLA_ERR_DTYPE;
  int cus = 0;
  st = device_cus(&cus);
  if (st != GLA_OK) return st;
  // whole value rows per workgroup (16 columns per wave; fp32: 64-column slices),
  // then sequence segments until the grid covers the compute units
  const long long BH = (long long)B * H;
  const long long nc = n_chunks(T);
  const int split = dtype == GLA_F32 ? dv / 64 : 1;
  int segs = 1;
  while (segs < GLA_MAX_SEGMENTS && BH * split * segs < cus && nc / (2LL * segs) >= 4) segs *= 2;
  plan->segments = segs;
  plan->dv_split = split;
  return gla_plan_check_delta(B, H, T, dk, dv, dtype, plan);
}

gla_status_t gla_chunk_fwd_delta(const void* q, const void* k, const void* v, const float* x, const float* beta,
                                 const float* S0, float* o, float* S_T, int B, int H, long long T, int dk, int dv,
                                 gla_dtype_t dtype, gla_gate_t gate, const gla_plan_t* plan, void* workspace,
                                 size_t* workspace_bytes, void* stream) {
  if (!workspace_bytes) return GLA_ERR_NULL;
  gla_status_t st = check_sizes(B, H, T, dk, dv);
  if (st != GLA_OK) return st;
  if (!valid_dtype(dtype)) return GLA_ERR_DTYPE;
  if (!valid_gate(gate)) return GLA_ERR_ARG;
  gla_plan_t pl;
  if (plan) {
    st = gla_plan_check_delta(B, H, T, dk, dv, dtype, plan);
    if (st != GLA_OK) return st;
    pl = *plan;
  } else {
    st = gla_plan_default_delta(B, H, T, dk, dv, dtype, &pl);
    if (st != GLA_OK) return st;
  }
  const long long BH = (long long)B * H;
  const int dt = dtype == GLA_BF16 ? 0 : 1;
  const size_t es = elem_size(dtype);
  const size_t b_bytes = align_up((size_t)BH * T * 4);
  const size_t t_bytes = align_up((size_t)BH * n_chunks(T) * GLA_CHUNK * GLA_CHUNK * es);  // Tinv per chunk
  const size_t h_bytes = pl.segments > 1 ? align_up((size_t)BH * (pl.segments - 1) * dk * dv * 4) : 0;
  const size_t f_bytes = pl.segments > 1 ? align_up((size_t)BH * (pl.segments - 1) * dk * dk * 4) : 0;
  const size_t r_bytes = pl.segments > 1 ? align_up((size_t)BH * n_chunks(T) * 4) : 0;
  const size_t need = std::max(b_bytes + t_bytes + h_bytes + f_bytes + r_bytes, kAlign);
  if (!workspace) {
    *workspace_bytes = need;
    return GLA_OK;
  }
  if (*workspace_bytes < need) return GLA_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return GLA_ERR_ALIGN;
  if (!S_T) return GLA_ERR_NULL;
  if (T > 0 && (!q || !k || !v || !x || !beta || !o)) return GLA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(S_T, 16) ||
      !aligned(S0, 16) || !aligned(x, 4) || !aligned(beta, 4))
    return GLA_ERR_ALIGN;
  const Range ins[] = {{q, (size_t)BH * T * dk * es}, {k, (size_t)BH * T * dk * es}, {v, (size_t)BH * T * dv * es},
                       {x, (size_t)BH * T * 4},       {beta, (size_t)BH * T * 4},    {S0, (size_t)BH * dk * dv * 4}};
  const Range outs[] = {{o, (size_t)BH * T * dv * 4}, {S_T, (size_t)BH * dk * dv * 4}, {workspace, need}};
  for (size_t i = 0; i < 3; ++i) {
    for (const Range& in : ins)
      if (overlap(outs[i], in)) return GLA_ERR_ALIAS;
    for (size_t j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return GLA_ERR_ALIAS;
  }
  char* w = (char*)workspace;
  gla::DeltaParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.b = (float*)w;
  p.beta = beta;
  p.S0 = S0;
  p.o = o;
  p.ST = S_T;
  p.Tinv = w + b_bytes;
  p.seg_state = pl.segments > 1 ? (float*)(w + b_bytes + t_bytes) : nullptr;
  p.seg_phi = pl.segments > 1 ? (float*)(w + b_bytes + t_bytes + h_bytes) : nullptr;
  p.reset = pl.segments > 1 ? (int*)(w + b_bytes + t_bytes + h_bytes + f_bytes) : nullptr;
  p.T = T;
  p.dk = dk;
  p.dv = dv;
  p.BH = (int)BH;
  p.nchunks = (int)n_chunks(T);
  p.nslices = pl.dv_split;
  p.segments = pl.segments;
  p.grid = (int)(BH * pl.dv_split * pl.segments);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (T > 0) {
    e = gla::launch_gate_cumsum(x, (float*)w, BH, T,
                                gate == GLA_GATE_BOUNDED_SIGMOID ? gla::kGateBoundedSigmoid : gla::kGateNegSoftplus,
                                false, s);
    if (e == hipSuccess) e = gla::launch_delta_prep(p, dt, s);
    if (e == hipSuccess) e = gla::launch_delta_segments(p, dt, s);
  }
  if (e == hipSuccess) e = gla::launch_delta_output(p, dt, s);
  return e == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

gla_status_t gla_plan_check_pc(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                               const gla_plan_t* plan) {
  gla_status_t st = check_sizes(B, H, T, dk, dv);
  if (st != GLA_OK) return st;
  if (!valid_dtype(dtype)) return GLA_ERR_DTYPE;
  if (!plan) return GLA_ERR_NULL;
  const long long nc = n_chunks(T);
  if (plan->segments < 1 || plan->segments > GLA_MAX_SEGMENTS) return GLA_ERR_PLAN;
  if (plan->segments > std::max(1LL, nc)) return GLA_ERR_PLAN;
  const int s = plan->dv_split;
  if (s != 1 && s != 2) return GLA_ERR_PLAN;
  if (dv % s) return GLA_ERR_PLAN;
  if (!gla::pc_config_built(dtype == GLA_BF16 ? 0 : 1, dk, dv / s))
    return (dtype == GLA_F32 && dk != 64) ? GLA_ERR_UNSUPPORTED : GLA_ERR_PLAN;
  return GLA_OK;
}

gla_status_t gla_plan_default_pc(int B, int H, long long T, int dk, int dv, gla_dtype_t dtype, gla_plan_t* plan) {
  if (!plan) return GLA_ERR_NULL;
  gla_status_t st = check_sizes(B, H, T, dk, dv);
  if (st != GLA_OK) return st;
  if (!valid_dtype(dtype)) return GLA_ERR_DTYPE;
  int cus = 0;
  st = device_cus(&cus);
  if (st != GLA_OK) return st;
  // whole value rows per workgroup (fp32: 64-column slices), then segments until
  // the grid covers the compute units
  const long long BH = (long long)B * H;
  const long long nc = n_chunks(T);
  const int split = (dtype == GLA_F32) ? dv / 64 : 1;
  const long long units = BH * split;
  int segs = 1;
  while (segs < GLA_MAX_SEGMENTS && units * segs < cus && nc / (2LL * segs) >= 4) segs *= 2;
  if (segs > std::max(1LL, nc)) segs = (int)std::max(1LL, nc);
  plan->segments = segs;
  plan->dv_split = split;
  return gla_plan_check_pc(B, H, T, dk, dv, dtype, plan);
}

gla_status_t gla_chunk_fwd_pc(const void* q, const void* k, const void* v, const float* x, const float* S0,
                              float* o, float* S_T, int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                              gla_gate_t gate, const gla_plan_t* plan, void* workspace, size_t* workspace_bytes,
                              void* stream) {
  if (!workspace_bytes) return GLA_ERR_NULL;
  gla_status_t st = check_sizes(B, H, T, dk, dv);
  if (st != GLA_OK) return st;
  if (!valid_dtype(dtype)) return GLA_ERR_DTYPE;
  if (!valid_gate(gate)) return GLA_ERR_ARG;
  gla_plan_t pl;
  if (plan) {
    st = gla_plan_check_pc(B, H, T, dk, dv, dtype, plan);
    if (st != GLA_OK) return st;
    pl = *plan;
  } else {
    st = gla_plan_default_pc(B, H, T, dk, dv, dtype, &pl);
    if (st != GLA_OK) return st;
  }
  const long long BH = (long long)B * H;
  const size_t hs = pl.segments > 1 ? align_up((size_t)BH * (pl.segments - 1) * dk * dv * 4) : 0;
  const size_t gs = pl.segments > 1 ? align_up((size_t)BH * pl.segments * dk * 4) : 0;
  if (!workspace) {
    *workspace_bytes = std::max<size_t>(hs + gs, kAlign);
    return GLA_OK;
  }
  if (*workspace_bytes < hs + gs) return GLA_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return GLA_ERR_ALIGN;
  if (!S_T) return GLA_ERR_NULL;
  if (T > 0 && (!q || !k || !v || !x || !o)) return GLA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(x, 16) || !aligned(o, 16) ||
      !aligned(S_T, 16) || !aligned(S0, 16))
    return GLA_ERR_ALIGN;
  const size_t es = elem_size(dtype);
  const Range ins[] = {{q, (size_t)BH * T * dk * es}, {k, (size_t)BH * T * dk * es}, {v, (size_t)BH * T * dv * es},
                       {x, (size_t)BH * T * dk * 4},  {S0, (size_t)BH * dk * dv * 4}};
  const Range outs[] = {{o, (size_t)BH * T * dv * 4}, {S_T, (size_t)BH * dk * dv * 4},
                        {pl.segments > 1 ? workspace : nullptr, hs + gs}};
  for (size_t i = 0; i < 3; ++i) {
    for (const Range& in : ins)
      if (overlap(outs[i], in)) return GLA_ERR_ALIAS;
    for (size_t j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return GLA_ERR_ALIAS;
  }
  gla::PcParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.x = x;
  p.S0 = S0;
  p.o = o;
  p.ST = S_T;
  p.seg_state = pl.segments > 1 ? (float*)workspace : nullptr;
  p.seg_decay = pl.segments > 1 ? (float*)((char*)workspace + hs) : nullptr;
  p.T = T;
  p.dk = dk;
  p.dv = dv;
  p.BH = (int)BH;
  p.nchunks = (int)n_chunks(T);
  p.segments = pl.segments;
  p.nslices = pl.dv_split;
  p.gate = gate == GLA_GATE_BOUNDED_SIGMOID ? gla::kGateBoundedSigmoid : gla::kGateNegSoftplus;
  const int dt = dtype == GLA_BF16 ? 0 : 1;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (T == 0) {
    // nothing decays: S_T = S0 (or zero), one workgroup per head writes it
    p.segments = 1;
    p.nchunks = 0;
    p.grid = (int)(BH * pl.dv_split);
    return gla::launch_pc_chunk_output(p, dt, s) == hipSuccess ? GLA_OK : GLA_ERR_HIP;
  }
  if (pl.segments > 1) {
    p.grid = (int)(BH * pl.dv_split * (pl.segments - 1));
    e = gla::launch_pc_segment_states(p, dt, s);
  }
  if (e == hipSuccess) {
    p.grid = (int)(BH * pl.dv_split * pl.segments);
    e = gla::launch_pc_chunk_output(p, dt, s);
  }
  return e == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

gla_status_t gla_chunk_fwd(const void* q, const void* k, const void* v, const float* x, const float* S0, float* o,
                           float* S_T, int B, int H, long long T, int dk, int dv, gla_dtype_t dtype,
                           gla_gate_t gate, gla_path_t path, void* workspace, size_t* workspace_bytes,
                           void* stream) {
  return gla_chunk_fwd_plan(q, k, v, x, S0, o, S_T, B, H, T, dk, dv, dtype, gate, path, nullptr, workspace,
                            workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- no-allocation forward
//
// The forward's only scratch memory is the segment workspace (the pre-pass's local
// and prefix states and segment log-decays).  gla_chunk_fwd_noalloc takes it from this
// file-scope device array instead of a caller's buffer.  Each GPU holds its own copy
// of the array (at its own address) until the process ends.  In host code the array's
// name is only a host-side stand-in: the device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is passed on.
// Nothing in it needs to start at zero: every byte a call reads is written earlier in
// the same call.  Calls that overlap on one GPU share the array and race.
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on first use there).
gla_status_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GLA_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GLA_ERR_HIP;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return GLA_OK;
}

}  // namespace

extern "C" gla_status_t gla_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* x,
                                              const float* S0, float* o, float* S_T, int B, int H, long long T,
                                              int dk, int dv, gla_dtype_t dtype, gla_gate_t gate, gla_path_t path,
                                              void* stream) {
  gla_status_t st = check_sizes(B, H, T, dk, dv);
  if (st != GLA_OK) return st;
  if (!valid_dtype(dtype)) return GLA_ERR_DTYPE;
  if (!valid_gate(gate) || !valid_path(path)) return GLA_ERR_ARG;
  gla_plan_t pl;
  st = gla_plan_default(B, H, T, dk, dv, dtype, path, &pl);
  if (st != GLA_OK) return st;
  // the workspace this plan needs must fit the array
  if (fwd_workspace_bytes((long long)B * H, dk, dv, pl.segments) > kScratchBytes) return GLA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != GLA_OK) return st;
  size_t n = kScratchBytes;
  return gla_chunk_fwd_plan(q, k, v, x, S0, o, S_T, B, H, T, dk, dv, dtype, gate, path, &pl, ws, &n, stream);
}

extern "C" gla_status_t gla_debug_flags(unsigned int* flags) {
  if (!flags) return GLA_ERR_NULL;
#ifdef GLA_DEBUG
  const unsigned int words[] = {gla::debug_word_gate_cumsum(), gla::debug_word_chunk_kernels(),
                                gla::debug_word_ws_kernels(),  gla::debug_word_bwd_kernels(),
                                gla::debug_word_pc_kernels(),  gla::debug_word_decode(),
                                gla::debug_word_delta_kernels()};
  unsigned int v = 0;
  for (unsigned int w : words) {
    if (w == ~0u) return GLA_ERR_HIP;
    v |= w;
  }
  *flags = v;
  return GLA_OK;
#else
  return GLA_ERR_UNSUPPORTED;
#endif
}

extern "C" gla_status_t gla_debug_selftest(const float* probe, float* out, void* stream) {
  if (!probe || !out) return GLA_ERR_NULL;
#ifdef GLA_DEBUG
  return gla::launch_debug_selftest(probe, out, (hipStream_t)stream) == hipSuccess ? GLA_OK : GLA_ERR_HIP;
#else
  return GLA_ERR_UNSUPPORTED;
#endif
}

extern "C" gla_status_t gla_lane_selftest(const float* in, float* out, void* stream) {
  if (!in || !out) return GLA_ERR_NULL;
  return gla::launch_lane_selftest(in, out, (hipStream_t)stream) == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}
