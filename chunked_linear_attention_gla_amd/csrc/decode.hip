// decode.hip -- one recurrent step of gated linear attention per (batch, head).
//
// Source: "Engineering Long-Context Training for Trillion-Parameter MoE Models:
// Three Key Breakthroughs" (§3.1 the state carried from position to position and
// multiplied by the per-position decay; §3.2 the bounded gate).  The chunked form
// exists for whole sequences; generating one token at a time is the recurrence
// itself:
//     S <- diag(a) S + k v^T,   o = S^T q,   a = e^{g(x)} (one scalar, or one per
//     key channel)
// with S the fp32 state carried between calls, updated in place.
//
// The step reads and writes the whole state (2 dk dv 4 bytes per head) and moves
// a few hundred bytes of q, k, v, x, o: it is bound by HBM bandwidth.  One
// workgroup per head; each thread owns 4 consecutive value columns of a set of
// state rows, so a wavefront reads and writes whole contiguous rows with 16-byte
// accesses, and the column sums of o are reduced through LDS.
#include "gla_device.h"
#include "gla_internal.h"

namespace gla {

namespace {

constexpr int kDecodeThreads = 256;

template <typename T>
__device__ __forceinline__ float load_f32(const T* p, long long i) {
  return static_cast<float>(p[i]);
}

template <typename T, bool PC>
__global__ void __launch_bounds__(kDecodeThreads) decode_step_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                                    const T* __restrict__ v, const float* __restrict__ x,
                                                                    float* __restrict__ S, float* __restrict__ o,
                                                                    int dk, int dv, int gate) {
  __shared__ float sq[128], sk[128], sa[128], sv[128];
  __shared__ float4 red[kDecodeThreads];
  const int tid = threadIdx.x;
  const long long bh = blockIdx.x;
  if (tid < dk) {
    sq[tid] = load_f32(q, bh * dk + tid);
    sk[tid] = load_f32(k, bh * dk + tid);
    if (PC) {
      const float xv = x[bh * dk + tid];
      sa[tid] = exp_e(gate == kGateBoundedSigmoid ? gate_bounded_sigmoid(xv) : gate_neg_softplus(xv));
    }
  }
  if (tid < dv) sv[tid] = load_f32(v, bh * dv + tid);
  float a_scalar = 1.0f;
  if (!PC) {
    const float xv = x[bh];
    a_scalar = exp_e(gate == kGateBoundedSigmoid ? gate_bounded_sigmoid(xv) : gate_neg_softplus(xv));
  }
  __syncthreads();

  const int ncg = dv / 4;                 // 4-column groups per row
  const int nrg = kDecodeThreads / ncg;   // row groups
  const int cg = tid % ncg, rg = tid / ncg;
  float* Sh = S + bh * (long long)dk * dv;
  const float4 vv = make_float4(sv[4 * cg], sv[4 * cg + 1], sv[4 * cg + 2], sv[4 * cg + 3]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // The state is read and written once per step, and a batch of states larger than the
  // caches is the case that matters: non-temporal accesses (measured: 56.2 -> 51.0 us per
  // step for 64 x 32 heads rotated over 768 MiB of state; non-temporal stores alone
  // changed nothing).
  for (int d = rg; d < dk; d += nrg) {
    floatx4* p = reinterpret_cast<floatx4*>(Sh + (long long)d * dv) + cg;
    floatx4 s = __builtin_nontemporal_load(p);
    const float a = PC ? sa[d] : a_scalar;
    const float kd = sk[d], qd = sq[d];
    s[0] = a * s[0] + kd * vv.x;
    s[1] = a * s[1] + kd * vv.y;
    s[2] = a * s[2] + kd * vv.z;
    s[3] = a * s[3] + kd * vv.w;
    __builtin_nontemporal_store(s, p);
    acc.x += qd * s[0];
    acc.y += qd * s[1];
    acc.z += qd * s[2];
    acc.w += qd * s[3];
  }
  red[tid] = acc;
  __syncthreads();
  if (rg == 0) {
    float4 t = acc;
    for (int r = 1; r < nrg; ++r) {
      const float4 u = red[r * ncg + cg];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    reinterpret_cast<float4*>(o + bh * dv)[cg] = t;
  }
}

}  // namespace

hipError_t launch_decode_step(const void* q, const void* k, const void* v, const float* x, float* S, float* o,
                              long long BH, int dk, int dv, int dtype, int gate, bool per_channel,
                              hipStream_t stream) {
  if (BH == 0) return hipSuccess;
  if (BH > 0x7FFFFFFFLL || dk > 128 || dv > 128 || dv % 4 || (kDecodeThreads % (dv / 4))) return hipErrorInvalidValue;
  const dim3 grid((unsigned)BH), block(kDecodeThreads);
#define GLA_DEC(TT, PCV)                                                                                       \
  hipLaunchKernelGGL((decode_step_kernel<TT, PCV>), grid, block, 0, stream, static_cast<const TT*>(q),         \
                     static_cast<const TT*>(k), static_cast<const TT*>(v), x, S, o, dk, dv, gate)
  if (dtype == 0) {
    if (per_channel) GLA_DEC(bf16, true);
    else GLA_DEC(bf16, false);
  } else {
    if (per_channel) GLA_DEC(float, true);
    else GLA_DEC(float, false);
  }
#undef GLA_DEC
  return hipGetLastError();
}

// debug builds: this unit's LDS-check word (see GLA_CHECK_LDS)
GLA_DEBUG_ACCESSOR(debug_word_decode)

}  // namespace gla
