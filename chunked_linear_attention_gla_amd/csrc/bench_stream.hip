// bench_stream.hip -- a measurement helper, not part of the method: the forward
// pass's byte mix as one flat grid-stride stream, the practical streaming rate of the
// device against which the output pass's achieved bandwidth is read.
//
// Per 16-byte unit j: one 16-byte load from each of three inputs at j and two
// 16-byte stores to the output at 2j and 2j + 1, i.e. 48 bytes read for 32 written --
// the 768 : 512 bytes of q, k, v (bf16) and o (fp32) per token-head at d = 128.
// Every workgroup walks units blockIdx * 1024 + k * gridDim * 1024, four units per
// thread per step with all loads of a step issued before its stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ void __launch_bounds__(kThreads) stream_mix_kernel(const uint4* __restrict__ a, const uint4* __restrict__ b,
                                                              const uint4* __restrict__ c, uint4* __restrict__ out,
                                                              unsigned long long n) {
  const unsigned long long step = (unsigned long long)gridDim.x * kThreads * kUnroll;
  for (unsigned long long base = (unsigned long long)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n;
       base += step) {
    uint4 x[kUnroll][3];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const unsigned long long j = base + (unsigned long long)u * kThreads;
      if (j < n) {
        x[u][0] = a[j];
        x[u][1] = b[j];
        x[u][2] = c[j];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const unsigned long long j = base + (unsigned long long)u * kThreads;
      if (j < n) {
        // a value that depends on all three loads, so none of them can be dropped
        const uint4 s = make_uint4(x[u][0].x ^ x[u][1].x ^ x[u][2].x, x[u][0].y ^ x[u][1].y ^ x[u][2].y,
                                   x[u][0].z ^ x[u][1].z ^ x[u][2].z, x[u][0].w ^ x[u][1].w ^ x[u][2].w);
        out[2 * j] = s;
        out[2 * j + 1] = s;
      }
    }
  }
}

}  // namespace

extern "C" gla_status_t gla_bench_stream(const void* a, const void* b, const void* c, void* out,
                                         unsigned long long units, int grid, void* stream) {
  if (units == 0) return GLA_OK;
  if (!a || !b || !c || !out) return GLA_ERR_NULL;
  if (grid < 1) return GLA_ERR_ARG;
  if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c | (uintptr_t)out) % 16) return GLA_ERR_ALIGN;
  const uintptr_t o0 = (uintptr_t)out, o1 = o0 + 32 * units;
  for (const void* in : {a, b, c}) {
    const uintptr_t i0 = (uintptr_t)in, i1 = i0 + 16 * units;
    if (i0 < o1 && o0 < i1) return GLA_ERR_ALIAS;
  }
  hipLaunchKernelGGL(stream_mix_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, (const uint4*)a,
                     (const uint4*)b, (const uint4*)c, (uint4*)out, units);
  return hipGetLastError() == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}
