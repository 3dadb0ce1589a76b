// bench_stream.hip -- a measurement helper, not part of the method: the forward
// pass's byte mix as one flat grid-stride stream, the practical streaming rate of the
// device against which the output pass's achieved bandwidth is read.
//
// Per 16-byte unit j: one 16-byte load from each of three inputs at j and two
// 16-byte stores to the output at 2j and 2j + 1, i.e. 48 bytes read for 32 written --
// the 768 : 512 bytes of q, k, v (bf16) and o (fp32) per token-head at d = 128.
// Every workgroup walks units blockIdx * 1024 + k * gridDim * 1024, four units per
// thread per step with all loads of a step issued before its stores.
//
// A second helper keeps the output pass's launch shape and order of access and drops
// its arithmetic: one workgroup of 512 threads per (head, segment), at most one per
// compute unit, each walking its segment's 64-token chunks in order with the next
// chunk's loads in flight while the current chunk's output is stored.  Its rate is
// the ceiling of that access pattern, below the flat stream's.
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

constexpr int kChunkThreads = 512;
constexpr int kChunkInUnits = 1024;   // 16-byte units of one input per chunk: 64 rows x 128 bf16
constexpr int kChunkOutUnits = 2048;  // of the output: 64 rows x 128 fp32
constexpr int kReserveUnits = 6144;   // 96 KB of LDS: no second workgroup fits a unit (160 KB)

__device__ __forceinline__ uint4 xor3(const uint4& a, const uint4& b, const uint4& c) {
  return make_uint4(a.x ^ b.x ^ c.x, a.y ^ b.y ^ c.y, a.z ^ b.z ^ c.z, a.w ^ b.w ^ c.w);
}

// Workgroup w: head w / segments, segment w % segments of chunks_per_head / segments
// chunks.  Thread t loads units t and t + 512 of each input's chunk and stores units
// t, t + 512, t + 1024, t + 1536 of the output's chunk; output unit j of a chunk is
// the xor of the three inputs' unit j mod 1024, so no load can be dropped.  `never`
// is always 0: its branch keeps the LDS reservation in the kernel and is not taken.
__global__ void __launch_bounds__(kChunkThreads) chunk_stream_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ v, uint4* __restrict__ o,
    long long chunks_per_head, int segments, int never) {
  __shared__ uint4 reserve[kReserveUnits];
  const int t = threadIdx.x;
  const long long head = blockIdx.x / segments, seg = blockIdx.x % segments;
  const long long per_seg = chunks_per_head / segments;
  const long long c0 = head * chunks_per_head + seg * per_seg, c1 = c0 + per_seg;
  uint4 cur[6];
  auto load = [&](long long c, uint4* r) {
    const long long u = c * kChunkInUnits + t;
    r[0] = q[u]; r[1] = q[u + kChunkThreads];
    r[2] = k[u]; r[3] = k[u + kChunkThreads];
    r[4] = v[u]; r[5] = v[u + kChunkThreads];
  };
  load(c0, cur);
  for (long long c = c0; c < c1; ++c) {
    // unconditional (the last chunk loads itself again, in bounds), so that the
    // stores below wait only for the current chunk's loads
    uint4 nxt[6];
    load(c + 1 < c1 ? c + 1 : c, nxt);
    const uint4 s0 = xor3(cur[0], cur[2], cur[4]), s1 = xor3(cur[1], cur[3], cur[5]);
    uint4* oc = o + c * kChunkOutUnits + t;
    oc[0] = s0;
    oc[kChunkThreads] = s1;
    oc[2 * kChunkThreads] = s0;
    oc[3 * kChunkThreads] = s1;
    if (never) {
      reserve[(t * 12) % kReserveUnits] = s0;
      oc[0] = reserve[(t * 12 + 12) % kReserveUnits];
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) cur[i] = nxt[i];
  }
}

}  // namespace

extern "C" gla_status_t gla_bench_chunk_stream(const void* q, const void* k, const void* v, void* o, int BH,
                                               long long T, int segments, void* stream) {
  if (BH == 0 || T == 0) return GLA_OK;
  if (!q || !k || !v || !o) return GLA_ERR_NULL;
  if (BH < 0 || T < 0 || segments < 1 || T % 64 != 0 || (T / 64) % segments != 0) return GLA_ERR_SHAPE;
  if ((long long)BH * segments > 0x7FFFFFFFLL) return GLA_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) % 16) return GLA_ERR_ALIGN;
  const unsigned long long in_bytes = (unsigned long long)BH * T * 256ull;
  const uintptr_t o0 = (uintptr_t)o, o1 = o0 + 2 * in_bytes;
  for (const void* in : {q, k, v}) {
    const uintptr_t i0 = (uintptr_t)in, i1 = i0 + in_bytes;
    if (i0 < o1 && o0 < i1) return GLA_ERR_ALIAS;
  }
  hipLaunchKernelGGL(chunk_stream_kernel, dim3((unsigned)(BH * segments)), dim3(kChunkThreads), 0,
                     (hipStream_t)stream, (const uint4*)q, (const uint4*)k, (const uint4*)v, (uint4*)o, T / 64,
                     segments, 0);
  return hipGetLastError() == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

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
