// gate_cumsum.hip -- log-decay gate and chunk-local cumulative log-decay.
//
// Sources: "Engineering Long-Context Training for Trillion-Parameter MoE Models:
// Three Key Breakthroughs" (§3.1 the per-position cumulative decay Gamma; §3.2 the
// gate g = g_min * sigmoid(x) with g_min = -5, replacing g = -softplus(.)).
//
// b[t] = sum_{i in chunk(t), i <= t} g(x[i]) is log Gamma restarted at each 64-token
// chunk.  The chunk kernels read every decay factor they need from b: the
// tile-start prefix r_u = b[16u - 1], the chunk total gamma = b[63] and
// differences of entries.  A 64-lane wavefront scans one chunk at a time, lane j
// owning token j, and forms the inclusive scan with DPP row shifts inside each
// 16-lane row followed by the three row totals read across lanes.
#include "gla_device.h"
#include "gla_internal.h"

namespace gla {

template <int CTRL>
__device__ __forceinline__ float dpp_or_zero(float v) {
  // row-local lane shift; lanes whose source falls outside the 16-lane row read 0
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}

// inclusive prefix sum over the 64 lanes of the wavefront
__device__ __forceinline__ float wave_inclusive_scan(float v, int lane) {
  v += dpp_or_zero<0x111>(v);  // row_shr:1
  v += dpp_or_zero<0x112>(v);  // row_shr:2
  v += dpp_or_zero<0x114>(v);  // row_shr:4
  v += dpp_or_zero<0x118>(v);  // row_shr:8
  const float t0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15));
  const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
  const float t2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47));
  const int row = lane >> 4;
  float off = 0.0f;
  if (row >= 1) off = t0;
  if (row >= 2) off = off + t1;
  if (row >= 3) off = off + t2;
  return v + off;
}

// Each wavefront takes kGateChunksPerWave consecutive chunks and issues all their
// loads before the first scan, so one memory round trip covers several chunks.
constexpr int kGateChunksPerWave = 8;

template <int GATE, bool REV>
__global__ void __launch_bounds__(256) gate_cumsum_kernel(const float* __restrict__ x,
                                                          float* __restrict__ b, long long T,
                                                          long long chunks_per_head,
                                                          long long total_chunks) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long first = ((long long)blockIdx.x * 4 + wave) * kGateChunksPerWave;
  if (first >= total_chunks) return;  // uniform across the wavefront
  // REV: the reversed sequence has pad absent tokens first, then original tokens
  // T-1 .. 0; logical token t > pad takes the gate of original token T + pad - t
  // (the token after it in original order), t <= pad none (g = 0)
  const long long pad = REV ? (kChunk - T % kChunk) % kChunk : 0;
  const long long Tl = T + pad;
  long long bh = first / chunks_per_head;
  long long c = first - bh * chunks_per_head;
  float g[kGateChunksPerWave];
  long long dst[kGateChunksPerWave];
  bool valid[kGateChunksPerWave];
#pragma unroll
  for (int i = 0; i < kGateChunksPerWave; ++i) {
    const long long t = c * kChunk + lane;
    valid[i] = first + i < total_chunks && t < Tl;
    dst[i] = bh * Tl + t;
    // unconditional load (token 0 of x stands in for absent tokens) so that the
    // compiler issues every load of the wavefront before the first gate
    const bool has_gate = valid[i] && (!REV || t > pad);
    const float xv = x[has_gate ? bh * T + (REV ? T + pad - t : t) : 0];
    const float gv = (GATE == kGateBoundedSigmoid) ? gate_bounded_sigmoid(xv) : gate_neg_softplus(xv);
    g[i] = has_gate ? gv : 0.0f;
    if (++c == chunks_per_head) {
      c = 0;
      ++bh;
    }
  }
#pragma unroll
  for (int i = 0; i < kGateChunksPerWave; ++i) {
    if (first + i >= total_chunks) break;  // uniform across the wavefront
    const float s = wave_inclusive_scan(g[i], lane);
    if (valid[i]) b[dst[i]] = s;
  }
}

// Packed sequences: wavefront `chunk` of unit bh = n * H + h covers tokens
// [cu[n] + 64 c, ...) of head h, so chunks restart at every sequence start.  Offsets
// are clamped into [0, T] and lengths to max_chunks chunks (inconsistent offsets give
// wrong values, never an access outside x or b).
template <int GATE>
__global__ void __launch_bounds__(256) gate_cumsum_varlen_kernel(const float* __restrict__ x,
                                                                 float* __restrict__ b,
                                                                 const long long* __restrict__ cu,
                                                                 int H, long long T, long long max_chunks,
                                                                 long long total_chunks) {
  const int lane = threadIdx.x & 63;
  const long long chunk = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (chunk >= total_chunks) return;  // uniform across the wavefront
  const long long bh = chunk / max_chunks;
  const long long c = chunk - bh * max_chunks;
  const long long n = bh / H, h = bh - n * H;
  long long a = cu[n], e = cu[n + 1];
  a = a < 0 ? 0 : (a > T ? T : a);
  e = e < a ? a : (e > T ? T : e);
  if (e - a > max_chunks * kChunk) e = a + max_chunks * kChunk;
  const long long t = c * kChunk + lane;
  if (c * kChunk >= e - a) return;  // uniform: the sequence has fewer chunks
  const bool valid = t < e - a;
  const long long row = h * T + a + t;
  float g = 0.0f;
  if (valid) g = (GATE == kGateBoundedSigmoid) ? gate_bounded_sigmoid(x[row]) : gate_neg_softplus(x[row]);
  const float s = wave_inclusive_scan(g, lane);
  if (valid) b[row] = s;
}

constexpr int kOrderThreads = 1024;
constexpr int kOrderBuckets = 8192;

__global__ void __launch_bounds__(kOrderThreads) varlen_order_kernel(const long long* __restrict__ cu, int N,
                                                                      long long T, long long max_chunks,
                                                                      int* __restrict__ order) {
  __shared__ int hist[kOrderBuckets];
  __shared__ int part[kOrderThreads];
  const int tid = threadIdx.x;
  const auto bucket = [&](int n) {
    long long a = cu[n], e = cu[n + 1];
    a = a < 0 ? 0 : (a > T ? T : a);
    e = e < a ? a : (e > T ? T : e);
    long long c = (e - a + kChunk - 1) / kChunk;
    if (c > max_chunks) c = max_chunks;
    // descending: the longest sequences get the first buckets
    const long long scaled = max_chunks < kOrderBuckets ? c : c * (kOrderBuckets - 1) / max_chunks;
    return (int)(kOrderBuckets - 1 - scaled);
  };
  for (int i = tid; i < kOrderBuckets; i += kOrderThreads) hist[i] = 0;
  __syncthreads();
  for (int n = tid; n < N; n += kOrderThreads) atomicAdd(&hist[bucket(n)], 1);
  __syncthreads();
  // exclusive prefix over the buckets: 8 per thread, then across threads
  constexpr int per = kOrderBuckets / kOrderThreads;
  int local = 0;
  for (int j = 0; j < per; ++j) local += hist[tid * per + j];
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < kOrderThreads; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - local;
  for (int j = 0; j < per; ++j) {
    const int h = hist[tid * per + j];
    hist[tid * per + j] = run;
    run += h;
  }
  __syncthreads();
  for (int n = tid; n < N; n += kOrderThreads) order[atomicAdd(&hist[bucket(n)], 1)] = n;
}

hipError_t launch_varlen_order(const long long* cu_seqlens, int N, long long T, long long max_chunks, int* order,
                               hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(varlen_order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, cu_seqlens, N, T,
                     max_chunks < 1 ? 1 : max_chunks, order);
  return hipGetLastError();
}

hipError_t launch_gate_cumsum_varlen(const float* x, float* b, const long long* cu_seqlens, int N, int H,
                                     long long T, long long max_chunks, int gate, hipStream_t stream) {
  const long long total = (long long)N * H * max_chunks;
  if (total == 0) return hipSuccess;
  const long long blocks = (total + 3) / 4;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(256);
  if (gate == kGateBoundedSigmoid)
    hipLaunchKernelGGL((gate_cumsum_varlen_kernel<kGateBoundedSigmoid>), grid, block, 0, stream, x, b, cu_seqlens,
                       H, T, max_chunks, total);
  else
    hipLaunchKernelGGL((gate_cumsum_varlen_kernel<kGateNegSoftplus>), grid, block, 0, stream, x, b, cu_seqlens, H,
                       T, max_chunks, total);
  return hipGetLastError();
}

hipError_t launch_gate_cumsum(const float* x, float* b, long long BH, long long T, int gate,
                              bool reversed_shift, hipStream_t stream) {
  const long long cph = (T + kChunk - 1) / kChunk;
  const long long total = BH * cph;
  if (total == 0) return hipSuccess;
  const long long blocks = (total + 4 * kGateChunksPerWave - 1) / (4 * kGateChunksPerWave);
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(256);
  if (gate == kGateBoundedSigmoid) {
    if (reversed_shift)
      hipLaunchKernelGGL((gate_cumsum_kernel<kGateBoundedSigmoid, true>), grid, block, 0, stream, x, b, T, cph, total);
    else
      hipLaunchKernelGGL((gate_cumsum_kernel<kGateBoundedSigmoid, false>), grid, block, 0, stream, x, b, T, cph, total);
  } else {
    if (reversed_shift)
      hipLaunchKernelGGL((gate_cumsum_kernel<kGateNegSoftplus, true>), grid, block, 0, stream, x, b, T, cph, total);
    else
      hipLaunchKernelGGL((gate_cumsum_kernel<kGateNegSoftplus, false>), grid, block, 0, stream, x, b, T, cph, total);
  }
  return hipGetLastError();
}

}  // namespace gla
