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
// owning token j (wave_inclusive_scan).  The forward kernels run the same scan on x
// themselves; this kernel serves the backward pass, the delta rule and the stage
// entry point gla_gate_cumsum.
#include "gla_device.h"
#include "gla_internal.h"

namespace gla {

// Each wavefront takes kGateChunksPerWave consecutive chunks and issues all their
// loads before the first scan, so one memory round trip covers several chunks.
constexpr int kGateChunksPerWave = 8;

// The scan of one workgroup's chunks (block = the workgroup's index within its scan).
template <int GATE, bool REV>
__device__ __forceinline__ void gate_cumsum_block(const float* __restrict__ x, float* __restrict__ b, long long T,
                                                  long long chunks_per_head, long long total_chunks, long long block) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long first = (block * 4 + wave) * kGateChunksPerWave;
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

template <int GATE, bool REV>
__global__ void __launch_bounds__(256) gate_cumsum_kernel(const float* __restrict__ x,
                                                          float* __restrict__ b, long long T,
                                                          long long chunks_per_head,
                                                          long long total_chunks) {
  gate_cumsum_block<GATE, REV>(x, b, T, chunks_per_head, total_chunks, blockIdx.x);
}

// Both scans of the backward pass in one launch: the first `fwd_blocks` workgroups write
// b, the others the reversed-padded b' (the two are independent).
template <int GATE>
__global__ void __launch_bounds__(256) gate_cumsum_pair_kernel(const float* __restrict__ x, float* __restrict__ b,
                                                               float* __restrict__ br, long long T,
                                                               long long chunks_per_head, long long total_chunks,
                                                               long long fwd_blocks) {
  const long long blk = blockIdx.x;
  if (blk < fwd_blocks) gate_cumsum_block<GATE, false>(x, b, T, chunks_per_head, total_chunks, blk);
  else gate_cumsum_block<GATE, true>(x, br, T, chunks_per_head, total_chunks, blk - fwd_blocks);
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

hipError_t launch_gate_cumsum_pair(const float* x, float* b, float* br, long long BH, long long T, int gate,
                                   hipStream_t stream) {
  const long long cph = (T + kChunk - 1) / kChunk;  // the reversed-padded sequence has as many chunks
  const long long total = BH * cph;
  if (total == 0) return hipSuccess;
  const long long blocks = (total + 4 * kGateChunksPerWave - 1) / (4 * kGateChunksPerWave);
  if (2 * blocks > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(2 * blocks)), block(256);
  if (gate == kGateBoundedSigmoid)
    hipLaunchKernelGGL((gate_cumsum_pair_kernel<kGateBoundedSigmoid>), grid, block, 0, stream, x, b, br, T, cph, total,
                       blocks);
  else
    hipLaunchKernelGGL((gate_cumsum_pair_kernel<kGateNegSoftplus>), grid, block, 0, stream, x, b, br, T, cph, total,
                       blocks);
  return hipGetLastError();
}

#ifdef GLA_DEBUG
// Self-test of the LDS checks: asks them about an address one element past this
// kernel's 256-byte LDS allocation and about a global pointer, and accesses neither;
// both bits must come up.
__global__ void __launch_bounds__(64) debug_selftest_kernel(const float* g, float* out) {
  __shared__ float tile[64];
  tile[threadIdx.x] = (float)threadIdx.x;
  __syncthreads();
  if (threadIdx.x == 0) {
    GLA_CHECK_LDS(tile + 64, 4);
    GLA_CHECK_LDS(g, 4);
  }
  out[threadIdx.x] = tile[63 - threadIdx.x];
}

hipError_t launch_debug_selftest(const float* g, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(debug_selftest_kernel, dim3(1), dim3(64), 0, stream, g, out);
  return hipGetLastError();
}
#endif

// One wavefront runs each cross-lane helper the kernels rely on over `in` (64
// values; the swaps pair it with in + 100) and writes slot k of `out` (64 values per
// slot), so that a test can hold every lane layout against its definition.
__global__ void __launch_bounds__(64) lane_selftest_kernel(const float* in, float* out) {
  const int l = threadIdx.x;
  const float v = in[l];
  float r[kLaneSelftestSlots];
  r[0] = group_max<8>(v);
  r[1] = group_max<16>(v);
  r[2] = group_sum<8>(v);
  r[3] = group_sum<16>(v);
  r[4] = strided_exclusive_scan<4>(v, l);
  r[5] = strided_exclusive_scan<8>(v, l);
  r[6] = strided_exclusive_scan<16>(v, l);
  r[7] = wave_inclusive_scan(v, l);
  r[8] = row_broadcast<0>(v);
  r[9] = row_broadcast<1>(v);
  r[10] = row_broadcast<2>(v);
  r[11] = row_broadcast<3>(v);
  r[12] = row_sum4(v);
  uint32_t a = __builtin_bit_cast(uint32_t, v), b = __builtin_bit_cast(uint32_t, v + 100.0f);
  permlane16_swap_pair(a, b);
  r[13] = __builtin_bit_cast(float, a);
  r[14] = __builtin_bit_cast(float, b);
  a = __builtin_bit_cast(uint32_t, v);
  b = __builtin_bit_cast(uint32_t, v + 100.0f);
  permlane32_swap_pair(a, b);
  r[15] = __builtin_bit_cast(float, a);
  r[16] = __builtin_bit_cast(float, b);
#pragma unroll
  for (int k = 0; k < kLaneSelftestSlots; ++k) out[k * 64 + l] = r[k];
}

hipError_t launch_lane_selftest(const float* in, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(lane_selftest_kernel, dim3(1), dim3(64), 0, stream, in, out);
  return hipGetLastError();
}

// debug builds: this unit's LDS-check word (see GLA_CHECK_LDS)
GLA_DEBUG_ACCESSOR(debug_word_gate_cumsum)

}  // namespace gla
