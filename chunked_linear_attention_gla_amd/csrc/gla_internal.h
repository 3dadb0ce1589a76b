// gla_internal.h -- host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace gla {

enum GateKind { kGateBoundedSigmoid = 0, kGateNegSoftplus = 1 };

// Everything a chunk kernel needs; passed by value to the kernels.
struct ChunkParams {
  const void* q;          // [BH][T][dk]
  const void* k;          // [BH][T][dk]
  const void* v;          // [BH][T][dv]
  const float* b;         // [BH][T] chunk-local cumulative log-decay
  const float* S0;        // [BH][dk][dv] or nullptr
  float* o;               // [BH][T][dv]
  float* ST;              // [BH][dk][dv]
  float* seg_state;       // [BH][segments-1][dk][dv]  local final states
  float* seg_decay;       // [BH][segments]            total log-decay per segment
  long long T;
  int dk, dv;
  int BH;
  int nchunks;            // ceil(T / 64)
  int segments;           // sequence segments per head; segment p owns chunks
                          // [p * nchunks / segments, (p + 1) * nchunks / segments)
  int nslices;            // value-column slices per head
  int grid;               // workgroups in this launch
};

hipError_t launch_gate_cumsum(const float* x, float* b, long long BH, long long T, int gate,
                              hipStream_t stream);

// dtype: 0 = bf16, 1 = fp32.  slice = dv / nslices.  diag: element-wise diagonal tiles.
bool chunk_config_built(int dtype, int dk, int slice, bool diag);
hipError_t launch_segment_states(const ChunkParams& p, int dtype, hipStream_t stream);
hipError_t launch_chunk_output(const ChunkParams& p, int dtype, bool diag, hipStream_t stream);
// The wave-specialised kernels (ws_kernels.hip) cover bf16, dk in {64, 128},
// slices of 32, 64 or 128 columns; launch_chunk_output and launch_segment_states
// route those to them.
bool ws_kernels_supported(int dtype, int dk, int slice);
hipError_t launch_chunk_output_ws(const ChunkParams& p, int dk, int slice, bool diag, hipStream_t stream);
hipError_t launch_segment_states_ws(const ChunkParams& p, int dk, int slice, hipStream_t stream);

}  // namespace gla
