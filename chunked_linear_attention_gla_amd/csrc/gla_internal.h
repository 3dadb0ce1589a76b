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
  const float* b;         // [BH][T] chunk-local cumulative log-decay, or nullptr: then the
                          //    kernels form it themselves from x (gate + 64-lane scan)
  const float* x;         // [BH][T] gate pre-activation (read when b is nullptr)
  int gate;               // GateKind of x
  const float* S0;        // [BH][dk][dv] or nullptr
  float* o;               // [BH][T][dv]
  float* ST;              // [BH][dk][dv]
  float* seg_state;       // [BH][segments-1][dk][dv]  local final states, then (after the prefix
                          //                           scan) the states reached from zero
  float* seg_decay;       // [BH][segments]            total log-decay per segment
  long long T;
  int dk, dv;
  int BH;
  int nchunks;            // ceil(T / 64)
  int segments;           // sequence segments per head; segment p owns chunks
                          // [p * nchunks / segments, (p + 1) * nchunks / segments)
  int nslices;            // value-column slices per head
  int grid;               // workgroups in this launch
  int reverse;            // 1: logical token t is stored at row T-1+pad-t of q, k, v and o
                          //    (b and the states are in logical order)
  int pad;                // reversed passes: absent logical tokens before the first real
                          //    one, so that logical chunks line up with the stored chunks
  long long Tl;           // logical length, T + pad: per-head length and stride of b
  int s0_transposed;      // 1: S0 is stored [dv][dk] (the transpose of the state)
  int seg_transposed;     // 1: the segment states are those of the transposed pass
                          //    ([dv][dk] per segment; same decays)
  void* state_out;        // optional: one state per pair of chunks, in the operand dtype,
                          //    in MFMA-fragment order (see store_chunk_state): the state
                          //    before each even chunk; a reversed pass stores the state after
                          //    each odd (logical) chunk and after the last one
  const long long* cu_seqlens;  // packed sequences: N+1 token offsets (device memory) into the
                          //    rows of every head; nullptr for the dense [BH][T] layout.  With
                          //    it, q, k, v, o, b are [H][T][.] (T = total tokens), the work
                          //    unit bh = n * H + h is sequence n of head h, and nchunks is
                          //    the largest sequence's chunk count
  int H;                  // heads (packed sequences only)
  const int* unit_order;  // packed sequences: sequence indices, longest first (the work
                          //    order); nullptr: dense order
  // Backward pass, gradient of the gate folded into the dq and dk passes (dense bf16
  // layout, one full-width slice; see the pair terms in bwd_kernels.hip):
  int gx_mode;            // 0: none.  1 (dq pass, forward time): the pairs inside each chunk
                          //    and the pairs entering it, W_t -> gx_out; the state before every
                          //    chunk whose crossing factor is not exactly 0 -> gx_states.
                          //    2 (dk pass, reversed time): the pairs leaving each chunk and
                          //    those crossing it, dx_t = g'(x_t) (W_t + ...) -> gx_out
  const void* gx_op;      // [BH][T][dv]: q (mode 1) or k (mode 2), the operand the pass lacks
  const float* gx_b;      // [BH][T] forward chunk-local cumulative log-decay
  const float* gx_x;      // [BH][T] gate pre-activation (mode 2: the slope g'(x))
  float* gx_out;          // [BH][T] W (mode 1 writes it, mode 2 reads it and writes dx)
  void* gx_states;        // [BH][nchunks][dk x dv] bf16 states in fragment order
};

// Byte offset of logical token t's row in a per-unit tensor of T rows with rows of
// row_bytes bytes.  Rows outside the unit (t >= T, or t < 0 once reversed) get an
// offset beyond every descriptor's range that cannot wrap round to a valid one
// when an instruction offset is added: loads there return zeros, stores are
// dropped.
// (Accepted sizes keep T * row_bytes below 2^32 - 2^16, so 32-bit arithmetic is exact.)
__host__ __device__ inline unsigned row_offset(const ChunkParams& p, unsigned T, unsigned t, unsigned row_bytes) {
  const int r = p.reverse ? (int)T - 1 + p.pad - (int)t : (int)t;
  return (r >= 0 && r < (int)T) ? (unsigned)r * row_bytes : 0xFFFFF000u;
}

// b = chunk-local cumsum of g(x), [BH][T].  reversed_shift: the gate of the time-reversed
// sequence, shifted by one token and preceded by pad = (-T mod 64) absent tokens,
// [BH][T + pad]: g'(tau) = g(x[T + pad - tau]) for tau > pad, 0 for tau <= pad -- the
// decays a_{t+1} that the state gradient crosses when run backwards, with chunks
// that line up with the forward chunks.
hipError_t launch_gate_cumsum(const float* x, float* b, long long BH, long long T, int gate,
                              bool reversed_shift, hipStream_t stream);
// Both of the above (b and the reversed-padded b') in one launch.
hipError_t launch_gate_cumsum_pair(const float* x, float* b, float* br, long long BH, long long T, int gate,
                                   hipStream_t stream);
// Packed sequences: q, k, v, x and o are [H][T][.] (T = total tokens), sequence n of
// every head covers rows [cu_seqlens[n], cu_seqlens[n+1]) and restarts its chunks
// there; at most max_chunks chunks per sequence.
// order[0..N) = the sequences by chunk count, longest first (one workgroup, counting
// sort; the order among equal counts is unspecified and changes no result).
hipError_t launch_varlen_order(const long long* cu_seqlens, int N, long long T, long long max_chunks, int* order,
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

// Per-channel decay (pc_kernels.hip): x [BH][T][dk]; the gate and the chunk-local
// cumulative sum are computed inside the kernels.
struct PcParams {
  const void* q;          // [BH][T][dk]
  const void* k;          // [BH][T][dk]
  const void* v;          // [BH][T][dv]
  const float* x;         // [BH][T][dk] gate pre-activation, one per key channel
  const float* S0;        // [BH][dk][dv] or nullptr
  float* o;               // [BH][T][dv]
  float* ST;              // [BH][dk][dv]
  float* seg_state;       // [BH][segments-1][dk][dv]  local final states
  float* seg_decay;       // [BH][segments][dk]        per-channel log2-decay of each segment
  long long T;
  int dk, dv;
  int BH;
  int nchunks;
  int segments;
  int nslices;
  int grid;
  int gate;               // GateKind
};
// Built (dtype, dk, slice) combinations: bf16 with dk, slice in {64, 128}; fp32 with 64, 64.
bool pc_config_built(int dtype, int dk, int slice);
hipError_t launch_pc_segment_states(const PcParams& p, int dtype, hipStream_t stream);
hipError_t launch_pc_chunk_output(const PcParams& p, int dtype, hipStream_t stream);

// Gated delta rule (delta_kernels.hip).
struct DeltaParams {
  const void* q;          // [BH][T][dk]
  const void* k;          // [BH][T][dk]
  const void* v;          // [BH][T][dv]
  const float* b;         // [BH][T] chunk-local cumulative log-decay
  const float* beta;      // [BH][T] write strength
  const float* S0;        // [BH][dk][dv] or nullptr
  float* o;               // [BH][T][dv]
  float* ST;              // [BH][dk][dv]
  void* Tinv;             // [BH][nchunks][64][64] operand dtype: (I + diag(beta) L)^-1 of each
                          //    chunk, zero above its diagonal 16x16 blocks
  float* seg_state;       // [BH][segments-1][dk][dv] local final state of each segment
  float* seg_phi;         // [BH][segments-1][dk][dk] state transition of each segment
  int* reset;             // [BH][nchunks] 1 where the chunk's transition e^gamma I - (k e^{gamma-b})^T W
                          //    scales any incoming state by less than 2^-114 (written by the
                          //    per-chunk pass; the local-state half starts at the last such
                          //    chunk of its segment), or nullptr
  long long T;
  int dk, dv;
  int BH;
  int nchunks;
  int nslices;
  int segments;
  int grid;
};
bool delta_config_built(int dtype, int dk, int dv, int slice);
hipError_t launch_delta_segments(const DeltaParams& p, int dtype, hipStream_t stream);
hipError_t launch_delta_prep(const DeltaParams& p, int dtype, hipStream_t stream);
hipError_t launch_delta_output(const DeltaParams& p, int dtype, hipStream_t stream);

// One recurrent step per head (decode.hip): S <- diag(a) S + k v^T in place, o = S^T q.
// q, k [BH][dk], v [BH][dv] in the operand dtype; x [BH] or, per_channel, [BH][dk];
// S [BH][dk][dv] and o [BH][dv] fp32.  dk, dv <= 128, dv a multiple of 4.
hipError_t launch_decode_step(const void* q, const void* k, const void* v, const float* x, float* S, float* o,
                              long long BH, int dk, int dv, int dtype, int gate, bool per_channel,
                              hipStream_t stream);

// Backward-pass kernels (bwd_kernels.hip).
//   dx from the pairs that span each token (see bwd_kernels.hip); Sfw and Sbw are the
//   per-chunk states stored by the dq pass (S^T before each chunk) and by the dk pass
//   (D^T after each chunk, before the next chunk's decay);
hipError_t launch_grad_dx(const void* q, const void* k, const void* v, const void* dO, const float* b,
                          const float* x, const void* Sfw, const void* Sbw, float* dx, long long BH, long long T,
                          int dk_, int dv_, int dtype, int gate, hipStream_t stream);
//   dS0 = e^{b[0]} D0 (dS_T, or zero, when T = 0).
hipError_t launch_grad_ds0(const float* D0, const float* b, const float* dST, float* dS0, long long BH,
                           long long T, int dk_, int dv_, hipStream_t stream);

#ifdef GLA_DEBUG
// read and clear the LDS-check word of each kernel translation unit (debug builds)
unsigned int debug_word_gate_cumsum();
unsigned int debug_word_chunk_kernels();
unsigned int debug_word_ws_kernels();
unsigned int debug_word_bwd_kernels();
unsigned int debug_word_pc_kernels();
unsigned int debug_word_decode();
unsigned int debug_word_delta_kernels();
// the LDS checks' self-test: one workgroup of 64 threads; out: 64 floats it writes
hipError_t launch_debug_selftest(const float* g, float* out, hipStream_t stream);
#endif
constexpr int kLaneSelftestSlots = 17;  // output slots of gla_lane_selftest (64 floats each)
hipError_t launch_lane_selftest(const float* in, float* out, hipStream_t stream);

}  // namespace gla
