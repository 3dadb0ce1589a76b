// chunk_common.h -- pieces shared by the chunk kernels: launch shape of the
// compute waves, causal tile numbering, chunk decay scalars and the MFMA state
// update.
#pragma once

#include "gla_device.h"
#include "gla_internal.h"

namespace gla {

template <typename T, int DK, int DVS>
struct Cfg {
  static constexpr int NB = DVS >= 32 ? 2 : 1;         // 16-column blocks per wave
  static constexpr int CPW = 16 * NB;                  // value columns per wave
  static constexpr int NW = DVS / CPW;                 // waves per workgroup
  static constexpr int NT = 64 * NW;                   // threads per workgroup

  static constexpr int PAD = Elem<T>::kPad;
  static constexpr int QLD = DK + PAD;   // row stride of Qh, Kh (and raw q, k)
  static constexpr int TLD = 64 + 4;     // row stride of the attention matrix A (8-byte stores and
                                         // fragment reads of the bf16 tile are conflict-free)
  static constexpr int QU = 8 * DK / NT;   // 8-element q (and k) units per thread per chunk
  static constexpr int VU = 8 * DVS / NT;  // 8-element v units per thread per chunk
  static constexpr int DB = DK / 16;       // 16-row blocks of the key dimension
  static constexpr int KS = DK / 32;       // K-steps over the key dimension
  static_assert(QU >= 1 && 8 * DK == QU * NT, "q staging must divide evenly");
  static_assert(VU >= 1 && 8 * DVS == VU * NT, "v staging must divide evenly");
};

// Causal 16x16 tiles of a 64x64 chunk, (query tile jb, key tile ib) with ib <= jb,
// numbered row by row: 0 -> (0,0), 1 -> (1,0), 2 -> (1,1), 3 -> (2,0), ...  The
// strictly-below-diagonal tiles are numbered the same way without the diagonal.
// Evaluated at compile time inside unrolled loops (no table in memory).
__host__ __device__ constexpr int tri_j(int t) { return t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0; }
__host__ __device__ constexpr int tri_i(int t) { return t - tri_j(t) * (tri_j(t) + 1) / 2; }
__host__ __device__ constexpr int off_j(int t) { return t >= 3 ? 3 : t >= 1 ? 2 : 1; }
__host__ __device__ constexpr int off_i(int t) { return t - (off_j(t) - 1) * off_j(t) / 2; }
static_assert(tri_j(9) == 3 && tri_i(9) == 3 && tri_j(4) == 2 && tri_i(4) == 1, "tile numbering");
static_assert(off_j(5) == 3 && off_i(5) == 2 && off_j(2) == 2 && off_i(2) == 1, "tile numbering");

// Work index of this workgroup: consecutive indices on one XCD for the dense layout;
// plain dispatch order for packed sequences, whose units are then taken longest first.
__device__ __forceinline__ int work_index(const ChunkParams& p) {
  return p.unit_order ? (int)blockIdx.x : xcd_linear_index(blockIdx.x, p.grid);
}

// Unit (sequence n, head h) -> n * H + h of the r-th unit in work order.
__device__ __forceinline__ int unit_of(const ChunkParams& p, int r) {
  if (!p.unit_order) return r;
  const int i = r / p.H;
  return p.unit_order[i] * p.H + (r - i * p.H);
}

// Rows of one work unit (a head of the dense layout, or one sequence of one head
// when sequences are packed) in the streamed tensors.
struct HeadSpan {
  long long row0;   // first row in q, k, v, o
  long long brow0;  // first entry in b
  uint32_t T;       // rows of the unit
  uint32_t Tl;      // entries of b (T + pad for a reversed pass)
  int nchunks;
};

// Packed sequences: the offsets are clamped into [0, total] and the length to the
// chunk count the launch was sized for, so inconsistent offsets give wrong values,
// never an access outside the tensors.
__device__ __forceinline__ HeadSpan head_span(const ChunkParams& p, int bh) {
  HeadSpan s;
  if (!p.cu_seqlens) {
    s.row0 = (long long)bh * p.T;
    s.brow0 = (long long)bh * p.Tl;
    s.T = (uint32_t)p.T;
    s.Tl = (uint32_t)p.Tl;
    s.nchunks = p.nchunks;
    return s;
  }
  const int n = bh / p.H, h = bh - n * p.H;
  long long a = p.cu_seqlens[n], e = p.cu_seqlens[n + 1];
  a = a < 0 ? 0 : (a > p.T ? p.T : a);
  e = e < a ? a : (e > p.T ? p.T : e);
  if (e - a > (long long)p.nchunks * kChunk) e = a + (long long)p.nchunks * kChunk;
  s.row0 = (long long)h * p.T + a;
  s.brow0 = s.row0;
  s.T = (uint32_t)(e - a);
  s.Tl = s.T;
  s.nchunks = (int)((e - a + kChunk - 1) / kChunk);
  return s;
}

// Per-unit buffer descriptors of the streamed tensors (sized to the unit's rows) and
// the unit's row counts.
struct HeadBuffers {
  rsrc_t q, k, v, b, x, o;
  uint32_t T, Tl;
};

template <typename T, int DK>
__device__ __forceinline__ HeadBuffers head_buffers(const ChunkParams& p, const HeadSpan& s) {
  HeadBuffers hb;
  const uint32_t es = (uint32_t)sizeof(T);
  hb.q = p.q ? make_rsrc(static_cast<const T*>(p.q) + s.row0 * DK, s.T * DK * es) : make_rsrc(nullptr, 0u);
  hb.k = make_rsrc(static_cast<const T*>(p.k) + s.row0 * DK, s.T * DK * es);
  hb.v = make_rsrc(static_cast<const T*>(p.v) + s.row0 * p.dv, s.T * (uint32_t)p.dv * es);
  hb.b = p.b ? make_rsrc(p.b + s.brow0, s.Tl * 4u) : make_rsrc(nullptr, 0u);
  hb.x = p.x ? make_rsrc(p.x + s.brow0, s.Tl * 4u) : make_rsrc(nullptr, 0u);
  hb.o = p.o ? make_rsrc(p.o + s.row0 * p.dv, s.T * (uint32_t)p.dv * 4u) : make_rsrc(nullptr, 0u);
  hb.T = s.T;
  hb.Tl = s.Tl;
  return hb;
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Cumulative log-decay of one chunk: lane j of every wave holds b_j; the tile
// boundaries are read out once per chunk as wave-uniform scalars.
struct ChunkDecay {
  float b;               // b_j for this lane's token j
  float r1, r2, r3, gam; // b_15, b_31, b_47, b_63
  __device__ __forceinline__ explicit ChunkDecay(float bl)
      : b(bl), r1(lane_value(bl, 15)), r2(lane_value(bl, 31)), r3(lane_value(bl, 47)), gam(lane_value(bl, 63)) {}
  // r_u = b_{16u-1}, the cumulative decay before tile u (r_0 = 0)
  __device__ __forceinline__ float r(int u) const { return u == 0 ? 0.0f : u == 1 ? r1 : u == 2 ? r2 : r3; }
  // E_u = b_{16u+15}, the cumulative decay at the end of tile u
  __device__ __forceinline__ float end(int u) const { return u == 0 ? r1 : u == 1 ? r2 : u == 2 ? r3 : gam; }
  // b of another token of the chunk
  __device__ __forceinline__ float at(int j) const { return __shfl(b, j); }
};

// ---------------------------------------------------------------- log-decays of a chunk
//
// Lane j of a wave needs b_j, the chunk-local cumulative log-decay of token j of the
// chunk.  It comes either from the b buffer (the backward pass's reversed passes) or
// from the gate input x: g = gate(x) per token and the 64-lane inclusive scan, the
// same routine as the gate kernel, so both give the same bits.  The load is issued
// with the chunk's other prefetch loads (decay_load) and finished when the chunk is
// staged (decay_finish), so prefetching never waits for it.  Tokens past the unit's
// end have g = 0: their b repeats the last token's (x path: the scan adds zeros; b
// path: the load is clamped to the last entry).
__device__ __forceinline__ float decay_load(const HeadBuffers& hb, const ChunkParams& p, uint32_t t0, int lane) {
  const uint32_t t = t0 + (uint32_t)lane;
  if (p.b) return buf_load4(hb.b, (t < hb.Tl ? t : hb.Tl - 1) * 4u);
  return buf_load4(hb.x, t * 4u);  // past the end: out of range, reads 0 (replaced in decay_finish)
}

__device__ __forceinline__ float gate_of(int gate, float x) {
  return gate == kGateBoundedSigmoid ? gate_bounded_sigmoid(x) : gate_neg_softplus(x);
}

__device__ __forceinline__ float decay_finish(const HeadBuffers& hb, const ChunkParams& p, float v, uint32_t t0,
                                              int lane) {
  if (p.b) return v;
  const float g = t0 + (uint32_t)lane < hb.Tl ? gate_of(p.gate, v) : 0.0f;
  return wave_inclusive_scan(g, lane);
}

__device__ __forceinline__ float sigmoid_f(float x) {
  if (x >= 0.0f) return 1.0f / (1.0f + exp_e(-x));
  const float e = exp_e(x);
  return e / (1.0f + e);
}

// Slope g'(x) of the gate (backward pass).
template <int GATE>
__device__ __forceinline__ float gate_slope(float x) {
  if (GATE == kGateNegSoftplus) return sigmoid_f(-x);  // d/dx log sigmoid(x)
  const float sg = sigmoid_f(x);
  return -5.0f * sg * (1.0f - sg);                      // d/dx -5 sigmoid(x)
}

// Shared memory for the workgroup-wide search below (x path).
struct SegScanSmem {
  int last_zero[16];
  float gsum[16];
};

// First chunk of [c_begin, c_end) that a segment pre-pass has to run, and the
// segment's total log-decay.  The state update multiplies the carried state by
// e^{gamma_c}; where that factor is exactly zero in fp32 (gamma_c below about -103.3),
// the state after chunk c does not depend on anything before it.  So the pass may
// start at the last such chunk from a zero state and end with the same local state,
// bit for bit (up to the sign of an exact zero).  gamma_c = b at the chunk's last token,
// read as the pass itself reads it.  Same results in every lane of the wave.
__device__ __forceinline__ int segment_first_live_chunk(const HeadBuffers& hb, int c_begin, int c_end,
                                                        float& gsum) {
  const int lane = threadIdx.x & 63;
  int last_zero = -1;
  float s = 0.0f;
  for (int c0 = c_begin; c0 < c_end; c0 += 64) {  // wave-uniform
    const int c = c0 + lane;
    if (c < c_end) {
      const uint32_t t = (uint32_t)c * kChunk + (kChunk - 1);
      const float gam = buf_load4(hb.b, (t < hb.Tl ? t : hb.Tl - 1) * 4u);
      if (exp_e(gam) == 0.0f) last_zero = c;
      s += gam;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    last_zero = max(last_zero, __shfl_xor(last_zero, off));
    s += __shfl_xor(s, off);
  }
  gsum = s;
  return last_zero >= 0 ? last_zero : c_begin;
}

// The same from the gate input x, with every wave of the workgroup taking part: wave w
// scans chunks c_begin + 8w .. +7, then + 8 NW, ... (all loads of a batch issued before
// its first scan), the per-wave results meet in LDS.  gamma_c = lane 63 of the chunk's
// scan, exactly the value the pass forms when it runs chunk c.  Contains a barrier:
// every wave of the workgroup must call it.  Same results in every lane.
template <int NW>
__device__ __forceinline__ int segment_first_live_chunk_x(const HeadBuffers& hb, const ChunkParams& p, int c_begin,
                                                          int c_end, float& gsum, SegScanSmem& sh) {
  static_assert(NW <= 16, "one LDS slot per wave");
  constexpr int kBatch = 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  int last_zero = -1;
  float s = 0.0f;
  for (int c0 = c_begin + wave * kBatch; c0 < c_end; c0 += NW * kBatch) {  // wave-uniform
    float xv[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) xv[i] = decay_load(hb, p, (uint32_t)min(c0 + i, c_end - 1) * kChunk, lane);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = c0 + i;
      if (c < c_end) {  // wave-uniform
        const float gam = lane_value(decay_finish(hb, p, xv[i], (uint32_t)c * kChunk, lane), 63);
        if (exp_e(gam) == 0.0f) last_zero = c;
        s += gam;
      }
    }
  }
  if (lane == 0) {
    sh.last_zero[wave] = last_zero;
    sh.gsum[wave] = s;
  }
  __syncthreads();
  last_zero = -1;
  s = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    last_zero = max(last_zero, sh.last_zero[w]);
    s += sh.gsum[w];
  }
  gsum = s;
  return last_zero >= 0 ? last_zero : c_begin;
}

// fp32 state slice of one wave: S[d = 16 db + 4 g + e][n = 16 nb + r16], e = 0..3
template <typename T, int DK, int DVS>
struct StateAcc {
  floatx4 s[Cfg<T, DK, DVS>::NB][Cfg<T, DK, DVS>::DB];
};

// v[n][i] operand fragments of one wave for the chunk's two token K-steps
template <typename T, int DK, int DVS>
struct VFrags {
  typename Elem<T>::Frag f[Cfg<T, DK, DVS>::NB][2];
};

// kp: token-major [64][KLD]
template <typename T, int DK, int DVS, int KLD = DK + 16>
__device__ __forceinline__ void state_update(StateAcc<T, DK, DVS>& S, const VFrags<T, DK, DVS>& Vf,
                                             const T* kp, float decay, int lane) {
  using E = Elem<T>;
  using C = Cfg<T, DK, DVS>;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) S.s[nb][db] *= decay;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const typename E::Frag ka = TokTile<T, DK, KLD>::load(kp, ks * 32, db * 16, lane);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) E::mfma(S.s[nb][db], ka, Vf.f[nb][ks]);
    }
  }
}

// v fragments of one wave's columns for both token K-steps of the chunk; vv: [64][VLD]
template <typename T, int DK, int DVS, int VLD = DVS + 16>
__device__ __forceinline__ void load_v_frags(VFrags<T, DK, DVS>& Vf, const T* vv, int wave, int lane) {
  using C = Cfg<T, DK, DVS>;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      Vf.f[nb][ks] = TokTile<T, DVS, VLD>::load(vv, ks * 32, wave * C::CPW + nb * 16, lane);
}

// Initial state of a segment: S0 (or zero; stored [dv][dk] when s0_transposed)
// decayed over the earlier segments of the same unit, plus the state P_{seg-1}
// that the segment prefix scan leaves for them (reached from a zero state at the
// unit's start; stored transposed when seg_transposed):
//   S = e^{Gamma_0 + .. + Gamma_{seg-1}} S0 + P_{seg-1}.
// All loads are issued before the first use, so this is one round trip to memory.
// The wave's slice of S: d = 16 db + 4 g + e, n = wcol + 16 nb + r16.
template <typename T, int DK, int DVS>
__device__ __forceinline__ void load_initial_state(StateAcc<T, DK, DVS>& S, const ChunkParams& p, int bh, int seg,
                                                   int wcol, int g, int r16) {
  using C = Cfg<T, DK, DVS>;
  const long long i0 = (long long)bh * DK * p.dv;
  floatx4 s0[C::NB][C::DB], pre[C::NB][C::DB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = db * 16 + 4 * g + e;
        const int n = wcol + nb * 16 + r16;
        s0[nb][db][e] = !p.S0 ? 0.0f
                        : p.s0_transposed ? p.S0[i0 + (long long)n * DK + d]
                                          : p.S0[i0 + (long long)d * p.dv + n];
      }
  const float* P = seg > 0 ? p.seg_state + ((long long)bh * (p.segments - 1) + seg - 1) * DK * p.dv : nullptr;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = db * 16 + 4 * g + e;
        const int n = wcol + nb * 16 + r16;
        pre[nb][db][e] = !P ? 0.0f : p.seg_transposed ? P[(long long)n * DK + d] : P[(long long)d * p.dv + n];
      }
  // e^{sum of the earlier segments' log-decays}: lane ps holds Gamma_ps (seg <= 63)
  float f0 = 1.0f;
  if (p.S0 && seg > 0) {
    const int lane = g * 16 + r16;
    float gl = lane < seg ? p.seg_decay[(long long)bh * p.segments + lane] : 0.0f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) gl += __shfl_xor(gl, off);
    f0 = exp_e(gl);
  }
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) S.s[nb][db][e] = f0 * s0[nb][db][e] + pre[nb][db][e];
}

// Per-chunk state storage (for the backward pass), one state per pair of chunks: the
// forward pass stores the state before every even chunk, the reversed pass the state
// after every odd chunk and after the last one (logical chunk index cc, slot cc / 2);
// the other state of each pair is one chunk step away from the stored one, and the dx
// kernel takes that step itself.  In the operand dtype, in MFMA-fragment order
//     [bh][slot][g32 = value column / 32][nb][db][lane][e]
// so that each lane writes (and a kernel with the same fragment layout later reads)
// its own 4 consecutive elements: S[16 db + 4 g + e][32 g32 + 16 nb + r16].
template <typename T, int DK, int DVS>
__device__ __forceinline__ void store_chunk_state(const StateAcc<T, DK, DVS>& S, const ChunkParams& p, int bh,
                                                  int c, int wcol, int lane) {
  using C = Cfg<T, DK, DVS>;
  static_assert(C::NB == 2, "chunk states are stored in groups of 32 value columns");
  const int cc = p.reverse ? p.nchunks - 1 - c : c;
  const bool keep = p.reverse ? ((cc & 1) != 0 || cc == p.nchunks - 1) : (cc & 1) == 0;
  if (!keep) return;  // wave-uniform
  const long long slots = (p.nchunks + 1) / 2;
  T* base = static_cast<T*>(p.state_out) +
            ((((long long)bh * slots + (cc >> 1)) * (p.dv / 32) + wcol / 32) * 2) * (long long)C::DB * 256;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      T* dst = base + ((nb * C::DB + db) * 64 + lane) * 4;
      if constexpr (sizeof(T) == 2) {
        typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
        bf16x4v w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = static_cast<__bf16>(S.s[nb][db][e]);
        *reinterpret_cast<bf16x4v*>(dst) = w;
      } else {
        *reinterpret_cast<floatx4*>(dst) = S.s[nb][db];
      }
    }
}

// Writes the wave's slice of a state to dst [dk][dv] (one head).
template <typename T, int DK, int DVS>
__device__ __forceinline__ void store_state(const StateAcc<T, DK, DVS>& S, float* dst, int dv, int wcol, int g,
                                            int r16) {
  using C = Cfg<T, DK, DVS>;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = db * 16 + 4 * g + e;
        const int n = wcol + nb * 16 + r16;
        dst[(long long)d * dv + n] = S.s[nb][db][e];
      }
}

}  // namespace gla
