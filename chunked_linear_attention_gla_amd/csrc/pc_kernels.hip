// pc_kernels.hip -- chunked GLA forward with a per-channel decay on gfx950 matrix cores.
//
// Source: "Engineering Long-Context Training for Trillion-Parameter MoE Models:
// Three Key Breakthroughs" (§3.1 the per-position cumulative decay Gamma and its
// reciprocal inside a chunk; §3.2 the bounded gate g = -5 sigmoid(x); §3.3 all
// causal tiles on the dense matrix product).
//
// Here the decay has one value per key channel d:
//     S_t[d][n] = a_t[d] S_{t-1}[d][n] + k_t[d] v_t[n],   o_t = S_t^T q_t,
// with x of layout [BH][T][dk].  With b_j[d] the chunk-local cumulative log-decay of
// channel d, r_u[d] = b_{16u-1}[d] (r_0 = 0) and gamma[d] = b_63[d]:
//   weight of k_i[d] v_i in o_j (i <= j)   = e^{b_j[d] - b_i[d]}
//   weight of row d of S_{c-1} in o_j      = e^{b_j[d]}
//   weight of k_i[d] v_i in row d of S_c   = e^{gamma[d] - b_i[d]}
// The decay cannot be taken out of the sum over d, so it has to sit inside the
// matrix-product operands.  With the query tile's start as reference for both sides,
//   Qh_j[d]      = q_j[d] e^{b_j[d] - r_u(j)[d]}                 in q * [e^-80, 1]
//   K^(u)_i[d]   = k_i[d] e^{r_u[d] - b_i[d]}   for i in tiles <= u
// give A_ji = sum_d Qh_j[d] K^(u(j))_i[d] exactly, for every causal tile: inside the
// diagonal tile K^(u) is the reciprocal decay, in [1, e^80] because g >= -5 bounds a
// 16-token tile's log-decay by 80 [§3.2]; for earlier key tiles it is <= 1 and
// underflows only where the true weight is below e^-87.  One code path, no
// diagonal branch [§3.3].  The inter-chunk term puts e^{r_u[d]} (<= 1) on the rows of
// the state:  o_j += sum_d Qh_j[d] e^{r_u(j)[d]} S_{c-1}[d][:].  The state update is
//   S_c[d][:] = e^{gamma[d]} S_{c-1}[d][:] + sum_i k_i[d] e^{gamma[d] - b_i[d]} v_i.
//
// The gate and the cumulative sum are fused into the kernels: each of the four
// waves stages one 16-token tile of the chunk (lane = column group x row group),
// scans g down its rows in registers and across lanes with shuffles, and publishes
// the tile's total per channel; r_u and gamma are sums of those totals.  Inside
// these kernels every log-decay (g, b, r, gamma, the segment totals) is kept in
// base 2, g log2 e, so that each weight is one hardware exp2 of a difference.
//
// The inter-chunk term is computed as (q_j e^{b_j}) S_{c-1}: the same product as
// Qh_j e^{r_u} S_{c-1}, with the state converted to the matrix-core type once per
// chunk instead of once per query tile.
//
// Work decomposition as in the scalar kernels: one workgroup per (head, value slice,
// segment); segments after the first start from the state assembled from the
// pre-pass's local final states H_p and per-channel segment log-decays.
#include "chunk_common.h"

namespace gla {

namespace {

// 16 value columns per wave; in staging, HALVES waves share one 16-token tile of
// the chunk, each taking DK / HALVES of its columns.
template <typename T, int DK, int DVS>
struct PcCfg {
  static constexpr int HALVES = DVS / 64;      // waves staging one tile
  static constexpr int NW = 4 * HALVES;
  static constexpr int NT = 64 * NW;
  static constexpr int CPW = DVS / NW;         // value columns per wave (16)
  static constexpr int NB = CPW / 16;          // 16-column blocks per wave (1)
  static constexpr int PAD = Elem<T>::kPad;
  static constexpr int QLD = DK + PAD;
  static constexpr int TLD = 64 + 4;   // A row stride: its 8-byte stores and fragment reads are conflict-free
  static constexpr int C8 = DK / 8;            // 8-column groups of a row
  static constexpr int C8W = C8 / HALVES;      // ... staged by one wave
  static constexpr int RG = 64 / C8W;          // lanes of one column group within a tile
  static constexpr int R = 16 / RG;            // rows of the tile per lane
  static constexpr int VU = 8 * DVS / NT;      // 8-element v units per thread
  static constexpr int DB = DK / 16;
  static constexpr int KS = DK / 32;
  static_assert(NB == 1 && R >= 1 && VU >= 1 && C8W >= 1, "unsupported shape");
};

// Staging position of a lane: the tile its wave stages, its 8-column group and its
// row group within the tile (rows rg * R .. rg * R + R - 1).
template <typename C>
struct PcLane {
  int tile, c8, rg;
  __device__ __forceinline__ PcLane(int wave, int lane)
      : tile(wave & 3), c8((wave >> 2) * C::C8W + lane % C::C8W), rg(lane / C::C8W) {}
};

template <typename T, int DK, int DVS>
struct PcSmem {
  using C = PcCfg<T, DK, DVS>;
  T qh[64 * C::QLD];                // Qh_j = q_j e^{b_j - r_u(j)}
  T qe[64 * C::QLD];                // q_j e^{b_j}
  T kt[10 * 16 * C::QLD];           // causal tile t = (u, v): k_i e^{r_u - b_i}, i in tile v
  T kp[TokTile<T, DK>::SIZE];       // k_i e^{gamma - b_i}, token-major
  T vv[TokTile<T, DVS>::SIZE];      // v, token-major
  T a[64 * C::TLD];                 // A[j][i]
  float tau[2][4][DK];              // per-tile sums of g, per channel, by chunk parity
  float eg[DK];                     // e^{gamma}
};

template <typename T, int DK, int DVS>
struct PcSegSmem {
  T kp[TokTile<T, DK>::SIZE];
  T vv[TokTile<T, DVS>::SIZE];
  float tau[2][4][DK];
  float eg[DK];
};

struct PcBuffers {
  rsrc_t q, k, v, x, o;
};

// Byte offset of token t's row; rows past the end get an offset beyond every
// descriptor's range (loads return zeros, stores are dropped).
__device__ __forceinline__ uint32_t pc_row(uint32_t t, uint32_t Tn, uint32_t row_bytes) {
  return t < Tn ? t * row_bytes : kDroppedOffset;
}

// One chunk of q, k, x (the wave's tile) and v (token-tile units) on its way to LDS.
template <typename T, int DK, int DVS, bool LOAD_Q>
struct PcStaged {
  using E = Elem<T>;
  using C = PcCfg<T, DK, DVS>;
  typename E::Vec8 q[LOAD_Q ? C::R : 1];
  typename E::Vec8 k[C::R];
  float4 x[C::R][2];
  typename E::Vec8 v[C::VU];

  __device__ __forceinline__ void load(const PcBuffers& hb, uint32_t Tn, int dv, uint32_t t0, int col0, int wave,
                                       int lane, int tid) {
    const PcLane<C> pl(wave, lane);
    const int c8 = pl.c8;
#pragma unroll
    for (int m = 0; m < C::R; ++m) {
      const uint32_t t = t0 + 16 * pl.tile + pl.rg * C::R + m;
      const uint32_t off = pc_row(t, Tn, DK * (uint32_t)sizeof(T)) + c8 * 8 * (uint32_t)sizeof(T);
      if (LOAD_Q) q[m] = E::load8(hb.q, off);
      k[m] = E::load8(hb.k, off);
      const uint32_t xo = pc_row(t, Tn, DK * 4u) + c8 * 32u;
      const uint4 a = buf_load16(hb.x, xo), b = buf_load16(hb.x, xo + 16u);
      x[m][0] = make_float4(__builtin_bit_cast(float, a.x), __builtin_bit_cast(float, a.y),
                            __builtin_bit_cast(float, a.z), __builtin_bit_cast(float, a.w));
      x[m][1] = make_float4(__builtin_bit_cast(float, b.x), __builtin_bit_cast(float, b.y),
                            __builtin_bit_cast(float, b.z), __builtin_bit_cast(float, b.w));
    }
#pragma unroll
    for (int m = 0; m < C::VU; ++m) {
      const int u = tid + m * C::NT;
      const int row = u / (DVS / 8), cv = u % (DVS / 8);
      v[m] = E::load8(hb.v, pc_row(t0 + row, Tn, (uint32_t)dv * (uint32_t)sizeof(T)) +
                                (col0 + cv * 8) * (uint32_t)sizeof(T));
    }
  }
};

// Qh, q e^b and the key tiles are read as MFMA fragments, swizzled by frag_swz
// (gla_device.h).

// Log-decay of one channel in base 2: g log2 e.  The bounded gate evaluates
// sigmoid(x) = 1 / (1 + e^{-x}) directly: a sum of positive terms, so no
// cancellation; e^{-x} = inf (x below about -88.7) gives exactly 0 and x = +inf gives
// 1, the limits.  One multiply, two transcendentals, one add and the final scale per
// element, where the sign-split form needs three more operations.
__device__ __forceinline__ float pc_log2_gate(float x, int gate) {
  return gate == kGateBoundedSigmoid ? (-5.0f * kLog2e) * __builtin_amdgcn_rcpf(1.0f + exp2_hw(x * -kLog2e))
                                     : kLog2e * gate_neg_softplus(x);
}

// Tile-local cumulative log2-decay of the lane's rows (see tile_log_decay).
template <typename T, int DK, int DVS>
struct PcLam {
  float v[PcCfg<T, DK, DVS>::R][8];
};

__device__ __forceinline__ float f4_get(const float4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// Tile-local inclusive cumulative log2-decay lam.v[m][e] = b - r_u of the lane's rows
// (row rg*R + m of the wave's tile, channel 8*c8 + e); absent tokens have g = 0.
// The lanes of the tile's last row group publish the tile totals to tau[tile].
template <typename T, int DK, int DVS, bool LOAD_Q>
__device__ __forceinline__ void tile_log_decay(PcLam<T, DK, DVS>& lam,
                                               const PcStaged<T, DK, DVS, LOAD_Q>& st, float (*tau)[DK],
                                               uint32_t t0, uint32_t Tn, int gate, int wave, int lane) {
  using C = PcCfg<T, DK, DVS>;
  const PcLane<C> pl(wave, lane);
  const int c8 = pl.c8, rg = pl.rg;
#pragma unroll
  for (int m = 0; m < C::R; ++m) {
    const bool valid = t0 + 16 * pl.tile + rg * C::R + m < Tn;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xv = f4_get(st.x[m][e >> 2], e & 3);
      const float g = pc_log2_gate(xv, gate);
      lam.v[m][e] = (valid ? g : 0.0f) + (m > 0 ? lam.v[m - 1][e] : 0.0f);
    }
  }
  // exclusive prefix of the lane totals over the row groups of the same columns
  // (lane = rg * C8W + column group)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float ex = strided_exclusive_scan<C::C8W>(lam.v[C::R - 1][e], lane);
#pragma unroll
    for (int m = 0; m < C::R; ++m) lam.v[m][e] += ex;
  }
  if (rg == C::RG - 1) {
    *reinterpret_cast<float4*>(&tau[pl.tile][c8 * 8]) =
        make_float4(lam.v[C::R - 1][0], lam.v[C::R - 1][1], lam.v[C::R - 1][2], lam.v[C::R - 1][3]);
    *reinterpret_cast<float4*>(&tau[pl.tile][c8 * 8 + 4]) =
        make_float4(lam.v[C::R - 1][4], lam.v[C::R - 1][5], lam.v[C::R - 1][6], lam.v[C::R - 1][7]);
  }
}

// Reads the four tile totals at the lane's 8 channels.
template <int DK>
__device__ __forceinline__ void read_tau(float (&tv)[4][8], const float (*tau)[DK], int col) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float4 a = *reinterpret_cast<const float4*>(&tau[u][col]);
    const float4 b = *reinterpret_cast<const float4*>(&tau[u][col + 4]);
    tv[u][0] = a.x; tv[u][1] = a.y; tv[u][2] = a.z; tv[u][3] = a.w;
    tv[u][4] = b.x; tv[u][5] = b.y; tv[u][6] = b.z; tv[u][7] = b.w;
  }
}

// The key-side chain of the wave's tile: row i starts at k_i e^{-b_i + r_tile} (lam is
// b - r_tile) and is multiplied by e^{tau_u} for u = tile, ..., 3 (tile u's total per
// channel), passing through k_i e^{r_u - b_i} (the key operand of query tile u) and
// ending at k_i e^{gamma - b_i}, the state-side operand.  The values only shrink, so a
// step underflows only where the true weight does.  Both kernels run this same
// sequence of fp32 operations, so their state-side operands are bit-identical.
template <typename T, int DK, int DVS, bool LOAD_Q, int R>
__device__ __forceinline__ void key_chain_start(float (&kf)[R][8], const PcStaged<T, DK, DVS, LOAD_Q>& st,
                                                const PcLam<T, DK, DVS>& lam) {
#pragma unroll
  for (int m = 0; m < R; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) kf[m][e] = Elem<T>::get(st.k[m], e) * exp2_hw(-lam.v[m][e]);
}
template <int R>
__device__ __forceinline__ void key_chain_step(float (&kf)[R][8], const float (&tau)[8]) {
  float step[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) step[e] = exp2_hw(tau[e]);
#pragma unroll
  for (int m = 0; m < R; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) kf[m][e] *= step[e];
}

// k_i e^{gamma - b_i} (token-major) for the wave's tile and, from the lanes of tile 0's
// waves and row group 0 (which together cover every channel once), e^{gamma}.
template <typename T, int DK, int DVS, bool LOAD_Q>
__device__ __forceinline__ void stage_state_side(T* kp, float* eg, const PcStaged<T, DK, DVS, LOAD_Q>& st,
                                                 const PcLam<T, DK, DVS>& lam,
                                                 const float (&tv)[4][8], int wave, int lane) {
  using C = PcCfg<T, DK, DVS>;
  const PcLane<C> pl(wave, lane);
  const int c8 = pl.c8, rg = pl.rg;
  float G[8];  // sum of the totals of this tile and the later ones: gamma - r_tile
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u >= pl.tile) s += tv[u][e];
    G[e] = s;
  }
  float kf[C::R][8];
  key_chain_start<T, DK, DVS, LOAD_Q, C::R>(kf, st, lam);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (u >= pl.tile) key_chain_step<C::R>(kf, tv[u]);  // wave-uniform
#pragma unroll
  for (int m = 0; m < C::R; ++m) TokTile<T, DK>::store8_f32(kp, 16 * pl.tile + rg * C::R + m, c8 * 8, kf[m]);
  if (pl.tile == 0 && rg == 0) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = exp2_hw(G[e]);
    *reinterpret_cast<float4*>(&eg[c8 * 8]) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(&eg[c8 * 8 + 4]) = make_float4(f[4], f[5], f[6], f[7]);
  }
}

template <typename T, int DK, int DVS, bool LOAD_Q>
__device__ __forceinline__ void stage_v(T* vv, const PcStaged<T, DK, DVS, LOAD_Q>& st, int tid) {
  using C = PcCfg<T, DK, DVS>;
#pragma unroll
  for (int m = 0; m < C::VU; ++m) {
    const int u = tid + m * C::NT;
    TokTile<T, DVS>::store8_raw(vv, u / (DVS / 8), (u % (DVS / 8)) * 8, st.v[m]);
  }
}

// fp32 state slice of one wave: S[d = 16 db + 4 g + e][n = wcol + 16 nb + r16]
template <typename T, int DK, int DVS>
struct PcState {
  floatx4 s[PcCfg<T, DK, DVS>::NB][PcCfg<T, DK, DVS>::DB];
};

template <typename T, int DK, int DVS>
struct PcVFrags {
  typename Elem<T>::Frag f[PcCfg<T, DK, DVS>::NB][2];
};

// S[d][:] <- e^{gamma[d]} S[d][:] + sum_i kp[i][d] v_i
template <typename T, int DK, int DVS>
__device__ __forceinline__ void pc_state_update(PcState<T, DK, DVS>& S, const PcVFrags<T, DK, DVS>& Vf,
                                                const T* kp, const float* eg, int lane) {
  using E = Elem<T>;
  using C = PcCfg<T, DK, DVS>;
  const int g = lane >> 4;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    const floatx4 f = *reinterpret_cast<const floatx4*>(&eg[16 * db + 4 * g]);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) S.s[nb][db] *= f;
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const typename E::Frag ka = TokTile<T, DK>::load(kp, ks * 32, db * 16, lane);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) E::mfma(S.s[nb][db], ka, Vf.f[nb][ks]);
    }
  }
}

template <typename T, int DK, int DVS>
__device__ __forceinline__ void pc_load_v_frags(PcVFrags<T, DK, DVS>& Vf, const T* vv, int wave, int lane) {
  using C = PcCfg<T, DK, DVS>;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) Vf.f[nb][ks] = TokTile<T, DVS>::load(vv, ks * 32, wave * C::CPW + nb * 16, lane);
}

template <typename T, int DK, int DVS>
__device__ __forceinline__ void pc_store_state(const PcState<T, DK, DVS>& S, float* dst, int dv, int wcol, int g,
                                               int r16) {
  using C = PcCfg<T, DK, DVS>;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(long long)(db * 16 + 4 * g + e) * dv + wcol + nb * 16 + r16] = S.s[nb][db][e];
}

// ============================================================================
// Segment pre-pass: local final state (from zero) and per-channel total log-decay
// of every segment but the last.
// ============================================================================
template <typename T, int DK, int DVS>
__global__ void __launch_bounds__((PcCfg<T, DK, DVS>::NT)) pc_segment_state_kernel(PcParams p) {
  using C = PcCfg<T, DK, DVS>;
  __shared__ __attribute__((aligned(16))) PcSegSmem<T, DK, DVS> sm;  // 16-byte aligned: row stores compile to ds_write_b128
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int nseg = p.segments - 1;
  const int L = xcd_linear_index(blockIdx.x, p.grid);
  const int slice = L % p.nslices;
  const int rest = L / p.nslices;
  const int seg = rest % nseg;
  const int bh = rest / nseg;
  const int col0 = slice * DVS;
  const int wcol = col0 + wave * C::CPW;
  const int c_begin = (int)((long long)seg * p.nchunks / p.segments);
  const int c_end = (int)((long long)(seg + 1) * p.nchunks / p.segments);
  const uint32_t Tn = (uint32_t)p.T;

  PcBuffers hb;
  hb.k = make_rsrc(static_cast<const T*>(p.k) + (long long)bh * p.T * DK, Tn * DK * (uint32_t)sizeof(T));
  hb.v = make_rsrc(static_cast<const T*>(p.v) + (long long)bh * p.T * p.dv, Tn * p.dv * (uint32_t)sizeof(T));
  hb.x = make_rsrc(p.x + (long long)bh * p.T * DK, Tn * DK * 4u);

  PcState<T, DK, DVS> S;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) S.s[nb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float gsum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // tile 0, row group 0: segment log-decay
  const PcLane<C> pl(wave, lane);

  // Exact truncation: the state update multiplies state row d by e^{gamma_c[d]}; if
  // that factor is exactly zero in fp32 for every channel of chunk c, the state after
  // c does not depend on anything before it, and the pass may start there from a zero
  // state with the same result.  The last two chunks of the segment are candidates;
  // their factors are computed by the same code, in the same order, as in the pass.
  // The segment log-decay then sums only the chunks run; the skipped decay would not
  // change it: it is below -150 (base 2) either way, so its exp2 is the same zero.
  __shared__ int live_flag[2];  // one per candidate: no flag is cleared while it may be read
  if (tid < 2) live_flag[tid] = 0;
  int c_first = c_begin;
  for (int cand = c_end - 1, i = 0; cand >= c_begin && i < 2; --cand, ++i) {  // uniform
    PcStaged<T, DK, DVS, false> sc;
    sc.load(hb, Tn, p.dv, (uint32_t)cand * kChunk, col0, wave, lane, tid);
    PcLam<T, DK, DVS> lc;
    tile_log_decay<T, DK, DVS, false>(lc, sc, sm.tau[0], (uint32_t)cand * kChunk, Tn, p.gate, wave, lane);
    __syncthreads();
    for (int d = tid; d < DK; d += C::NT) {
      float s = 0.0f;
#pragma unroll
      for (int u = 0; u < 4; ++u) s += sm.tau[0][u][d];
      if (exp2_hw(s) != 0.0f) live_flag[i] = 1;
    }
    __syncthreads();  // also orders the reads of tau before it is written again
    if (!live_flag[i]) {
      c_first = cand;
      break;
    }
  }

  PcStaged<T, DK, DVS, false> st;
  if (c_first < c_end) st.load(hb, Tn, p.dv, (uint32_t)c_first * kChunk, col0, wave, lane, tid);
  // Two barriers per chunk: the tile totals alternate between two buffers, so a wave
  // may publish chunk c + 1's totals while others still update the state of chunk c;
  // everything else chunk c + 1 writes comes after the barrier that all waves reach
  // only once they are done with chunk c.
  for (int c = c_first; c < c_end; ++c) {
    const uint32_t t0 = (uint32_t)c * kChunk;
    float (*tau)[DK] = sm.tau[(c - c_first) & 1];
    PcLam<T, DK, DVS> lam;
    tile_log_decay<T, DK, DVS, false>(lam, st, tau, t0, Tn, p.gate, wave, lane);
    __syncthreads();
    float tv[4][8];
    read_tau<DK>(tv, tau, pl.c8 * 8);
    stage_state_side<T, DK, DVS, false>(sm.kp, sm.eg, st, lam, tv, wave, lane);
    stage_v<T, DK, DVS, false>(sm.vv, st, tid);
#pragma unroll
    for (int e = 0; e < 8; ++e) gsum[e] += tv[0][e] + tv[1][e] + tv[2][e] + tv[3][e];
    st.load(hb, Tn, p.dv, (uint32_t)min(c + 1, c_end - 1) * kChunk, col0, wave, lane, tid);
    __syncthreads();
    PcVFrags<T, DK, DVS> Vf;
    pc_load_v_frags<T, DK, DVS>(Vf, sm.vv, wave, lane);
    pc_state_update<T, DK, DVS>(S, Vf, sm.kp, sm.eg, lane);
  }
  pc_store_state<T, DK, DVS>(S, p.seg_state + ((long long)bh * nseg + seg) * DK * p.dv, p.dv, wcol, g, r16);
  if (slice == 0 && pl.tile == 0 && pl.rg == 0) {
    float* dst = p.seg_decay + ((long long)bh * p.segments + seg) * DK + pl.c8 * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = gsum[e];
  }
}

// ============================================================================
// Fused output pass.
// ============================================================================
template <typename T, int DK, int DVS>
__global__ void __launch_bounds__((PcCfg<T, DK, DVS>::NT)) pc_chunk_output_kernel(PcParams p) {
  using E = Elem<T>;
  using C = PcCfg<T, DK, DVS>;
  __shared__ __attribute__((aligned(16))) PcSmem<T, DK, DVS> sm;  // 16-byte aligned: row stores compile to ds_write_b128
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const PcLane<C> pl(wave, lane);
  const int c8 = pl.c8, rg = pl.rg, tile = pl.tile;
  const int L = xcd_linear_index(blockIdx.x, p.grid);
  const int slice = L % p.nslices;
  const int rest = L / p.nslices;
  const int seg = rest % p.segments;
  const int bh = rest / p.segments;
  const int col0 = slice * DVS;
  const int wcol = col0 + wave * C::CPW;
  const int c_begin = (int)((long long)seg * p.nchunks / p.segments);
  const int c_end = (int)((long long)(seg + 1) * p.nchunks / p.segments);
  const uint32_t Tn = (uint32_t)p.T;

  PcBuffers hb;
  hb.q = make_rsrc(static_cast<const T*>(p.q) + (long long)bh * p.T * DK, Tn * DK * (uint32_t)sizeof(T));
  hb.k = make_rsrc(static_cast<const T*>(p.k) + (long long)bh * p.T * DK, Tn * DK * (uint32_t)sizeof(T));
  hb.v = make_rsrc(static_cast<const T*>(p.v) + (long long)bh * p.T * p.dv, Tn * p.dv * (uint32_t)sizeof(T));
  hb.x = make_rsrc(p.x + (long long)bh * p.T * DK, Tn * DK * 4u);
  hb.o = make_rsrc(p.o + (long long)bh * p.T * p.dv, Tn * p.dv * 4u);

  // ---- initial state: S0 (or zero) folded with the earlier segments' local states
  PcState<T, DK, DVS> S;
  {
    const long long i0 = (long long)bh * DK * p.dv;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          S.s[nb][db][e] = p.S0 ? p.S0[i0 + (long long)(db * 16 + 4 * g + e) * p.dv + wcol + nb * 16 + r16] : 0.0f;
    for (int ps = 0; ps < seg; ++ps) {
      const float* H = p.seg_state + ((long long)bh * (p.segments - 1) + ps) * DK * p.dv;
      const float* G = p.seg_decay + ((long long)bh * p.segments + ps) * DK;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int d = db * 16 + 4 * g + e;
            S.s[nb][db][e] = exp2_hw(G[d]) * S.s[nb][db][e] + H[(long long)d * p.dv + wcol + nb * 16 + r16];
          }
    }
  }

  // A is read in 32-key steps: the two tiles above the diagonal that such a step
  // covers, (0, 1) and (2, 3), stay zero.
  for (int e = tid; e < 2 * 256; e += C::NT) {
    const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
    sm.a[(blk * 32 + rr) * C::TLD + blk * 32 + 16 + cc] = E::cvt(0.0f);
  }

  PcStaged<T, DK, DVS, true> st;
  if (c_begin < c_end) st.load(hb, Tn, p.dv, (uint32_t)c_begin * kChunk, col0, wave, lane, tid);

  for (int c = c_begin; c < c_end; ++c) {
    const uint32_t t0 = (uint32_t)c * kChunk;

    // ---- (1) gate and tile-local cumulative log-decay; Qh needs nothing else
    PcLam<T, DK, DVS> lam;
    float (*tau)[DK] = sm.tau[(c - c_begin) & 1];
    tile_log_decay<T, DK, DVS, true>(lam, st, tau, t0, Tn, p.gate, wave, lane);
    float qf[C::R][8];  // q_j e^{b_j - r_u} in fp32 (kept for q e^{b} below)
#pragma unroll
    for (int m = 0; m < C::R; ++m) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[m][e] = E::get(st.q[m], e) * exp2_hw(lam.v[m][e]);
      E::store8_f32_sw(sm.qh + (16 * tile + rg * C::R + m) * C::QLD + c8 * 8, qf[m], frag_swz<T>(rg * C::R + m) != 0);
    }
    __syncthreads();

    // ---- (2) key operands of every query tile, the state-side operands, q e^{b}
    {
      float tv[4][8];
      read_tau<DK>(tv, tau, c8 * 8);
      {
        float er[8];  // e^{r_tile}
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float s = 0.0f;
#pragma unroll
          for (int w = 0; w < 4; ++w)
            if (w < tile) s += tv[w][e];
          er[e] = exp2_hw(s);
        }
#pragma unroll
        for (int m = 0; m < C::R; ++m) {
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[m][e] *= er[e];
          E::store8_f32_sw(sm.qe + (16 * tile + rg * C::R + m) * C::QLD + c8 * 8, qf[m], frag_swz<T>(rg * C::R + m) != 0);
        }
      }
      // Key tile `tile` serves the query tiles u >= tile as K^(u) = k e^{r_u - b} and the
      // state update as k e^{gamma - b}: the key chain (above), with each K^(u) stored on
      // the way.
      float kf[C::R][8];
      key_chain_start<T, DK, DVS, true, C::R>(kf, st, lam);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (u < tile) continue;  // wave-uniform
        T* kt = sm.kt + (u * (u + 1) / 2 + tile) * 16 * C::QLD;
#pragma unroll
        for (int m = 0; m < C::R; ++m)
          E::store8_f32_sw(kt + (rg * C::R + m) * C::QLD + c8 * 8, kf[m], frag_swz<T>(rg * C::R + m) != 0);
        key_chain_step<C::R>(kf, tv[u]);
      }
#pragma unroll
      for (int m = 0; m < C::R; ++m) TokTile<T, DK>::store8_f32(sm.kp, 16 * tile + rg * C::R + m, c8 * 8, kf[m]);
      if (tile == 0 && rg == 0) {  // e^{gamma}: these lanes cover every channel once
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = exp2_hw(tv[0][e] + tv[1][e] + tv[2][e] + tv[3][e]);
        *reinterpret_cast<float4*>(&sm.eg[c8 * 8]) = make_float4(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<float4*>(&sm.eg[c8 * 8 + 4]) = make_float4(f[4], f[5], f[6], f[7]);
      }
      stage_v<T, DK, DVS, true>(sm.vv, st, tid);
    }
    // prefetch chunk c + 1 (the last iteration re-reads its own chunk so that every
    // iteration issues the same loads)
    st.load(hb, Tn, p.dv, (uint32_t)min(c + 1, c_end - 1) * kChunk, col0, wave, lane, tid);
    __syncthreads();

    // ---- (3) A_ji = Qh_j . K^(u(j))_i over the 10 causal tiles, one code path
#pragma unroll
    for (int t = 0; t < 10; ++t) {
      if (t % C::NW != wave) continue;  // wave-uniform
      const int jb = tri_j(t), ib = tri_i(t);
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        E::mfma(acc, E::load_frag(sm.kt + (t * 16 + r16) * C::QLD, ks * 32 + ((4 * g) ^ frag_swz<T>(r16))),
                E::load_frag(sm.qh + (jb * 16 + r16) * C::QLD, ks * 32 + ((4 * g) ^ frag_swz<T>(r16))));
      // acc[e]: j = 16 jb + r16, i = 16 ib + 4 g + e; causal select on the diagonal tile
      float vals[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) vals[e] = (jb != ib || 4 * g + e <= r16) ? acc[e] : 0.0f;
      E::store4(sm.a + (jb * 16 + r16) * C::TLD + ib * 16 + 4 * g, vals[0], vals[1], vals[2], vals[3]);
    }
    __syncthreads();

    // ---- (4) o = (q e^{b}) S_{c-1} + A V for this wave's columns; then S_c
    {
      PcVFrags<T, DK, DVS> Vf;
      pc_load_v_frags<T, DK, DVS>(Vf, sm.vv, wave, lane);
      // rows 32 ks + 4 g + e and 32 ks + 16 + 4 g + e of the state
      typename E::Frag sf[C::NB][C::KS];
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) sf[nb][ks] = E::from_acc(S.s[nb][2 * ks], S.s[nb][2 * ks + 1]);
      floatx4 O[4][C::NB];
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) O[jb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const typename E::Frag qb = E::load_frag(sm.qe + (jb * 16 + r16) * C::QLD, ks * 32 + ((4 * g) ^ frag_swz<T>(r16)));
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) E::mfma(O[jb][nb], sf[nb][ks], qb);
        }
#pragma unroll
        for (int ks = 0; ks <= jb / 2; ++ks) {
          const typename E::Frag ab = E::load_frag(sm.a + (jb * 16 + r16) * C::TLD, ks * 32 + 4 * g);
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) E::mfma(O[jb][nb], Vf.f[nb][ks], ab);
        }
      }
      pc_state_update<T, DK, DVS>(S, Vf, sm.kp, sm.eg, lane);
      // lane holds o[t0 + 16 jb + r16][wcol + 16 nb + 4 g + 0..3]
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
          buf_store16(hb.o, pc_row(t0 + jb * 16 + r16, Tn, (uint32_t)p.dv * 4u) + (wcol + nb * 16 + 4 * g) * 4u,
                      O[jb][nb]);
    }
    // no barrier here: chunk c + 1 writes Qh (read only in step 3, before the last
    // barrier) and the other tile-total buffer before its first barrier, and the rest of
    // its operands after it
  }

  if (seg == p.segments - 1) pc_store_state<T, DK, DVS>(S, p.ST + (long long)bh * DK * p.dv, p.dv, wcol, g, r16);
}

template <typename F>
hipError_t pc_dispatch(int dtype, int dk, int slice, F&& f) {
  if (dtype == 0) {
    if (dk == 128 && slice == 128) return f.template operator()<bf16, 128, 128>();
    if (dk == 128 && slice == 64) return f.template operator()<bf16, 128, 64>();
    if (dk == 64 && slice == 128) return f.template operator()<bf16, 64, 128>();
    if (dk == 64 && slice == 64) return f.template operator()<bf16, 64, 64>();
  } else {
    if (dk == 64 && slice == 64) return f.template operator()<float, 64, 64>();
  }
  return hipErrorInvalidValue;
}

struct PcOutFn {
  const PcParams& p;
  hipStream_t s;
  template <typename T, int DK, int DVS>
  hipError_t operator()() const {
    hipLaunchKernelGGL((pc_chunk_output_kernel<T, DK, DVS>), dim3(p.grid), dim3(PcCfg<T, DK, DVS>::NT), 0, s, p);
    return hipGetLastError();
  }
};

struct PcSegFn {
  const PcParams& p;
  hipStream_t s;
  template <typename T, int DK, int DVS>
  hipError_t operator()() const {
    hipLaunchKernelGGL((pc_segment_state_kernel<T, DK, DVS>), dim3(p.grid), dim3(PcCfg<T, DK, DVS>::NT), 0, s, p);
    return hipGetLastError();
  }
};

struct PcProbeFn {
  template <typename T, int DK, int DVS>
  hipError_t operator()() const {
    return hipSuccess;
  }
};

}  // namespace

bool pc_config_built(int dtype, int dk, int slice) { return pc_dispatch(dtype, dk, slice, PcProbeFn{}) == hipSuccess; }

hipError_t launch_pc_segment_states(const PcParams& p, int dtype, hipStream_t stream) {
  if (p.segments <= 1 || p.grid == 0) return hipSuccess;
  return pc_dispatch(dtype, p.dk, p.dv / p.nslices, PcSegFn{p, stream});
}

hipError_t launch_pc_chunk_output(const PcParams& p, int dtype, hipStream_t stream) {
  if (p.grid == 0) return hipSuccess;
  return pc_dispatch(dtype, p.dk, p.dv / p.nslices, PcOutFn{p, stream});
}

// debug builds: this unit's LDS-check word (see GLA_CHECK_LDS)
GLA_DEBUG_ACCESSOR(debug_word_pc_kernels)

}  // namespace gla
