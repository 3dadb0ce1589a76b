// chunk_kernels.hip -- chunked gated-linear-attention forward on gfx950 matrix cores.
//
// Sources (web pages; cited by title and section):
//   [LCT] "Engineering Long-Context Training for Trillion-Parameter MoE Models:
//          Three Key Breakthroughs"
//   [ESU] "Engineering Stability in Ultra-Long Context and Trillion-Parameter
//          Sparse Models"
//
// Chunked form of S_t = a_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t [LCT §3.1],
// [ESU §2.1]: the sequence is cut into 64-token chunks, each made of four
// 16-token tiles u = 0..3.  With b_j the chunk-local cumulative log-decay,
// r_u = b_{16u-1} (r_0 = 0) and gamma = b_63, for query j and key i of one chunk:
//   weight of k_i v_i^T in o_j  (i <= j)  = e^{b_j - b_i}
//                                        = e^{b_j - r_u(j)} e^{r_u(j) - r_u(i)} e^{r_u(i) - b_i}
//   weight of S_{c-1} in o_j              = e^{b_j}    = e^{r_u(j)} e^{b_j - r_u(j)}
//   weight of k_i v_i^T in S_c            = e^{gamma - b_i}
// so, with Qh_j = q_j e^{b_j - r_u(j)} ("q * Gamma") and Kh_i = k_i e^{r_u(i) - b_i}
// ("k / Gamma"):
//   A_ji = (Qh_j . Kh_i) e^{r_u(j) - r_u(i)}  for i <= j, 0 above the diagonal
//   o_j  = e^{r_u(j)} (Qh_j^T S_{c-1}) + sum_i A_ji v_i
//   S_c  = e^gamma S_{c-1} + sum_i (k_i e^{gamma - b_i}) v_i^T
// Because g >= -5, the tile-relative factors lie in [e^-80, 1] and [1, e^80],
// inside the fp32/bf16 exponent range [LCT §3.2], [ESU §2.2], so every causal
// 16x16 tile of A, diagonal or not, comes out of the same matrix-core product
// with no separate diagonal branch [LCT §3.3].  The remaining scalars
// e^{r_u(j) - r_u(i)}, e^{r_u(j)} and e^gamma are all <= 1.
//
// The conventional design kept for the ablation (DIAG = true) computes only the
// off-diagonal tiles on matrix cores, with factors referenced to the end of the
// key tile, E_u = b_{16u+15} (Kh_i = k_i e^{E_u(i) - b_i} <= 1 and a tile scalar
// e^{r_u(j) - E_u(i)} <= 1), and the diagonal tiles by explicit position pairs,
// A_ji = e^{b_j - b_i} (q_j . k_i), on the vector ALUs [LCT §3.1], [ESU §2.1].
//
// Work decomposition: one workgroup per (head, slice of DVS value columns,
// segment of consecutive chunks).  A workgroup streams its chunks in order,
// holding its slice of the state in fp32 MFMA accumulators; wave w owns value
// columns [w*CPW, (w+1)*CPW) of the slice for o and S.  Segments after the first
// start from the state assembled from the pre-pass (segment_state_kernel).
#include "chunk_common.h"

namespace gla {

template <typename T, int DK, int DVS, bool DIAG>
struct OutSmem {
  using C = Cfg<T, DK, DVS>;
  T qh[64 * C::QLD];                 // Qh[j][d]  row-major
  T kh[64 * C::QLD];                 // Kh[i][d]  row-major
  T kp[TokTile<T, DK>::SIZE];        // k_i e^{gamma - b_i}, token-major tile
  T vv[TokTile<T, DVS>::SIZE];       // v, token-major tile
  T a[64 * C::TLD];                  // A[j][i]   row-major
  T qr[DIAG ? 64 * C::QLD : 1];      // raw q, diagonal-branch path only
  T kr[DIAG ? 64 * C::QLD : 1];      // raw k, diagonal-branch path only
  float sb[DIAG ? 64 : 1];           // b of the chunk, diagonal-branch path only
};

template <typename T, int DK, int DVS>
struct SegSmem {
  T kp[TokTile<T, DK>::SIZE];
  T vv[TokTile<T, DVS>::SIZE];
  SegScanSmem scan;  // first chunk to run (x path)
};

// Per-thread registers holding one chunk of q, k, v (and b) on its way to LDS.
// Rows past the end of the sequence read as zeros (buffer range check); b past
// the end repeats its last value (absent tokens have g = 0).
template <typename T, int DK, int DVS, bool LOAD_Q>
struct Staged {
  using E = Elem<T>;
  using C = Cfg<T, DK, DVS>;
  typename E::Vec8 q[LOAD_Q ? C::QU : 1];
  typename E::Vec8 k[C::QU];
  typename E::Vec8 v[C::VU];
  float b;      // b of the lane's token, or its x until decay() (see decay_load)
  uint32_t t0;  // first token of the chunk held

  // chunk starting at logical token t0 (rows in logical order; see row_offset)
  __device__ __forceinline__ void load(const HeadBuffers& hb, const ChunkParams& p, uint32_t t0_, int col0,
                                       int tid) {
    t0 = t0_;
    b = decay_load(hb, p, t0, tid & 63);
#pragma unroll
    for (int m = 0; m < C::QU; ++m) {
      const int u = tid + m * C::NT;
      const int row = u / (DK / 8), c8 = u % (DK / 8);
      const uint32_t off = row_offset(p, hb.T, t0 + row, DK * (uint32_t)sizeof(T)) + c8 * 8 * (uint32_t)sizeof(T);
      if (LOAD_Q) q[m] = E::load8(hb.q, off);
      k[m] = E::load8(hb.k, off);
    }
#pragma unroll
    for (int m = 0; m < C::VU; ++m) {
      const int u = tid + m * C::NT;
      const int row = u / (DVS / 8), c8 = u % (DVS / 8);
      v[m] = E::load8(hb.v, row_offset(p, hb.T, t0 + row, (uint32_t)p.dv * (uint32_t)sizeof(T)) +
                                (col0 + c8 * 8) * (uint32_t)sizeof(T));
    }
  }

  // b of the lane's token (lane = token of the chunk)
  __device__ __forceinline__ float decay(const HeadBuffers& hb, const ChunkParams& p, int lane) const {
    return decay_finish(hb, p, b, t0, lane);
  }
};

// b of the rows this thread stages (one shuffle each, issued together)
template <typename T, int DK, int DVS>
struct RowB {
  float v[Cfg<T, DK, DVS>::QU];
  __device__ __forceinline__ RowB(const ChunkDecay& cd, int tid) {
#pragma unroll
    for (int m = 0; m < Cfg<T, DK, DVS>::QU; ++m) v[m] = cd.at((tid + m * Cfg<T, DK, DVS>::NT) / (DK / 8));
  }
};

// Writes k e^{gamma - b} and v into their token-major LDS tiles.
template <typename T, int DK, int DVS, bool LOAD_Q>
__device__ __forceinline__ void stage_state_operands(T* kp, T* vv, const Staged<T, DK, DVS, LOAD_Q>& st,
                                                     const ChunkDecay& cd, const RowB<T, DK, DVS>& brow, int tid) {
  using C = Cfg<T, DK, DVS>;
#pragma unroll
  for (int m = 0; m < C::QU; ++m) {
    const int u = tid + m * C::NT;
    const int row = u / (DK / 8), c8 = u % (DK / 8);
    TokTile<T, DK>::store8(kp, row, c8 * 8, st.k[m], exp_e(cd.gam - brow.v[m]));
  }
#pragma unroll
  for (int m = 0; m < C::VU; ++m) {
    const int u = tid + m * C::NT;
    const int row = u / (DVS / 8), c8 = u % (DVS / 8);
    TokTile<T, DVS>::store8_raw(vv, row, c8 * 8, st.v[m]);
  }
}

// ============================================================================
// Segment pre-pass: local final state of every segment but the last.
// ============================================================================
template <typename T, int DK, int DVS>
__global__ void __launch_bounds__((Cfg<T, DK, DVS>::NT)) segment_state_kernel(ChunkParams p) {
  using C = Cfg<T, DK, DVS>;
  __shared__ __attribute__((aligned(16))) SegSmem<T, DK, DVS> sm;  // 16-byte aligned: row stores compile to ds_write_b128
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int nseg = p.segments - 1;
  const int L = work_index(p);
  const int slice = L % p.nslices;
  const int rest = L / p.nslices;
  const int seg = rest % nseg;
  const int bh = unit_of(p, rest / nseg);
  const int col0 = slice * DVS;
  const int wcol = col0 + wave * C::CPW;
  const HeadSpan span = head_span(p, bh);
  const int c_begin = (int)((long long)seg * span.nchunks / p.segments);
  const int c_end = (int)((long long)(seg + 1) * span.nchunks / p.segments);
  const HeadBuffers hb = head_buffers<T, DK>(p, span);

  StateAcc<T, DK, DVS> S;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) S.s[nb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float gsum;  // total log-decay of the segment
  const int c_first = p.b ? segment_first_live_chunk(hb, c_begin, c_end, gsum)
                          : segment_first_live_chunk_x<C::NW>(hb, p, c_begin, c_end, gsum, sm.scan);

  Staged<T, DK, DVS, false> st;
  if (c_first < c_end) st.load(hb, p, (uint32_t)c_first * kChunk, col0, tid);
  for (int c = c_first; c < c_end; ++c) {
    const ChunkDecay cd(st.decay(hb, p, lane));
    const RowB<T, DK, DVS> brow(cd, tid);
    stage_state_operands<T, DK, DVS, false>(sm.kp, sm.vv, st, cd, brow, tid);
    // prefetch the next chunk (the last iteration re-reads its own chunk so that
    // every iteration issues the same loads)
    st.load(hb, p, (uint32_t)min(c + 1, c_end - 1) * kChunk, col0, tid);
    __syncthreads();
    VFrags<T, DK, DVS> Vf;
    load_v_frags<T, DK, DVS>(Vf, sm.vv, wave, lane);
    state_update<T, DK, DVS>(S, Vf, sm.kp, exp_e(cd.gam), lane);
    __syncthreads();
  }

  store_state<T, DK, DVS>(S, p.seg_state + ((long long)bh * nseg + seg) * DK * p.dv, p.dv, wcol, g, r16);
  if (slice == 0 && tid == 0) p.seg_decay[(long long)bh * p.segments + seg] = gsum;
}

// ============================================================================
// Fused output pass.
// ============================================================================
// Register budget of the output kernel: two waves per SIMD where it then still fits
// without spilling (the bf16 unified kernels with 4 waves of 32 columns, and dk = 64
// with 2); this also keeps the MFMA accumulators in VGPRs instead of AGPR copies.
template <typename T, int DK, int DVS, bool DIAG>
constexpr int out_waves_per_simd() {
  return (sizeof(T) == 2 && !DIAG && (DVS == 128 || (DK == 64 && DVS == 64))) ? 2 : 1;
}

template <typename T, int DK, int DVS, bool DIAG>
__global__ void __launch_bounds__((Cfg<T, DK, DVS>::NT))
__attribute__((amdgpu_waves_per_eu(out_waves_per_simd<T, DK, DVS, DIAG>()))) chunk_output_kernel(ChunkParams p) {
  using E = Elem<T>;
  using C = Cfg<T, DK, DVS>;
  __shared__ __attribute__((aligned(16))) OutSmem<T, DK, DVS, DIAG> sm;  // 16-byte aligned: row stores compile to ds_write_b128
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int L = work_index(p);
  const int slice = L % p.nslices;
  const int rest = L / p.nslices;
  const int seg = rest % p.segments;
  const int bh = unit_of(p, rest / p.segments);
  const int col0 = slice * DVS;
  const int wcol = col0 + wave * C::CPW;
  const HeadSpan span = head_span(p, bh);
  const int c_begin = (int)((long long)seg * span.nchunks / p.segments);
  const int c_end = (int)((long long)(seg + 1) * span.nchunks / p.segments);
  const HeadBuffers hb = head_buffers<T, DK>(p, span);

  // ---- initial state of this segment
  StateAcc<T, DK, DVS> S;
  load_initial_state<T, DK, DVS>(S, p, bh, seg, wcol, g, r16);

  // The two key tiles that a 32-wide K-step reads above the diagonal, (jb 0, ib 1)
  // and (jb 2, ib 3), are never written by the loop: zero them once.
  for (int e = tid; e < 2 * 256; e += C::NT) {
    const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
    sm.a[(blk * 32 + rr) * C::TLD + blk * 32 + 16 + cc] = E::cvt(0.0f);
  }

  Staged<T, DK, DVS, true> st;
  if (c_begin < c_end) st.load(hb, p, (uint32_t)c_begin * kChunk, col0, tid);
  __syncthreads();

  // o of a chunk is stored at the end of its iteration, after that iteration's
  // prefetch loads; lane (g, r16) holds row r16 of tile jb at columns 16 nb + 4g.
  // Rows outside the head get an out-of-range offset and are dropped.
  auto store_o = [&](const floatx4 (&O)[4][C::NB], uint32_t row0, bool none) {
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        // dropped stores get distinct addresses: identical ones would be merged
        // into one, and the loop's wait counts assume all of them are issued
        const uint32_t off = none ? kDroppedOffset + 16u * (jb * C::NB + nb)
                                  : row_offset(p, hb.T, row0 + jb * 16 + r16, (uint32_t)p.dv * 4u) +
                                        (wcol + nb * 16 + 4 * g) * 4u;
        buf_store16<kAuxStream>(hb.o, off, O[jb][nb]);
      }
  };
  // Issuing the same number of (dropped) stores after the first loads gives both
  // entries into the loop the same outstanding memory operations, so the wait for
  // the prefetched data never waits for the stores behind it.
  {
    floatx4 Oz[4][C::NB];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) Oz[jb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    store_o(Oz, 0, true);
  }

  for (int c = c_begin; c < c_end; ++c) {
    const uint32_t t0 = (uint32_t)c * kChunk;
    if constexpr (C::NB == 2) {
      if (p.state_out) store_chunk_state<T, DK, DVS>(S, p, bh, c, wcol, lane);
    }
    const ChunkDecay cd(st.decay(hb, p, lane));

    // ---- (1) chunk c: registers -> LDS with the tile-relative decay factors
    {
      const RowB<T, DK, DVS> brow(cd, tid);
#pragma unroll
      for (int m = 0; m < C::QU; ++m) {
        const int u = tid + m * C::NT;
        const int row = u / (DK / 8), c8 = u % (DK / 8);
        const int tile = row >> 4;
        const float rj = cd.r(tile);
        E::store8_scaled(sm.qh + row * C::QLD + c8 * 8, st.q[m], exp_e(brow.v[m] - rj));
        const float kref = DIAG ? cd.end(tile) : rj;
        E::store8_scaled(sm.kh + row * C::QLD + c8 * 8, st.k[m], exp_e(kref - brow.v[m]));
        if (DIAG) {
          E::store8_raw(sm.qr + row * C::QLD + c8 * 8, st.q[m]);
          E::store8_raw(sm.kr + row * C::QLD + c8 * 8, st.k[m]);
        }
      }
      stage_state_operands<T, DK, DVS, true>(sm.kp, sm.vv, st, cd, brow, tid);
      if (DIAG && tid < 64) sm.sb[tid] = cd.b;
    }

    // ---- (2) prefetch chunk c + 1 while c is computed.  The last iteration re-reads
    //      its own chunk so every iteration issues the same loads.
    st.load(hb, p, (uint32_t)min(c + 1, c_end - 1) * kChunk, col0, tid);
    __syncthreads();

    // ---- (3) attention matrix A of the chunk (bf16 / fp32 in LDS)
    {
      constexpr int NBLK = DIAG ? 6 : 10;
#pragma unroll
      for (int bi = 0; bi < NBLK; ++bi) {
        if (bi % C::NW != wave) continue;  // wave-uniform
        const int jb = DIAG ? off_j(bi) : tri_j(bi);
        const int ib = DIAG ? off_i(bi) : tri_i(bi);
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const typename E::Frag ka = E::load_frag(sm.kh + (ib * 16 + r16) * C::QLD, ks * 32 + 4 * g);
          const typename E::Frag qb = E::load_frag(sm.qh + (jb * 16 + r16) * C::QLD, ks * 32 + 4 * g);
          E::mfma(acc, ka, qb);
        }
        // acc[e] = (Qh_j . Kh_i), j = 16 jb + r16, i = 16 ib + 4 g + e
        const float ri = DIAG ? cd.end(ib) : cd.r(ib);
        const float f = (jb == ib) ? 1.0f : exp_e(cd.r(jb) - ri);
        float vals[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool keep = (jb != ib) || (4 * g + e <= r16);
          vals[e] = keep ? acc[e] * f : 0.0f;
        }
        E::store4(sm.a + (jb * 16 + r16) * C::TLD + ib * 16 + 4 * g, vals[0], vals[1], vals[2], vals[3]);
      }
      if (DIAG) {
        // diagonal tiles by explicit position pairs: A_ji = e^{b_j - b_i} (q_j . k_i), i <= j
        for (int e = tid; e < 4 * 256; e += C::NT) {
          const int u = e >> 8, j = (e >> 4) & 15, i = e & 15;
          float val = 0.0f;
          if (i <= j) {
            const T* qrow = sm.qr + (u * 16 + j) * C::QLD;
            const T* krow = sm.kr + (u * 16 + i) * C::QLD;
            float dot = 0.0f;
#pragma unroll 8
            for (int d = 0; d < DK; ++d) dot += E::to_f32(qrow[d]) * E::to_f32(krow[d]);
            val = dot * exp_e(sm.sb[u * 16 + j] - sm.sb[u * 16 + i]);
          }
          sm.a[(u * 16 + j) * C::TLD + u * 16 + i] = E::cvt(val);
        }
      }
    }
    __syncthreads();

    // ---- (4) o = e^{r_u(j)} Qh S_{c-1} + A V  for this wave's columns; then S_c
    {
      typename E::Frag Sf[C::NB][C::KS];
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) Sf[nb][ks] = E::from_acc(S.s[nb][2 * ks], S.s[nb][2 * ks + 1]);
      VFrags<T, DK, DVS> Vf;
      load_v_frags<T, DK, DVS>(Vf, sm.vv, wave, lane);

      floatx4 O[4][C::NB];
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) O[jb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
      // inter-chunk: O^T[n][j] = sum_d S[d][n] Qh[j][d]
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          const typename E::Frag qb = E::load_frag(sm.qh + (jb * 16 + r16) * C::QLD, ks * 32 + 4 * g);
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) E::mfma(O[jb][nb], Sf[nb][ks], qb);
        }
      }
#pragma unroll
      for (int jb = 1; jb < 4; ++jb) {
        const float f = exp_e(cd.r(jb));
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) O[jb][nb] *= f;
      }
      // intra-chunk: O^T[n][j] += sum_i v[n][i] A[j][i], keys up to the end of tile jb
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
        for (int ks = 0; ks <= jb / 2; ++ks) {
          const typename E::Frag ab = E::load_frag(sm.a + (jb * 16 + r16) * C::TLD, ks * 32 + 4 * g);
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) E::mfma(O[jb][nb], Vf.f[nb][ks], ab);
        }
      }
      state_update<T, DK, DVS>(S, Vf, sm.kp, exp_e(cd.gam), lane);
      // lane holds o[t0 + 16 jb + r16][wcol + 16 nb + 4 g + 0..3]
      store_o(O, t0, false);
    }
    __syncthreads();
  }

  if (seg == p.segments - 1) store_state<T, DK, DVS>(S, p.ST + (long long)bh * DK * p.dv, p.dv, wcol, g, r16);
}

// ============================================================================
// Host dispatch.
// ============================================================================
namespace {

template <typename T, int DK, int DVS>
hipError_t seg_launch(const ChunkParams& p, hipStream_t s) {
  hipLaunchKernelGGL((segment_state_kernel<T, DK, DVS>), dim3(p.grid), dim3(Cfg<T, DK, DVS>::NT), 0, s, p);
  return hipGetLastError();
}

template <typename T, int DK, int DVS, bool DIAG>
hipError_t out_launch(const ChunkParams& p, hipStream_t s) {
  hipLaunchKernelGGL((chunk_output_kernel<T, DK, DVS, DIAG>), dim3(p.grid), dim3(Cfg<T, DK, DVS>::NT), 0, s,
                     p);
  return hipGetLastError();
}

// Built (dtype, dk, slice) combinations.  fp32 keeps slices <= 64 columns (LDS and
// registers); the fp32 diagonal-branch path needs dk = 64 (raw q, k in LDS).
template <typename F>
hipError_t dispatch(int dtype, int dk, int slice, bool diag, F&& f) {
#define GLA_CASE(TT, DKV, DVSV)                                                   \
  if (dk == DKV && slice == DVSV) {                                                \
    return diag ? f.template operator()<TT, DKV, DVSV, true>()                     \
                : f.template operator()<TT, DKV, DVSV, false>();                   \
  }
  if (dtype == 0) {
    GLA_CASE(bf16, 128, 128) GLA_CASE(bf16, 128, 64) GLA_CASE(bf16, 128, 32) GLA_CASE(bf16, 128, 16)
    GLA_CASE(bf16, 64, 64) GLA_CASE(bf16, 64, 32) GLA_CASE(bf16, 64, 16)
  } else {
    if (!diag || dk == 64) {
      GLA_CASE(float, 128, 64) GLA_CASE(float, 128, 32) GLA_CASE(float, 128, 16)
      GLA_CASE(float, 64, 64) GLA_CASE(float, 64, 32) GLA_CASE(float, 64, 16)
    }
  }
#undef GLA_CASE
  return hipErrorInvalidValue;
}

struct OutFn {
  const ChunkParams& p;
  hipStream_t s;
  template <typename T, int DK, int DVS, bool DIAG>
  hipError_t operator()() const {
    if constexpr (DIAG && sizeof(T) == 4 && DK == 128) {
      return hipErrorInvalidValue;
    } else {
      return out_launch<T, DK, DVS, DIAG>(p, s);
    }
  }
};

struct SegFn {
  const ChunkParams& p;
  hipStream_t s;
  template <typename T, int DK, int DVS, bool DIAG>
  hipError_t operator()() const {
    if constexpr (DIAG) {
      return hipErrorInvalidValue;  // the pre-pass has no diagonal tiles
    } else {
      return seg_launch<T, DK, DVS>(p, s);
    }
  }
};

struct ProbeFn {
  template <typename T, int DK, int DVS, bool DIAG>
  hipError_t operator()() const {
    if constexpr (DIAG && sizeof(T) == 4 && DK == 128) return hipErrorInvalidValue;
    return hipSuccess;
  }
};

}  // namespace

bool chunk_config_built(int dtype, int dk, int slice, bool diag) {
  if (ws_kernels_supported(dtype, dk, slice)) return true;
  return dispatch(dtype, dk, slice, diag, ProbeFn{}) == hipSuccess;
}

// Segment prefix scan, in place: the local final states H_0 .. H_{P-2} of a unit
// (from zero states, as the pre-pass leaves them) become the states reached from a
// zero state at the start of the unit,
//   P_0 = H_0,   P_p = e^{Gamma_p} P_{p-1} + H_p,
// so that segment p > 0 starts from e^{Gamma_0 + .. + Gamma_{p-1}} S0 + P_{p-1}: one
// state read per output workgroup instead of a chain of p dependent reads.  Thread =
// 4 consecutive elements of one unit's states; its loads are issued in batches of 8
// segments ahead of the arithmetic that consumes them.  A workgroup lies within one
// unit (per_state4 is a multiple of the block size), so whether a batch can be
// skipped is uniform, and its decays are read before any state moves.  Where
// e^{Gamma_p} is exactly zero in fp32, P_p = H_p (up to the sign of an exact zero) is
// already in place; a batch whose factors are all zero, and whose last state the next
// batch does not carry forward, is skipped without touching memory.
constexpr int kPrefixThreads = 256;
constexpr int kPrefixBatch = 8;

__global__ void __launch_bounds__(kPrefixThreads) segment_prefix_kernel(float* __restrict__ seg_state,
                                                                        const float* __restrict__ seg_decay,
                                                                        int segments, int per_state4, int units) {
  const long long gid = (long long)blockIdx.x * kPrefixThreads + threadIdx.x;
  const int unit = __builtin_amdgcn_readfirstlane((int)(gid / per_state4));
  if (unit >= units) return;
  const int e4 = (int)(gid - (long long)unit * per_state4);
  const int nseg = segments - 1;
  floatx4* H = reinterpret_cast<floatx4*>(seg_state) + (long long)unit * nseg * per_state4 + e4;
  const float* G = seg_decay + (long long)unit * segments;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < nseg; p0 += kPrefixBatch) {
    // f[j] = e^{Gamma_{p0+j}} for 0 < p0 + j < nseg, else 0 (no carry into P_0 or past the end)
    // (lane j reads Gamma_{p0+j}: one load for the batch, then one readlane per factor)
    const float el = exp_e(G[min(p0 + (int)(threadIdx.x & 63), nseg - 1)]);
    float f[kPrefixBatch + 1];
    bool live = false;
#pragma unroll
    for (int j = 0; j <= kPrefixBatch; ++j) {
      const int ps = p0 + j;
      const float e = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, el), j));
      f[j] = ps > 0 && ps < nseg ? e : 0.0f;
      live |= f[j] != 0.0f;
    }
    if (!live) {  // uniform across the workgroup
      acc = floatx4{0.f, 0.f, 0.f, 0.f};
      continue;
    }
    floatx4 h[kPrefixBatch];
#pragma unroll
    for (int j = 0; j < kPrefixBatch; ++j) h[j] = H[(long long)min(p0 + j, nseg - 1) * per_state4];
#pragma unroll
    for (int j = 0; j < kPrefixBatch; ++j) {
      const int ps = p0 + j;
      if (ps >= nseg) break;
      acc = ps == 0 ? h[j] : f[j] * acc + h[j];
      if (ps > 0) H[(long long)ps * per_state4] = acc;
    }
  }
}

hipError_t launch_segment_prefix(const ChunkParams& p, hipStream_t stream) {
  const int per_state4 = p.dk * p.dv / 4;
  const long long threads = (long long)p.BH * per_state4;
  const int blocks = (int)((threads + kPrefixThreads - 1) / kPrefixThreads);
  hipLaunchKernelGGL(segment_prefix_kernel, dim3(blocks), dim3(kPrefixThreads), 0, stream, p.seg_state,
                     p.seg_decay, p.segments, per_state4, p.BH);
  return hipGetLastError();
}

hipError_t launch_segment_states(const ChunkParams& p, int dtype, hipStream_t stream) {
  if (p.segments <= 1 || p.grid == 0) return hipSuccess;
  hipError_t e = ws_kernels_supported(dtype, p.dk, p.dv / p.nslices)
                     ? launch_segment_states_ws(p, p.dk, p.dv / p.nslices, stream)
                     : dispatch(dtype, p.dk, p.dv / p.nslices, false, SegFn{p, stream});
  if (e != hipSuccess || p.segments <= 2) return e;  // a single local state is already its own prefix
  return launch_segment_prefix(p, stream);
}

hipError_t launch_chunk_output(const ChunkParams& p, int dtype, bool diag, hipStream_t stream) {
  if (p.grid == 0) return hipSuccess;
  if (ws_kernels_supported(dtype, p.dk, p.dv / p.nslices))
    return launch_chunk_output_ws(p, p.dk, p.dv / p.nslices, diag, stream);
  return dispatch(dtype, p.dk, p.dv / p.nslices, diag, OutFn{p, stream});
}

// debug builds: this unit's LDS-check word (see GLA_CHECK_LDS)
GLA_DEBUG_ACCESSOR(debug_word_chunk_kernels)

}  // namespace gla
