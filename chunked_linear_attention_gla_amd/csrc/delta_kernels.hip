// delta_kernels.hip -- chunked gated delta rule on gfx950 matrix cores.
//
// Source: "Engineering Long-Context Training for Trillion-Parameter MoE Models:
// Three Key Breakthroughs" (§3.1: Delta-Net-style structures share the chunked
// computation and its diagonal-tile problem; §3.2 the bounded gate; §3.3 every
// causal tile on the dense matrix product).  The recurrence, in the plainest
// reading of a gated delta rule with that decay:
//     S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t.
//
// Chunked form.  S_t = a_t S_{t-1} + k_t u_t^T with the effective write
// u_t = beta_t (v_t - a_t S_{t-1}^T k_t).  Inside a 64-token chunk with
// cumulative log-decay b (as in the linear-attention kernels) and S_0 the state
// before the chunk, a_t S_{t-1} = e^{b_t} S_0 + sum_{s<t} e^{b_t - b_s} k_s u_s^T, so
//     (I + diag(beta) L) U = diag(beta) V - diag(beta e^b) K S_0,
//     L[t][s] = e^{b_t - b_s} (k_t . k_s)  for s < t.
// With Tinv = (I + diag(beta) L)^-1 (unit lower triangular):
//     W = Tinv diag(beta e^b) K,  Ut = Tinv diag(beta) V   (no dependence on S_0)
//     U = Ut - W S_0
//     o = e^b (Q S_0) + A U,   A[t][s] = e^{b_t - b_s} (q_t . k_s), s <= t
//     S_c = e^gamma S_0 + (K e^{gamma - b})^T U
// i.e. the linear-attention chunk with the values replaced by U.  L and A are
// causal 64x64 decay-weighted Gram matrices: both come out of the unified tile
// product of the linear-attention kernels (q or k scaled by e^{b - r_u}, k by
// e^{r_u - b}, tile scalar e^{r_u(t) - r_u(s)}), safe because the bounded gate
// keeps a 16-token tile's reciprocal decay below e^80 [§3.2].
//
// Two passes:
//   delta_prep_kernel   one workgroup per (head, chunk), all chunks in parallel:
//                       L, Tinv (fp32, 16x16 blocks: forward substitution on the
//                       diagonal blocks, matrix-core products for the others),
//                       written to the workspace in the operand dtype, and with
//                       segments each chunk's reset flag (below).
//   delta_segment_kernel for sequence segments: the affine map S_end = Phi S_start
//                       + H of every segment but the last (Phi = prod of the chunk
//                       transitions e^gamma I - (k e^{gamma-b})^T W, run as dk extra
//                       columns from the identity with no writes).
//   delta_output_kernel one workgroup per (head, slice of value columns, segment),
//                       chunks in order from the folded start state: the effective
//                       writes U = Tinv (diag(beta) V - diag(beta e^b) K S_0) (= Ut -
//                       W S_0) on the matrix cores from Tinv and the staged k and v,
//                       then o and the state update as in the linear-attention output
//                       pass.
#include "chunk_common.h"

namespace gla {

namespace {

__device__ __forceinline__ uint32_t dl_row(uint32_t t, uint32_t Tn, uint32_t row_bytes) {
  return t < Tn ? t * row_bytes : kDroppedOffset;
}

// Row-major tiles read as MFMA fragments (Qh, Kh, beta e^b k, the key operands of L)
// use the swizzle frag_swz of gla_device.h; the staging loops below give each wave
// whole 8-row groups (the row advances by a multiple of 16 per pass), so a store's swap
// is wave-uniform (frag_swap).

// acc += X Z for 16x16 fp32 blocks in LDS (X row stride ldx, Z row stride ldz):
// afterwards lane (g, r16) holds (X Z)[4 g + e][r16] in acc[e].
__device__ __forceinline__ void mm16(floatx4& acc, const float* X, int ldx, const float* Z, int ldz, int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[r * ldx + 4 * s + g], Z[(4 * s + g) * ldz + r], acc, 0, 0, 0);
}

__device__ __forceinline__ void store16(float* dst, int ld, const floatx4& acc, float sign, int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int e = 0; e < 4; ++e) dst[(4 * g + e) * ld + r] = sign * acc[e];
}

// ============================================================================
// Pass 1: Tinv = (I + diag(beta) L)^-1 of every chunk (and its reset flag).
// ============================================================================
// Steps Q..14 of the right-looking forward substitution of a unit lower triangular
// 16x16 block (strictly lower part in m, row stride LD) on 64 lanes: lane (g, r16)
// holds rows 4 k + g of column r16 in x[k]; step q broadcasts the final x_q from row
// group q % 4 and subtracts m[i][q] x_q from every row i > q.
template <int Q, int LD>
__device__ __forceinline__ void substitute_rows(float (&x)[4], const float* m, int g) {
  if constexpr (Q < 15) {
    const float xq = row_broadcast<Q % 4>(x[Q / 4]);
#pragma unroll
    for (int k = Q / 4; k < 4; ++k) {
      const float u = fmaf(-m[(4 * k + g) * LD + Q], xq, x[k]);
      x[k] = (k > Q / 4 || g > Q % 4) ? u : x[k];  // rows 4 k + g > Q only
    }
    substitute_rows<Q + 1, LD>(x, m, g);
  }
}

template <typename T, int DK, int DV>
struct PrepCfg {
  static constexpr int NT = 256;
  static constexpr int PAD = Elem<T>::kPad;
  static constexpr int QLD = DK + PAD;
  static constexpr int QU = 8 * DK / NT;
  static constexpr int KS = DK / 32;
  static constexpr int KL = DK / 8;   // lanes that stage one key row
  // M is held as its 10 lower 16x16 blocks (block (I, J), J <= I, at index
  // I (I + 1) / 2 + J; the diagonal ones later hold Tinv's), Tinv's six blocks below the
  // diagonal apart (J < I, at index I (I - 1) / 2 + J), 16 rows each at a padded
  // stride: M's 18 puts the left-operand reads of the fp32 block products (row r,
  // column 4 s + g) on banks 18 r + g, distinct within each half-wave; Tinv's 20 does
  // the same for store16 (banks 16 g + r).
  static constexpr int MLD = 18;
  static constexpr int FLD = 20;
};

__device__ __forceinline__ constexpr int lblk(int I, int J) { return I * (I + 1) / 2 + J; }
__device__ __forceinline__ constexpr int sblk(int I, int J) { return I * (I - 1) / 2 + J; }  // J < I

// LDS: the staged keys, then (over them, once M is formed in registers) M and Tinv's
// blocks below the diagonal in fp32 (M's diagonal blocks become Tinv's once inverted);
// per-row factors.  At d = 128 that is 20 KB, eight workgroups per compute unit (the
// pass is a chain of short phases between barriers, so the workgroups in flight set its
// speed).
template <typename T, int DK, int DV>
struct PrepSmem {
  using C = PrepCfg<T, DK, DV>;
  union {
    T kr[64 * C::QLD];               // k as loaded
    struct {
      float tf[6][16 * C::FLD];      // Tinv (fp32), blocks below the diagonal
      float mf[10][16 * C::MLD];     // M = diag(beta) L, lower blocks; diagonal ones then D_I of Tinv
    } t;
  } u1;
  float sb[64];                      // b
  float sbeta[64];
  float lk[64];                      // log2 of max_d |k_t[d] e^{gamma - b_t}|, per row
  float fac[64];                     // beta_s e^{b_s} max_d |k_s[d]|, per row
  int vote[4];
};

template <typename T, int DK, int DV>
__global__ void __launch_bounds__(256) delta_prep_kernel(DeltaParams p) {
  using E = Elem<T>;
  using C = PrepCfg<T, DK, DV>;
  __shared__ __attribute__((aligned(16))) PrepSmem<T, DK, DV> sm;  // 16-byte aligned: row stores compile to ds_write_b128
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const long long bh = blockIdx.x / p.nchunks;
  const int c = (int)(blockIdx.x - bh * p.nchunks);
  const uint32_t t0 = (uint32_t)c * kChunk;
  const uint32_t Tn = (uint32_t)p.T;
  const bool test = p.reset != nullptr;  // uniform: the reset test only runs for plans with segments
  const rsrc_t rk = make_rsrc(static_cast<const T*>(p.k) + bh * p.T * DK, Tn * DK * (uint32_t)sizeof(T));

  // ---- operands: loads first, decays after the barrier that publishes b and beta
  typename E::Vec8 kv[C::QU];
#pragma unroll
  for (int m = 0; m < C::QU; ++m) {
    const int u = tid + m * C::NT, row = u / C::KL, c8 = u % C::KL;
    kv[m] = E::load8(rk, dl_row(t0 + row, Tn, DK * (uint32_t)sizeof(T)) + c8 * 8 * (uint32_t)sizeof(T));
  }
  if (tid < 64) {
    const long long t = (long long)t0 + tid;
    const long long tc = t < p.T ? t : p.T - 1;  // absent tokens: g = 0, beta = 0
    sm.sb[tid] = p.b[bh * p.T + tc];
    sm.sbeta[tid] = t < p.T ? p.beta[bh * p.T + t] : 0.0f;
  }
  __syncthreads();
  const int last = (int)(((long long)Tn - 1 - t0) < 63 ? ((long long)Tn - 1 - t0) : 63);
  const float gam = sm.sb[last];  // the chunk's total log-decay
#pragma unroll
  for (int m = 0; m < C::QU; ++m) {
    const int u = tid + m * C::NT, row = u / C::KL, c8 = u % C::KL;
    E::store8_scaled_sw(sm.u1.kr + row * C::QLD + c8 * 8, kv[m], 1.0f, frag_swap<T>(row));
    if (test) {
      // max_d |k_row[d]| over the row's KL consecutive lanes: the key side of the reset
      // test and the row's factor in the bound on |W| below
      float mx = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(E::get(kv[m], e)));
      mx = group_max<C::KL>(mx);
      if (c8 == 0) {
        const float br = sm.sb[row];
        sm.lk[row] = __builtin_amdgcn_logf(mx) + (gam - br) * kLog2e;
        sm.fac[row] = sm.sbeta[row] * exp_e(br) * mx;
      }
    }
  }
  __syncthreads();

  // ---- M = diag(beta) L over the 10 causal tiles, strictly below the diagonal:
  //      k_t . k_s on the matrix cores, then the decay e^{b_t - b_s} (<= 1 where kept;
  //      the masked entries are selected away, never multiplied).  Wave I forms its
  //      diagonal tile and one or two of the six below the diagonal in registers; they
  //      go to LDS over the keys once every wave is done with those.
  const auto m_tile = [&](int jb, int ib, floatx4& out) {  // block row, block column
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      E::mfma(acc, E::load_frag(sm.u1.kr + (ib * 16 + r16) * C::QLD, ks * 32 + ((4 * g) ^ frag_swz<T>(r16))),
              E::load_frag(sm.u1.kr + (jb * 16 + r16) * C::QLD, ks * 32 + ((4 * g) ^ frag_swz<T>(r16))));
    // acc[e]: row t = 16 jb + r16, column s = 16 ib + 4 g + e
    const int tr = jb * 16 + r16;
    const float bt = sm.sb[tr], bet = sm.sbeta[tr];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int sc = ib * 16 + 4 * g + e;
      out[e] = (jb != ib || 4 * g + e < r16) ? acc[e] * (exp_e(bt - sm.sb[sc]) * bet) : 0.0f;
    }
  };
  const auto m_store = [&](int jb, int ib, const floatx4& v) {
    float* mb = &sm.u1.t.mf[lblk(jb, ib)][0];
#pragma unroll
    for (int e = 0; e < 4; ++e) mb[r16 * C::MLD + 4 * g + e] = v[e];
  };
  // wave I: (I, I), then (1, 0) and (3, 0) | (2, 0) and (3, 1) | (2, 1) | (3, 2)
  const int ja = wave == 2 ? 2 : 3, ia = wave == 0 ? 0 : wave == 1 ? 1 : wave == 2 ? 1 : 2;
  const int jb2 = wave == 0 ? 1 : 2;  // second tile of waves 0 and 1: (1, 0), (2, 0)
  floatx4 md, m1, m2;
  m_tile(wave, wave, md);
  m_tile(ja, ia, m1);
  if (wave < 2) m_tile(jb2, 0, m2);  // wave-uniform
  __syncthreads();  // the keys are read; M goes over them
  m_store(wave, wave, md);
  m_store(ja, ia, m1);
  if (wave < 2) m_store(jb2, 0, m2);
  // ---- diagonal block D_I of Tinv = (I + M)^-1 by forward substitution, right-looking
  //      (each x_q, once final, is subtracted from the later rows at once: a 15-step
  //      chain) on all 64 lanes: lane (g, r16) holds rows 4 k + g (k = 0..3) of column
  //      r16, and x_q passes from row group q % 4 to the others by a row broadcast.  D_I
  //      replaces M's diagonal block, which nothing reads afterwards; the wave's own LDS
  //      writes and reads stay in order.
  {
    float* mb = &sm.u1.t.mf[lblk(wave, wave)][0];
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = (4 * k + g == r16) ? 1.0f : 0.0f;
    substitute_rows<0, C::MLD>(x, mb, g);
#pragma unroll
    for (int k = 0; k < 4; ++k) mb[(4 * k + g) * C::MLD + r16] = x[k];
  }
  // ---- blocks below the diagonal, wave J taking block column J from the top:
  //      X_IJ = -D_I sum_{J <= K < I} M_IK X_KJ needs only blocks of its own column and
  //      the diagonal blocks D, so the column needs no barrier until it is complete.
  //      X_JJ = D_J sits in M's diagonal block (stride MLD), the others in tf; the block
  //      being formed is its own scratch (mm16 reads all of it before the store).
  {
    const int J = wave;
    for (int I = J + 1; I < 4; ++I) {  // wave-uniform
      float* dst = &sm.u1.t.tf[sblk(I, J)][0];
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      mm16(acc, &sm.u1.t.mf[lblk(I, J)][0], C::MLD, &sm.u1.t.mf[lblk(J, J)][0], C::MLD, lane);
      for (int K = J + 1; K < I; ++K)
        mm16(acc, &sm.u1.t.mf[lblk(I, K)][0], C::MLD, &sm.u1.t.tf[sblk(K, J)][0], C::FLD, lane);
      store16(dst, C::FLD, acc, 1.0f, lane);
      floatx4 x = {0.f, 0.f, 0.f, 0.f};
      mm16(x, &sm.u1.t.mf[lblk(I, I)][0], C::MLD, dst, C::FLD, lane);
      store16(dst, C::FLD, x, -1.0f, lane);
    }
  }
  __syncthreads();

  // ---- Tinv in the operand dtype to the workspace, row-major [64][64] and zero above
  //      the diagonal blocks (the later passes form W and Ut from it and the chunk's k
  //      and v); 8 consecutive elements of a row per thread and step.  With the reset
  //      test, the same values bound each row of W = Tinv diag(beta e^b) K:
  //      max_d |W[t][d]| <= sum_s |Tinv[t][s]| beta_s e^{b_s} max_d |k_s[d]|.
  T* Tg = static_cast<T*>(p.Tinv) + ((long long)bh * p.nchunks + c) * (64 * 64);
  bool ok = gam * kLog2e < -127.0f;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int e = tid + m * C::NT, t = e >> 3, s = (e & 7) * 8;
    const int I = t >> 4, J = s >> 4;
    const bool keep = J <= I;
    // diagonal blocks in M's place (stride MLD), the others in tf; 8-byte reads (a row
    // of M's blocks starts at a multiple of 8 bytes only)
    const float* src = J < I ? &sm.u1.t.tf[sblk(I, J)][(t & 15) * C::FLD + (s & 15)]
                             : &sm.u1.t.mf[lblk(I, I)][(t & 15) * C::MLD + (s & 15)];
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      const float2 pr = *reinterpret_cast<const float2*>(src + k);
      v[k] = pr.x;
      v[k + 1] = pr.y;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = keep ? v[k] : 0.0f;
    if constexpr (sizeof(T) == 2) {
      typename E::Frag o;
#pragma unroll
      for (int k = 0; k < 8; ++k) o.v[k] = E::cvt(v[k]);
      *reinterpret_cast<bf16x8*>(Tg + t * 64 + s) = o.v;
    } else {
      *reinterpret_cast<float4*>(Tg + t * 64 + s) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(Tg + t * 64 + s + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
    if (test) {
      const float4 f0 = *reinterpret_cast<const float4*>(&sm.fac[s]);
      const float4 f1 = *reinterpret_cast<const float4*>(&sm.fac[s + 4]);
      float wb = fabsf(v[0]) * f0.x + fabsf(v[1]) * f0.y + fabsf(v[2]) * f0.z + fabsf(v[3]) * f0.w +
                 fabsf(v[4]) * f1.x + fabsf(v[5]) * f1.y + fabsf(v[6]) * f1.z + fabsf(v[7]) * f1.w;
      wb = group_sum<8>(wb);  // the row's 8 threads are consecutive lanes
      ok = ok && (sm.lk[t] + __builtin_amdgcn_logf(wb) < -128.0f);
    }
  }
  if (!test) return;  // uniform
  // Reset test of the chunk.  The transition P = e^gamma I - (k e^{gamma-b})^T W has
  // |P[d][e]| <= e^gamma + sum_t |kt_t|max |w_t|max, so |P H| <= 2^13 2^-127 max|H| once
  // every term is below 2^-127 (64 rows, 128 columns): the state after this chunk then
  // does not depend on the state before it, to 2^-114 relative.  The terms are compared
  // in log2 (no product underflows on the way) against 2^-128, which leaves a factor 2
  // for the rounding of Tinv, k and the factors in the operand dtype; NaN terms fail
  // the comparison, so they never mark a reset.
  const unsigned long long no = __ballot(!ok);
  if (lane == 0) sm.vote[wave] = no == 0ull;
  __syncthreads();
  if (tid == 0) p.reset[bh * p.nchunks + c] = sm.vote[0] & sm.vote[1] & sm.vote[2] & sm.vote[3];
}

// ============================================================================
// Pass 2 (and the segment pre-pass): chunks in order.  Each wave forms the effective
// writes of its own value columns from the chunk's Tinv (pass 1) and the k and v these
// passes stage anyway, U = Tinv (diag(beta) V - diag(beta e^b) K S_0): the same U as
// Ut - W S_0, without forming W.
// ============================================================================
template <typename T, int DK, int DVS>
struct DoCfg {
  static constexpr int NW = DVS / 16;        // waves, 16 value columns each
  static constexpr int NT = 64 * NW;
  static constexpr int PAD = Elem<T>::kPad;
  static constexpr int QLD = DK + PAD;
  static constexpr int TLD = 64 + 4;   // row stride of A and Tinv: their 8-byte stores and fragment reads are conflict-free
  static constexpr int QU = 8 * DK / NT;
  static constexpr int VU = 8 * DVS / NT;      // 8-element v pieces per thread
  static constexpr int TU = 64 * 64 / 8 / NT;  // 8-element Tinv pieces per thread
  static constexpr int DB = DK / 16;
  static constexpr int KS = DK / 32;
  static_assert(QU >= 1 && QU * NT == 8 * DK, "staging must divide evenly");
  static_assert(VU >= 1 && VU * NT == 8 * DVS, "v staging must divide evenly");
  static_assert(TU >= 1 && TU * NT * 8 == 64 * 64, "Tinv staging must divide evenly");
};

template <typename T, int DK, int DVS>
struct DoSmem {
  using C = DoCfg<T, DK, DVS>;
  T qh[64 * C::QLD];
  T kh[64 * C::QLD];
  T kp[2][TokTile<T, DK>::SIZE];  // k e^{gamma - b}, token-major, by chunk parity
  T kb[64 * C::QLD];              // beta e^b k, row-major, read as fragments (swizzled as qh)
  T vb[TokTile<T, DVS>::SIZE];    // beta v of the slice, token-major
  T tv[64 * C::TLD];              // Tinv
  T a[64 * C::TLD];
};

template <typename T, int DK, int DVS>
struct DsSmem {
  using C = DoCfg<T, DK, DVS>;
  T kp[TokTile<T, DK>::SIZE];
  T kb[64 * C::QLD];
  T vb[TokTile<T, DVS>::SIZE];
  T tv[64 * C::TLD];
  int nonzero[2][C::NW];  // transition half: per wave, whether its columns are nonzero, by chunk parity
};

// One chunk of (q,) k, (v,) Tinv, b and beta on its way to LDS, in row-contiguous
// 16-byte pieces (rows past the end read zeros; b past the end repeats the last value,
// beta past the end is 0).
template <typename T, int DK, int DVS, bool LOAD_Q, bool LOAD_V>
struct DoStaged {
  using E = Elem<T>;
  using C = DoCfg<T, DK, DVS>;
  typename E::Vec8 q[LOAD_Q ? C::QU : 1], k[C::QU], v[LOAD_V ? C::VU : 1], ti[C::TU];
  float b, be;

  // chunk c (first token t0) of the slice starting at value column col0
  __device__ __forceinline__ void load(const rsrc_t& rq, const rsrc_t& rk, const rsrc_t& rv, const rsrc_t& rt,
                                       const rsrc_t& rb, const rsrc_t& rbe, uint32_t Tn, int dv, int c, int col0,
                                       int tid) {
    const int lane = tid & 63;
    const uint32_t t0 = (uint32_t)c * kChunk, tb = t0 + lane;
    b = buf_load4(rb, (tb < Tn ? tb : Tn - 1) * 4u);
    be = buf_load4(rbe, tb * 4u);  // past the end: out of range, reads 0
#pragma unroll
    for (int m = 0; m < C::QU; ++m) {
      const int u = tid + m * C::NT, row = u / (DK / 8), c8 = u % (DK / 8);
      const uint32_t off = dl_row(t0 + row, Tn, DK * (uint32_t)sizeof(T)) + c8 * 8 * (uint32_t)sizeof(T);
      if (LOAD_Q) q[m] = E::load8(rq, off);
      k[m] = E::load8(rk, off);
    }
    if constexpr (LOAD_V) {
#pragma unroll
      for (int m = 0; m < C::VU; ++m) {
        const int u = tid + m * C::NT, row = u / (DVS / 8), c8 = u % (DVS / 8);
        v[m] = E::load8(rv, dl_row(t0 + row, Tn, (uint32_t)dv * (uint32_t)sizeof(T)) +
                                (col0 + c8 * 8) * (uint32_t)sizeof(T));
      }
    }
#pragma unroll
    for (int m = 0; m < C::TU; ++m) {
      const int u = tid + m * C::NT;  // row u / 8, columns 8 (u % 8)..+7 of chunk c's Tinv
      ti[m] = E::load8(rt, ((uint32_t)c * 4096u + (uint32_t)u * 8u) * (uint32_t)sizeof(T));
    }
  }
};

// The state-side operands of the staged chunk into LDS: k e^{gamma - b} (token-major),
// beta e^b k (row-major, swizzled for fragment reads), beta v (token-major, with v) and
// Tinv (row-major).
template <typename T, int DK, int DVS, bool LOAD_Q, bool LOAD_V>
__device__ __forceinline__ void stage_state_side(T* kp, T* kb, T* vb, T* tv,
                                                 const DoStaged<T, DK, DVS, LOAD_Q, LOAD_V>& st,
                                                 const ChunkDecay& cd, int tid) {
  using C = DoCfg<T, DK, DVS>;
#pragma unroll
  for (int m = 0; m < C::QU; ++m) {
    const int u = tid + m * C::NT, row = u / (DK / 8), c8 = u % (DK / 8);
    const float br = cd.at(row), ber = __shfl(st.be, row);
    TokTile<T, DK>::store8(kp, row, c8 * 8, st.k[m], exp_e(cd.gam - br));
    Elem<T>::store8_scaled_sw(kb + row * C::QLD + c8 * 8, st.k[m], ber * exp_e(br), frag_swap<T>(row));
  }
  if constexpr (LOAD_V) {
#pragma unroll
    for (int m = 0; m < C::VU; ++m) {
      const int u = tid + m * C::NT, row = u / (DVS / 8), c8 = u % (DVS / 8);
      TokTile<T, DVS>::store8(vb, row, c8 * 8, st.v[m], __shfl(st.be, row));
    }
  }
#pragma unroll
  for (int m = 0; m < C::TU; ++m) {
    const int u = tid + m * C::NT, row = u >> 3, c8 = u & 7;
    T* dst = tv + row * C::TLD + c8 * 8;
    GLA_CHECK_LDS(dst, 8 * (unsigned)sizeof(T));
    if constexpr (sizeof(T) == 2) {  // rows are 8-byte aligned at this stride
      *reinterpret_cast<uint2*>(dst) = make_uint2(st.ti[m].u.x, st.ti[m].u.y);
      *reinterpret_cast<uint2*>(dst + 4) = make_uint2(st.ti[m].u.z, st.ti[m].u.w);
    } else {
      *reinterpret_cast<float4*>(dst) = st.ti[m].a;
      *reinterpret_cast<float4*>(dst + 4) = st.ti[m].b;
    }
  }
}

// The effective writes of the wave's 16 value columns (slice column colr), S_0 given
// as operand fragments Sf: U = Tinv R with R = diag(beta) V - Y, Y = diag(beta e^b) K S_0.
// Y comes out with tokens as accumulator rows -- Y[jb][e] = Y[16 jb + 4 g + e][colr + r16]
// -- so two stacked 16-token blocks are already the right-hand operand of the product
// with Tinv (the fragment convention of gla_device.h), beta v entering through the
// transposing read of the same tokens and columns; U's accumulators again hold tokens as
// rows, so Uf are the operand fragments of A.U and the state update.  Tinv is zero
// above its diagonal 16x16 blocks, so token block tb needs K-steps up to tb / 2 only.
// Without v (LOAD_V = false: the transition half) R = -Y.
template <typename T, int DK, int DVS, bool LOAD_V>
__device__ __forceinline__ void effective_writes(typename Elem<T>::Frag (&Uf)[2],
                                                 const typename Elem<T>::Frag (&Sf)[DK / 32], const T* kb,
                                                 const T* vb, const T* tv, int colr, int lane) {
  using E = Elem<T>;
  using C = DoCfg<T, DK, DVS>;
  const int r16 = lane & 15, g = lane >> 4;
  floatx4 Y[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    Y[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      E::mfma(Y[jb], E::load_frag(kb + (jb * 16 + r16) * C::QLD, ks * 32 + ((4 * g) ^ frag_swz<T>(r16))), Sf[ks]);
  }
  typename E::Frag R[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    floatx4 lo = -Y[2 * ks], hi = -Y[2 * ks + 1];
    if constexpr (LOAD_V) {
      const typename E::Frag vf = TokTile<T, DVS>::load(vb, ks * 32, colr, lane);
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] += static_cast<float>(vf.v[e]);
          hi[e] += static_cast<float>(vf.v[4 + e]);
        }
      } else {
        lo += vf.lo;
        hi += vf.hi;
      }
    }
    R[ks] = E::from_acc(lo, hi);
  }
  floatx4 U[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    U[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks <= tb / 2; ++ks) E::mfma(U[tb], E::load_frag(tv + (tb * 16 + r16) * C::TLD, ks * 32 + 4 * g), R[ks]);
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) Uf[ks] = E::from_acc(U[2 * ks], U[2 * ks + 1]);
}

// S <- e^gamma S + (k e^{gamma - b})^T U
template <typename T, int DK, int DVS>
__device__ __forceinline__ void delta_state_update(floatx4 (&S)[DK / 16], const typename Elem<T>::Frag (&Uf)[2],
                                                   const T* kp, float dec, int lane) {
  using E = Elem<T>;
  using C = DoCfg<T, DK, DVS>;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) S[db] *= dec;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) E::mfma(S[db], TokTile<T, DK>::load(kp, ks * 32, db * 16, lane), Uf[ks]);
}

// Segment pre-pass: for every segment but the last, run its chunks from a zero
// state (PHI = false: the local state H, value columns) or from the identity with
// no writes (PHI = true: the segment's state transition, dk columns), i.e. the
// affine map S_end = Phi S_start + H.  One workgroup per (head, segment, slice).
template <typename T, int DK, int NCOL, bool PHI>
__global__ void __launch_bounds__((DoCfg<T, DK, NCOL>::NT)) delta_segment_kernel(DeltaParams p) {
  using E = Elem<T>;
  using C = DoCfg<T, DK, NCOL>;
  __shared__ __attribute__((aligned(16))) DsSmem<T, DK, NCOL> sm;  // 16-byte aligned: row stores compile to ds_write_b128
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int nseg = p.segments - 1;
  const int ncol = PHI ? DK : p.dv;
  const int nsl = ncol / NCOL;
  const int L = xcd_linear_index(blockIdx.x, p.BH * nseg * nsl);
  const int slice = L % nsl;
  const int rest = L / nsl;
  const int seg = rest % nseg;
  const int bh = rest / nseg;
  const int col0 = slice * NCOL;
  const int wcol = col0 + wave * 16;
  const int c_begin = (int)((long long)seg * p.nchunks / p.segments);
  const int c_end = (int)((long long)(seg + 1) * p.nchunks / p.segments);
  const uint32_t Tn = (uint32_t)p.T;
  const uint32_t es = (uint32_t)sizeof(T);
  const rsrc_t rk = make_rsrc(static_cast<const T*>(p.k) + (long long)bh * p.T * DK, Tn * DK * es);
  const rsrc_t rv = make_rsrc(static_cast<const T*>(p.v) + (long long)bh * p.T * p.dv, Tn * (uint32_t)p.dv * es);
  const rsrc_t rt = make_rsrc(static_cast<const T*>(p.Tinv) + (long long)bh * p.nchunks * 4096,
                              (uint32_t)p.nchunks * 4096u * es);
  const rsrc_t rb = make_rsrc(p.b + (long long)bh * p.T, Tn * 4u);
  const rsrc_t rbe = make_rsrc(p.beta + (long long)bh * p.T, Tn * 4u);

  floatx4 S[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) S[db][e] = (PHI && db * 16 + 4 * g + e == wcol + r16) ? 1.0f : 0.0f;

  // The local state (from zero at the segment start) does not depend, to 2^-114 relative,
  // on anything before the segment's last chunk whose transition marks a reset: start
  // there from zero.  (The transition half keeps every chunk: it stops by itself once its
  // product is exactly zero.)
  int c_first = c_begin;
  if (!PHI && p.reset) {
    int lastr = -1;
    for (int c0 = c_begin; c0 < c_end; c0 += 64) {  // wave-uniform
      const int cc = c0 + lane;
      if (cc < c_end && p.reset[(long long)bh * p.nchunks + cc] != 0) lastr = cc;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lastr = max(lastr, __shfl_xor(lastr, off));
    if (lastr >= 0) c_first = lastr;
  }

  DoStaged<T, DK, NCOL, false, !PHI> st;
  if (c_first < c_end) st.load(rk, rk, rv, rt, rb, rbe, Tn, p.dv, c_first, col0, tid);
  for (int c = c_first; c < c_end; ++c) {
    const ChunkDecay cd(st.b);
    stage_state_side<T, DK, NCOL, false, !PHI>(sm.kp, sm.kb, sm.vb, sm.tv, st, cd, tid);
    st.load(rk, rk, rv, rt, rb, rbe, Tn, p.dv, min(c + 1, c_end - 1), col0, tid);
    __syncthreads();
    typename E::Frag Sf[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) Sf[ks] = E::from_acc(S[2 * ks], S[2 * ks + 1]);
    typename E::Frag Uf[2];
    effective_writes<T, DK, NCOL, !PHI>(Uf, Sf, sm.kb, sm.vb, sm.tv, wave * 16, lane);
    delta_state_update<T, DK, NCOL>(S, Uf, sm.kp, exp_e(cd.gam), lane);
    if constexpr (PHI) {
      // Once this workgroup's columns of the running transition product are all
      // exactly zero, every later chunk leaves them zero: stop.  Each wave posts
      // whether its columns hold a nonzero value (slots by chunk parity, so that no
      // slot is written while another wave may still read it).
      bool nz = false;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) nz |= S[db][e] != 0.0f;
      if (lane == 0) sm.nonzero[(c - c_first) & 1][wave] = __ballot(nz) != 0ull;
    }
    __syncthreads();
    if constexpr (PHI) {
      const int par = (c - c_first) & 1;
      int any = 0;
#pragma unroll
      for (int w = 0; w < C::NW; ++w) any |= sm.nonzero[par][w];
      if (!any) break;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the prefetch of a chunk not run is not left in flight
  float* dst = PHI ? p.seg_phi + ((long long)bh * nseg + seg) * DK * DK
                   : p.seg_state + ((long long)bh * nseg + seg) * DK * p.dv;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[(long long)(db * 16 + 4 * g + e) * ncol + wcol + r16] = S[db][e];
}

template <typename T, int DK, int DVS>
__global__ void __launch_bounds__((DoCfg<T, DK, DVS>::NT)) delta_output_kernel(DeltaParams p) {
  using E = Elem<T>;
  using F = Elem<float>;
  using C = DoCfg<T, DK, DVS>;
  __shared__ __attribute__((aligned(16))) DoSmem<T, DK, DVS> sm;  // 16-byte aligned: row stores compile to ds_write_b128
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int L = xcd_linear_index(blockIdx.x, p.grid);
  const int slice = L % p.nslices;
  const int rest = L / p.nslices;
  const int seg = rest % p.segments;
  const int bh = rest / p.segments;
  const int col0 = slice * DVS;
  const int wcol = col0 + wave * 16;
  const int c_begin = (int)((long long)seg * p.nchunks / p.segments);
  const int c_end = (int)((long long)(seg + 1) * p.nchunks / p.segments);
  const uint32_t Tn = (uint32_t)p.T;
  const uint32_t es = (uint32_t)sizeof(T);
  const rsrc_t rq = make_rsrc(static_cast<const T*>(p.q) + (long long)bh * p.T * DK, Tn * DK * es);
  const rsrc_t rk = make_rsrc(static_cast<const T*>(p.k) + (long long)bh * p.T * DK, Tn * DK * es);
  const rsrc_t rv = make_rsrc(static_cast<const T*>(p.v) + (long long)bh * p.T * p.dv, Tn * (uint32_t)p.dv * es);
  const rsrc_t rt = make_rsrc(static_cast<const T*>(p.Tinv) + (long long)bh * p.nchunks * 4096,
                              (uint32_t)p.nchunks * 4096u * es);
  const rsrc_t rb = make_rsrc(p.b + (long long)bh * p.T, Tn * 4u);
  const rsrc_t rbe = make_rsrc(p.beta + (long long)bh * p.T, Tn * 4u);
  const rsrc_t ro = make_rsrc(p.o + (long long)bh * p.T * p.dv, Tn * (uint32_t)p.dv * 4u);

  // ---- initial state: S0 (or zero), then S <- Phi_p S + H_p over the earlier
  //      segments, in fp32 on the matrix cores.  Slice of the wave: S[16 db + 4 g + e][wcol + r16]
  floatx4 S[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const long long i = (long long)bh * DK * p.dv + (long long)(db * 16 + 4 * g + e) * p.dv + wcol + r16;
      S[db][e] = p.S0 ? p.S0[i] : 0.0f;
    }
  for (int ps = 0; ps < seg; ++ps) {
    const float* Phi = p.seg_phi + ((long long)bh * (p.segments - 1) + ps) * DK * DK;
    const float* Hs = p.seg_state + ((long long)bh * (p.segments - 1) + ps) * DK * p.dv;
    floatx4 N[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) N[db] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const F::Frag sf = F::from_acc(S[2 * ks], S[2 * ks + 1]);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const float* row = Phi + (long long)(db * 16 + r16) * DK + ks * 32 + 4 * g;
        F::Frag pf;
        pf.lo = *reinterpret_cast<const floatx4*>(row);
        pf.hi = *reinterpret_cast<const floatx4*>(row + 16);
        F::mfma(N[db], pf, sf);  // N[db][e] = (Phi S)[16 db + 4 g + e][wcol + r16]
      }
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[db][e] = N[db][e] + Hs[(long long)(db * 16 + 4 * g + e) * p.dv + wcol + r16];
  }
  for (int e = tid; e < 2 * 256; e += C::NT) {
    const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
    sm.a[(blk * 32 + rr) * C::TLD + blk * 32 + 16 + cc] = E::cvt(0.0f);
  }

  DoStaged<T, DK, DVS, true, true> st;
  if (c_begin < c_end) st.load(rq, rk, rv, rt, rb, rbe, Tn, p.dv, c_begin, col0, tid);
  for (int c = c_begin; c < c_end; ++c) {
    const uint32_t t0 = (uint32_t)c * kChunk;
    const ChunkDecay cd(st.b);
    // ---- (1) operands of chunk c
#pragma unroll
    for (int m = 0; m < C::QU; ++m) {
      const int u = tid + m * C::NT, row = u / (DK / 8), c8 = u % (DK / 8);
      const float br = cd.at(row), r = cd.r(row >> 4);
      const bool sw = frag_swap<T>(row);
      E::store8_scaled_sw(sm.qh + row * C::QLD + c8 * 8, st.q[m], exp_e(br - r), sw);
      E::store8_scaled_sw(sm.kh + row * C::QLD + c8 * 8, st.k[m], exp_e(r - br), sw);
    }
    T* const kp = sm.kp[(c - c_begin) & 1];
    stage_state_side<T, DK, DVS, true, true>(kp, sm.kb, sm.vb, sm.tv, st, cd, tid);
    // ---- (2) prefetch chunk c + 1 (the last iteration re-reads its own chunk)
    st.load(rq, rk, rv, rt, rb, rbe, Tn, p.dv, min(c + 1, c_end - 1), col0, tid);
    __syncthreads();

    // ---- (3) A over the 10 causal tiles; the effective writes U of the wave's columns;
    //      o_inter = e^{r_u} Qh S_0
#pragma unroll
    for (int t = 0; t < 10; ++t) {
      if (t % C::NW != wave) continue;  // wave-uniform
      const int jb = tri_j(t), ib = tri_i(t);
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        E::mfma(acc, E::load_frag(sm.kh + (ib * 16 + r16) * C::QLD, ks * 32 + ((4 * g) ^ frag_swz<T>(r16))),
                E::load_frag(sm.qh + (jb * 16 + r16) * C::QLD, ks * 32 + ((4 * g) ^ frag_swz<T>(r16))));
      const float f = (jb == ib) ? 1.0f : exp_e(cd.r(jb) - cd.r(ib));
      float vals[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) vals[e] = (jb != ib || 4 * g + e <= r16) ? acc[e] * f : 0.0f;
      E::store4(sm.a + (jb * 16 + r16) * C::TLD + ib * 16 + 4 * g, vals[0], vals[1], vals[2], vals[3]);
    }
    typename E::Frag Sf[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) Sf[ks] = E::from_acc(S[2 * ks], S[2 * ks + 1]);
    typename E::Frag Uf[2];
    effective_writes<T, DK, DVS, true>(Uf, Sf, sm.kb, sm.vb, sm.tv, wave * 16, lane);
    floatx4 O[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      O[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        E::mfma(O[jb], Sf[ks], E::load_frag(sm.qh + (jb * 16 + r16) * C::QLD, ks * 32 + ((4 * g) ^ frag_swz<T>(r16))));
      if (jb > 0) O[jb] *= exp_e(cd.r(jb));
    }
    __syncthreads();

    // ---- (4) o += A U (every wave's A tiles are in); S_c = e^gamma S_0 + (k e^{gamma - b})^T U
    {
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int ks = 0; ks <= jb / 2; ++ks)
          E::mfma(O[jb], Uf[ks], E::load_frag(sm.a + (jb * 16 + r16) * C::TLD, ks * 32 + 4 * g));
      delta_state_update<T, DK, DVS>(S, Uf, kp, exp_e(cd.gam), lane);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
        buf_store16(ro, dl_row(t0 + jb * 16 + r16, Tn, (uint32_t)p.dv * 4u) + (wcol + 4 * g) * 4u, O[jb]);
    }
    // No barrier here: the next chunk's staging writes Qh, Kh, beta e^b k, beta v and
    // Tinv, last read in (3) before this chunk's second barrier, and the other
    // k e^{gamma - b} buffer; A is rewritten only after its first barrier.
  }
  if (seg == p.segments - 1) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p.ST[(long long)bh * DK * p.dv + (long long)(db * 16 + 4 * g + e) * p.dv + wcol + r16] = S[db][e];
  }
}

}  // namespace

bool delta_config_built(int dtype, int dk, int dv, int slice) {
  if (dk != 64 && dk != 128) return false;
  if (dv != 64 && dv != 128) return false;
  if (dtype == 0) return slice == 32 || slice == 64 || slice == 128;
  return dk == 64 && dv == 64 && (slice == 32 || slice == 64);
}

hipError_t launch_delta_prep(const DeltaParams& p, int dtype, hipStream_t stream) {
  const long long blocks = (long long)p.BH * p.nchunks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
#define GLA_DP(TT, DKV, DVV) \
  hipLaunchKernelGGL((delta_prep_kernel<TT, DKV, DVV>), dim3((unsigned)blocks), dim3(256), 0, stream, p)
  if (dtype == 0) {
    if (p.dk == 128 && p.dv == 128) GLA_DP(bf16, 128, 128);
    else if (p.dk == 128 && p.dv == 64) GLA_DP(bf16, 128, 64);
    else if (p.dk == 64 && p.dv == 128) GLA_DP(bf16, 64, 128);
    else if (p.dk == 64 && p.dv == 64) GLA_DP(bf16, 64, 64);
    else return hipErrorInvalidValue;
  } else {
    if (p.dk == 64 && p.dv == 64) GLA_DP(float, 64, 64);
    else return hipErrorInvalidValue;
  }
#undef GLA_DP
  return hipGetLastError();
}

// Segment pre-pass: 64-column slices of the local states (dv columns) and of the
// transitions (dk columns).
hipError_t launch_delta_segments(const DeltaParams& p, int dtype, hipStream_t stream) {
  if (p.segments <= 1) return hipSuccess;
  const long long units = (long long)p.BH * (p.segments - 1);
  const long long gh = units * (p.dv / 64), gp = units * (p.dk / 64);
  if (gh > 0x7FFFFFFFLL || gp > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
#define GLA_DS(TT, DKV)                                                                                         \
  do {                                                                                                          \
    hipLaunchKernelGGL((delta_segment_kernel<TT, DKV, 64, false>), dim3((unsigned)gh), dim3(256), 0, stream, p); \
    hipLaunchKernelGGL((delta_segment_kernel<TT, DKV, 64, true>), dim3((unsigned)gp), dim3(256), 0, stream, p);  \
  } while (0)
  if (dtype == 0) {
    if (p.dk == 128) GLA_DS(bf16, 128);
    else if (p.dk == 64) GLA_DS(bf16, 64);
    else return hipErrorInvalidValue;
  } else {
    if (p.dk == 64) GLA_DS(float, 64);
    else return hipErrorInvalidValue;
  }
#undef GLA_DS
  return hipGetLastError();
}

hipError_t launch_delta_output(const DeltaParams& p, int dtype, hipStream_t stream) {
  if (p.grid == 0) return hipSuccess;
  const int slice = p.dv / p.nslices;
#define GLA_DO(TT, DKV, DVSV)                                                                                   \
  if (p.dk == DKV && slice == DVSV) {                                                                            \
    hipLaunchKernelGGL((delta_output_kernel<TT, DKV, DVSV>), dim3(p.grid), dim3(DoCfg<TT, DKV, DVSV>::NT), 0, \
                       stream, p);                                                                              \
    return hipGetLastError();                                                                                    \
  }
  if (dtype == 0) {
    GLA_DO(bf16, 128, 128) GLA_DO(bf16, 128, 64) GLA_DO(bf16, 128, 32)
    GLA_DO(bf16, 64, 128) GLA_DO(bf16, 64, 64) GLA_DO(bf16, 64, 32)
  } else {
    GLA_DO(float, 64, 64) GLA_DO(float, 64, 32)
  }
#undef GLA_DO
  return hipErrorInvalidValue;
}

// debug builds: this unit's LDS-check word (see GLA_CHECK_LDS)
GLA_DEBUG_ACCESSOR(debug_word_delta_kernels)

}  // namespace gla
