// bwd_kernels.hip -- the parts of the backward pass that are not forward-shaped.
//
// The gradients dq, dk, dv and dS0 come from forward-shaped passes over remapped
// operands (see gla_chunk_bwd in api.hip).  This file computes the gradient of the
// gate pre-activation x and dS0.
//
// dL/dg_t.  In the recurrence S_t = a_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t of the
// chunked linear attention with per-position decay ("Engineering Long-Context
// Training for Trillion-Parameter MoE Models: Three Key Breakthroughs", §3.1), the
// loss is a sum over pairs: the key/value of token s reaches the output of token
// j >= s (and the final state) with weight prod_{s<i<=j} a_i.  So g_t = log a_t
// enters exactly the pairs that span it, s < t <= j, and dL/dg_t is the sum of
// their contributions.  For t in chunk c those pairs are
//   (1) s and j both in chunk c:       sum_{s<t<=j} P_js,
//       P_js = e^{b_j - b_s} (q_j . k_s)(dO_j . v_s)
//   (2) s before chunk c, j in chunk c: sum_{j>=t} r_j,  r_j = e^{b_j} q_j^T S_{c-1} dO_j
//   (3) s in chunk c, j after chunk c:  sum_{s<t} u_s,   u_s = e^{gamma - b_s} k_s^T dH_c v_s
//   (4) s before and j after chunk c:  Z_c = e^gamma <dH_c, S_{c-1}>
// with b the chunk-local cumulative log-decay, gamma its chunk total, S_{c-1} the
// state before the chunk and dH_c = dL/dS after the chunk.  Each pair is counted
// once, so nothing cancels: summing per-token inflows and outflows over the whole
// sequence (dL/dg_t = sum_{t'>=t} (q.dq - k.dk)_t') is equivalent in exact arithmetic
// but turns the rounding of dq and dk into errors that grow with T.
// S_{c-1} (transposed) is stored per chunk by the dq pass, D_{c+1 start} (transposed)
// by the dk pass; dH_c = a_{first token of c+1} D (dS_T after the last chunk).
// dx_t = g'(x_t) dL/dg_t with g' the slope of the gate of §3.2.
#include "chunk_common.h"

namespace gla {

namespace {

template <typename T, int DK, int DV>
struct DxCfg {
  static constexpr int NW = DK / 32;            // waves, one per 32 state columns (over dk)
  static constexpr int NT = 64 * NW;
  static constexpr int PAD = Elem<T>::kPad;
  static constexpr int LDK = DK + PAD;          // row stride of q, k in LDS
  static constexpr int LDV = DV + PAD;          // row stride of v, dO in LDS
  static constexpr int DB = DV / 16;            // state row blocks (state rows run over dv)
  static constexpr int KS = DV / 32;
};

template <typename T, int DK, int DV>
struct DxSmem {
  using X = DxCfg<T, DK, DV>;
  T q[64 * X::LDK];
  T k[64 * X::LDK];
  T v[64 * X::LDV];
  T g[64 * X::LDV];                             // dO
  float b[64];
  float rpart[X::NW][64];
  float upart[X::NW][64];
  float zpart[X::NW];
  float prow[10][16];
  float pcol[10][16];
};

__device__ __forceinline__ float sigmoid_f(float x) {
  if (x >= 0.0f) return 1.0f / (1.0f + exp_e(-x));
  const float e = exp_e(x);
  return e / (1.0f + e);
}

template <int GATE>
__device__ __forceinline__ float gate_slope(float x) {
  if (GATE == kGateNegSoftplus) return sigmoid_f(-x);  // d/dx log sigmoid(x)
  const float sg = sigmoid_f(x);
  return -5.0f * sg * (1.0f - sg);                      // d/dx -5 sigmoid(x)
}

// 64 rows of a per-head [T][ncol] tensor, 8-element units spread over the threads:
// all loads are issued first (load), the LDS stores come after (store), so a
// workgroup has its whole chunk in flight at once.  Rows past the end read zeros.
template <typename T, int NCOL, int LD, int NT>
struct RowStage {
  static constexpr int U = 64 * NCOL / 8 / NT;
  static_assert(U >= 1 && U * NT * 8 == 64 * NCOL, "units must divide evenly");
  typename Elem<T>::Vec8 r[U];
  __device__ __forceinline__ void load(rsrc_t src, uint32_t t0, int tid) {
#pragma unroll
    for (int m = 0; m < U; ++m) {
      const int u = tid + m * NT, row = u / (NCOL / 8), c8 = u % (NCOL / 8);
      r[m] = Elem<T>::load8(src, ((t0 + row) * NCOL + c8 * 8) * (uint32_t)sizeof(T));
    }
  }
  __device__ __forceinline__ void store(T* dst, int tid) const {
#pragma unroll
    for (int m = 0; m < U; ++m) {
      const int u = tid + m * NT, row = u / (NCOL / 8), c8 = u % (NCOL / 8);
      Elem<T>::store8_raw(dst + row * LD + c8 * 8, r[m]);
    }
  }
};

// A stored chunk state (fragment order, see store_chunk_state) of one 32-column group.
template <typename T, int DB>
__device__ __forceinline__ floatx4 load_state4(const T* base, int nb, int db, int lane) {
  const T* src = base + ((nb * DB + db) * 64 + lane) * 4;
  floatx4 r;
  if constexpr (sizeof(T) == 2) {
    typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
    const bf16x4v w = *reinterpret_cast<const bf16x4v*>(src);
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = static_cast<float>(w[e]);
  } else {
    r = *reinterpret_cast<const floatx4*>(src);
  }
  return r;
}

template <typename T, int DK, int DV, int GATE>
__global__ void __launch_bounds__((DxCfg<T, DK, DV>::NT)) grad_dx_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dO,
    const float* __restrict__ b, const float* __restrict__ x, const T* __restrict__ Sfw, const T* __restrict__ Sbw,
    float* __restrict__ dx, long long Tlen, int nchunks) {
  using X = DxCfg<T, DK, DV>;
  using E = Elem<T>;
  __shared__ __attribute__((aligned(16))) DxSmem<T, DK, DV> sm;  // 16-byte aligned: row stores compile to ds_write_b128
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const long long bh = blockIdx.x / nchunks;
  const int c = (int)(blockIdx.x - bh * nchunks);
  const uint32_t t0 = (uint32_t)c * kChunk;
  const uint32_t Tn = (uint32_t)Tlen;

  // ---- operands of the chunk (raw) and its cumulative log-decay: every load of the
  //      chunk, including this wave's 32-column slices of S^T (before the chunk) and D^T
  //      (after it), is issued before the first LDS store
  float bval = 0.0f;
  if (tid < 64) {
    const long long tt = (long long)t0 + tid;
    bval = b[bh * Tlen + (tt < Tlen ? tt : Tlen - 1)];
  }
  RowStage<T, DK, X::LDK, X::NT> sq, sk;
  RowStage<T, DV, X::LDV, X::NT> svv, sg;
  sq.load(make_rsrc(q + bh * Tlen * DK, Tn * DK * (uint32_t)sizeof(T)), t0, tid);
  sk.load(make_rsrc(k + bh * Tlen * DK, Tn * DK * (uint32_t)sizeof(T)), t0, tid);
  svv.load(make_rsrc(v + bh * Tlen * DV, Tn * DV * (uint32_t)sizeof(T)), t0, tid);
  sg.load(make_rsrc(dO + bh * Tlen * DV, Tn * DV * (uint32_t)sizeof(T)), t0, tid);
  const long long sidx = (((bh * nchunks + c) * (DK / 32) + w) * 2) * (long long)X::DB * 256;
  floatx4 sv[2][X::DB], ev[2][X::DB];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int db = 0; db < X::DB; ++db) {
      sv[nb][db] = load_state4<T, X::DB>(Sfw + sidx, nb, db, lane);
      ev[nb][db] = load_state4<T, X::DB>(Sbw + sidx, nb, db, lane);
    }
  sq.store(sm.q, tid);
  sk.store(sm.k, tid);
  svv.store(sm.v, tid);
  sg.store(sm.g, tid);
  if (tid < 64) sm.b[tid] = bval;
  float z = 0.0f;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int db = 0; db < X::DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) z += sv[nb][db][e] * ev[nb][db][e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
  if (lane == 0) sm.zpart[w] = z;
  __syncthreads();

  // ---- (2) and (3): dO_j^T S^T and v_i^T D^T on the matrix cores, dotted with q_j, k_i
  {
    typename E::Frag Sf[2][X::KS], Ef[2][X::KS];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int ks = 0; ks < X::KS; ++ks) {
        Sf[nb][ks] = E::from_acc(sv[nb][2 * ks], sv[nb][2 * ks + 1]);
        Ef[nb][ks] = E::from_acc(ev[nb][2 * ks], ev[nb][2 * ks + 1]);
      }
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      floatx4 M[2], N[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) M[nb] = N[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < X::KS; ++ks) {
        const typename E::Frag gf = E::load_frag(sm.g + (jb * 16 + r16) * X::LDV, ks * 32 + 4 * g);
        const typename E::Frag vf = E::load_frag(sm.v + (jb * 16 + r16) * X::LDV, ks * 32 + 4 * g);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          E::mfma(M[nb], Sf[nb][ks], gf);  // M[nb][e] = (dO_j^T S^T)[n], j = 16 jb + r16
          E::mfma(N[nb], Ef[nb][ks], vf);  // N[nb][e] = (v_j^T D^T)[n]
        }
      }
      // n = 32 w + 16 nb + 4 g + e
      float rp = 0.0f, up = 0.0f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = 32 * w + 16 * nb + 4 * g + e;
          rp += M[nb][e] * E::to_f32(sm.q[(jb * 16 + r16) * X::LDK + n]);
          up += N[nb][e] * E::to_f32(sm.k[(jb * 16 + r16) * X::LDK + n]);
        }
      rp += __shfl_xor(rp, 16);
      rp += __shfl_xor(rp, 32);
      up += __shfl_xor(up, 16);
      up += __shfl_xor(up, 32);
      if (g == 0) {
        sm.rpart[w][jb * 16 + r16] = rp;
        sm.upart[w][jb * 16 + r16] = up;
      }
    }
  }

  // ---- (1): P_js = e^{b_j - b_s} (q_j . k_s)(dO_j . v_s) on the 10 causal tiles,
  //      reduced to row sums (over s < j) and column sums (over j > s) per tile
#pragma unroll
  for (int t = 0; t < 10; ++t) {
    if (t % X::NW != w) continue;  // wave-uniform
    const int jb = tri_j(t), ib = tri_i(t);
    floatx4 qk = {0.f, 0.f, 0.f, 0.f}, gv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks)
      E::mfma(qk, E::load_frag(sm.k + (ib * 16 + r16) * X::LDK, ks * 32 + 4 * g),
              E::load_frag(sm.q + (jb * 16 + r16) * X::LDK, ks * 32 + 4 * g));
#pragma unroll
    for (int ks = 0; ks < DV / 32; ++ks)
      E::mfma(gv, E::load_frag(sm.v + (ib * 16 + r16) * X::LDV, ks * 32 + 4 * g),
              E::load_frag(sm.g + (jb * 16 + r16) * X::LDV, ks * 32 + 4 * g));
    // lane (g, r16), element e: j = 16 jb + r16, s = 16 ib + 4 g + e
    const float bj = sm.b[jb * 16 + r16];
    float pe[4], row = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool keep = jb != ib || 4 * g + e < r16;
      pe[e] = keep ? qk[e] * gv[e] * exp_e(bj - sm.b[ib * 16 + 4 * g + e]) : 0.0f;
      row += pe[e];
    }
    row += __shfl_xor(row, 16);
    row += __shfl_xor(row, 32);
    if (g == 0) sm.prow[t][r16] = row;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float col = pe[e];
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) col += __shfl_xor(col, off);
      if (r16 == 0) sm.pcol[t][4 * g + e] = col;
    }
  }
  __syncthreads();

  // ---- combine: one lane per token of the chunk
  if (w == 0) {
    const int j = lane, jb = j >> 4, jr = j & 15;
    const int last = (int)((Tlen - 1 - (long long)t0) < 63 ? (Tlen - 1 - (long long)t0) : 63);
    const float gam = sm.b[last];
    // dH_c = a D with a the decay of the first token of the next chunk (1 after the last chunk)
    const long long tn = (long long)t0 + kChunk;
    const float a = tn < Tlen ? exp_e(b[bh * Tlen + tn]) : 1.0f;
    float rs = 0.0f, us = 0.0f, zs = 0.0f;
#pragma unroll
    for (int ww = 0; ww < X::NW; ++ww) {
      rs += sm.rpart[ww][j];
      us += sm.upart[ww][j];
      zs += sm.zpart[ww];
    }
    const float bj = sm.b[j];
    const float r = exp_e(bj) * rs;
    const float u = a * exp_e(gam - bj) * us;
    const float Z = a * exp_e(gam) * zs;
    // row sum of P over s < j: tiles (jb, 0..jb); column sum over j' > j: tiles (jb..3, jb)
    float rowsum = 0.0f, colsum = 0.0f;
#pragma unroll
    for (int t = 0; t < 10; ++t) {
      if (tri_j(t) == jb) rowsum += sm.prow[t][jr];
      if (tri_i(t) == jb) colsum += sm.pcol[t][jr];
    }
    // R_j = sum_{s<j<=j'} P = sum_{t<j} (colsum - rowsum)_t ; inflow suffix ; outflow prefix
    float d = colsum - rowsum, dincl = d;
    float rsuf = r, upre = u;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float a1 = __shfl_up(dincl, off);
      const float a2 = __shfl_down(rsuf, off);
      const float a3 = __shfl_up(upre, off);
      if (lane >= off) {
        dincl += a1;
        upre += a3;
      }
      if (lane + off < 64) rsuf += a2;
    }
    const float R = dincl - d;  // exclusive prefix
    const float uex = upre - u;  // exclusive prefix
    const float dg = R + rsuf + uex + Z;
    const long long tt = (long long)t0 + j;
    if (tt < Tlen) dx[bh * Tlen + tt] = gate_slope<GATE>(x[bh * Tlen + tt]) * dg;
  }
}

__global__ void __launch_bounds__(256) grad_ds0_kernel(const float* __restrict__ D0, const float* __restrict__ b,
                                                       const float* __restrict__ dST, float* __restrict__ dS0,
                                                       long long Tlen, long long nst, long long total) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const long long bh = i / nst;
  if (Tlen == 0)
    dS0[i] = dST ? dST[i] : 0.0f;
  else
    dS0[i] = exp_e(b[bh * Tlen]) * D0[i];  // a_0 D_0
}

}  // namespace

hipError_t launch_grad_dx(const void* q, const void* k, const void* v, const void* dO, const float* b,
                          const float* x, const void* Sfw, const void* Sbw, float* dx, long long BH, long long T,
                          int dk_, int dv_, int dtype, int gate, hipStream_t stream) {
  const long long nc = (T + kChunk - 1) / kChunk;
  const long long blocks = BH * nc;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
#define GLA_DX(TT, DKV, DVV, GT)                                                                                  \
  hipLaunchKernelGGL((grad_dx_kernel<TT, DKV, DVV, GT>), dim3((unsigned)blocks), dim3(DxCfg<TT, DKV, DVV>::NT), 0, \
                     stream, static_cast<const TT*>(q), static_cast<const TT*>(k), static_cast<const TT*>(v),     \
                     static_cast<const TT*>(dO), b, x, static_cast<const TT*>(Sfw), static_cast<const TT*>(Sbw), dx, \
                     T, (int)nc)
#define GLA_DX_G(TT, DKV, DVV)                                             \
  do {                                                                     \
    if (gate == kGateBoundedSigmoid) GLA_DX(TT, DKV, DVV, kGateBoundedSigmoid); \
    else GLA_DX(TT, DKV, DVV, kGateNegSoftplus);                           \
  } while (0)
#define GLA_DX_D(TT)                                            \
  do {                                                          \
    if (dk_ == 128 && dv_ == 128) GLA_DX_G(TT, 128, 128);       \
    else if (dk_ == 128 && dv_ == 64) GLA_DX_G(TT, 128, 64);    \
    else if (dk_ == 64 && dv_ == 128) GLA_DX_G(TT, 64, 128);    \
    else if (dk_ == 64 && dv_ == 64) GLA_DX_G(TT, 64, 64);      \
    else return hipErrorInvalidValue;                           \
  } while (0)
  if (dtype == 0) GLA_DX_D(bf16);
  else GLA_DX_D(float);
#undef GLA_DX_D
#undef GLA_DX_G
#undef GLA_DX
  return hipGetLastError();
}

hipError_t launch_grad_ds0(const float* D0, const float* b, const float* dST, float* dS0, long long BH,
                           long long T, int dk_, int dv_, hipStream_t stream) {
  const long long nst = (long long)dk_ * dv_;
  const long long total = BH * nst;
  if (total == 0) return hipSuccess;
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(grad_ds0_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, D0, b, dST, dS0, T, nst, total);
  return hipGetLastError();
}

}  // namespace gla
