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
// S_{c-1} (transposed) is stored by the dq pass before every even chunk and D_{c+1 start}
// (transposed) by the dk pass after every odd chunk and the last one; the dx kernel
// rebuilds the other state of each chunk from its pair's neighbour chunk.
// dH_c = a_{first token of c+1} D (dS_T after the last chunk).
// dx_t = g'(x_t) dL/dg_t with g' the slope of the gate of §3.2.
// This kernel serves the fp32 operands and the diagonal-branch path; for bf16 on the
// unified path the same four groups are formed inside the dq and dk passes (the gate-
// gradient terms of chunk_output_ws_kernel in ws_kernels.hip).
#include "chunk_common.h"

namespace gla {

namespace {

template <typename T, int DK, int DV>
struct DxCfg {
  // 16-column blocks of state columns per wave: two for bf16 (four waves at d = 128; eight
  // waves of one block each measured 8 % slower), one for fp32 (whose two-block waves
  // spill registers)
  static constexpr int NB = sizeof(T) == 2 ? 2 : 1;
  static constexpr int NW = DK / (16 * NB);     // waves, one per 16 NB state columns (over dk)
  static constexpr int NT = 64 * NW;
  static constexpr int PAD = Elem<T>::kPad;
  static constexpr int LDK = DK + PAD;          // row stride of q, k in LDS
  static constexpr int LDV = DV + PAD;          // row stride of v, dO in LDS
  static constexpr int DB = DV / 16;            // state row blocks (state rows run over dv)
  static constexpr int KS = DV / 32;
  // bf16: two workgroups per CU (LDS allows it); register budget held to match.  fp32
  // tiles fill the LDS of one CU.
  static constexpr int kWavesPerSimd = sizeof(T) == 2 ? 2 : 1;
};

template <typename T, int DK, int DV>
struct DxSmem {
  using X = DxCfg<T, DK, DV>;
  T q[64 * X::LDK];
  T k[64 * X::LDK];
  T v[64 * X::LDV];
  T g[64 * X::LDV];                             // dO
  float b[64];
  float bn[64];                                 // the neighbouring chunk's cumulative log-decay
  float rpart[X::NW][64];
  float upart[X::NW][64];
  float zpart[X::NW];
  float prow[10][16];
  float pcol[10][16];
};

// The four chunk tiles are read both as MFMA fragments and transposed
// (ds_read_tr16_b64); they are swizzled by frag_swz (gla_device.h) and every read
// applies the same swap.

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
      if constexpr (sizeof(T) == 2) {
        const uint4 u = r[m].u;
        GLA_CHECK_LDS(dst + row * LD + c8 * 8, 16);
        *reinterpret_cast<uint4*>(dst + row * LD + c8 * 8) = frag_swz<T>(row) ? make_uint4(u.z, u.w, u.x, u.y) : u;
      } else {
        Elem<T>::store8_raw(dst + row * LD + c8 * 8, r[m]);
      }
    }
  }
};

// Four elements of a stored chunk state (fragment order, see store_chunk_state) as they
// are stored: bf16 states stay packed (two to a register) until they are used.
template <typename T> struct StateRaw;
template <> struct StateRaw<bf16> {
  using V = bf16x4;
  __device__ static __forceinline__ V load(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
  __device__ static __forceinline__ floatx4 f32(V v) {
    floatx4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = static_cast<float>(v[e]);
    return r;
  }
  __device__ static __forceinline__ V raw(const floatx4& a) {
    V r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = static_cast<bf16>(a[e]);
    return r;
  }
  // operand fragment of two accumulator blocks (rows 16 apart), as Elem::from_acc
  __device__ static __forceinline__ Elem<bf16>::Frag frag(V lo, V hi) {
    Elem<bf16>::Frag f;
    f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return f;
  }
};
template <> struct StateRaw<float> {
  using V = floatx4;
  __device__ static __forceinline__ V load(const float* p) { return *reinterpret_cast<const floatx4*>(p); }
  __device__ static __forceinline__ floatx4 f32(V v) { return v; }
  __device__ static __forceinline__ V raw(const floatx4& a) { return a; }
  __device__ static __forceinline__ Elem<float>::Frag frag(V lo, V hi) { return Elem<float>::from_acc(lo, hi); }
};

// Operand fragment whose contraction index is the token (kappa order), for column
// c0 + r16 of a row-major [64][LD] tile (bf16: transposing reads of the swizzled rows).
template <typename T, int LD>
__device__ __forceinline__ typename Elem<T>::Frag tok_frag(const T* tile, int k0, int c0, int lane) {
  if constexpr (sizeof(T) == 2) {
    typedef short shortx4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
    const int s = lane & 15, g = lane >> 4;
    const int row = k0 + 4 * g + (s >> 2);  // rows row and row + 16 share bit 3
    const T* p0 = tile + row * LD + c0 + ((4 * (s & 3)) ^ frag_swz<T>(row));
    const T* p1 = p0 + 16 * LD;
    GLA_CHECK_LDS(p0, 8);
    GLA_CHECK_LDS(p1, 8);
    const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p0));
    const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p1));
    typename Elem<T>::Frag f;
    f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    return f;
  } else {
    const int g = lane >> 4, r = lane & 15;
    GLA_CHECK_LDS(tile + (k0 + 4 * g) * LD + c0 + r, 4);
    GLA_CHECK_LDS(tile + (k0 + 16 + 4 * g + 3) * LD + c0 + r, 4);
    typename Elem<T>::Frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f.lo[e] = tile[(k0 + 4 * g + e) * LD + c0 + r];
      f.hi[e] = tile[(k0 + 16 + 4 * g + e) * LD + c0 + r];
    }
    return f;
  }
}

// The same fragment with element e (token k0 + 16 (e / 4) + 4 g + e % 4) multiplied by fac[e].
template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag scale_frag(typename Elem<T>::Frag f, const float (&fac)[8]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = static_cast<bf16>(static_cast<float>(f.v[e]) * fac[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f.lo[e] *= fac[e];
      f.hi[e] *= fac[4 + e];
    }
  }
  return f;
}

// One workgroup per chunk c of one head; wave w owns 16 NB state columns (over dk).  The
// forward pass stored S^T before each even chunk and the reversed pass D^T after each odd
// chunk (and after the last chunk), one state per pair of chunks (2m, 2m + 1).  The state
// missing for chunk c is one chunk step from the stored one of its pair:
//   odd c:  S^T before c = e^{gamma'} S^T + sum_{s in c-1} e^{gamma' - b'_s} v_s k_s^T,
//   even c: D^T after c  = sum_{j in c+1} e^{b'_j - b'_0} dO_j q_j^T + e^{gamma' - b'_0} a' D^T,
// with b', gamma' those of the neighbour chunk c -/+ 1 and a' the decay of the token after
// chunk c + 1.  The neighbour's two operand tiles pass through the LDS tiles of the same
// names before the chunk's own; the workgroups of one pair run on one XCD (consecutive
// work items, see xcd_linear_index), so their shared reads meet in its L2.
template <typename T, int DK, int DV, int GATE>
__global__ void __launch_bounds__((DxCfg<T, DK, DV>::NT)) __attribute__((amdgpu_waves_per_eu(DxCfg<T, DK, DV>::kWavesPerSimd))) grad_dx_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dO,
    const float* __restrict__ b, const float* __restrict__ x, const T* __restrict__ Sfw, const T* __restrict__ Sbw,
    float* __restrict__ dx, long long Tlen, int nchunks) {
  using X = DxCfg<T, DK, DV>;
  using E = Elem<T>;
  __shared__ __attribute__((aligned(16))) DxSmem<T, DK, DV> sm;  // 16-byte aligned: row stores compile to ds_write_b128
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int item = xcd_linear_index((int)blockIdx.x, (int)gridDim.x);
  const long long bh = item / nchunks;
  const int c = (int)(item - bh * nchunks);
  const bool odd = (c & 1) != 0;
  const bool nbr = odd || c + 1 < nchunks;  // uniform: a state to rebuild from the neighbour
  const int cn = odd ? c - 1 : c + 1;       // the neighbour chunk
  const uint32_t t0 = (uint32_t)c * kChunk, tn0 = (uint32_t)cn * kChunk;
  const uint32_t Tn = (uint32_t)Tlen;
  const float* bh_b = b + bh * Tlen;

  // ---- every load first: the chunk's b and operands, the neighbour's b and two operand
  //      tiles (k, v of c - 1 or q, dO of c + 1), this wave's slices of the pair's states
  float bval = 0.0f;
  // the combine's per-token inputs (wave 0), loaded now so that they are in by then
  float xslope = 0.0f, bnext = 0.0f;
  if (w == 0) {
    const long long tt = (long long)t0 + lane;
    xslope = gate_slope<GATE>(x[bh * Tlen + (tt < Tlen ? tt : Tlen - 1)]);
    const long long tn = (long long)t0 + kChunk;
    bnext = tn < Tlen ? bh_b[tn] : 0.0f;
  }
  if (tid < 64) {
    const long long tt = (long long)t0 + tid;
    bval = bh_b[tt < Tlen ? tt : Tlen - 1];
  } else if (tid < 128 && nbr) {
    const long long tt = (long long)tn0 + (tid - 64);
    bval = bh_b[tt < Tlen ? tt : Tlen - 1];
  }
  const rsrc_t rq = make_rsrc(q + bh * Tlen * DK, Tn * DK * (uint32_t)sizeof(T));
  const rsrc_t rk = make_rsrc(k + bh * Tlen * DK, Tn * DK * (uint32_t)sizeof(T));
  const rsrc_t rv = make_rsrc(v + bh * Tlen * DV, Tn * DV * (uint32_t)sizeof(T));
  const rsrc_t rg = make_rsrc(dO + bh * Tlen * DV, Tn * DV * (uint32_t)sizeof(T));
  // The two own tiles that wait for the neighbour's (k, v for odd c; q, dO for even c)
  // are loaded with everything else where registers allow (bf16 at dk = 128), else
  // after the rebuild.
  constexpr bool kEarly = sizeof(T) == 2 && DK == 128;
  RowStage<T, DK, X::LDK, X::NT> sq, sk, nA;
  RowStage<T, DV, X::LDV, X::NT> svv, sg, nB;
  if (nbr) {
    nA.load(odd ? rk : rq, tn0, tid);
    nB.load(odd ? rv : rg, tn0, tid);
    if (odd) {
      sq.load(rq, t0, tid);
      sg.load(rg, t0, tid);
      if constexpr (kEarly) {
        sk.load(rk, t0, tid);
        svv.load(rv, t0, tid);
      }
    } else {
      sk.load(rk, t0, tid);
      svv.load(rv, t0, tid);
      if constexpr (kEarly) {
        sq.load(rq, t0, tid);
        sg.load(rg, t0, tid);
      }
    }
  } else {
    sq.load(rq, t0, tid);
    sk.load(rk, t0, tid);
    svv.load(rv, t0, tid);
    sg.load(rg, t0, tid);
  }
  // the pair's stored states: 16-column block n of the state at ((n DB + db) 64 + lane) 4
  const long long sidx = (bh * ((nchunks + 1) / 2) + (c >> 1)) * (DK / 16) * (long long)X::DB * 256;
  using RS = StateRaw<T>;
  typename RS::V sv[X::NB][X::DB], ev[X::NB][X::DB];
#pragma unroll
  for (int nb = 0; nb < X::NB; ++nb)
#pragma unroll
    for (int db = 0; db < X::DB; ++db) {
      sv[nb][db] = RS::load(Sfw + sidx + (((X::NB * w + nb) * X::DB + db) * 64 + lane) * 4);
      ev[nb][db] = RS::load(Sbw + sidx + (((X::NB * w + nb) * X::DB + db) * 64 + lane) * 4);
    }
  if (tid < 64) sm.b[tid] = bval;
  else if (tid < 128) sm.bn[tid - 64] = bval;

  // st <- f0 st + sum over the neighbour's tokens s of fexp(s) ta_s tb_s^T: ta the tile
  // over dv (v or dO), tb the tile over dk (k or q), in fp32 and back to the stored form
  const auto rebuild = [&](typename RS::V (&st)[X::NB][X::DB], const T* ta, const T* tb, float f0, auto&& fexp) {
    floatx4 acc[X::NB][X::DB];
#pragma unroll
    for (int nb = 0; nb < X::NB; ++nb)
#pragma unroll
      for (int db = 0; db < X::DB; ++db) acc[nb][db] = RS::f32(st[nb][db]) * f0;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float fac[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) fac[e] = fexp(ks * 32 + 16 * (e >> 2) + 4 * g + (e & 3));
      // the per-token factor goes on the NB fragments of tb rather than the DB of ta
      typename E::Frag fb[X::NB];
#pragma unroll
      for (int nb = 0; nb < X::NB; ++nb)
        fb[nb] = scale_frag<T>(tok_frag<T, X::LDK>(tb, ks * 32, 16 * (X::NB * w + nb), lane), fac);
#pragma unroll
      for (int db = 0; db < X::DB; ++db) {
        const typename E::Frag fa = tok_frag<T, X::LDV>(ta, ks * 32, db * 16, lane);
#pragma unroll
        for (int nb = 0; nb < X::NB; ++nb) E::mfma(acc[nb][db], fa, fb[nb]);
      }
    }
#pragma unroll
    for (int nb = 0; nb < X::NB; ++nb)
#pragma unroll
      for (int db = 0; db < X::DB; ++db) st[nb][db] = RS::raw(acc[nb][db]);
  };

  if (nbr) {
    // the neighbour's tiles go where the chunk's own tiles of those names go later
    if (odd) {
      nA.store(sm.k, tid);
      nB.store(sm.v, tid);
      sq.store(sm.q, tid);
      sg.store(sm.g, tid);
    } else {
      nA.store(sm.q, tid);
      nB.store(sm.g, tid);
      sk.store(sm.k, tid);
      svv.store(sm.v, tid);
    }
    __syncthreads();
    if (odd) {
      // S^T before c from S^T before c - 1 (a whole chunk)
      const float gn = sm.bn[63];
      rebuild(sv, sm.v, sm.k, exp_e(gn), [&](int s) { return exp_e(gn - sm.bn[s]); });
    } else {
      // D^T after c from D^T after c + 1 (rows of c + 1 past the end are zeros)
      const long long rem = Tlen - 1 - (long long)tn0;
      const float gn = sm.bn[rem < 63 ? (int)rem : 63], bn0 = sm.bn[0];
      const long long tnext = (long long)tn0 + kChunk;
      const float an = tnext < Tlen ? exp_e(bh_b[tnext]) : 1.0f;
      rebuild(ev, sm.g, sm.q, exp_e(gn - bn0) * an, [&](int j) { return exp_e(sm.bn[j] - bn0); });
    }
    if constexpr (!kEarly) {
      if (odd) {
        sk.load(rk, t0, tid);
        svv.load(rv, t0, tid);
      } else {
        sq.load(rq, t0, tid);
        sg.load(rg, t0, tid);
      }
    }
    __syncthreads();
    if (odd) {
      sk.store(sm.k, tid);
      svv.store(sm.v, tid);
    } else {
      sq.store(sm.q, tid);
      sg.store(sm.g, tid);
    }
  } else {
    sq.store(sm.q, tid);
    sk.store(sm.k, tid);
    svv.store(sm.v, tid);
    sg.store(sm.g, tid);
  }
  float z = 0.0f;
#pragma unroll
  for (int nb = 0; nb < X::NB; ++nb)
#pragma unroll
    for (int db = 0; db < X::DB; ++db) {
      const floatx4 a4 = RS::f32(sv[nb][db]), b4 = RS::f32(ev[nb][db]);
#pragma unroll
      for (int e = 0; e < 4; ++e) z += a4[e] * b4[e];
    }
  z = row_sum4(group_sum<16>(z));  // all 64 lanes
  if (lane == 0) sm.zpart[w] = z;
  __syncthreads();

  // ---- (2) and (3): dO_j^T S^T and v_i^T D^T on the matrix cores, dotted with q_j, k_i
  {
    typename E::Frag Sf[X::NB][X::KS], Ef[X::NB][X::KS];
#pragma unroll
    for (int nb = 0; nb < X::NB; ++nb)
#pragma unroll
      for (int ks = 0; ks < X::KS; ++ks) {
        Sf[nb][ks] = RS::frag(sv[nb][2 * ks], sv[nb][2 * ks + 1]);
        Ef[nb][ks] = RS::frag(ev[nb][2 * ks], ev[nb][2 * ks + 1]);
      }
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      floatx4 M[X::NB], N[X::NB];
#pragma unroll
      for (int nb = 0; nb < X::NB; ++nb) M[nb] = N[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < X::KS; ++ks) {
        const typename E::Frag gf = E::load_frag(sm.g + (jb * 16 + r16) * X::LDV, ks * 32 + ((4 * g) ^ frag_swz<T>(r16)));
        const typename E::Frag vf = E::load_frag(sm.v + (jb * 16 + r16) * X::LDV, ks * 32 + ((4 * g) ^ frag_swz<T>(r16)));
#pragma unroll
        for (int nb = 0; nb < X::NB; ++nb) {
          E::mfma(M[nb], Sf[nb][ks], gf);  // M[nb][e] = (dO_j^T S^T)[n], j = 16 jb + r16
          E::mfma(N[nb], Ef[nb][ks], vf);  // N[nb][e] = (v_j^T D^T)[n]
        }
      }
      // n = 16 (NB w + nb) + 4 g + e: four consecutive columns (also after the swap,
      // which moves whole 8-byte halves), read as one 8-byte (bf16) or 16-byte piece
      float rp = 0.0f, up = 0.0f;
#pragma unroll
      for (int nb = 0; nb < X::NB; ++nb) {
        const int n0 = (16 * (X::NB * w + nb) + 4 * g) ^ frag_swz<T>(r16);
        const T* qrow = sm.q + (jb * 16 + r16) * X::LDK + n0;
        const T* krow = sm.k + (jb * 16 + r16) * X::LDK + n0;
        float qv[4], kv[4];
        if constexpr (sizeof(T) == 2) {
          GLA_CHECK_LDS(qrow, 8);
          GLA_CHECK_LDS(krow, 8);
          const bf16x4 q4 = *reinterpret_cast<const bf16x4*>(qrow), k4 = *reinterpret_cast<const bf16x4*>(krow);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            qv[e] = static_cast<float>(q4[e]);
            kv[e] = static_cast<float>(k4[e]);
          }
        } else {
          GLA_CHECK_LDS(qrow, 16);
          GLA_CHECK_LDS(krow, 16);
          const floatx4 q4 = *reinterpret_cast<const floatx4*>(qrow), k4 = *reinterpret_cast<const floatx4*>(krow);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            qv[e] = q4[e];
            kv[e] = k4[e];
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          rp += M[nb][e] * qv[e];
          up += N[nb][e] * kv[e];
        }
      }
      rp = row_sum4(rp);
      up = row_sum4(up);
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
      E::mfma(qk, E::load_frag(sm.k + (ib * 16 + r16) * X::LDK, ks * 32 + ((4 * g) ^ frag_swz<T>(r16))),
              E::load_frag(sm.q + (jb * 16 + r16) * X::LDK, ks * 32 + ((4 * g) ^ frag_swz<T>(r16))));
#pragma unroll
    for (int ks = 0; ks < DV / 32; ++ks)
      E::mfma(gv, E::load_frag(sm.v + (ib * 16 + r16) * X::LDV, ks * 32 + ((4 * g) ^ frag_swz<T>(r16))),
              E::load_frag(sm.g + (jb * 16 + r16) * X::LDV, ks * 32 + ((4 * g) ^ frag_swz<T>(r16))));
    // lane (g, r16), element e: j = 16 jb + r16, s = 16 ib + 4 g + e
    const float bj = sm.b[jb * 16 + r16];
    float pe[4], row = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool keep = jb != ib || 4 * g + e < r16;
      pe[e] = keep ? qk[e] * gv[e] * exp_e(bj - sm.b[ib * 16 + 4 * g + e]) : 0.0f;
      row += pe[e];
    }
    row = row_sum4(row);
    if (g == 0) sm.prow[t][r16] = row;
    // column sums over the 16 lanes of a row group: DPP row shifts, the total lands in
    // the row's last lane
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float col = pe[e];
      col += dpp_or_zero<0x111>(col);  // row_shr:1
      col += dpp_or_zero<0x112>(col);  // row_shr:2
      col += dpp_or_zero<0x114>(col);  // row_shr:4
      col += dpp_or_zero<0x118>(col);  // row_shr:8
      if (r16 == 15) sm.pcol[t][4 * g + e] = col;
    }
  }
  __syncthreads();

  // ---- combine: one lane per token of the chunk
  if (w == 0) {
    const int j = lane, jb = j >> 4, jr = j & 15;
    const int last = (int)((Tlen - 1 - (long long)t0) < 63 ? (Tlen - 1 - (long long)t0) : 63);
    const float gam = sm.b[last];
    // dH_c = a D with a the decay of the first token of the next chunk (1 after the last chunk)
    const float a = (nbr && !odd) ? exp_e(sm.bn[0]) : ((long long)t0 + kChunk < Tlen ? exp_e(bnext) : 1.0f);
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
    // (64-lane scans on DPP row shifts; the suffix is the total minus the exclusive prefix)
    const float d = colsum - rowsum;
    const float R = wave_inclusive_scan(d, lane) - d;      // exclusive prefix
    const float rincl = wave_inclusive_scan(r, lane);
    const float rtot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rincl), 63));
    const float rsuf = rtot - (rincl - r);                 // inclusive suffix
    const float uex = wave_inclusive_scan(u, lane) - u;    // exclusive prefix
    const float dg = R + rsuf + uex + Z;
    const long long tt = (long long)t0 + j;
    if (tt < Tlen) dx[bh * Tlen + tt] = xslope * dg;
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

// debug builds: this unit's LDS-check word (see GLA_CHECK_LDS)
GLA_DEBUG_ACCESSOR(debug_word_bwd_kernels)

}  // namespace gla
