// ws_kernels.hip -- wave-specialised kernels of the chunked GLA forward (bf16
// operands, fp32 accumulation) for gfx950: the output pass and the segment
// pre-pass.
//
// Sources (web pages; cited by title and section):
//   [LCT] "Engineering Long-Context Training for Trillion-Parameter MoE Models:
//          Three Key Breakthroughs"
//   [ESU] "Engineering Stability in Ultra-Long Context and Trillion-Parameter
//          Sparse Models"
//
// The arithmetic is the chunked form described at the top of chunk_kernels.hip:
// Qh_j = q_j e^{b_j - r_u(j)}, Kh_i = k_i e^{r_u(i) - b_i} ("q * Gamma", "k / Gamma",
// [LCT §3.2-§3.3], [ESU §2.2]), every causal 16x16 tile of the attention matrix
// A_ji = (Qh_j . Kh_i) e^{r_u(j) - r_u(i)} on the matrix cores, and
//   o_j = e^{r_u(j)} (Qh_j^T S_{c-1}) + sum_i A_ji v_i,
//   S_c = e^gamma S_{c-1} + sum_i (k_i e^{gamma - b_i}) v_i^T.
// The ablation (DIAG) keys the off-diagonal tiles to the end of the key tile and
// computes the diagonal tiles by position pairs, A_ji = e^{b_j - b_i} (q_j . k_i)
// [LCT §3.1], [ESU §2.1].
//
// Work split.  One workgroup per (head, slice of DVS value columns, segment of
// chunks), as in the plain output pass, but with two kinds of waves so that the
// vector-ALU work of preparing a chunk runs beside the matrix-core work on the
// previous one (a compute wave and a staging wave share each SIMD):
//   NCW compute waves, one per 32 value columns, hold the fp32 state slice in
//     MFMA accumulators;
//   4 staging waves load chunk c+1 from HBM into registers and write its
//     operands to LDS.
// Per chunk c (slot = c's LDS buffer set):
//   part 1: compute waves: the 6 off-diagonal tiles of A(c);
//           staging waves: the 4 diagonal tiles of A(c), one each (matrix cores;
//           position pairs on the vector ALUs for DIAG);
//   -- barrier --
//   part 2: compute waves: o(c) = e^{r_u} Qh S + A V, the state update, o stores;
//           staging waves: chunk c+1 -> LDS (Qh, k e^{gamma-b}, v into the other
//           slot; Kh, b into the single buffers read only in part 1), then issue
//           the loads of chunk c+2;
//   -- barrier --
// Qh, k e^{gamma-b} and v are double-buffered because both parts of an
// iteration read them while part 2 writes the next chunk; Kh, A, b and the raw
// q, k of the ablation are read only in part 1 and written only in part 2 (or
// read only in part 2 and written only in part 1), so one copy suffices.
#include "chunk_common.h"

namespace gla {

template <int DK, int DVS, bool DIAG>
struct WsCfg {
  using C = Cfg<bf16, DK, DVS>;
  static constexpr int NCW = C::NW;          // compute waves (C::CPW columns each)
  static constexpr int NSW = 4;              // staging waves
  static constexpr int NT = 64 * (NCW + NSW);
  static constexpr int SNT = 64 * NSW;       // staging threads
  static constexpr int LD = DK + 8;          // row stride of qh, kh (row-major fragment reads)
  // row strides of the token-major kp and vv: 16 elements of padding make their
  // transposing reads conflict-free; the ablation, 4 KB short of room, keeps 8
  static constexpr int KLD = DK + (DIAG ? 8 : 16);
  static constexpr int VLD = DVS + (DIAG ? 8 : 16);
  static constexpr int TLD = 64 + 4;         // row stride of A
  static constexpr int QU = 8 * DK / SNT;    // 16-byte q (and k) pieces per staging thread
  static constexpr int VU = 8 * DVS / SNT;   // 16-byte v pieces per staging thread
  static constexpr int PIECES = DK / 8;      // 16-byte pieces per q/k row
  static_assert(QU >= 1 && QU * SNT == 8 * DK, "q staging must divide evenly");
  static_assert(VU >= 1 && VU * SNT == 8 * DVS, "v staging must divide evenly");

};

template <int DK, int DVS, bool DIAG, int GX = 0>
struct WsSmem {
  using W = WsCfg<DK, DVS, DIAG>;
  bf16 qh[2][64 * W::LD];          // Qh[j][d]
  bf16 kp[2][64 * W::KLD];         // k_i e^{gamma - b_i}, [i][d]
  bf16 vv[2][64 * W::VLD];         // v[i][n]
  bf16 kh[64 * W::LD];             // Kh[i][d]
  bf16 a[64 * W::TLD];             // A[j][i]
  float sb[64];                    // b of the chunk
  bf16 qr[DIAG ? 64 * DK : 1];     // raw q, 16-byte pieces swizzled by row (ablation)
  bf16 kr[DIAG ? 64 * DK : 1];     // raw k, same layout (ablation)
  // gate-gradient terms (GX), per chunk parity and compute wave, per token of the chunk:
  // GX 1: column sums of P, row sums of P, r; GX 2: u, and the crossing term in gx_r[.][.][0]
  static constexpr int GXP = GX ? 2 : 1, GXW = GX ? W::NCW : 1, GXT = GX ? 64 : 1;
  float gx_a[GXP][GXW][GXT];
  float gx_c[GX == 1 ? 2 : 1][GX == 1 ? W::NCW : 1][GX == 1 ? 64 : 1];
  float gx_r[GXP][GXW][GXT];
};

// Physical 16-byte piece of logical piece p in row r of the raw q/k tiles: the
// position-pair reads of one 16-lane group touch 4 rows 4 apart at one logical
// piece; the swizzle puts them in different banks.
__device__ __forceinline__ int raw_piece(int p, int r) { return p ^ ((r >> 2) & 3); }

// Registers of one staging thread holding a chunk of q (LOAD_Q), k, v and b
// between its loads and its LDS writes.  Rows past the end read as zeros (buffer
// range check); b past the end repeats the last value (absent tokens have g = 0).
template <int DK, int DVS, bool LOAD_Q = true>
struct WsStaged {
  static constexpr int QU = 8 * DK / 256, VU = 8 * DVS / 256;
  // The segment pre-pass (LOAD_Q = false) streams k and v past the caches: its loads
  // then do not evict the previous output pass's dirty o lines from L2 and the MALL
  // (measured: pre-pass 0.206 -> 0.158 ms at 64K); the output pass keeps ordinary
  // loads (streaming ones made it 1 % slower).
  static constexpr int kLoadAux = LOAD_Q ? 0 : kAuxStream;
  uint4 q[LOAD_Q ? QU : 1], k[QU], v[VU];
  float b;      // b of the lane's token, or its x until decay() (see decay_load)
  uint32_t t0;  // first token of the chunk held

  // chunk starting at logical token t0 (rows in logical order; see row_offset)
  __device__ __forceinline__ void load(const HeadBuffers& hb, const ChunkParams& p, uint32_t t0_, int col0, int st) {
    t0 = t0_;
    b = decay_load(hb, p, t0, st & 63);
#pragma unroll
    for (int m = 0; m < QU; ++m) {
      const int u = st + m * 256;
      const int row = u / (DK / 8), c8 = u % (DK / 8);
      const uint32_t off = row_offset(p, hb.T, t0 + row, DK * 2u) + c8 * 16u;
      if (LOAD_Q) q[m] = buf_load16<kLoadAux>(hb.q, off);
      k[m] = buf_load16<kLoadAux>(hb.k, off);
    }
#pragma unroll
    for (int m = 0; m < VU; ++m) {
      const int u = st + m * 256;
      const int row = u / (DVS / 8), c8 = u % (DVS / 8);
      v[m] = buf_load16<kLoadAux>(hb.v, row_offset(p, hb.T, t0 + row, (uint32_t)p.dv * 2u) + (col0 + c8 * 8) * 2u);
    }
  }

  // b of the lane's token (lane = token of the chunk)
  __device__ __forceinline__ float decay(const HeadBuffers& hb, const ChunkParams& p, int lane) const {
    return decay_finish(hb, p, b, t0, lane);
  }
};

// One attention tile (query tile jb, key tile ib) on the matrix cores, scaled by f
// and, on the diagonal, masked to i <= j; written to A as bf16.
template <int DK, int TLD, int LD>
__device__ __forceinline__ void attention_tile(bf16* a, const bf16* qh, const bf16* kh, int jb, int ib, float f,
                                               int g, int r16) {
  using E = Elem<bf16>;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < DK / 32; ++ks) {
    const E::Frag ka = E::load_frag(kh + (ib * 16 + r16) * LD, ks * 32 + ((4 * g) ^ frag_swz<bf16>(r16)));
    const E::Frag qb = E::load_frag(qh + (jb * 16 + r16) * LD, ks * 32 + ((4 * g) ^ frag_swz<bf16>(r16)));
    E::mfma(acc, ka, qb);
  }
  // acc[e] = Qh_j . Kh_i for j = 16 jb + r16, i = 16 ib + 4 g + e
  float vals[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) vals[e] = (jb != ib || 4 * g + e <= r16) ? acc[e] * f : 0.0f;
  E::store4(a + (jb * 16 + r16) * TLD + ib * 16 + 4 * g, vals[0], vals[1], vals[2], vals[3]);
}

// Diagonal tile u of the ablation by explicit position pairs on the vector ALUs:
// A_ji = e^{b_j - b_i} (q_j . k_i) for i <= j.  Lane (dq, jq, iq) forms the 16
// partial dot products of query rows 4jq.. and key rows 4iq.. over its quarter dq
// of the key dimension (packed bf16 dot2), the quarters are summed across lanes,
// and the lane then finishes query row 4jq + dq.
template <int DK, int TLD>
__device__ __forceinline__ void diagonal_pairs(bf16* a, const bf16* qr, const bf16* kr, const float* sb, int u,
                                               int lane) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  constexpr int PQ = DK / 32;  // 16-byte pieces per quarter of the key dimension
  const int dq = lane >> 4, jq = (lane >> 2) & 3, iq = lane & 3;
  float acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.0f;
#pragma unroll
  for (int s = 0; s < PQ; ++s) {
    const int p = dq * PQ + s;
    uint4 qv[4], kv[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int rq = u * 16 + jq * 4 + x, rk = u * 16 + iq * 4 + x;
      GLA_CHECK_LDS(qr + rq * DK + raw_piece(p, rq) * 8, 16);
      GLA_CHECK_LDS(kr + rk * DK + raw_piece(p, rk) * 8, 16);
      qv[x] = *reinterpret_cast<const uint4*>(qr + rq * DK + raw_piece(p, rq) * 8);
      kv[x] = *reinterpret_cast<const uint4*>(kr + rk * DK + raw_piece(p, rk) * 8);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        float t = acc[x][y];
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qv[x].x), __builtin_bit_cast(bf16x2, kv[y].x), t, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qv[x].y), __builtin_bit_cast(bf16x2, kv[y].y), t, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qv[x].z), __builtin_bit_cast(bf16x2, kv[y].z), t, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qv[x].w), __builtin_bit_cast(bf16x2, kv[y].w), t, false);
        acc[x][y] = t;
      }
  }
  // Sum the four quarters (lanes l, l^16, l^32, l^48) while handing each row's
  // sums to one quarter: across lanes 16 apart, keep the rows whose low bit
  // matches this lane's quarter and send the others; across lanes 32 apart, keep
  // row dq.  Lane (dq, jq, iq) ends with the dot products of row 4jq + dq.
  const int b0 = dq & 1, b1 = dq >> 1;
  float half[2][4];
#pragma unroll
  for (int xh = 0; xh < 2; ++xh)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const float keep = b0 ? acc[2 * xh + 1][y] : acc[2 * xh][y];
      const float send = b0 ? acc[2 * xh][y] : acc[2 * xh + 1][y];
      half[xh][y] = keep + __shfl_xor(send, 16);
    }
  const int j = jq * 4 + dq;
  const float bj = sb[u * 16 + j];
  float vals[4];
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const float keep = b1 ? half[1][y] : half[0][y];
    const float send = b1 ? half[0][y] : half[1][y];
    const float dot = keep + __shfl_xor(send, 32);
    const int i = iq * 4 + y;
    vals[y] = (i <= j) ? dot * exp_e(bj - sb[u * 16 + i]) : 0.0f;
  }
  Elem<bf16>::store4(a + (u * 16 + j) * TLD + u * 16 + iq * 4, vals[0], vals[1], vals[2], vals[3]);
}

// ---------------------------------------------------------------- gate-gradient terms
// The backward pass's dL/dg_t is the sum over the pairs (key token s, output token j)
// that span t (s < t <= j); per chunk c they fall into four groups (listed with the dx
// kernel in bwd_kernels.hip).  With GX != 0 the dq pass (forward time, holding S_{c-1})
// and the dk pass (reversed time, holding D = dL/dS after the chunk) form them beside
// their own outputs, so that no further pass re-reads q, k, v and dO:
//   GX 1, dq pass: (1) the pairs inside the chunk, P_js = A_js (q_j . k_s) for s < j, from
//     the pass's own score tile A_js = e^{b_j - b_s}(dO_j . v_s) and q, which the compute
//     waves read themselves, 32 columns each (a wave's share of q_j . k_s is one MFMA per
//     tile, and the row and column sums of P are linear in it); (2) the pairs entering,
//     r_j = q_j . (e^{b_j} S_{c-1}^T dO_j), q dotted with the pass's inter-chunk output
//     term before the intra-chunk term is added.  W_t = (exclusive prefix over the chunk of
//     column sum - row sum of P) + (inclusive suffix of r) -> gx_out.  It also stores
//     S_{c-1} (bf16) wherever the crossing factor a e^gamma of chunk c is not exactly 0.
//   GX 2, dk pass: (3) the pairs leaving, u_s = k_s . (a e^{gamma - b_s} D v_s): the pass's
//     inter-chunk output term for token s dotted with k (the reversed pass's cumulative
//     decay at s is exactly log a + gamma - b_s); (4) the pairs crossing the chunk whole,
//     a e^gamma <D, S_{c-1}>, with S_{c-1} from the dq pass; then
//     dx_t = g'(x_t) (W_t + exclusive prefix of u + (4)) -> gx_out.
// a e^gamma (a the decay of the first token after the chunk, 1 after the last chunk) is
// formed by both passes from the same two entries of the forward b buffer with the same
// operations, so they agree exactly on the chunks where it is 0: there the dq pass stores
// no state and the dk pass reads none (the term is exactly 0).
__device__ __forceinline__ float gx_cross_factor(float b_end, float b_next) { return exp_e(b_end + b_next); }

// Offset (elements) of compute wave cw's 32-column group of the bf16 state stored for chunk
// pc, in the fragment order of store_chunk_state.
template <int DK>
__device__ __forceinline__ long long gx_state_offset(const ChunkParams& p, int bh, int pc, int cw) {
  return (((long long)bh * p.nchunks + pc) * (p.dv / 32) + cw) * 2LL * (DK / 16) * 256;
}

template <int DK, int DVS, bool DIAG, int GX = 0>
__global__ void __launch_bounds__((WsCfg<DK, DVS, DIAG>::NT)) chunk_output_ws_kernel(ChunkParams p) {
  using W = WsCfg<DK, DVS, DIAG>;
  using C = typename W::C;
  using E = Elem<bf16>;
  static_assert(GX == 0 || (!DIAG && DVS >= 64), "gate-gradient terms: unified path, one full-width slice");
  __shared__ __attribute__((aligned(16))) WsSmem<DK, DVS, DIAG, GX> sm;  // 16-byte aligned: row stores compile to ds_write_b128
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool compute = wave < W::NCW;  // wave-uniform role
  const int r16 = lane & 15, g = lane >> 4;
  const int L = work_index(p);
  const int slice = L % p.nslices;
  const int rest = L / p.nslices;
  const int seg = rest % p.segments;
  const int bh = unit_of(p, rest / p.segments);
  const int col0 = slice * DVS;
  const int cw = compute ? wave : 0;             // compute-wave index
  const int sw = compute ? 0 : wave - W::NCW;    // staging-wave index
  const int st = compute ? 0 : tid - 64 * W::NCW;
  const int wcol = col0 + cw * C::CPW;
  const HeadSpan span = head_span(p, bh);
  const int c_begin = (int)((long long)seg * span.nchunks / p.segments);
  const int c_end = (int)((long long)(seg + 1) * span.nchunks / p.segments);
  const HeadBuffers hb = head_buffers<bf16, DK>(p, span);

  // The two key tiles that a 32-wide K-step of A.V reads above the diagonal,
  // (jb 0, ib 1) and (jb 2, ib 3), are never written by the loop: zero them once.
  for (int e = tid; e < 2 * 256; e += W::NT) {
    const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
    sm.a[(blk * 32 + rr) * W::TLD + blk * 32 + 16 + cc] = E::cvt(0.0f);
  }

  // gate-gradient terms: physical chunk of logical chunk c, and the operands of the
  // crossing factor of chunk c (last token's b, next chunk's first b) from the forward b
  const float* gxb = GX ? p.gx_b + span.row0 : nullptr;
  const long long Tg = (long long)hb.T;
  const auto gx_phys = [&](int c) { return p.reverse ? p.nchunks - 1 - c : c; };
  const auto gx_cross_load = [&](int c, float& be, float& bn) {
    const int pc = gx_phys(c);
    const long long e = min((long long)pc * kChunk + kChunk - 1, Tg - 1), n = (long long)(pc + 1) * kChunk;
    be = gxb[e];
    bn = n < Tg ? gxb[n] : 0.0f;
  };

  // The two roles run separate loops with the same barriers (one before the
  // loop, two per chunk), so that the registers of one role are free for the
  // other: the compute waves hold the state and o accumulators, the staging waves
  // two register sets of prefetched chunks.
  if (compute) {
    StateAcc<bf16, DK, DVS> S;
    load_initial_state<bf16, DK, DVS>(S, p, bh, seg, wcol, g, r16);
    // GX: the operand this pass lacks (q or k), rows of the unit, p.dv columns
    const rsrc_t gxop = GX ? make_rsrc(static_cast<const bf16*>(p.gx_op) + span.row0 * p.dv, hb.T * (uint32_t)p.dv * 2u)
                           : make_rsrc(nullptr, 0u);
    bf16* gx_st = GX ? static_cast<bf16*>(p.gx_states) : nullptr;
    float gx_be = 0.0f, gx_bn = 0.0f;  // GX 2: crossing-factor operands, loaded one chunk ahead
    if constexpr (GX == 2) {
      if (c_begin < c_end) gx_cross_load(c_begin, gx_be, gx_bn);
    }
    __syncthreads();
    for (int c = c_begin; c < c_end; ++c) {
      const int slot = (c - c_begin) & 1;
      const uint32_t t0 = (uint32_t)c * kChunk;
      if (p.state_out) store_chunk_state<bf16, DK, DVS>(S, p, bh, c, wcol, lane);
      // GX: this wave's 32 columns of q (GX 1) or k (GX 2) for the chunk's tokens, four
      // consecutive columns per lane: [t0 + 16 jb + r16][wcol + 16 nb + 4 g ..]
      [[maybe_unused]] uint2 gxo[4][2];
      [[maybe_unused]] float gxf = 0.0f;         // crossing factor a e^gamma of this chunk (wave-uniform)
      [[maybe_unused]] uint2 gxs[C::NB][C::DB];  // GX 2: S_{c-1} where gxf != 0
      if constexpr (GX != 0) {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            gxo[jb][nb] = buf_load8(gxop, row_offset(p, hb.T, t0 + jb * 16 + r16, (uint32_t)p.dv * 2u) +
                                              (uint32_t)(wcol + nb * 16 + 4 * g) * 2u);
        if constexpr (GX == 1) {
          float be, bn;
          gx_cross_load(c, be, bn);
          gxf = gx_cross_factor(be, bn);
        } else {
          gxf = gx_cross_factor(gx_be, gx_bn);
          if (c + 1 < c_end) gx_cross_load(c + 1, gx_be, gx_bn);
        }
        gxf = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, gxf)));
        if constexpr (GX == 2) {
          if (gxf != 0.0f) {
            const bf16* src = gx_st + gx_state_offset<DK>(p, bh, gx_phys(c), cw);
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
              for (int db = 0; db < C::DB; ++db)
                gxs[nb][db] = *reinterpret_cast<const uint2*>(src + ((nb * C::DB + db) * 64 + lane) * 4);
          }
        }
      }

      // ---- part 1: off-diagonal tiles of A(c)
      const ChunkDecay cd(sm.sb[lane]);
#pragma unroll
      for (int t = 0; t < 6; ++t) {
        if (t % W::NCW != cw) continue;  // wave-uniform
        const int jb = off_j(t), ib = off_i(t);
        const float ri = DIAG ? cd.end(ib) : cd.r(ib);
        attention_tile<DK, W::TLD, W::LD>(sm.a, sm.qh[slot], sm.kh, jb, ib, exp_e(cd.r(jb) - ri), g, r16);
      }
      if constexpr (GX == 2) {
        // (4): <D, S_{c-1}> over this wave's slice, times a e^gamma; at the end of part 1
        // so that S_{c-1} is not held into part 2
        float z = 0.0f;
        if (gxf != 0.0f) {
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
              const bf16x4 s4 = __builtin_bit_cast(bf16x4, gxs[nb][db]);
#pragma unroll
              for (int e = 0; e < 4; ++e) z += S.s[nb][db][e] * static_cast<float>(s4[e]);
            }
          z = row_sum4(group_sum<16>(z));  // all 64 lanes
        }
        if (lane == 0) sm.gx_r[slot][cw][0] = gxf * z;
      }
      __syncthreads();

      // ---- part 2: o(c) and S_c
      if constexpr (GX == 1) {
        // (1): this wave's share of q_j . k_s (its 32 columns) on the 10 causal tiles, times
        // A_js, reduced to row sums (over s < j) and column sums (over j > s)
        typename E::Frag qf[4], kf[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
          qf[jb].v = __builtin_shufflevector(__builtin_bit_cast(bf16x4, gxo[jb][0]), __builtin_bit_cast(bf16x4, gxo[jb][1]),
                                             0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) kf[ib] = E::load_frag(sm.vv[slot] + (ib * 16 + r16) * W::VLD, cw * C::CPW + 4 * g);
        floatx4 colP[4];
        float rowP[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          colP[u] = floatx4{0.f, 0.f, 0.f, 0.f};
          rowP[u] = 0.0f;
        }
#pragma unroll
        for (int t = 0; t < 10; ++t) {
          const int jb = tri_j(t), ib = tri_i(t);
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          E::mfma(acc, kf[ib], qf[jb]);  // acc[e]: k_s . q_j over the wave's columns, j = 16 jb + r16, s = 16 ib + 4 g + e
          GLA_CHECK_LDS(sm.a + (jb * 16 + r16) * W::TLD + ib * 16 + 4 * g, 8);
          const bf16x4 a4 = *reinterpret_cast<const bf16x4*>(sm.a + (jb * 16 + r16) * W::TLD + ib * 16 + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pe = (jb != ib || 4 * g + e < r16) ? acc[e] * static_cast<float>(a4[e]) : 0.0f;
            colP[ib][e] += pe;
            rowP[jb] += pe;
          }
        }
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          const float rs = row_sum4(rowP[jb]);
          if (g == 0) sm.gx_c[slot][cw][jb * 16 + r16] = rs;
        }
        // column sums over the 16 lanes of a row group (DPP row shifts; total in the last lane)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float col = colP[ib][e];
            col += dpp_or_zero<0x111>(col);  // row_shr:1
            col += dpp_or_zero<0x112>(col);  // row_shr:2
            col += dpp_or_zero<0x114>(col);  // row_shr:4
            col += dpp_or_zero<0x118>(col);  // row_shr:8
            if (r16 == 15) sm.gx_a[slot][cw][ib * 16 + 4 * g + e] = col;
          }
      }
      typename E::Frag Sf[C::NB][C::KS];
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) Sf[nb][ks] = E::from_acc(S.s[nb][2 * ks], S.s[nb][2 * ks + 1]);
      if constexpr (GX == 1) {
        // S_{c-1} for the dk pass's crossing term, where its factor is not exactly 0
        if (gxf != 0.0f) {
          bf16* dst = gx_st + gx_state_offset<DK>(p, bh, c, cw);
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
              *reinterpret_cast<bf16x4*>(dst + ((nb * C::DB + 2 * ks) * 64 + lane) * 4) =
                  __builtin_shufflevector(Sf[nb][ks].v, Sf[nb][ks].v, 0, 1, 2, 3);
              *reinterpret_cast<bf16x4*>(dst + ((nb * C::DB + 2 * ks + 1) * 64 + lane) * 4) =
                  __builtin_shufflevector(Sf[nb][ks].v, Sf[nb][ks].v, 4, 5, 6, 7);
            }
        }
      }
      VFrags<bf16, DK, DVS> Vf;
      load_v_frags<bf16, DK, DVS, W::VLD>(Vf, sm.vv[slot], cw, lane);

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
          const E::Frag qb = E::load_frag(sm.qh[slot] + (jb * 16 + r16) * W::LD, ks * 32 + ((4 * g) ^ frag_swz<bf16>(r16)));
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
      if constexpr (GX != 0) {
        // (2) r_j (GX 1) or (3) u_s (GX 2): the inter-chunk term of the output row dotted
        // with q or k over this wave's columns
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          float d = 0.0f;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const bf16x4 o4 = __builtin_bit_cast(bf16x4, gxo[jb][nb]);
#pragma unroll
            for (int e = 0; e < 4; ++e) d += static_cast<float>(o4[e]) * O[jb][nb][e];
          }
          d = row_sum4(d);
          if (g == 0) (GX == 1 ? sm.gx_r : sm.gx_a)[slot][cw][jb * 16 + r16] = d;
        }
      }
      // intra-chunk: O^T[n][j] += sum_i v[n][i] A[j][i], keys up to the end of tile jb
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
        for (int ks = 0; ks <= jb / 2; ++ks) {
          const E::Frag ab = E::load_frag(sm.a + (jb * 16 + r16) * W::TLD, ks * 32 + 4 * g);
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) E::mfma(O[jb][nb], Vf.f[nb][ks], ab);
        }
      }
      state_update<bf16, DK, DVS, W::KLD>(S, Vf, sm.kp[slot], exp_e(cd.gam), lane);
      // lane holds o[t0 + 16 jb + r16][wcol + 16 nb + 4 g + 0..3]; rows outside the
      // head get an out-of-range offset and are dropped
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
          buf_store16<0>(hb.o, row_offset(p, hb.T, t0 + jb * 16 + r16, (uint32_t)p.dv * 4u) + (wcol + nb * 16 + 4 * g) * 4u,
                         O[jb][nb]);
      __syncthreads();
    }
    if (seg == p.segments - 1) store_state<bf16, DK, DVS>(S, p.ST + (long long)bh * DK * p.dv, p.dv, wcol, g, r16);
  } else {
    // Staging of one chunk from a register set: -> LDS slot ns (Qh, k e^{gamma-b},
    // v), Kh and b (single buffers), and the raw q, k of the ablation.
    const auto stage = [&](const WsStaged<DK, DVS>& stg, int ns) {
      const float bl = stg.decay(hb, p, lane);
      const ChunkDecay cd(bl);
      float brow[W::QU];
#pragma unroll
      for (int m = 0; m < W::QU; ++m) brow[m] = cd.at((st + m * 256) / (DK / 8));
#pragma unroll
      for (int m = 0; m < W::QU; ++m) {
        const int u = st + m * 256;
        const int row = u / (DK / 8), c8 = u % (DK / 8);
        const int tile = row >> 4;
        const float rj = cd.r(tile);
        E::Vec8 qv, kv;
        qv.u = stg.q[m];
        kv.u = stg.k[m];
        const bool swap = frag_swap<bf16>(row);  // Qh and Kh rows swizzled for the fragment reads
        E::store8_scaled_sw(sm.qh[ns] + row * W::LD + c8 * 8, qv, exp_e(brow[m] - rj), swap);
        E::store8_scaled_sw(sm.kh + row * W::LD + c8 * 8, kv, exp_e((DIAG ? cd.end(tile) : rj) - brow[m]), swap);
        E::store8_scaled(sm.kp[ns] + row * W::KLD + c8 * 8, kv, exp_e(cd.gam - brow[m]));
        if (DIAG) {
          GLA_CHECK_LDS(sm.qr + row * DK + raw_piece(c8, row) * 8, 16);
          GLA_CHECK_LDS(sm.kr + row * DK + raw_piece(c8, row) * 8, 16);
          *reinterpret_cast<uint4*>(sm.qr + row * DK + raw_piece(c8, row) * 8) = stg.q[m];
          *reinterpret_cast<uint4*>(sm.kr + row * DK + raw_piece(c8, row) * 8) = stg.k[m];
        }
      }
#pragma unroll
      for (int m = 0; m < W::VU; ++m) {
        const int u = st + m * 256;
        const int row = u / (DVS / 8), c8 = u % (DVS / 8);
        GLA_CHECK_LDS(sm.vv[ns] + row * W::VLD + c8 * 8, 16);
        *reinterpret_cast<uint4*>(sm.vv[ns] + row * W::VLD + c8 * 8) = stg.v[m];
      }
      if (sw == 0) sm.sb[lane] = bl;
    };
    // Chunk index of a load: every load is issued, the ones past the segment
    // re-read its last chunk (already in L2), so that the number of loads in
    // flight is the same at every wait.
    const auto chunk_t0 = [&](int c) { return (uint32_t)min(c, c_end - 1) * kChunk; };
    // Part 1 of chunk c: the diagonal tile sw of A(c).
    const auto diagonal = [&](int c) {
      if (DIAG) {
        diagonal_pairs<DK, W::TLD>(sm.a, sm.qr, sm.kr, sm.sb, sw, lane);
      } else {
        attention_tile<DK, W::TLD, W::LD>(sm.a, sm.qh[(c - c_begin) & 1], sm.kh, sw, sw, 1.0f, g, r16);
      }
    };
    // GX: the last staging wave combines the compute waves' sums of chunk c during part 1
    // of chunk c + 1 (the sums alternate between two LDS buffers by chunk parity), the
    // last chunk's after the loop.  One lane per token of the chunk.
    const bool gx_wave = GX != 0 && sw == W::NSW - 1;
    float* gx_out = GX ? p.gx_out + span.row0 : nullptr;
    const float* gx_x = GX == 2 ? p.gx_x + span.row0 : nullptr;
    float gx_xv = 0.0f, gx_wv = 0.0f;  // GX 2: x and W of the chunk combined next (loaded one chunk ahead)
    const auto gx_token = [&](int cc) -> long long {  // physical token of this lane's row of chunk cc
      const long long tl = (long long)cc * kChunk + lane;
      return p.reverse ? Tg - 1 + p.pad - tl : tl;
    };
    const auto gx_fetch = [&](int cc) {
      const long long t = gx_token(cc);
      const bool in = t >= 0 && t < Tg;
      gx_xv = in ? gx_x[t] : 0.0f;
      gx_wv = in ? gx_out[t] : 0.0f;
    };
    const auto gx_combine = [&](int cc) {
      const int par = (cc - c_begin) & 1;
      const long long t = gx_token(cc);
      if constexpr (GX == 1) {
        float col = 0.0f, row = 0.0f, r = 0.0f;
#pragma unroll
        for (int w = 0; w < W::NCW; ++w) {
          col += sm.gx_a[par][w][lane];
          row += sm.gx_c[par][w][lane];
          r += sm.gx_r[par][w][lane];
        }
        // pairs inside: exclusive prefix of (column sum - row sum); entering: inclusive suffix of r
        const float d = col - row;
        const float R = wave_inclusive_scan(d, lane) - d;
        const float rincl = wave_inclusive_scan(r, lane);
        const float rsuf = lane_value(rincl, 63) - rincl + r;
        if (t < Tg) gx_out[t] = R + rsuf;
      } else if constexpr (GX == 2) {
        float u = 0.0f, z = 0.0f;
#pragma unroll
        for (int w = 0; w < W::NCW; ++w) {
          u += sm.gx_a[par][w][lane];
          z += sm.gx_r[par][w][0];
        }
        // leaving: the sum over the physically earlier tokens of the chunk = later rows here
        const float uincl = wave_inclusive_scan(u, lane);
        const float uex = lane_value(uincl, 63) - uincl;
        const float slope = p.gate == kGateBoundedSigmoid ? gate_slope<kGateBoundedSigmoid>(gx_xv)
                                                          : gate_slope<kGateNegSoftplus>(gx_xv);
        if (t >= 0 && t < Tg) gx_out[t] = slope * (gx_wv + uex + z);
        if (cc + 1 < c_end) gx_fetch(cc + 1);
      }
    };
    // Register set s0 holds the chunks at even offsets from c_begin, s1 the odd
    // ones; chunk c+1 is staged during chunk c, and the loads of chunk c+3 are
    // issued right after into the freed set, two chunks ahead of their use.
    WsStaged<DK, DVS> s0, s1;
    if (c_begin < c_end) {
      s0.load(hb, p, chunk_t0(c_begin), col0, st);
      stage(s0, 0);
      s1.load(hb, p, chunk_t0(c_begin + 1), col0, st);
      s0.load(hb, p, chunk_t0(c_begin + 2), col0, st);
      if (GX == 2 && gx_wave) gx_fetch(c_begin);
    }
    __syncthreads();
    // Chunks are taken in pairs so that each set is named statically; staging and
    // loads inside the loop are unconditional (past the last chunk they repeat it
    // into buffers nobody reads any more), so that every wait sees the same loads
    // in flight: one set is waited for while the other set's loads stay outstanding.
    int c = c_begin;
    for (; c + 1 < c_end; c += 2) {
      diagonal(c);
      if (gx_wave && c > c_begin) gx_combine(c - 1);
      __syncthreads();
      stage(s1, 1);
      s1.load(hb, p, chunk_t0(c + 3), col0, st);
      __syncthreads();
      diagonal(c + 1);
      if (gx_wave) gx_combine(c);
      __syncthreads();
      stage(s0, 0);
      s0.load(hb, p, chunk_t0(c + 4), col0, st);
      __syncthreads();
    }
    if (c < c_end) {  // odd number of chunks: the last one has nothing to stage after it
      diagonal(c);
      if (gx_wave && c > c_begin) gx_combine(c - 1);
      __syncthreads();
      __syncthreads();
    }
    if (gx_wave && c_begin < c_end) gx_combine(c_end - 1);
    // no loads left in flight when the wave ends
    __builtin_amdgcn_s_waitcnt(0);
  }
}

// ============================================================================
// Segment pre-pass: local final state (from a zero state) and total log-decay of
// every segment but the last, for the output pass to fold into its initial state.
// Same split as the output pass: staging waves load chunk c+2 and write
// k e^{gamma - b} and v of chunk c+1 into the second buffer set while the compute
// waves apply chunk c to their state slice; one barrier per chunk.
// ============================================================================
template <int DK, int DVS>
struct WsSegSmem {
  using W = WsCfg<DK, DVS, false>;
  bf16 kp[2][64 * W::KLD];  // k_i e^{gamma - b_i}, [i][d]
  bf16 vv[2][64 * W::VLD];  // v[i][n]
  float gam[2];             // gamma of the chunk in each buffer set
  SegScanSmem scan;         // first chunk to run (x path)
};

template <int DK, int DVS>
__global__ void __launch_bounds__((WsCfg<DK, DVS, false>::NT)) segment_state_ws_kernel(ChunkParams p) {
  using W = WsCfg<DK, DVS, false>;
  using C = typename W::C;
  using E = Elem<bf16>;
  __shared__ __attribute__((aligned(16))) WsSegSmem<DK, DVS> sm;  // 16-byte aligned: row stores compile to ds_write_b128
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool compute = wave < W::NCW;
  const int r16 = lane & 15, g = lane >> 4;
  const int nseg = p.segments - 1;
  const int L = work_index(p);
  const int slice = L % p.nslices;
  const int rest = L / p.nslices;
  const int seg = rest % nseg;
  const int bh = unit_of(p, rest / nseg);
  const int col0 = slice * DVS;
  const int cw = compute ? wave : 0;
  const int sw = compute ? 0 : wave - W::NCW;
  const int st = compute ? 0 : tid - 64 * W::NCW;
  const int wcol = col0 + cw * C::CPW;
  const HeadSpan span = head_span(p, bh);
  const int c_begin = (int)((long long)seg * span.nchunks / p.segments);
  const int c_end = (int)((long long)(seg + 1) * span.nchunks / p.segments);
  const HeadBuffers hb = head_buffers<bf16, DK>(p, span);
  // first chunk to run and the segment's log-decay: from b every wave finds them
  // itself; from x the waves share the chunk scans (one barrier)
  float gsum;  // total log-decay of the segment
  const int c_first = p.b ? segment_first_live_chunk(hb, c_begin, c_end, gsum)
                          : segment_first_live_chunk_x<W::NCW + W::NSW>(hb, p, c_begin, c_end, gsum, sm.scan);

  if (compute) {
    StateAcc<bf16, DK, DVS> S;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) S.s[nb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    for (int c = c_first; c < c_end; ++c) {
      const int slot = (c - c_first) & 1;
      const float gam = sm.gam[slot];
      VFrags<bf16, DK, DVS> Vf;
      load_v_frags<bf16, DK, DVS, W::VLD>(Vf, sm.vv[slot], cw, lane);
      state_update<bf16, DK, DVS, W::KLD>(S, Vf, sm.kp[slot], exp_e(gam), lane);
      __syncthreads();
    }
    store_state<bf16, DK, DVS>(S, p.seg_state + ((long long)bh * nseg + seg) * DK * p.dv, p.dv, wcol, g, r16);
    if (slice == 0 && tid == 0) p.seg_decay[(long long)bh * p.segments + seg] = gsum;
  } else {
    const auto stage = [&](const WsStaged<DK, DVS, false>& stg, int ns) {
      const ChunkDecay cd(stg.decay(hb, p, lane));
      float brow[W::QU];
#pragma unroll
      for (int m = 0; m < W::QU; ++m) brow[m] = cd.at((st + m * 256) / (DK / 8));
#pragma unroll
      for (int m = 0; m < W::QU; ++m) {
        const int u = st + m * 256;
        const int row = u / (DK / 8), c8 = u % (DK / 8);
        E::Vec8 kv;
        kv.u = stg.k[m];
        E::store8_scaled(sm.kp[ns] + row * W::KLD + c8 * 8, kv, exp_e(cd.gam - brow[m]));
      }
#pragma unroll
      for (int m = 0; m < W::VU; ++m) {
        const int u = st + m * 256;
        const int row = u / (DVS / 8), c8 = u % (DVS / 8);
        GLA_CHECK_LDS(sm.vv[ns] + row * W::VLD + c8 * 8, 16);
        *reinterpret_cast<uint4*>(sm.vv[ns] + row * W::VLD + c8 * 8) = stg.v[m];
      }
      if (sw == 0 && lane == 0) sm.gam[ns] = cd.gam;
    };
    const auto chunk_t0 = [&](int c) { return (uint32_t)min(c, c_end - 1) * kChunk; };
    // register set s0: chunks at even offsets from c_first, s1: odd offsets
    WsStaged<DK, DVS, false> s0, s1;
    if (c_first < c_end) {
      s0.load(hb, p, chunk_t0(c_first), col0, st);
      stage(s0, 0);
      s1.load(hb, p, chunk_t0(c_first + 1), col0, st);
      s0.load(hb, p, chunk_t0(c_first + 2), col0, st);
    }
    __syncthreads();
    int c = c_first;
    for (; c + 1 < c_end; c += 2) {
      stage(s1, 1);
      s1.load(hb, p, chunk_t0(c + 3), col0, st);
      __syncthreads();
      stage(s0, 0);
      s0.load(hb, p, chunk_t0(c + 4), col0, st);
      __syncthreads();
    }
    if (c < c_end) __syncthreads();
    // no loads left in flight when the wave ends
    __builtin_amdgcn_s_waitcnt(0);
  }
}

template <int DK, int DVS>
hipError_t ws_seg_launch(const ChunkParams& p, hipStream_t s) {
  hipLaunchKernelGGL((segment_state_ws_kernel<DK, DVS>), dim3(p.grid), dim3(WsCfg<DK, DVS, false>::NT), 0, s, p);
  return hipGetLastError();
}

template <int DK, int DVS, bool DIAG>
hipError_t ws_launch(const ChunkParams& p, hipStream_t s) {
  if constexpr (DVS >= 64 && !DIAG) {
    // the gate-gradient terms need the whole value width in one workgroup
    if (p.gx_mode != 0 && p.nslices != 1) return hipErrorInvalidValue;
    if (p.gx_mode == 1) {
      hipLaunchKernelGGL((chunk_output_ws_kernel<DK, DVS, DIAG, 1>), dim3(p.grid), dim3(WsCfg<DK, DVS, DIAG>::NT), 0, s, p);
      return hipGetLastError();
    }
    if (p.gx_mode == 2) {
      hipLaunchKernelGGL((chunk_output_ws_kernel<DK, DVS, DIAG, 2>), dim3(p.grid), dim3(WsCfg<DK, DVS, DIAG>::NT), 0, s, p);
      return hipGetLastError();
    }
  }
  if (p.gx_mode != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((chunk_output_ws_kernel<DK, DVS, DIAG>), dim3(p.grid), dim3(WsCfg<DK, DVS, DIAG>::NT), 0, s, p);
  return hipGetLastError();
}

bool ws_kernels_supported(int dtype, int dk, int slice) {
  return dtype == 0 && (dk == 64 || dk == 128) && (slice == 32 || slice == 64 || slice == 128);
}

hipError_t launch_chunk_output_ws(const ChunkParams& p, int dk, int slice, bool diag, hipStream_t stream) {
#define GLA_WS_CASE(DKV, DVSV)                                                                   \
  if (dk == DKV && slice == DVSV) return diag ? ws_launch<DKV, DVSV, true>(p, stream) : ws_launch<DKV, DVSV, false>(p, stream);
  GLA_WS_CASE(128, 128) GLA_WS_CASE(128, 64) GLA_WS_CASE(128, 32)
  GLA_WS_CASE(64, 128) GLA_WS_CASE(64, 64) GLA_WS_CASE(64, 32)
#undef GLA_WS_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_segment_states_ws(const ChunkParams& p, int dk, int slice, hipStream_t stream) {
#define GLA_WS_CASE(DKV, DVSV) \
  if (dk == DKV && slice == DVSV) return ws_seg_launch<DKV, DVSV>(p, stream);
  GLA_WS_CASE(128, 128) GLA_WS_CASE(128, 64) GLA_WS_CASE(128, 32)
  GLA_WS_CASE(64, 128) GLA_WS_CASE(64, 64) GLA_WS_CASE(64, 32)
#undef GLA_WS_CASE
  return hipErrorInvalidValue;
}

// debug builds: this unit's LDS-check word (see GLA_CHECK_LDS)
GLA_DEBUG_ACCESSOR(debug_word_ws_kernels)

}  // namespace gla
