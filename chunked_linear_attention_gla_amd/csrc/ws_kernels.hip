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

template <int DK, int DVS, bool DIAG>
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

template <int DK, int DVS, bool DIAG>
__global__ void __launch_bounds__((WsCfg<DK, DVS, DIAG>::NT)) chunk_output_ws_kernel(ChunkParams p) {
  using W = WsCfg<DK, DVS, DIAG>;
  using C = typename W::C;
  using E = Elem<bf16>;
  __shared__ __attribute__((aligned(16))) WsSmem<DK, DVS, DIAG> sm;  // 16-byte aligned: row stores compile to ds_write_b128
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

  // The two roles run separate loops with the same barriers (one before the
  // loop, two per chunk), so that the registers of one role are free for the
  // other: the compute waves hold the state and o accumulators, the staging waves
  // two register sets of prefetched chunks.
  if (compute) {
    StateAcc<bf16, DK, DVS> S;
    load_initial_state<bf16, DK, DVS>(S, p, bh, seg, wcol, g, r16);
    __syncthreads();
    for (int c = c_begin; c < c_end; ++c) {
      const int slot = (c - c_begin) & 1;
      const uint32_t t0 = (uint32_t)c * kChunk;
      if (p.state_out) store_chunk_state<bf16, DK, DVS>(S, p, bh, c, wcol, lane);

      // ---- part 1: off-diagonal tiles of A(c)
      const ChunkDecay cd(sm.sb[lane]);
#pragma unroll
      for (int t = 0; t < 6; ++t) {
        if (t % W::NCW != cw) continue;  // wave-uniform
        const int jb = off_j(t), ib = off_i(t);
        const float ri = DIAG ? cd.end(ib) : cd.r(ib);
        attention_tile<DK, W::TLD, W::LD>(sm.a, sm.qh[slot], sm.kh, jb, ib, exp_e(cd.r(jb) - ri), g, r16);
      }
      __syncthreads();

      // ---- part 2: o(c) and S_c
      typename E::Frag Sf[C::NB][C::KS];
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) Sf[nb][ks] = E::from_acc(S.s[nb][2 * ks], S.s[nb][2 * ks + 1]);
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
    // Register set s0 holds the chunks at even offsets from c_begin, s1 the odd
    // ones; chunk c+1 is staged during chunk c, and the loads of chunk c+3 are
    // issued right after into the freed set, two chunks ahead of their use.
    WsStaged<DK, DVS> s0, s1;
    if (c_begin < c_end) {
      s0.load(hb, p, chunk_t0(c_begin), col0, st);
      stage(s0, 0);
      s1.load(hb, p, chunk_t0(c_begin + 1), col0, st);
      s0.load(hb, p, chunk_t0(c_begin + 2), col0, st);
    }
    __syncthreads();
    // Chunks are taken in pairs so that each set is named statically; staging and
    // loads inside the loop are unconditional (past the last chunk they repeat it
    // into buffers nobody reads any more), so that every wait sees the same loads
    // in flight: one set is waited for while the other set's loads stay outstanding.
    int c = c_begin;
    for (; c + 1 < c_end; c += 2) {
      diagonal(c);
      __syncthreads();
      stage(s1, 1);
      s1.load(hb, p, chunk_t0(c + 3), col0, st);
      __syncthreads();
      diagonal(c + 1);
      __syncthreads();
      stage(s0, 0);
      s0.load(hb, p, chunk_t0(c + 4), col0, st);
      __syncthreads();
    }
    if (c < c_end) {  // odd number of chunks: the last one has nothing to stage after it
      diagonal(c);
      __syncthreads();
      __syncthreads();
    }
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
