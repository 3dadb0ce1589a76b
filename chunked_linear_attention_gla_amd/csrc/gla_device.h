// gla_device.h -- device-side building blocks for the gfx950 (CDNA4) GLA kernels.
//
// MFMA fragment convention used by every kernel in this library.
// A 16x16 output tile is produced by v_mfma_f32_16x16x32_bf16 (bf16 operands)
// or by eight v_mfma_f32_16x16x4_f32 (fp32 operands).  Lane l = 16*g + r
// (g = l / 16 in 0..3, r = l % 16) holds, for a K-step of 32 starting at k0,
// eight operand elements e = 0..7 at the logical contraction indices
//     kappa(g, e) = k0 + 16*(e / 4) + 4*g + (e % 4),
// for row/column r of its operand.  kappa is a permutation of k0..k0+31, so any
// such assignment computes the same sum as long as both operands use it.  This
// one is chosen because the accumulator of a 16x16 tile holds rows 4g..4g+3 of
// column r in lane l: two vertically adjacent accumulator tiles are therefore
// already a K-step fragment, and the state S (an accumulator) feeds the q.S
// product and the attention matrix feeds A.V without any shuffle.
//   bf16: the 8 elements are the hardware K positions 8g..8g+7 of one 16x16x32.
//   fp32: element e is the (lane-group g) K position of the e-th 16x16x4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;  // tokens per chunk
constexpr int kTile = 16;   // tokens per tile (the bounded-decay safe length)

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- debug checks
// A library built with -DGLA_DEBUG checks, inside the shared LDS helpers below, that
// every access reaches LDS and falls inside the workgroup's static LDS allocation.  A
// failed check sets a bit in a device word of its translation unit and the kernel goes
// on (the hardware drops LDS accesses past the allocation): checks never trap.  The C
// entry point gla_debug_flags reads and clears the words.  Release builds compile
// every check away.
enum : unsigned { kDebugLdsRange = 1u, kDebugNotLds = 2u };
#ifdef GLA_DEBUG
static __device__ unsigned int g_debug_word;
__device__ __forceinline__ void debug_fail(unsigned bit) { atomicOr(&g_debug_word, bit); }
__device__ __forceinline__ void debug_check_lds(const void* p, unsigned bytes) {
  if (!__builtin_amdgcn_is_shared((const __attribute__((address_space(0))) void*)p)) {
    debug_fail(kDebugNotLds);
    return;
  }
  const unsigned off = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
  if (off + bytes > __builtin_amdgcn_groupstaticsize()) debug_fail(kDebugLdsRange);
}
#define GLA_CHECK_LDS(p, bytes) ::gla::debug_check_lds((const void*)(p), (bytes))
// Host side, one per translation unit: read and clear that unit's word (~0u if the
// read fails).
#define GLA_DEBUG_ACCESSOR(NAME)                                                              \
  unsigned int NAME() {                                                                        \
    unsigned int v = 0, z = 0;                                                                 \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_word), sizeof v, 0, hipMemcpyDeviceToHost) != \
        hipSuccess)                                                                            \
      return ~0u;                                                                              \
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_debug_word), &z, sizeof z, 0, hipMemcpyHostToDevice) !=   \
        hipSuccess)                                                                            \
      return ~0u;                                                                              \
    return v;                                                                                  \
  }
#else
#define GLA_CHECK_LDS(p, bytes) ((void)0)
#define GLA_DEBUG_ACCESSOR(NAME)
#endif

// 2^x on the hardware exp2 (v_exp_f32).  2^-inf = 0, 2^+inf = inf.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// e^x as 2^(x log2 e).
__device__ __forceinline__ float exp_e(float x) { return exp2_hw(x * kLog2e); }

// Log-decay gates ("Engineering Long-Context Training for Trillion-Parameter MoE
// Models: Three Key Breakthroughs", §3.2).
// g = -5 * sigmoid(x).  With t = e^{-|x|} in [0, 1], sigmoid(x) is 1 / (1 + t) for
// x >= 0 and t / (1 + t) for x < 0: nothing overflows for either sign, and one
// hardware reciprocal (1 ulp) replaces an IEEE division per branch, so the gate costs
// two transcendentals and no divergent branch (it runs once per token and channel
// inside the per-channel kernels).
__device__ __forceinline__ float sigmoid_hw(float x) {
  const float t = exp_e(-fabsf(x));
  const float r = __builtin_amdgcn_rcpf(1.0f + t);
  return x >= 0.0f ? r : t * r;
}

__device__ __forceinline__ float gate_bounded_sigmoid(float x) { return -5.0f * sigmoid_hw(x); }

// g = -softplus(-x) = -(max(-x, 0) + log1p(e^-|x|)) = log sigmoid(x), floored at
// kSoftplusFloor.  The gate is unbounded below (x = -inf gives g = -inf, a = 0); the
// chunked paths take differences of cumulative sums of g, where -inf - -inf would be
// NaN.  At the floor e^g is already exactly 0 in fp32 (2^-184.7), so a = 0 is kept and
// every decay product through such a token is an exact zero, while the cumulative
// sums stay finite.  NaN input still gives NaN (the comparison is false for NaN).
constexpr float kSoftplusFloor = -128.0f;
__device__ __forceinline__ float gate_neg_softplus(float x) {
  const float z = -x;
  const float g = -(fmaxf(z, 0.0f) + log1pf(exp_e(-fabsf(z))));
  return g < kSoftplusFloor ? kSoftplusFloor : g;
}

template <int CTRL>
__device__ __forceinline__ float dpp_or_zero(float v) {
  // row-local lane shift; lanes whose source falls outside the 16-lane row read 0
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}

// Maximum and sum over aligned groups of N consecutive lanes (N = 2, 4, 8 or 16), left
// in every lane of the group: lane swaps within quads (xor 1, xor 2), then the mirror
// images within 8 and 16 lanes, each of which maps the group's two halves onto each
// other.  Every lane of the wavefront must be active.
template <int N>
__device__ __forceinline__ float group_max(float v) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "group of 2, 4, 8 or 16 lanes");
  v = fmaxf(v, dpp_or_zero<0xB1>(v));                          // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v = fmaxf(v, dpp_or_zero<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v = fmaxf(v, dpp_or_zero<0x141>(v));   // row_half_mirror
  if constexpr (N >= 16) v = fmaxf(v, dpp_or_zero<0x140>(v));  // row_mirror
  return v;
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "group of 2, 4, 8 or 16 lanes");
  v += dpp_or_zero<0xB1>(v);
  if constexpr (N >= 4) v += dpp_or_zero<0x4E>(v);
  if constexpr (N >= 8) v += dpp_or_zero<0x141>(v);
  if constexpr (N >= 16) v += dpp_or_zero<0x140>(v);
  return v;
}

// v_permlane16_swap_b32 with both of its results: the odd 16-lane rows of a trade
// places with the even rows of b, so a = (a0, b0, a2, b2) and b = (a1, b1, a3, b3) by
// row.  Written out because this compiler's builtin hands back its first result for
// either index; the s_nop gives the two wait states the instruction needs after a
// VALU write of its operands.
__device__ __forceinline__ void permlane16_swap_pair(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// v_permlane32_swap_b32 with both of its results: the high 32 lanes of a trade places
// with the low 32 lanes of b, so a = (a_lo, b_lo) and b = (a_hi, b_hi) by half-wave.
// Written out for the reason given above.
__device__ __forceinline__ void permlane32_swap_pair(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// Row R0's value at the lane's position, in every row (a broadcast across the four
// 16-lane rows): a row-pair swap picks row R0 % 2 of each pair, a half-wave swap the
// pair R0 / 2.
template <int R0>
__device__ __forceinline__ float row_broadcast(float v) {
  static_assert(R0 >= 0 && R0 < 4, "row of a wavefront");
  uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
  permlane16_swap_pair(a, b);  // a: the pair's even row, b: its odd row
  uint32_t c = (R0 & 1) ? b : a, d = c;
  permlane32_swap_pair(c, d);  // c: the low pair's, d: the high pair's
  return __builtin_bit_cast(float, (R0 & 2) ? d : c);
}

// Sum over the four 16-lane rows of the lanes at the same position (lanes l, l ^ 16,
// l ^ 32, l ^ 48), left in all four: a row-pair swap, then a half-wave swap.
__device__ __forceinline__ float row_sum4(float v) {
  uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
  permlane16_swap_pair(a, b);  // a: the pair's even row, b: its odd row
  const float pair = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  uint32_t c = __builtin_bit_cast(uint32_t, pair), d = c;
  permlane32_swap_pair(c, d);  // c: the low pair's sum, d: the high pair's
  return __builtin_bit_cast(float, c) + __builtin_bit_cast(float, d);
}

// Exclusive prefix sum of v over the lanes l - S, l - 2S, ... (S = STRIDE in 1, 2, 4, 8
// or 16: lanes that hold the same item of earlier groups of S lanes).  Inside each
// 16-lane row: DPP row shifts for the prefix and rotations for the row total (both
// keep a lane's position modulo S); across the four rows: the row-pair and half-wave
// swap permutes of gfx950, which hand every lane the totals of the rows before its
// own at the same position.
template <int STRIDE>
__device__ __forceinline__ float strided_exclusive_scan(float v, int lane) {
  static_assert(STRIDE == 1 || STRIDE == 2 || STRIDE == 4 || STRIDE == 8 || STRIDE == 16, "stride");
  float incl = v, rt = v;
  if constexpr (STRIDE <= 1) { incl += dpp_or_zero<0x111>(incl); rt += dpp_or_zero<0x121>(rt); }  // row_shr / row_ror 1
  if constexpr (STRIDE <= 2) { incl += dpp_or_zero<0x112>(incl); rt += dpp_or_zero<0x122>(rt); }
  if constexpr (STRIDE <= 4) { incl += dpp_or_zero<0x114>(incl); rt += dpp_or_zero<0x124>(rt); }
  if constexpr (STRIDE <= 8) { incl += dpp_or_zero<0x118>(incl); rt += dpp_or_zero<0x128>(rt); }
  // Across rows (R_r: the row totals at the lane's position): one row-pair swap of rt
  // with itself gives every lane the totals of both rows of its pair, a half-wave swap
  // moves the sum of rows 0 and 1 into the high half of a zero register.
  uint32_t ev = __builtin_bit_cast(uint32_t, rt), od = ev;
  permlane16_swap_pair(ev, od);
  const float even = __builtin_bit_cast(float, ev), odd = __builtin_bit_cast(float, od);
  const float low = __builtin_bit_cast(
      float, __builtin_amdgcn_permlane32_swap(0u, __builtin_bit_cast(uint32_t, even + odd), false, false)[0]);
  return (incl - v) + ((lane & 16) ? even : 0.0f) + low;  // rows 0..3: + 0, R0, R0 + R1, R2 + R0 + R1
}

// Inclusive prefix sum over the 64 lanes of the wavefront: DPP row shifts inside each
// 16-lane row, then the three row totals read across lanes.  Every kernel that forms
// the chunk-local cumulative log-decay uses this one routine, so they all get the
// same bits.
__device__ __forceinline__ float wave_inclusive_scan(float v, int lane) {
  v += dpp_or_zero<0x111>(v);  // row_shr:1
  v += dpp_or_zero<0x112>(v);  // row_shr:2
  v += dpp_or_zero<0x114>(v);  // row_shr:4
  v += dpp_or_zero<0x118>(v);  // row_shr:8
  const float t0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15));
  const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
  const float t2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47));
  const int row = lane >> 4;
  float off = 0.0f;
  if (row >= 1) off = t0;
  if (row >= 2) off = off + t1;
  if (row >= 3) off = off + t2;
  return v + off;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// ---------------------------------------------------------------- buffer access
//
// Streaming tensors are read and written through raw buffer instructions with a
// per-head resource descriptor whose size is the head's extent in bytes.  The
// hardware range check returns zeros for loads past the end and drops stores
// past the end, so the ragged last chunk needs no branches: every wave issues
// the same memory instructions every chunk and the compiler can wait on exact
// counts instead of draining all outstanding loads and stores.
// Descriptor word 3 for gfx9-family raw buffers: DATA_FORMAT (bits 15..18) = 4,
// 32-bit elements; no swizzle, no stride.
constexpr int kBufferWord3 = 0x00020000;
// cache-policy operand of the buffer builtins: bit 1 marks a streaming
// (non-temporal) access
constexpr int kAuxStream = 2;
// Largest extent of one head's tensor (bytes) that a descriptor may describe, and
// an offset beyond it that leaves room for a few 16-byte accesses without
// wrapping: a store there is always out of range and dropped.
constexpr uint32_t kMaxHeadBytes = 0xFFFF0000u;
constexpr uint32_t kDroppedOffset = 0xFFFFF000u;

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}
template <int AUX = 0>
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 buf_load8(rsrc_t r, uint32_t off) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ float buf_load4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
template <int AUX = 0>
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, const floatx4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, AUX);
}

// ---------------------------------------------------------------- element traits

template <typename T> struct Elem;

template <> struct Elem<bf16> {
  // 8 consecutive elements as loaded from global memory (16 bytes)
  struct Vec8 { uint4 u; };
  struct Frag { bf16x8 v; };
  static constexpr int kPad = 8;  // LDS row padding in elements (16 bytes)

  __device__ static __forceinline__ Vec8 zero8() { Vec8 r; r.u = make_uint4(0, 0, 0, 0); return r; }
  // operands are streamed once per kernel: non-temporal loads (per-channel call
  // 0.791 -> 0.774 ms; the delta rule's unchanged)
  __device__ static __forceinline__ Vec8 load8(rsrc_t r, uint32_t byte_off) {
    Vec8 v; v.u = buf_load16<kAuxStream>(r, byte_off); return v;
  }
  __device__ static __forceinline__ float get(const Vec8& v, int e) {
    const uint32_t w = (e < 2) ? v.u.x : (e < 4) ? v.u.y : (e < 6) ? v.u.z : v.u.w;
    return bf16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFFu));
  }
  __device__ static __forceinline__ bf16 cvt(float f) { return static_cast<bf16>(f); }
  // store 8 scaled elements as one 16-byte LDS write
  __device__ static __forceinline__ void store8_scaled(bf16* dst, const Vec8& v, float s) {
    GLA_CHECK_LDS(dst, 16);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = cvt(get(v, e) * s);
    *reinterpret_cast<bf16x8*>(dst) = o;
  }
  __device__ static __forceinline__ void store8_raw(bf16* dst, const Vec8& v) {
    GLA_CHECK_LDS(dst, 16);
    *reinterpret_cast<uint4*>(dst) = v.u;
  }
  // store -v (sign bits flipped: exact)
  __device__ static __forceinline__ void store8_neg(bf16* dst, const Vec8& v) {
    GLA_CHECK_LDS(dst, 16);
    constexpr uint32_t m = 0x80008000u;
    *reinterpret_cast<uint4*>(dst) = make_uint4(v.u.x ^ m, v.u.y ^ m, v.u.z ^ m, v.u.w ^ m);
  }
  // The same two stores into a row that holds each 16-byte group with its two 8-byte
  // halves swapped when `swap` (a fragment-read swizzle; see the kernels using it).
  static constexpr bool kSwizzle = true;
  __device__ static __forceinline__ void store8_scaled_sw(bf16* dst, const Vec8& v, float s, bool swap) {
    GLA_CHECK_LDS(dst, 16);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = cvt(get(v, e) * s);
    if (swap) o = __builtin_shufflevector(o, o, 4, 5, 6, 7, 0, 1, 2, 3);
    *reinterpret_cast<bf16x8*>(dst) = o;
  }
  __device__ static __forceinline__ void store8_vscaled_sw(bf16* dst, const Vec8& v, const float (&s)[8], bool swap) {
    GLA_CHECK_LDS(dst, 16);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = cvt(get(v, e) * s[e]);
    if (swap) o = __builtin_shufflevector(o, o, 4, 5, 6, 7, 0, 1, 2, 3);
    *reinterpret_cast<bf16x8*>(dst) = o;
  }
  // 8 fp32 values rounded to bf16, as one 16-byte LDS write (halves swapped when `swap`)
  __device__ static __forceinline__ void store8_f32_sw(bf16* dst, const float (&x)[8], bool swap) {
    GLA_CHECK_LDS(dst, 16);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = cvt(x[e]);
    if (swap) o = __builtin_shufflevector(o, o, 4, 5, 6, 7, 0, 1, 2, 3);
    *reinterpret_cast<bf16x8*>(dst) = o;
  }
  __device__ static __forceinline__ void store8_neg_sw(bf16* dst, const Vec8& v, bool swap) {
    GLA_CHECK_LDS(dst, 16);
    constexpr uint32_t m = 0x80008000u;
    const uint4 n = make_uint4(v.u.x ^ m, v.u.y ^ m, v.u.z ^ m, v.u.w ^ m);
    *reinterpret_cast<uint4*>(dst) = swap ? make_uint4(n.z, n.w, n.x, n.y) : n;
  }
  // store 8 elements, each with its own scale
  __device__ static __forceinline__ void store8_vscaled(bf16* dst, const Vec8& v, const float (&s)[8]) {
    GLA_CHECK_LDS(dst, 16);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = cvt(get(v, e) * s[e]);
    *reinterpret_cast<bf16x8*>(dst) = o;
  }
  // two 4-element (8-byte) LDS reads at cols c and c + 16 of one row
  __device__ static __forceinline__ Frag load_frag(const bf16* row, int c) {
    GLA_CHECK_LDS(row + c, 8);
    GLA_CHECK_LDS(row + c + 16, 8);
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + c);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + c + 16);
    Frag f;
    f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return f;
  }
  __device__ static __forceinline__ Frag from_acc(const floatx4& a, const floatx4& b) {
    Frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = cvt(a[e]); f.v[4 + e] = cvt(b[e]); }
    return f;
  }
  __device__ static __forceinline__ void store4(bf16* dst, float a, float b, float c, float d) {
    GLA_CHECK_LDS(dst, 8);
    bf16x4 o;
    o[0] = cvt(a); o[1] = cvt(b); o[2] = cvt(c); o[3] = cvt(d);
    *reinterpret_cast<bf16x4*>(dst) = o;
  }
  __device__ static __forceinline__ void mfma(floatx4& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
  }
  __device__ static __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
};

template <> struct Elem<float> {
  struct Vec8 { float4 a, b; };
  struct Frag { floatx4 lo, hi; };
  static constexpr int kPad = 4;  // 16 bytes

  __device__ static __forceinline__ Vec8 zero8() {
    Vec8 r; r.a = make_float4(0, 0, 0, 0); r.b = r.a; return r;
  }
  __device__ static __forceinline__ Vec8 load8(rsrc_t r, uint32_t byte_off) {
    Vec8 v;
    const uint4 a = buf_load16(r, byte_off), b = buf_load16(r, byte_off + 16);
    v.a = make_float4(__builtin_bit_cast(float, a.x), __builtin_bit_cast(float, a.y),
                      __builtin_bit_cast(float, a.z), __builtin_bit_cast(float, a.w));
    v.b = make_float4(__builtin_bit_cast(float, b.x), __builtin_bit_cast(float, b.y),
                      __builtin_bit_cast(float, b.z), __builtin_bit_cast(float, b.w));
    return v;
  }
  __device__ static __forceinline__ float get(const Vec8& v, int e) {
    switch (e) {
      case 0: return v.a.x; case 1: return v.a.y; case 2: return v.a.z; case 3: return v.a.w;
      case 4: return v.b.x; case 5: return v.b.y; case 6: return v.b.z; default: return v.b.w;
    }
  }
  __device__ static __forceinline__ float cvt(float f) { return f; }
  __device__ static __forceinline__ void store8_scaled(float* dst, const Vec8& v, float s) {
    GLA_CHECK_LDS(dst, 32);
    float4 a = v.a, b = v.b;
    a.x *= s; a.y *= s; a.z *= s; a.w *= s;
    b.x *= s; b.y *= s; b.z *= s; b.w *= s;
    *reinterpret_cast<float4*>(dst) = a;
    *reinterpret_cast<float4*>(dst + 4) = b;
  }
  __device__ static __forceinline__ void store8_raw(float* dst, const Vec8& v) {
    GLA_CHECK_LDS(dst, 32);
    *reinterpret_cast<float4*>(dst) = v.a;
    *reinterpret_cast<float4*>(dst + 4) = v.b;
  }
  __device__ static __forceinline__ void store8_neg(float* dst, const Vec8& v) {
    GLA_CHECK_LDS(dst, 32);
    constexpr uint32_t m = 0x80000000u;
    const auto flip = [](float f) { return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f) ^ m); };
    *reinterpret_cast<float4*>(dst) = make_float4(flip(v.a.x), flip(v.a.y), flip(v.a.z), flip(v.a.w));
    *reinterpret_cast<float4*>(dst + 4) = make_float4(flip(v.b.x), flip(v.b.y), flip(v.b.z), flip(v.b.w));
  }
  // fp32 tiles are not swizzled (their fragment reads are 16-byte pieces)
  static constexpr bool kSwizzle = false;
  __device__ static __forceinline__ void store8_scaled_sw(float* dst, const Vec8& v, float s, bool) {
    store8_scaled(dst, v, s);
  }
  __device__ static __forceinline__ void store8_f32_sw(float* dst, const float (&x)[8], bool) {
    GLA_CHECK_LDS(dst, 32);
    *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
  __device__ static __forceinline__ void store8_neg_sw(float* dst, const Vec8& v, bool) { store8_neg(dst, v); }
  __device__ static __forceinline__ void store8_vscaled_sw(float* dst, const Vec8& v, const float (&s)[8], bool) {
    store8_vscaled(dst, v, s);
  }
  __device__ static __forceinline__ void store8_vscaled(float* dst, const Vec8& v, const float (&s)[8]) {
    GLA_CHECK_LDS(dst, 32);
    *reinterpret_cast<float4*>(dst) = make_float4(v.a.x * s[0], v.a.y * s[1], v.a.z * s[2], v.a.w * s[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(v.b.x * s[4], v.b.y * s[5], v.b.z * s[6], v.b.w * s[7]);
  }
  __device__ static __forceinline__ Frag load_frag(const float* row, int c) {
    GLA_CHECK_LDS(row + c, 16);
    GLA_CHECK_LDS(row + c + 16, 16);
    Frag f;
    f.lo = *reinterpret_cast<const floatx4*>(row + c);
    f.hi = *reinterpret_cast<const floatx4*>(row + c + 16);
    return f;
  }
  __device__ static __forceinline__ Frag from_acc(const floatx4& a, const floatx4& b) {
    Frag f; f.lo = a; f.hi = b; return f;
  }
  __device__ static __forceinline__ void store4(float* dst, float a, float b, float c, float d) {
    GLA_CHECK_LDS(dst, 16);
    floatx4 o = {a, b, c, d};
    *reinterpret_cast<floatx4*>(dst) = o;
  }
  __device__ static __forceinline__ void mfma(floatx4& acc, const Frag& a, const Frag& b) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[s], b.lo[s], acc, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[s], b.hi[s], acc, 0, 0, 0);
  }
  __device__ static __forceinline__ float to_f32(float x) { return x; }
};

// ---------------------------------------------------------------- token-major tiles
//
// Tiles whose token index is the MFMA contraction index: k e^{gamma-b} and v in the
// state update, v in A.V.  An operand fragment needs, in lane (g, r16), eight
// tokens (kappa order) of one feature column c0 + r16.
//
// bf16: the tile is stored row-major [64 tokens][NCOL] and the fragment is read
// with the gfx950 LDS transpose read ds_read_b64_tr_b16.  Within each group of
// 16 lanes that instruction hands destination lane 4a + b, as its element e,
// element b of the 8 bytes addressed by source lane a + 4e.  Source lane s of
// lane group g therefore points at row k0 + 4g + s/4, columns c0 + 4(s%4)..+3,
// and every lane receives tokens k0 + 4g + 0..3 of its own column c0 + r16: the
// first half of the fragment; rows 16 further give the second half.
// fp32: there is no 32-bit transpose read, so the tile is stored transposed
// [NCOL][64 tokens] and read with ordinary fragment loads.
// LDX: row stride in elements.  One transposing read covers 8 rows x 32 bytes per
// 32-lane half; a stride of NCOL + 16 (an odd multiple of 8 banks) puts those rows in
// disjoint banks, where NCOL + 8 costs a 2-way bank conflict on every read (measured
// with SQ_LDS_BANK_CONFLICT).  A tile that is also written with 8-byte stores in the
// accumulator layout (16 rows of one column piece per store cycle) is better at
// NCOL + 8: those stores are 2-way there and 4-way at NCOL + 16.
// Row-major bf16 tiles read as MFMA fragments (ds_read2_b64: one 8-byte piece from each
// of 16 rows, columns c and c + 16): at a row stride of 136 elements rows r and r + 8
// fall on the same bank pair, a 2-way conflict on every read.  Rows with bit 3 set
// therefore hold each 16-byte group with its 8-byte halves swapped: element column c of
// row r is at c ^ frag_swz<T>(r) (bf16 only; the swap moves whole 8-byte halves, so
// four consecutive columns starting at a multiple of 4 stay consecutive).  frag_swap is
// the same test for a store whose rows share bit 3 across the wavefront.
template <typename T>
__device__ __forceinline__ int frag_swz(int row) {
  return Elem<T>::kSwizzle ? (row & 8) >> 1 : 0;
}
template <typename T>
__device__ __forceinline__ bool frag_swap(int row) {
  return __builtin_amdgcn_readfirstlane(frag_swz<T>(row)) != 0;
}

template <typename T, int NCOL, int LDX = NCOL + 16> struct TokTile;

template <int NCOL, int LDX> struct TokTile<bf16, NCOL, LDX> {
  static constexpr int LD = LDX;         // row stride (elements) of [token][col]
  static constexpr int SIZE = 64 * LD;
  using E = Elem<bf16>;
  __device__ static __forceinline__ void store8(bf16* t, int row, int col, const E::Vec8& v, float s) {
    E::store8_scaled(t + row * LD + col, v, s);
  }
  __device__ static __forceinline__ void store8_raw(bf16* t, int row, int col, const E::Vec8& v) {
    E::store8_raw(t + row * LD + col, v);
  }
  __device__ static __forceinline__ void store8_v(bf16* t, int row, int col, const E::Vec8& v, const float (&s)[8]) {
    E::store8_vscaled(t + row * LD + col, v, s);
  }
  __device__ static __forceinline__ void store8_f32(bf16* t, int row, int col, const float (&x)[8]) {
    E::store8_f32_sw(t + row * LD + col, x, false);
  }
  __device__ static __forceinline__ E::Frag load(const bf16* t, int k0, int c0, int lane) {
    typedef short shortx4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
    const int s = lane & 15, g = lane >> 4;
    const bf16* p0 = t + (k0 + 4 * g + (s >> 2)) * LD + c0 + 4 * (s & 3);
    const bf16* p1 = p0 + 16 * LD;
    GLA_CHECK_LDS(p0, 8);
    GLA_CHECK_LDS(p1, 8);
    const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p0));
    const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p1));
    E::Frag f;
    f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    return f;
  }
};

template <int NCOL, int LDX> struct TokTile<float, NCOL, LDX> {
  static constexpr int LD = 64 + 4;      // row stride (elements) of [col][token]
  static constexpr int SIZE = NCOL * LD;
  using E = Elem<float>;
  __device__ static __forceinline__ void store8(float* t, int row, int col, const E::Vec8& v, float s) {
    GLA_CHECK_LDS(t + col * LD + row, 4);
    GLA_CHECK_LDS(t + (col + 7) * LD + row, 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) t[(col + e) * LD + row] = E::get(v, e) * s;
  }
  __device__ static __forceinline__ void store8_raw(float* t, int row, int col, const E::Vec8& v) {
    GLA_CHECK_LDS(t + col * LD + row, 4);
    GLA_CHECK_LDS(t + (col + 7) * LD + row, 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) t[(col + e) * LD + row] = E::get(v, e);
  }
  __device__ static __forceinline__ void store8_v(float* t, int row, int col, const E::Vec8& v, const float (&s)[8]) {
    GLA_CHECK_LDS(t + col * LD + row, 4);
    GLA_CHECK_LDS(t + (col + 7) * LD + row, 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) t[(col + e) * LD + row] = E::get(v, e) * s[e];
  }
  __device__ static __forceinline__ void store8_f32(float* t, int row, int col, const float (&x)[8]) {
    GLA_CHECK_LDS(t + col * LD + row, 4);
    GLA_CHECK_LDS(t + (col + 7) * LD + row, 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) t[(col + e) * LD + row] = x[e];
  }
  __device__ static __forceinline__ E::Frag load(const float* t, int k0, int c0, int lane) {
    return E::load_frag(t + (c0 + (lane & 15)) * LD, k0 + 4 * (lane >> 4));
  }
};

// Workgroup index -> linear work index, so that consecutive work indices land on
// the same XCD.  The dispatcher hands workgroups to the 8 XCDs round-robin
// (workgroup w runs on XCD w % 8); grouping consecutive work items on one XCD
// lets value-column slices of the same head share q and k through that XCD's L2.
__device__ __forceinline__ int xcd_linear_index(int w, int G) {
  const int x = w & 7, y = w >> 3;
  const int base = G >> 3, rem = G & 7;
  return x * base + (x < rem ? x : rem) + y;
}

}  // namespace gla
