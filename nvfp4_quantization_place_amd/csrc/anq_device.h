// Device building blocks of the fused tail kernels (gfx950 / CDNA4).
//
// Every helper here is exact or correctly rounded: the kernels must reproduce
// the binary32 definition of the op bit for bit, so no result is approximated
// and nothing is contracted (the library is built with -ffp-contract=off; the
// only fused multiply-adds are the explicit ones below, where they are exact
// or part of a correction step). Where a correction rests on a property of the
// hardware estimate or conversion instructions rather than on a proof, the
// property is checked over every input on the GPU by anq_selfcheck_arith.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "anq_internal.h"

namespace anq {

// 8 activations = 16 bytes, the unit of every global load and store.
struct alignas(16) U4 {
  uint32_t w[4];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ U4 ld16(const void* p) {
  return *reinterpret_cast<const U4*>(p);
}
// stored as a vector, not as a struct copy: the copy kept arrays of U4 that
// only some lanes fill in scratch memory
__device__ __forceinline__ void st16(void* p, const U4& v) {
  const u32x4 x = {v.w[0], v.w[1], v.w[2], v.w[3]};
  *reinterpret_cast<u32x4*>(p) = x;
}

// Row streams are read once and written once: with NT they carry the
// non-temporal hint (the `nt` bit of gfx950 global loads and stores). Measured
// on MI355X: at 8192 x 7168 and 65536 x 1024 the 16-byte row loads and stores
// hinted together cut the kernel time by ~10% (either alone does little); from
// 1 to 32 MiB of input, with inputs coming from HBM, the hinted loads alone cut
// it by 5-15%. The launchers choose NT by call size.

template <bool NT>
__device__ __forceinline__ U4 ld16s(const void* p) {
  if constexpr (NT) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    U4 r;
    r.w[0] = v.x;
    r.w[1] = v.y;
    r.w[2] = v.z;
    r.w[3] = v.w;
    return r;
  }
  return ld16(p);
}
template <bool NT>
__device__ __forceinline__ void st16s(void* p, const U4& v) {
  if constexpr (NT) {
    const u32x4 x = {v.w[0], v.w[1], v.w[2], v.w[3]};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
  } else {
    st16(p, v);
  }
}
template <bool NT>
__device__ __forceinline__ void st8s(void* p, uint32_t lo, uint32_t hi) {
  const u32x2 x = {lo, hi};
  if constexpr (NT) __builtin_nontemporal_store(x, reinterpret_cast<u32x2*>(p));
  else *reinterpret_cast<u32x2*>(p) = x;
}
template <bool NT>
__device__ __forceinline__ void st4s(void* p, uint32_t v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
  else *reinterpret_cast<uint32_t*>(p) = v;
}
template <bool NT>
__device__ __forceinline__ void st1s(void* p, uint8_t v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<uint8_t*>(p));
  else *reinterpret_cast<uint8_t*>(p) = v;
}

// A 64-bit value known to be the same in every lane, moved to scalar
// registers. Used for row offsets so that a global pointer plus the offset
// stays a global pointer (no flat addressing) and is addressed as SGPR base +
// 32-bit lane offset.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------- T <-> f32

template <int DT>
__device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi) {
  if constexpr (DT == kBF16) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xFFFF0000u);
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 v = __builtin_bit_cast(h2, w);
    lo = (float)v.x;
    hi = (float)v.y;
  }
}

// Round two binary32 values to T (nearest even) and pack them, lo in bits 0-15.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == kBF16) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    b2 v;
    v.x = (__bf16)lo;  // v_cvt_pk_bf16_f32: round to nearest even
    v.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 v;
    v.x = (_Float16)lo;  // v_cvt_f16_f32: round to nearest even
    v.y = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
  }
}

template <int DT>
__device__ __forceinline__ void unpack8(const U4& v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack2<DT>(v.w[i], f[2 * i], f[2 * i + 1]);
}

template <int DT>
__device__ __forceinline__ U4 pack8(const float (&f)[8]) {
  U4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v.w[i] = pack2<DT>(f[2 * i], f[2 * i + 1]);
  return v;
}

// ------------------------------------------------------------ E4M3 / E2M1

// gfx950 conversion instructions, used exactly where their semantics match the
// definition of the op (checked against definition-based encoders over every
// rounding interval, exact ties included, on the target):
//  * v_cvt_pk_fp8_f32 converts to OCP E4M3FN, nearest even, signed zeros kept,
//    subnormals kept; it returns NaN beyond +-448, so its inputs are either
//    bounded by construction (div_rn_sat) or first clamped with v_med3_f32
//    (saturation to +-448 is the nearest-even result there).
//  * v_cvt_scalef32_pk_fp4_f32 with scale 1.0 converts to E2M1, nearest even,
//    sign copied, and saturates every value past +-6 (infinities included) to
//    the signed top code, which is the nearest-even result there; the first
//    operand goes to the low nibble.

// Four binary32 values within +-448 (the quotients of div_rn_sat) -> four
// E4M3FN codes, element i in byte i.
__device__ __forceinline__ uint32_t e4m3x4_in_range(float a, float b, float c, float d) {
  // the first conversion's untouched upper half is overwritten by the second;
  // `a` (dead after it) fills it, so no register has to be zeroed first
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)__float_as_uint(a), false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
}

// One non-negative binary32 value -> its E4M3FN code.
__device__ __forceinline__ uint32_t e4m3_pos(float a) {
  a = __builtin_amdgcn_fmed3f(a, 448.0f, -448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, 0.0f, 0, false) & 0xFFu;
}

// Value of a non-negative E4M3FN code (the NVFP4 block scale), exact:
// E >= 1: 2^(E-7) (1 + M/8); E = 0: M 2^-9.
__device__ __forceinline__ float e4m3_value_pos(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// Eight binary32 values -> eight E2M1 codes, element i in bits 4i..4i+3. The
// converter's own saturation covers the infinities a block's n * mult can
// reach, so no clamp precedes it.
__device__ __forceinline__ uint32_t e2m1x8(const float (&v)[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// ---------------------------------------------------------------- division


// 1 / b rounded once, for a normal b < 2^126: the hardware reciprocal estimate
// y and one residual correction, y + y (1 - b y), the residual exact in one
// FMA. An exhaustive GPU check over every normal binary32 b below 2^120 gave
// the IEEE quotient bit for bit. From 2^126 up the quotient is subnormal and
// the estimate flushes it to zero, so callers stay below that.
__device__ __forceinline__ float recip_rn(float d) {
  const float y = __builtin_amdgcn_rcpf(d);
  const float e = __builtin_fmaf(-d, y, 1.0f);
  return __builtin_fmaf(e, y, y);
}

// recip_rn extended to d = +0 and d = +inf (r = 1 / sqrt(mean + eps) with eps = 0
// or an overflowing mean): there the correction is NaN, and the estimate alone
// is already the IEEE result (+inf, +0).
__device__ __forceinline__ float recip_rn_ext(float d) {
  const float y = __builtin_amdgcn_rcpf(d);
  const float y1 = __builtin_fmaf(__builtin_fmaf(-d, y, 1.0f), y, y);
  return __builtin_isfinite(y1) ? y1 : y;
}

// amax / 6 rounded once, for amax >= +0 (the NVFP4 block scale's quotient):
// q0 = RN(amax RN(1/6)), the remainder amax - 6 q0 exact in one FMA, and
// q0 + rem RN(1/6) rounded once (Markstein's correction). An exhaustive GPU
// check over every non-negative binary32 found it exact for amax >= 2^-125 and
// an ulp off for some smaller amax, where the quotient is subnormal; a large G
// (>= 2^120 in the same check) carries that ulp into the scale code. Those
// blocks, whose every |n| is below 2^-125, take a branch: amax = k 2^-149 with
// k < 2^24 is scaled by 2^48 (exact), divided in the normal range and scaled
// back. k/6 has at most 22 integer bits, so the first rounding keeps at least
// two fraction bits; a fraction of 1/6, 1/3, 2/3 or 5/6 then cannot round
// across one half, and a half stays exact, so the second rounding gives
// RN(amax / 6). amax = +inf makes the correction NaN; q0 = inf stands and the
// code saturates.
__device__ __forceinline__ float amax_div6(float am) {
  constexpr float kInv6 = 0x1.555556p-3f;  // RN(1/6)
  const float q0 = am * kInv6;
  float q = q0 < __builtin_inff() ? __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, am), kInv6, q0) : q0;
  if (__float_as_uint(am) - 1u < 0x00FFFFFFu) {  // 0 < amax < 2^-125
    asm volatile("");  // keeps this a branch: it is almost never taken
    const float a = am * 0x1p48f;
    const float p0 = a * kInv6;
    q = __builtin_fmaf(__builtin_fmaf(-p0, 6.0f, a), kInv6, p0) * 0x1p-48f;
  }
  return q;
}

// a / b rounded once, for an E4M3 code decision, from y = RN(1/b): q0 = RN(a y)
// is within an ulp of a/b, the remainder a - b q0 is exact in one FMA, and
// q0 + rem y rounded once is RN(a/b) while the quotient is normal (Markstein's
// correction). a is first clamped to +-c with c = the largest binary32
// <= 448 b (sat_bound), so the quotient is at most 448 in magnitude (the
// converter needs no clamp of its own) and a clamped quotient lies in
// [432, 448], which has the saturated code 448 that every |a / b| >= 448 has.
// The residual is negated after the FMA (-(q0 b - a) = a - q0 b, exact), which
// keeps the sign of a zero quotient without a copysign. 4 operations. Requires 448 b finite. Checked exhaustively at the
// code level: for every binary32 a (subnormal quotients included) and 13
// scales from 2^-126 to 2^119, the E4M3 code equals that of the IEEE quotient.
__device__ __forceinline__ float sat_bound(float b) {
  float c = 448.0f * b;                                        // RN(448 b)
  if (__builtin_fmaf(-448.0f, b, c) > 0.0f) c = __uint_as_float(__float_as_uint(c) - 1u);
  return c;                                                    // the largest binary32 <= 448 b
}
__device__ __forceinline__ float div_rn_sat(float a, float b, float y, float c) {
  const float ac = __builtin_amdgcn_fmed3f(a, c, -c);
  const float q0 = ac * y;
  const float t = __builtin_fmaf(q0, b, -ac);
  return __builtin_fmaf(-t, y, q0);
}

// ------------------------------------------------------ cross-lane sums

// DPP lane moves inside a 16-lane row (VALU, no LDS round trip):
//   0xB1 quad_perm [1,0,3,2] (lane ^ 1), 0x4E quad_perm [2,3,0,1] (lane ^ 2),
//   0x141 row_half_mirror (lane i <-> 7 - i within 8), 0x140 row_mirror (i <-> 15 - i).
// Every lane has a valid source under these patterns and all lanes are active
// where they are used, so no "old" value is needed (bound_ctrl set): the move
// needs no register seeded beforehand.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  static_assert(CTRL == 0xB1 || CTRL == 0x4E || CTRL == 0x141 || CTRL == 0x140,
                "only patterns with a source lane for every lane");
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = dpp_u32<CTRL>((uint32_t)b), hi = dpp_u32<CTRL>((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, (hi << 32) | lo);
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __builtin_bit_cast(double, (hi << 32) | lo);
}

// Sum over aligned groups of W lanes (W a power of two, 2..64). Every lane of a
// group ends with the same bits: each step adds a value and its partner's, and
// IEEE addition commutes; groups of 32 and 64 combine their 16-lane rows read
// with readlane in one fixed order. A group's lanes must all be active.
template <int W>
__device__ __forceinline__ double lanes_sum(double v) {
  if constexpr (W >= 2) v += dpp_f64<0xB1>(v);
  if constexpr (W >= 4) v += dpp_f64<0x4E>(v);
  if constexpr (W >= 8) v += dpp_f64<0x141>(v);
  if constexpr (W >= 16) v += dpp_f64<0x140>(v);
  if constexpr (W == 32) {
    const double lo = readlane_f64(v, 0) + readlane_f64(v, 16);
    const double hi = readlane_f64(v, 32) + readlane_f64(v, 48);
    v = (__lane_id() < 32) ? lo : hi;
  } else if constexpr (W == 64) {
    v = (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
  }
  return v;
}

// ------------------------------------------------- exact sum of squares

// a + b = s + e exactly (Knuth's TwoSum; no contraction allowed).
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

__device__ __forceinline__ void dd_add(double& hi, double& lo, double bh, double bl) {
  double s, e;
  two_sum(hi, bh, s, e);
  e += lo + bl;
  hi = s + e;
  lo = e - (hi - s);
}

// Double-double sum over aligned groups of W lanes, same pattern as lanes_sum.
template <int CTRL>
__device__ __forceinline__ void dd_step(double& hi, double& lo) {
  const double oh = dpp_f64<CTRL>(hi), ol = dpp_f64<CTRL>(lo);
  dd_add(hi, lo, oh, ol);
}
template <int W>
__device__ __forceinline__ void lanes_sum_dd(double& hi, double& lo) {
  if constexpr (W >= 2) dd_step<0xB1>(hi, lo);
  if constexpr (W >= 4) dd_step<0x4E>(hi, lo);
  if constexpr (W >= 8) dd_step<0x141>(hi, lo);
  if constexpr (W >= 16) dd_step<0x140>(hi, lo);
  if constexpr (W >= 32) {
    double r[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      r[q][0] = readlane_f64(hi, 16 * q);
      r[q][1] = readlane_f64(lo, 16 * q);
    }
    double h0 = r[0][0], l0 = r[0][1], h1 = r[2][0], l1 = r[2][1];
    dd_add(h0, l0, r[1][0], r[1][1]);
    dd_add(h1, l1, r[3][0], r[3][1]);
    if constexpr (W == 64) {
      dd_add(h0, l0, h1, l1);
      hi = h0;
      lo = l0;
    } else {
      const bool low = __lane_id() < 32;
      hi = low ? h0 : h1;
      lo = low ? l0 : l1;
    }
  }
}

__device__ __forceinline__ float f32_next_up(float f) {
  return __uint_as_float(__float_as_uint(f) + 1u);  // f >= 0 and finite here
}
__device__ __forceinline__ float f32_next_down(float f) {
  return f > 0.0f ? __uint_as_float(__float_as_uint(f) - 1u) : 0.0f;
}

// The binary32 rounding of the exact sum is in doubt when S (>= 0, the
// float64 sum of `width` exact squares, within width * 2^-53 * S of it) lies
// within that bound of a midpoint between two binary32 values. In S's binade
// the bound is below 2 * width float64 ulps, and a binary32 midpoint is a
// float64 whose low 29 significand bits are 2^28 (midpoints of other binades
// are at least 2^27 ulps away); so the test is on those bits alone. Nonzero S
// below the binary32 normal range is always settled exactly; S = 0 is exact.
__device__ __forceinline__ bool near_f32_midpoint(double S, int32_t width) {
  if (!(S >= 0x1p-126)) return S != 0.0;
  const uint32_t low29 = (uint32_t)__builtin_bit_cast(uint64_t, S) & 0x1FFFFFFFu;
  const uint32_t w2 = 2u * (uint32_t)width;
  return low29 - (0x10000000u - w2) <= 2u * w2;
}

// Round hi + lo (a double-double with |lo| <= ulp(hi)/2) to binary32, nearest
// even. Only when hi is itself a binary32 midpoint can lo change the result,
// and then its sign picks the side (lo == 0: an exact tie, keep the even one).
__device__ __forceinline__ float dd_to_f32(double hi, double lo) {
  const float f = (float)hi;
  const double fd = (double)f;
  if (fd == hi) return f;
  const float flo = fd < hi ? f : f32_next_down(f);
  const float fhi = fd < hi ? f32_next_up(f) : f;
  const double mid = 0.5 * ((double)flo + (double)fhi);
  if (hi != mid) return f;
  return lo > 0.0 ? fhi : (lo < 0.0 ? flo : f);
}

// ------------------------------------------------------------- epilogues
// Shared by the fused tail and the standalone quantisers, so both encode with
// the same instructions.

// FP8: codes of n_i / s for eight values (s = dequant scale, inv_s = RN(1/s)).
__device__ __forceinline__ void fp8_codes8(const float (&n)[8], float s, float inv_s, uint32_t& lo,
                                           uint32_t& hi) {
  float t[8];
  const float c = sat_bound(s);
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = div_rn_sat(n[i], s, inv_s, c);
  lo = e4m3x4_in_range(t[0], t[1], t[2], t[3]);
  hi = e4m3x4_in_range(t[4], t[5], t[6], t[7]);
}

// NVFP4 multipliers G / value(c) for the 127 non-negative E4M3 codes (0 for c = 0
// and the unused slot 127), filled by the workgroup; IEEE divisions.
__device__ __forceinline__ void fill_mult_tab(float* tab, float G) {
  for (int c = threadIdx.x; c < 128; c += blockDim.x) {
    const float S = c < 127 ? e4m3_value_pos((uint32_t)c) : 0.0f;
    tab[c] = S > 0.0f ? G / S : 0.0f;
  }
}

// NVFP4: one lane holds one half (8 values) of a 16-element block, its partner
// (lane ^ 1) the other half. Returns the lane's eight E2M1 codes packed low
// nibble first, and the block's E4M3 scale code (the same in both lanes).
__device__ __forceinline__ void nvfp4_half_block(const float (&n)[8], float G, const float* mult_tab,
                                                 uint32_t& codes, uint32_t& sfc) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(n[i]));
  // the other half's amax; both are non-negative (fmaxf drops NaN), and such
  // binary32 values order as their bit patterns
  const uint32_t ab = __float_as_uint(am);
  am = __uint_as_float(max(ab, dpp_u32<0xB1>(ab)));
  sfc = e4m3_pos(G * amax_div6(am));
  const float mult = mult_tab[sfc & 0x7Fu];  // in the table whatever the input (NaN gives 0x7F)
  float t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = n[i] * mult;
  codes = e2m1x8(t);
}

// ------------------------------------------------------------ SiLU gate

// 2^(j/64) for j < 64, each rounded to the nearest binary64: the table of the
// gate's exp. Each workgroup copies it into LDS.
__device__ const double kExp2Tab[64] = {
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0,
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0,
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0,
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0,
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0,
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0,
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0,
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0,
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0,
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0,
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0,
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0,
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0,
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0,
};

__device__ __forceinline__ void fill_exp2_tab(double* tab) {
  for (int j = threadIdx.x; j < 64; j += blockDim.x) tab[j] = kExp2Tab[j];
}

// exp(-z) rounded once to binary32, for binary32 z. Table-driven in binary64:
// -z = (n / 64) ln 2 + r with n = rint(-z 64 / ln 2) and a two-part ln 2 / 64
// (its high part has 37 bits, so n * high is exact for |n| < 2^15), |r| <= ln 2 / 128;
// exp(-z) = 2^(n >> 6) * 2^((n & 63) / 64) * p(r), p the degree-5 Taylor
// polynomial (truncation below 2^-54 relative). The binary64 value is within
// about 2^-50 of exp(-z), far inside a binary32 rounding step; that the one
// final rounding then lands where exp(-z) itself would is checked over every
// fp16 and bf16 z. |z| >= 200 is clamped: exp(-+200) already round to 0 / inf.
__device__ __forceinline__ float exp_neg_rn(float z, const double* exp2_tab) {
  const double zc = (double)__builtin_amdgcn_fmed3f(z, 200.0f, -200.0f);
  const double n = __builtin_rint(-zc * 0x1.71547652b82fep+6);  // -z * 64 / ln 2
  double r = __builtin_fma(-n, 0x1.62e42fefa0000p-7, -zc);       // exact
  r = __builtin_fma(-n, 0x1.cf79abc9e3b3ap-46, r);
  double p = __builtin_fma(0x1.1111111111111p-7, r, 0x1.5555555555555p-5);
  p = __builtin_fma(p, r, 0x1.5555555555555p-3);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p = __builtin_fma(p, r, 1.0);
  const int ni = (int)n;
  return (float)__builtin_ldexp(exp2_tab[ni & 63] * p, ni >> 6);
}

// The gate's sigma = 1 / d uses recip_rn for d < 2^126 and binary64 division
// (recip_big) above, where the estimate would flush the subnormal quotient.
constexpr float kRecipBig = 0x1p126f;
__device__ __forceinline__ float recip_big(float d) { return (float)(1.0 / (double)d); }

// The SiLU gate applied to x, in binary32 steps: E = exp(-z) rounded once,
// d = 1 + E, sigma = 1 / d rounded once, s = z * sigma, u = x * s.
__device__ __forceinline__ float silu_gate(float x, float z, const double* exp2_tab) {
  const float d = 1.0f + exp_neg_rn(z, exp2_tab);
  const float sigma = d >= kRecipBig ? recip_big(d) : recip_rn(d);
  return x * (z * sigma);
}

// Eight gates at once: the common path is branch-free so the eight exp
// chains interleave; one branch per vector (never taken unless some z is
// below about -87.3) redoes the reciprocals of d >= 2^126.
__device__ __forceinline__ void silu_gate8(const float (&x)[8], const float (&z)[8],
                                           const double* exp2_tab, float (&u)[8]) {
  float d[8], sigma[8];
  bool big = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    d[i] = 1.0f + exp_neg_rn(z[i], exp2_tab);
    sigma[i] = recip_rn(d[i]);
    big |= d[i] >= kRecipBig;
  }
  if (big) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (d[i] >= kRecipBig) sigma[i] = recip_big(d[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = x[i] * (z[i] * sigma[i]);
}

// ------------------------------------------------ bf16 gate lookup table
//
// For bf16 z the gate value s(z) = z * sigma(z) (the silu_gate steps with x = 1)
// depends on z's 16 bits only. With |z| < 2^-25, exp(-z) rounds to 1, so
// s = z / 2; with |z| >= 128 it rounds to 0 (z > 0, s = z) or overflows
// (z < 0, s = -0). Between, there are 32 binades x 128 significands per sign:
// an 8192-entry binary32 table, index (bf16 bits & 0x7FFF) - (102 << 7) plus
// 4096 for negative z. The library holds it as constants (anq_gate_table.h,
// written by gen_gate_table.py from the same binary32 steps; a CPU test pins
// every entry to the oracle's gate and the GPU tests run every in-range z
// through it); each workgroup copies it into LDS. Values outside the table
// take the computed path.
constexpr int kGateTab = 8192;
constexpr uint32_t kGateTabLo = 102u << 7;  // bf16 exponent field 102: 2^-25

// u_i = x_i * s(z_i) for the eight bf16 z of zv (the silu_gate8 result).
// With b a bf16 pattern and t = b - (102 << 7) (32-bit, wrapping below the
// table), b is in the table iff bits 12..14 of t are clear: positive z in
// range give t < 4096, negative ones 0x8000 <= t < 0x9000, and every other b
// sets one of those bits. The entry is (t & 4095) | (b's sign at bit 12), one
// bitfield insert of b >> 3 (b has 16 bits, so b >> 3 has nothing above bit
// 12); every index is below kGateTab whatever b is.
__device__ __forceinline__ void gate_lut8(const float (&x)[8], const U4& zv, const float* tab,
                                          const double* exp2_tab, float (&u)[8]) {
  float s[8];
  uint32_t any = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = zv.w[i >> 1];
    const uint32_t b = (i & 1) ? (w >> 16) : (w & 0xFFFFu);
    const uint32_t t = b - kGateTabLo;
    any |= t;
    s[i] = tab[(t & 4095u) | ((b >> 3) & ~4095u)];
  }
  if (any & 0x7000u) {  // rare for activations: |z| < 2^-25 or |z| >= 128 somewhere in the vector
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = (i & 1) ? (zv.w[i >> 1] >> 16) : (zv.w[i >> 1] & 0xFFFFu);
      if ((b & 0x7FFFu) - kGateTabLo >= 4096u) s[i] = silu_gate(1.0f, __uint_as_float(b << 16), exp2_tab);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = x[i] * s[i];
}

// Byte offset of the block scale of row r, block column c in the 128x4-tiled
// scale layout of block-scaled GEMM operands: rows padded to 128, scale
// columns to 4; tile (r / 128, c / 4) is 512 contiguous bytes, tiles row-major
// with `tiles_c` tiles per tile row; inside a tile, (r % 32, (r / 32) % 4, c % 4)
// with strides 16, 4, 1. The four columns of a tile row are one 4-byte word.
__device__ __forceinline__ size_t sf_swizzled_offset(int64_t r, int32_t c, int32_t tiles_c) {
  return ((size_t)(r >> 7) * (size_t)tiles_c + (size_t)(c >> 2)) * 512u + (size_t)(r & 31) * 16u +
         (size_t)((r >> 5) & 3) * 4u + (size_t)(c & 3);
}

// Store the block scale of (row, c) in the swizzled layout. The owner of a
// row's last block also zeroes the (at most 3) padding columns of that row's
// last tile.
__device__ __forceinline__ void store_block_scale_swizzled(uint8_t* sf, int64_t row, int32_t c,
                                                           int32_t nblk, int32_t tiles_c,
                                                           uint8_t code) {
  const size_t o = sf_swizzled_offset(row, c, tiles_c);
  sf[o] = code;
  if (c == nblk - 1) {
    for (int32_t z = c + 1; z < tiles_c * 4; ++z) sf[o + (size_t)(z - c)] = 0;
  }
}

// Zero the scale words of padded rows [tokens, roundup(tokens, 128)) in the
// swizzled layout: the caller's `worker` of `workers` takes rows tokens + worker,
// tokens + worker + workers, ...; `lane` of `lanes` takes tile columns.
__device__ __forceinline__ void zero_padded_scale_rows(uint8_t* sf, int64_t tokens, int32_t tiles_c,
                                                       int64_t worker, int64_t workers, int lane,
                                                       int lanes) {
  const int64_t rows_pad = (tokens + 127) & ~(int64_t)127;
  for (int64_t r = tokens + worker; r < rows_pad; r += workers)
    for (int32_t t = lane; t < tiles_c; t += lanes)
      *reinterpret_cast<uint32_t*>(sf + sf_swizzled_offset(r, 4 * t, tiles_c)) = 0u;
}

}  // namespace anq
