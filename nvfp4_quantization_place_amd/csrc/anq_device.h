// Device building blocks of the fused tail kernels (gfx950 / CDNA4).
//
// Every helper here is exact or correctly rounded: the kernels must reproduce
// the binary32 definition of the op bit for bit, so nothing is approximated
// and nothing is contracted (the library is built with -ffp-contract=off; the
// only fused multiply-adds are the explicit ones below, where they are exact
// or part of a proven correction step).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace anq {

constexpr int kF16 = 0;
constexpr int kBF16 = 1;

// 8 activations = 16 bytes, the unit of every global load and store.
struct alignas(16) U4 {
  uint32_t w[4];
};

__device__ __forceinline__ U4 ld16(const void* p) {
  return *reinterpret_cast<const U4*>(p);
}
__device__ __forceinline__ void st16(void* p, const U4& v) {
  *reinterpret_cast<U4*>(p) = v;
}

// A pointer known to be the same in every lane, moved to scalar registers so
// that loads and stores address it as SGPR base + 32-bit lane offset.
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
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
//    subnormals kept; it returns NaN beyond +-448, so inputs are first clamped
//    with v_med3_f32 (saturation to +-448 is the nearest-even result there).
//  * v_cvt_scalef32_pk_fp4_f32 with scale 1.0 converts to E2M1, nearest even,
//    saturating at +-6, sign copied; the first operand goes to the low nibble.

// Four binary32 values -> four E4M3FN codes, element i in byte i.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, 448.0f, -448.0f);
  b = __builtin_amdgcn_fmed3f(b, 448.0f, -448.0f);
  c = __builtin_amdgcn_fmed3f(c, 448.0f, -448.0f);
  d = __builtin_amdgcn_fmed3f(d, 448.0f, -448.0f);
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
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

// Eight binary32 values -> eight E2M1 codes, element i in bits 4i..4i+3.
__device__ __forceinline__ uint32_t e2m1x8(const float (&v)[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// ---------------------------------------------------------------- division

// Correctly rounded a / b from y = RN(1/b): q0 = RN(a*y) is within an ulp of
// a/b, the remainder a - b*q0 is exact in one FMA, and q0 + rem*y rounded once
// is RN(a/b) (Markstein's correction theorem; no underflow in this use). The
// sign of q0 is carried over so that a = -0 keeps its sign like IEEE division.
__device__ __forceinline__ float div_rn(float a, float b, float y) {
  const float q0 = a * y;
  const float rem = __builtin_fmaf(-q0, b, a);
  const float q1 = __builtin_fmaf(rem, y, q0);
  return __builtin_copysignf(q1, q0);
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

__device__ __forceinline__ float f32_next_up(float f) {
  return __uint_as_float(__float_as_uint(f) + 1u);  // f >= 0 and finite here
}
__device__ __forceinline__ float f32_next_down(float f) {
  return f > 0.0f ? __uint_as_float(__float_as_uint(f) - 1u) : 0.0f;
}

// The binary32 rounding of S (>= 0, a float64 sum of exact squares) is in
// doubt when S lies within `bound` of a midpoint between two binary32 values.
__device__ __forceinline__ bool near_f32_midpoint(double S, float f, double bound) {
  const double fd = (double)f;
  const double mid_hi = 0.5 * (fd + (double)f32_next_up(f));
  const double mid_lo = 0.5 * (fd + (double)f32_next_down(f));
  return __builtin_fabs(S - mid_hi) <= bound || (f > 0.0f && __builtin_fabs(S - mid_lo) <= bound);
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

}  // namespace anq
