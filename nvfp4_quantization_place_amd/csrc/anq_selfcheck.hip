// Self-check of the device arithmetic behind the kernels' exact results.
//
// The kernels replace four IEEE operations by cheaper forms whose exactness
// rests on properties of the gfx950 instructions (the reciprocal estimate's
// accuracy, the conversion instructions' saturation). This kernel compares each
// replacement with the operation it stands for over every input in its domain
// (for the FP8 quotient, every binary32 numerator at a set of scales), using
// the same device helpers the kernels use, on the GPU at hand.
#include "anq_device.h"
#include "anq_internal.h"

namespace anq {

namespace {

constexpr uint32_t kSignificands = 1u << 23;

__global__ void zero_counts(unsigned long long* counts) {
  if (threadIdx.x < kSelfcheckCounts) counts[threadIdx.x] = 0ull;
}

// E4M3 code of an IEEE quotient: saturation to +-448 is the nearest-even
// result past the top code, and the converter needs its input within range.
__device__ __forceinline__ uint32_t e4m3_code_sat(float q) {
  q = __builtin_amdgcn_fmed3f(q, 448.0f, -448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false) & 0xFFu;
}

// Thread m takes significand m (grid: exactly 2^23 threads) and walks the
// exponents (and signs) each check needs.
__global__ void __launch_bounds__(256) selfcheck_kernel(unsigned long long* counts) {
  const uint32_t m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= kSignificands) return;
  uint32_t bad[kSelfcheckCounts] = {0, 0, 0, 0};

  // 0: recip_rn against 1 / b for every normal b below 2^120 (biased exponent <= 246)
  for (uint32_t e = 1; e <= 246; ++e) {
    const float b = __uint_as_float((e << 23) | m);
    bad[0] += __float_as_uint(recip_rn(b)) != __float_as_uint(1.0f / b);
  }
  if (m == 0) {
    bad[0] += __float_as_uint(recip_rn_ext(0.0f)) != __float_as_uint(__builtin_inff());
    bad[0] += __float_as_uint(recip_rn_ext(__builtin_inff())) != 0u;
  }

  // 1: amax_div6 against amax / 6 for every non-negative binary32 (+inf included)
  for (uint32_t e = 0; e <= 255; ++e) {
    if (e == 255 && m != 0) break;  // NaN patterns
    const float a = __uint_as_float((e << 23) | m);
    bad[1] += __float_as_uint(amax_div6(a)) != __float_as_uint(a / 6.0f);
  }

  // 2: the FP8 code of div_rn_sat(a, s) against that of the IEEE a / s, every
  // binary32 a (both signs, infinities included), seven scales
  const float scales[7] = {0x1p-126f, 0.01f, 0.05f, 1.0f, 3.0f, 1e5f, 0x1p119f};
#pragma unroll 1
  for (int k = 0; k < 7; ++k) {
    const float s = scales[k], y = recip_rn(s), c = sat_bound(s);
    for (uint32_t sg = 0; sg < 2; ++sg)
      for (uint32_t e = 0; e <= 255; ++e) {
        if (e == 255 && m != 0) break;
        const float a = __uint_as_float((sg << 31) | (e << 23) | m);
        const uint32_t got = e4m3x4_in_range(div_rn_sat(a, s, y, c), 0.0f, 0.0f, 0.0f) & 0xFFu;
        bad[2] += got != e4m3_code_sat(a / s);
      }
  }

  // 3: e2m1x8 saturates every binary32 at or past +-6 (infinities included) to
  // the signed top code
  for (uint32_t sg = 0; sg < 2; ++sg)
    for (uint32_t e = 129; e <= 255; ++e) {
      if (e == 255 && m != 0) break;
      const float a = __uint_as_float((sg << 31) | (e << 23) | m);
      if (__builtin_fabsf(a) < 6.0f) continue;
      const float v[8] = {a, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      bad[3] += (e2m1x8(v) & 0xFu) != (sg ? 0xFu : 0x7u);
    }

#pragma unroll
  for (int i = 0; i < kSelfcheckCounts; ++i)
    if (bad[i]) atomicAdd(&counts[i], (unsigned long long)bad[i]);
}

}  // namespace

int launch_selfcheck(unsigned long long* counts, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(zero_counts, dim3(1), dim3(64), 0, s, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return (int)err;
  hipLaunchKernelGGL(selfcheck_kernel, dim3(kSignificands / 256), dim3(256), 0, s, counts);
  return (int)hipGetLastError();
}

}  // namespace anq
