// Fused residual add + RMSNorm + FP8 / NVFP4 epilogue, one HBM pass per row.
//
// Operation: the local tail of a transformer layer as the pages define it
// (TensorRT-LLM issue #17900 "Fuse local NVFP4 tail after NCCL fallback",
// Proposal: residual + RMSNorm + NVFP4 in one launch, with or without the norm
// output; TensorRT-LLM PR #17288, Description: RMSNorm with FP8 quantisation
// in the epilogue, in-place residual add).
//
// gfx950 mapping:
//  * A row is split into 16-byte vectors of 8 activations; lane l of the row's
//    lane group owns vectors l, l + L, l + 2L, ... (L lanes per row), so each
//    load/store instruction of a wavefront touches 1 KiB of contiguous bytes.
//  * The row stays in registers between the add and the epilogue: x and
//    residual are read once, residual / norm_out / codes written once.
//  * Small rows (<= 1024 elements) use 16, 32 or 64 lanes of one wavefront per
//    row and reduce with cross-lane shuffles; larger rows use one workgroup of
//    up to 1024 lanes per row and combine wavefront partials through LDS in a
//    fixed order.
//  * The sum of squares is accumulated in float64 (squares of fp16/bf16 values
//    are exact there) and rounded once to binary32. When that float64 total is
//    within its error bound of a binary32 rounding midpoint, the row is summed
//    again as a double-double, which settles the rounding of the exact sum.
//  * NVFP4: a 16-element block is two adjacent vectors held by lanes 2j and
//    2j+1; their amax meet through one lane swap.
#include <type_traits>

#include "anq_device.h"
#include "anq_internal.h"

namespace anq {

// ---------------------------------------------------------------- reducers

// G lanes of one wavefront, G in {16, 32, 64}: xor butterfly. Every lane ends
// with the same bits (IEEE addition commutes, and each step pairs the same
// partial sums in every lane).
template <int G>
struct GroupReduce {
  __device__ __forceinline__ double sum(double v) const {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
  }
  __device__ __forceinline__ void sum_dd(double& hi, double& lo) const {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) {
      const double oh = __shfl_xor(hi, m, 64);
      const double ol = __shfl_xor(lo, m, 64);
      dd_add(hi, lo, oh, ol);
    }
  }
};

// One row per workgroup: wavefront butterflies, then every lane adds the
// wavefront partials from LDS in wavefront order.
struct BlockReduce {
  double* lds;  // >= 2 * 16 doubles
  __device__ __forceinline__ double sum(double v) const {
    v = GroupReduce<64>().sum(v);
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[w] = v;
    __syncthreads();
    double s = 0.0;
    for (int i = 0; i < nw; ++i) s += lds[i];
    __syncthreads();
    return s;
  }
  __device__ __forceinline__ void sum_dd(double& hi, double& lo) const {
    GroupReduce<64>().sum_dd(hi, lo);
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      lds[2 * w] = hi;
      lds[2 * w + 1] = lo;
    }
    __syncthreads();
    double h = 0.0, l = 0.0;
    for (int i = 0; i < nw; ++i) dd_add(h, l, lds[2 * i], lds[2 * i + 1]);
    __syncthreads();
    hi = h;
    lo = l;
  }
};

// ---------------------------------------------------------------- the kernel

// Rounded-once binary32 sum of squares of the row's h values (see above).
template <int K, class Red>
__device__ __forceinline__ float row_sum_squares(const float (&h)[K][8], double acc,
                                                 int32_t width, const Red& red) {
  const double S = red.sum(acc);
  float ss = (float)S;
  // float64 error of a sum of `width` non-negative terms is below width * 2^-53 * S
  if (near_f32_midpoint(S, ss, S * (double)width * 0x1p-52)) {  // uniform over the row
    double hi = 0.0, lo = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double d = (double)h[k][i];
        dd_add(hi, lo, d * d, 0.0);
      }
    red.sum_dd(hi, lo);
    ss = dd_to_f32(hi, lo);
  }
  return ss;
}

template <int DT, int EPI, bool NORM, int K, int G>
__global__ void __launch_bounds__(1024) tail_kernel(TailParams p) {
  __shared__ double lds[32];
  const int32_t V = p.vec;
  int lane, L;
  int64_t row, step;
  if constexpr (G > 0) {
    lane = threadIdx.x & (G - 1);
    L = G;
    const int rpb = blockDim.x / G;
    row = (int64_t)blockIdx.x * rpb + threadIdx.x / G;
    step = (int64_t)gridDim.x * rpb;
  } else {
    lane = threadIdx.x;
    L = blockDim.x;
    row = blockIdx.x;
    step = gridDim.x;
  }

  const uint8_t* x = static_cast<const uint8_t*>(p.x);
  uint8_t* res = static_cast<uint8_t*>(p.residual);
  const uint8_t* gam = static_cast<const uint8_t*>(p.gamma);
  uint8_t* nout = static_cast<uint8_t*>(p.norm_out);

  float g[K][8];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int v = lane + k * L;
    if (v < V) {
      unpack8<DT>(ld16(gam + (size_t)v * 16), g[k]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) g[k][i] = 0.0f;
    }
  }

  const float sc = *p.scale;   // FP8: s, NVFP4: G
  const float inv_sc = 1.0f / sc;  // RN(1/s), correctly rounded division
  constexpr float kInv6 = 0x1.555556p-3f;  // RN(1/6)

  typename std::conditional<(G > 0), GroupReduce<(G > 0 ? G : 64)>, BlockReduce>::type red;
  if constexpr (G == 0) red.lds = lds;

  for (; row < p.tokens; row += step) {
    const size_t rbase = (size_t)row * (size_t)p.hidden * 2;  // byte offset of the row in T
    U4 xv[K], rv[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int v = lane + k * L;
      if (v < V) {
        xv[k] = ld16(x + rbase + (size_t)v * 16);
        rv[k] = ld16(res + rbase + (size_t)v * 16);
      }
    }
    float h[K][8];
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int v = lane + k * L;
      if (v < V) {
        float xf[8], rf[8], s[8];
        unpack8<DT>(xv[k], xf);
        unpack8<DT>(rv[k], rf);
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] = xf[i] + rf[i];
        const U4 hv = pack8<DT>(s);
        st16(res + rbase + (size_t)v * 16, hv);
        unpack8<DT>(hv, h[k]);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_fma((double)h[k][i], (double)h[k][i], acc);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) h[k][i] = 0.0f;
      }
    }

    const float ss = row_sum_squares<K>(h, acc, p.hidden, red);
    const float r = 1.0f / sqrtf(ss / (float)p.hidden + p.eps);

#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int v = lane + k * L;
      if (v >= V) continue;
      float n[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) n[i] = (h[k][i] * r) * g[k][i];
      if constexpr (NORM) st16(nout + rbase + (size_t)v * 16, pack8<DT>(n));
      if constexpr (EPI == kEpiFp8) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = div_rn(n[i], sc, inv_sc);
        uint2 o;
        o.x = e4m3x4(t[0], t[1], t[2], t[3]);
        o.y = e4m3x4(t[4], t[5], t[6], t[7]);
        *reinterpret_cast<uint2*>(p.q + (size_t)row * p.hidden + (size_t)v * 8) = o;
      } else {
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(n[i]));
        am = fmaxf(am, __shfl_xor(am, 1, 64));  // the other half of the 16-element block
        const float s_b = sc * div_rn(am, 6.0f, kInv6);
        const uint32_t sfc = e4m3_pos(s_b);
        const float S = e4m3_value_pos(sfc);
        const float mult = S > 0.0f ? sc / S : 0.0f;
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = n[i] * mult;
        const uint32_t w = e2m1x8(t);
        *reinterpret_cast<uint32_t*>(p.q + (size_t)row * (p.hidden / 2) + (size_t)v * 4) = w;
        if ((lane & 1) == 0) p.sf[(size_t)row * (p.hidden / 16) + (v >> 1)] = (uint8_t)sfc;
      }
    }
  }
}

// ---------------------------------------------------------------- dispatch

Tiling pick_tail_tiling(int32_t vec, int64_t tokens) {
  Tiling t{};
  const int64_t kMaxGrid = 1 << 22;
  if (vec <= 128) {
    t.group = vec <= 16 ? 16 : (vec <= 32 ? 32 : 64);
    t.vec_per_lane = vec <= 64 ? 1 : 2;
    t.block = 256;
    const int64_t rpb = 256 / t.group;
    t.grid = (tokens + rpb - 1) / rpb;
  } else {
    t.group = 0;
    t.vec_per_lane = vec <= 2048 ? 2 : (vec <= 4096 ? 4 : 8);
    const int lanes = (vec + t.vec_per_lane - 1) / t.vec_per_lane;
    t.block = (lanes + 63) / 64 * 64;
    t.grid = tokens;
  }
  if (t.grid > kMaxGrid) t.grid = kMaxGrid;
  return t;
}

template <int DT, int EPI, bool NORM>
static hipError_t launch3(const TailParams& p, const Tiling& t, hipStream_t s) {
  void* args[] = {const_cast<TailParams*>(&p)};
  const void* fn = nullptr;
  if (t.group == 16) fn = (const void*)&tail_kernel<DT, EPI, NORM, 1, 16>;
  else if (t.group == 32) fn = (const void*)&tail_kernel<DT, EPI, NORM, 1, 32>;
  else if (t.group == 64 && t.vec_per_lane == 1) fn = (const void*)&tail_kernel<DT, EPI, NORM, 1, 64>;
  else if (t.group == 64 && t.vec_per_lane == 2) fn = (const void*)&tail_kernel<DT, EPI, NORM, 2, 64>;
  else if (t.group == 0 && t.vec_per_lane == 1) fn = (const void*)&tail_kernel<DT, EPI, NORM, 1, 0>;
  else if (t.group == 0 && t.vec_per_lane == 2) fn = (const void*)&tail_kernel<DT, EPI, NORM, 2, 0>;
  else if (t.group == 0 && t.vec_per_lane == 4) fn = (const void*)&tail_kernel<DT, EPI, NORM, 4, 0>;
  else if (t.group == 0 && t.vec_per_lane == 8) fn = (const void*)&tail_kernel<DT, EPI, NORM, 8, 0>;
  if (!fn) return hipErrorInvalidConfiguration;
  return hipLaunchKernel(fn, dim3((unsigned)t.grid), dim3((unsigned)t.block), args, 0, s);
}

template <int DT, int EPI>
static hipError_t launch2(bool norm, const TailParams& p, const Tiling& t, hipStream_t s) {
  return norm ? launch3<DT, EPI, true>(p, t, s) : launch3<DT, EPI, false>(p, t, s);
}

template <int DT>
static hipError_t launch1(int epi, bool norm, const TailParams& p, const Tiling& t, hipStream_t s) {
  return epi == kEpiFp8 ? launch2<DT, kEpiFp8>(norm, p, t, s) : launch2<DT, kEpiNvfp4>(norm, p, t, s);
}

hipError_t launch_tail(int dtype, int epi, bool norm, const TailParams& p, const Tiling& t,
                       hipStream_t s) {
  return dtype == kBF16 ? launch1<kBF16>(epi, norm, p, t, s) : launch1<kF16>(epi, norm, p, t, s);
}

}  // namespace anq
