// Q/K per-head RMSNorm + NeoX RoPE + uniform FP8 E4M3 store of a fused QKV
// buffer (SGLang PR #32975 "fused norm + RoPE + uniform fp8 store"; the Q/K
// RMSNorm and RoPE of TensorRT-LLM PR #17288, Description).
//
// gfx950 mapping: a (token, head) pair is one unit of work for D/16 lanes of a
// wavefront. Lane j holds elements [8j, 8j+8) of the first half of the head and
// [D/2 + 8j, D/2 + 8j + 8) of the second half, so every NeoX rotation pair
// (k, k + D/2) lives in one lane and each lane issues two 16-byte loads and
// two 8-byte stores. The head's sum of squares meets through a DPP butterfly
// over the D/16 lanes. cos|sin rows are read per (token, head) and come from
// cache after the first head of a token.
#include <stdlib.h>

#include "anq_device.h"
#include "anq_internal.h"

namespace anq {

template <int DT, int LPH, bool NT>
__global__ void __launch_bounds__(256) qk_kernel(QKParams p) {
  constexpr int D = LPH * 16;
  constexpr int HALF = D / 2;
  const int lane = threadIdx.x & (LPH - 1);
  const int gpb = blockDim.x / LPH;
  const int heads = p.nq + p.nk + p.nv;
  const int qk_heads = p.nq + p.nk;
  const float sc = *p.scale;
  const float inv_sc = 1.0f / sc;
  const uint8_t* qkv = static_cast<const uint8_t*>(p.qkv);

  for (int64_t pair = (int64_t)blockIdx.x * gpb + threadIdx.x / LPH; pair < p.pairs;
       pair += (int64_t)gridDim.x * gpb) {
    const int64_t t = pair / heads;
    const int hd = (int)(pair - t * heads);
    const size_t e0 = (size_t)t * heads * D + (size_t)hd * D;  // first element of the head
    const size_t ea = e0 + 8 * lane, eb = e0 + HALF + 8 * lane;
    float a[8], b[8], oa[8], ob[8];
    unpack8<DT>(ld16s<NT>(qkv + ea * 2), a);
    unpack8<DT>(ld16s<NT>(qkv + eb * 2), b);
    if (hd < qk_heads) {  // uniform over the head's lanes
      const uint8_t* gp = static_cast<const uint8_t*>(hd < p.nq ? p.gamma_q : p.gamma_k);
      float ga[8], gb[8];
      unpack8<DT>(ld16(gp + (size_t)(8 * lane) * 2), ga);
      unpack8<DT>(ld16(gp + (size_t)(HALF + 8 * lane) * 2), gb);
      double acc = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc = __builtin_fma((double)a[i], (double)a[i], acc);
        acc = __builtin_fma((double)b[i], (double)b[i], acc);
      }
      const double S = lanes_sum<LPH>(acc);
      float ss = (float)S;
      if (near_f32_midpoint(S, ss, S * (double)D * 0x1p-52)) {
        double hi = 0.0, lo = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dd_add(hi, lo, (double)a[i] * (double)a[i], 0.0);
          dd_add(hi, lo, (double)b[i] * (double)b[i], 0.0);
        }
        lanes_sum_dd<LPH>(hi, lo);
        ss = dd_to_f32(hi, lo);
      }
      const float r = 1.0f / sqrtf(ss / (float)D + p.eps);
      const int64_t pos = p.positions[t];
      const float* cs = p.cos_sin + (size_t)pos * D;
      const float4 c0 = *reinterpret_cast<const float4*>(cs + 8 * lane);
      const float4 c1 = *reinterpret_cast<const float4*>(cs + 8 * lane + 4);
      const float4 s0 = *reinterpret_cast<const float4*>(cs + HALF + 8 * lane);
      const float4 s1 = *reinterpret_cast<const float4*>(cs + HALF + 8 * lane + 4);
      const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float na = (a[i] * r) * ga[i];
        const float nb = (b[i] * r) * gb[i];
        oa[i] = (na * c[i]) - (nb * s[i]);
        ob[i] = (nb * c[i]) + (na * s[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        oa[i] = a[i];
        ob[i] = b[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      oa[i] = div_rn(oa[i], sc, inv_sc);
      ob[i] = div_rn(ob[i], sc, inv_sc);
    }
    st8s<NT>(p.out + ea, e4m3x4(oa[0], oa[1], oa[2], oa[3]), e4m3x4(oa[4], oa[5], oa[6], oa[7]));
    st8s<NT>(p.out + eb, e4m3x4(ob[0], ob[1], ob[2], ob[3]), e4m3x4(ob[4], ob[5], ob[6], ob[7]));
  }
}

template <int DT, bool NT>
static hipError_t launch_qk_nt(const QKParams& p, hipStream_t s) {
  void* args[] = {const_cast<QKParams*>(&p)};
  const void* fn = nullptr;
  const int lph = p.head_dim / 16;
  switch (lph) {
    case 2: fn = (const void*)&qk_kernel<DT, 2, NT>; break;
    case 4: fn = (const void*)&qk_kernel<DT, 4, NT>; break;
    case 8: fn = (const void*)&qk_kernel<DT, 8, NT>; break;
    case 16: fn = (const void*)&qk_kernel<DT, 16, NT>; break;
    case 32: fn = (const void*)&qk_kernel<DT, 32, NT>; break;
    default: return hipErrorInvalidConfiguration;
  }
  const int block = 256;
  const int64_t gpb = block / lph;
  int64_t grid = (p.pairs + gpb - 1) / gpb;
  if (grid > (1 << 22)) grid = 1 << 22;
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(block), args, 0, s);
}

// Streaming hints (see ld16s) once qkv alone is >= 32 MiB; ANQ_STREAM=0/1 overrides.
template <int DT>
static hipError_t launch_qk_dt(const QKParams& p, hipStream_t s) {
  bool stream = p.pairs * (int64_t)p.head_dim * 2 >= ((int64_t)32 << 20);
  if (const char* e = getenv("ANQ_STREAM")) {
    if (*e) stream = atoi(e) != 0;
  }
  return stream ? launch_qk_nt<DT, true>(p, s) : launch_qk_nt<DT, false>(p, s);
}

hipError_t launch_qk(int dtype, const QKParams& p, hipStream_t s) {
  return dtype == kBF16 ? launch_qk_dt<kBF16>(p, s) : launch_qk_dt<kF16>(p, s);
}

}  // namespace anq
