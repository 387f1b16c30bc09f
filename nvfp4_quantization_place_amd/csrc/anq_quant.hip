// Standalone FP8 / NVFP4 quantisation of an activation tensor: the second
// kernel of the separated local tail, which launches a residual/RMSNorm
// kernel and then a quantisation kernel (TensorRT-LLM issue #17900 "Fuse local
// NVFP4 tail after NCCL fallback", Proposal). Together with add_rmsnorm it is
// the baseline the fused kernel is measured against.
//
// gfx950 mapping: one thread per 16-byte vector of 8 activations, one pass over
// the tensor (no grid-stride loop: single-pass stores stream best on MI355X).
// An NVFP4 block of 16 is two vectors in adjacent lanes; rows are multiples of
// 16 elements, so flattening [tokens, hidden] keeps every block inside a row.
// The encoders are the fused kernel's own (fp8_codes8, nvfp4_half_block).
// With the swizzled scale layout (its own instantiation), threads past the
// last vector zero the scale words of the padded rows (one 4-byte word each).
// NT: the streaming hint on the input load and on the code and linear scale
// stores (bf16, one GPU, with the hint on the stores: the separated FP8 tail at
// [65536, 1024] 120.8 -> 119.2 us, NVFP4 at [8192, 7168] 106.1 -> 103.7).
#include "anq_device.h"
#include "anq_internal.h"

namespace anq {

template <int DT, int EPI, bool NT>
__global__ void __launch_bounds__(256) quant_kernel(QuantParams p) {
  constexpr bool kNvfp4 = EPI == kEpiNvfp4 || EPI == kEpiNvfp4Swz;
  __shared__ float mult_tab[128];
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool ok = v < p.vecs;
  const int64_t vv = ok ? v : p.vecs - 1;  // past the end: a clamped load, no store
  // the vector's load goes out first; it lands while the multiplier table fills
  const U4 in = ld16s<NT>(static_cast<const uint8_t*>(p.in) + (size_t)vv * 16);
  const float sc = *p.scale;  // FP8: s, NVFP4: G
  const float inv_sc = recip_rn(sc);  // s is a positive normal <= 2^119
  if constexpr (kNvfp4) {
    fill_mult_tab(mult_tab, sc);
    __syncthreads();
  }
  if constexpr (EPI == kEpiNvfp4Swz) {
    if (v >= p.vecs) {  // threads past the tensor zero the padded scale rows, a word each
      const int64_t e = v - p.vecs;
      if (e < p.pad_rows * p.sf_tiles)
        *reinterpret_cast<uint32_t*>(p.sf + sf_swizzled_offset(p.tokens + e / p.sf_tiles,
                                                               4 * (int32_t)(e % p.sf_tiles),
                                                               p.sf_tiles)) = 0u;
    }
  }
  float f[8];
  unpack8<DT>(in, f);
  if constexpr (EPI == kEpiFp8) {
    uint32_t lo, hi;
    fp8_codes8(f, sc, inv_sc, lo, hi);
    if (ok) st8s<NT>(p.q + (size_t)v * 8, lo, hi);
  } else {
    uint32_t w, sfc;
    nvfp4_half_block(f, sc, mult_tab, w, sfc);
    if (ok) {
      st4s<NT>(p.q + (size_t)v * 4, w);
      if ((v & 1) == 0) {
        if constexpr (EPI != kEpiNvfp4Swz) {  // linear [tokens, hidden/16]: block v/2 of the tensor
          st1s<NT>(p.sf + (size_t)(v >> 1), (uint8_t)sfc);
        } else {
          const int64_t row = v / p.vec;
          store_block_scale_swizzled(p.sf, row, (int32_t)((v - row * p.vec) >> 1), p.vec / 2,
                                     p.sf_tiles, (uint8_t)sfc);
        }
      }
    }
  }
}

// The grid (one thread per vector, and per padded scale word with the swizzled
// layout, in 256-thread workgroups) and the streaming hint come from
// pick_quant_tiling.
template <int DT, int EPI>
static hipError_t launch_quant_epi(const QuantParams& p, const QuantTiling& t, hipStream_t s) {
  void* args[] = {const_cast<QuantParams*>(&p)};
  const void* fn = t.stream ? (const void*)&quant_kernel<DT, EPI, true>
                            : (const void*)&quant_kernel<DT, EPI, false>;
  return hipLaunchKernel(fn, dim3((unsigned)t.grid), dim3(256), args, 0, s);
}

template <int DT>
static hipError_t launch_quant_dt(int epi, const QuantParams& p, const QuantTiling& t,
                                  hipStream_t s) {
  switch (epi) {
    case kEpiFp8: return launch_quant_epi<DT, kEpiFp8>(p, t, s);
    case kEpiNvfp4: return launch_quant_epi<DT, kEpiNvfp4>(p, t, s);
    case kEpiNvfp4Swz: return launch_quant_epi<DT, kEpiNvfp4Swz>(p, t, s);
    default: return hipErrorInvalidValue;
  }
}

int launch_quant(int dtype, int epi, const QuantParams& p, const QuantTiling& t, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return (int)(dtype == kBF16 ? launch_quant_dt<kBF16>(epi, p, t, s)
                              : launch_quant_dt<kF16>(epi, p, t, s));
}

// u = x * SiLU(z) in binary32 (silu_gate), one thread per 8 elements: the gate
// of the gated RMSNorm as a standalone op.
template <int DT>
__global__ void __launch_bounds__(256) gate_kernel(const uint8_t* x, const uint8_t* z, float* u,
                                                   int64_t vecs) {
  __shared__ double exp2_tab[64];
  fill_exp2_tab(exp2_tab);
  __syncthreads();
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= vecs) return;
  float xf[8], zf[8], o[8];
  unpack8<DT>(ld16(x + (size_t)v * 16), xf);
  unpack8<DT>(ld16(z + (size_t)v * 16), zf);
  silu_gate8(xf, zf, exp2_tab, o);
  float4* dst = reinterpret_cast<float4*>(u + (size_t)v * 8);
  dst[0] = make_float4(o[0], o[1], o[2], o[3]);
  dst[1] = make_float4(o[4], o[5], o[6], o[7]);
}

int launch_gate(int dtype, const void* x, const void* z, float* u, int64_t vecs, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t grid = (vecs + 255) / 256;  // <= 2^31 - 1, checked by the front end
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const uint8_t* zb = static_cast<const uint8_t*>(z);
  if (dtype == kBF16)
    hipLaunchKernelGGL(gate_kernel<kBF16>, dim3((unsigned)grid), dim3(256), 0, s, xb, zb, u, vecs);
  else
    hipLaunchKernelGGL(gate_kernel<kF16>, dim3((unsigned)grid), dim3(256), 0, s, xb, zb, u, vecs);
  return (int)hipGetLastError();
}

}  // namespace anq
