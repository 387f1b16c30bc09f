// Q/K per-head RMSNorm + NeoX RoPE + uniform FP8 E4M3 store of a fused QKV
// buffer (SGLang PR #32975 "fused norm + RoPE + uniform fp8 store"; the Q/K
// RMSNorm and RoPE of TensorRT-LLM PR #17288, Description).
//
// gfx950 mapping: one or a few wavefronts per token. 64 lanes form 64/(D/16) head
// slots of D/16 lanes; lane j of a slot holds elements [8j, 8j+8) of the first
// half of a head and [D/2 + 8j, D/2 + 8j + 8) of the second half, so every
// NeoX rotation pair (k, k + D/2) lives in one lane. A wavefront loads the
// token's cos|sin slice and both gammas once, then walks its share of the
// token's head groups, loading the next group while it finishes the current
// one. A head's sum of squares meets through a DPP butterfly over its
// D/16 lanes. Q and K heads are normalised, rotated and quantised; V heads
// are only quantised.
//
// STORE selects the KV-store epilogue (the "store" of the norm + RoPE + store
// kernel in SGLang PR #32975, with its uniform FP8 pool): Q codes go to a
// dense [tokens, nq*D] buffer, and the token's K and V codes go to its slot of
// the pool, a row of (nk+nv)*D bytes; a slot outside [0, num_slots) stores
// nothing.
#include <stdlib.h>

#include "anq_device.h"
#include "anq_internal.h"

namespace anq {

template <int DT, int LPH, bool NT, bool STORE>
__global__ void __launch_bounds__(1024) qk_kernel(QKParams p) {
  constexpr int D = LPH * 16;
  constexpr int HALF = D / 2;
  constexpr int HPP = 64 / LPH;  // heads per pass of a wavefront
  const int lane = threadIdx.x & 63;
  const int j = lane & (LPH - 1);
  const int slot = lane / LPH;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t t = wave / p.waves_per_token;
  const int w = (int)(wave - t * p.waves_per_token);
  if (t >= p.tokens) return;  // the whole wavefront
  const int heads = p.nq + p.nk + p.nv;
  const int qk_heads = p.nq + p.nk;
  const float sc = *p.scale;
  const float inv_sc = recip_rn(sc);  // s is a positive normal <= 2^119
  const float sat = sat_bound(sc);  // the numerator clamp of div_rn_sat
  const size_t row_elems = (size_t)heads * D;
  const uint8_t* row = static_cast<const uint8_t*>(p.qkv) + (size_t)t * row_elems * 2;
  uint8_t* orow = p.out + (size_t)t * (STORE ? (size_t)p.nq * D : row_elems);
  uint8_t* kvrow = nullptr;  // KV store: the token's pool row, or none
  if constexpr (STORE) {
    if (p.num_slots > 0) {  // 0 also when there are no K/V heads (slots may then be NULL)
      const int64_t sl = p.slots[t];
      if (sl >= 0 && sl < p.num_slots) kvrow = p.kv + (size_t)sl * (size_t)(heads - p.nq) * D;
    }
  }
  const uint32_t oa_off = 8 * j, ob_off = HALF + 8 * j;  // element offsets inside a head

  // per-token constants: the lane's cos|sin values and gamma slices
  float c[8], s[8];
  U4 gqa{}, gqb{}, gka{}, gkb{};
  if (qk_heads > 0) {
    int64_t pos = p.positions[t];
    pos = pos < 0 ? 0 : (pos >= p.max_pos ? p.max_pos - 1 : pos);  // never read outside the table
    const float* cs = p.cos_sin + (size_t)pos * D;
    const float4 c0 = *reinterpret_cast<const float4*>(cs + oa_off);
    const float4 c1 = *reinterpret_cast<const float4*>(cs + oa_off + 4);
    const float4 s0 = *reinterpret_cast<const float4*>(cs + HALF + oa_off);
    const float4 s1 = *reinterpret_cast<const float4*>(cs + HALF + oa_off + 4);
    c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
    c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
    s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
    s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
    if (p.nq > 0) {
      gqa = ld16(static_cast<const uint8_t*>(p.gamma_q) + oa_off * 2);
      gqb = ld16(static_cast<const uint8_t*>(p.gamma_q) + ob_off * 2);
    }
    if (p.nk > 0) {
      gka = ld16(static_cast<const uint8_t*>(p.gamma_k) + oa_off * 2);
      gkb = ld16(static_cast<const uint8_t*>(p.gamma_k) + ob_off * 2);
    }
  }

  const int passes = (heads + HPP - 1) / HPP;
  const int W = p.waves_per_token;  // this wavefront takes passes w, w + W, ...
  // loads of the first pass (heads past the end re-read the last head; never stored)
  int hl = w * HPP + slot < heads ? w * HPP + slot : heads - 1;
  U4 av = ld16s<NT>(row + ((size_t)hl * D + oa_off) * 2);
  U4 bv = ld16s<NT>(row + ((size_t)hl * D + ob_off) * 2);
  for (int pass = w; pass < passes; pass += W) {
    const int h = pass * HPP + slot;
    float a[8], b[8], oa[8], ob[8];
    unpack8<DT>(av, a);
    unpack8<DT>(bv, b);
    if (pass + W < passes) {  // next group of heads, landing while this one is processed
      hl = h + W * HPP < heads ? h + W * HPP : heads - 1;
      av = ld16s<NT>(row + ((size_t)hl * D + oa_off) * 2);
      bv = ld16s<NT>(row + ((size_t)hl * D + ob_off) * 2);
    }
    if (h < qk_heads) {  // uniform over the head's lanes
      float ga[8], gb[8];
      unpack8<DT>(h < p.nq ? gqa : gka, ga);
      unpack8<DT>(h < p.nq ? gqb : gkb, gb);
      double acc = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc = __builtin_fma((double)a[i], (double)a[i], acc);
        acc = __builtin_fma((double)b[i], (double)b[i], acc);
      }
      const double S = lanes_sum<LPH>(acc);
      float ss = (float)S;
      if (near_f32_midpoint(S, D)) {
        double hi = 0.0, lo = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dd_add(hi, lo, (double)a[i] * (double)a[i], 0.0);
          dd_add(hi, lo, (double)b[i] * (double)b[i], 0.0);
        }
        lanes_sum_dd<LPH>(hi, lo);
        ss = dd_to_f32(hi, lo);
      }
      const float r = recip_rn_ext(sqrtf(ss * (1.0f / D) + p.eps));  // D = 2^k: exact, as ss / D
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
      oa[i] = div_rn_sat(oa[i], sc, inv_sc, sat);
      ob[i] = div_rn_sat(ob[i], sc, inv_sc, sat);
    }
    // Lanes 2m and 2m+1 swap one 8-byte half so that each stores 16 contiguous
    // codes: the even lane elements [16m, 16m+16), the odd lane the same range
    // of the second half. Every head's output then leaves as whole lines.
    const uint32_t a0 = e4m3x4_in_range(oa[0], oa[1], oa[2], oa[3]);
    const uint32_t a1 = e4m3x4_in_range(oa[4], oa[5], oa[6], oa[7]);
    const uint32_t b0 = e4m3x4_in_range(ob[0], ob[1], ob[2], ob[3]);
    const uint32_t b1 = e4m3x4_in_range(ob[4], ob[5], ob[6], ob[7]);
    const bool odd = (j & 1) != 0;
    const uint32_t r0 = dpp_u32<0xB1>(odd ? a0 : b0), r1 = dpp_u32<0xB1>(odd ? a1 : b1);
    uint8_t* dst = orow + (size_t)h * D;
    if constexpr (STORE) {
      if (h >= p.nq) dst = kvrow ? kvrow + (size_t)(h - p.nq) * D : nullptr;
    }
    if (h < heads && dst) {
      U4 v;
      v.w[0] = odd ? r0 : a0;
      v.w[1] = odd ? r1 : a1;
      v.w[2] = odd ? b0 : r0;
      v.w[3] = odd ? b1 : r1;
      st16s<NT>(dst + (odd ? HALF + 8 * (j - 1) : 8 * j), v);
    }
  }
}

template <int DT, bool NT, bool STORE>
static hipError_t launch_qk_nt(const QKParams& p, hipStream_t s) {
  void* args[] = {const_cast<QKParams*>(&p)};
  const void* fn = nullptr;
  const int lph = p.head_dim / 16;
  switch (lph) {
    case 2: fn = (const void*)&qk_kernel<DT, 2, NT, STORE>; break;
    case 4: fn = (const void*)&qk_kernel<DT, 4, NT, STORE>; break;
    case 8: fn = (const void*)&qk_kernel<DT, 8, NT, STORE>; break;
    case 16: fn = (const void*)&qk_kernel<DT, 16, NT, STORE>; break;
    case 32: fn = (const void*)&qk_kernel<DT, 32, NT, STORE>; break;
    default: return hipErrorInvalidConfiguration;
  }
  int block = 256;  // four wavefronts
  if (const char* e = getenv("ANQ_QK_BLOCK")) {
    const int b = atoi(e);
    if (b >= 64 && b <= 1024 && b % 64 == 0) block = b;
  }
  const int64_t wpb = block / 64;
  const int64_t grid = (p.tokens * p.waves_per_token + wpb - 1) / wpb;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(block), args, 0, s);
}

// Streaming hints (see ld16s) once qkv alone is >= 32 MiB; ANQ_STREAM=0/1 overrides.
template <int DT, bool STORE>
static hipError_t launch_qk_dt(QKParams p, hipStream_t s) {
  // wavefronts per token: one, walking all of the token's head groups, once
  // the call has enough tokens to fill the GPU (~2048 wavefronts); more, up to
  // one per head group, for fewer tokens. At 4096 tokens x 32 heads of 128
  // (bf16) one wavefront per token measured 11.8 us against 12.8 with two.
  // ANQ_QK_WAVES and ANQ_QK_BLOCK override, for sweeps.
  const int passes = (p.nq + p.nk + p.nv + 64 / (p.head_dim / 16) - 1) / (64 / (p.head_dim / 16));
  const int64_t want = p.tokens > 0 ? (2048 + p.tokens - 1) / p.tokens : 1;
  int W = (int)(want < passes ? want : passes);
  if (W < 1) W = 1;
  if (const char* e = getenv("ANQ_QK_WAVES")) {
    if (*e && atoi(e) > 0) W = atoi(e);
  }
  p.waves_per_token = W < passes ? W : passes;
  bool stream = p.pairs * (int64_t)p.head_dim * 2 >= ((int64_t)32 << 20);
  if (const char* e = getenv("ANQ_STREAM")) {
    if (*e) stream = atoi(e) != 0;
  }
  return stream ? launch_qk_nt<DT, true, STORE>(p, s) : launch_qk_nt<DT, false, STORE>(p, s);
}

hipError_t launch_qk(int dtype, bool kv_store, const QKParams& p, hipStream_t s) {
  if (kv_store)
    return dtype == kBF16 ? launch_qk_dt<kBF16, true>(p, s) : launch_qk_dt<kF16, true>(p, s);
  return dtype == kBF16 ? launch_qk_dt<kBF16, false>(p, s) : launch_qk_dt<kF16, false>(p, s);
}

}  // namespace anq
