// Q/K per-head RMSNorm + NeoX RoPE + uniform FP8 E4M3 store of a fused QKV
// buffer (SGLang PR #32975 "fused norm + RoPE + uniform fp8 store"; the Q/K
// RMSNorm and RoPE of TensorRT-LLM PR #17288, Description).
//
// gfx950 mapping: one or a few wavefronts per token. 64 lanes form 64/(D/16) head
// slots of D/16 lanes; lane j of a slot holds elements [8j, 8j+8) of the first
// half of a head and [D/2 + 8j, D/2 + 8j + 8) of the second half, so every
// NeoX rotation pair (k, k + D/2) lives in one lane. A wavefront takes at most
// four groups of heads of its token and issues all of their loads at once,
// with the token's cos|sin slice; the workgroup shares gamma_q and gamma_k as
// binary32 in LDS. A head's sum of squares meets through a DPP butterfly over
// its D/16 lanes. Q and K heads are normalised, rotated and quantised; V heads
// are only quantised.
//
// STORE selects the KV-store epilogue (the "store" of the norm + RoPE + store
// kernel in SGLang PR #32975, with its uniform FP8 pool): Q codes go to a
// dense [tokens, nq*D] buffer, and the token's K and V codes go to its slot of
// the pool, a row of (nk+nv)*D bytes; a slot outside [0, num_slots) stores
// nothing.
#include "anq_device.h"
#include "anq_internal.h"

namespace anq {

template <int DT, int LPH, bool NT, bool STORE, int PF>
__global__ void __launch_bounds__(1024) qk_kernel(QKParams p) {
  constexpr int D = LPH * 16;
  constexpr int HALF = D / 2;
  constexpr int HPP = 64 / LPH;  // heads per pass of a wavefront
  const int lane = threadIdx.x & 63;
  const int j = lane & (LPH - 1);
  const int slot = lane / LPH;
  // wavefront-uniform indices and row bases live in scalar registers; the
  // lanes add 32-bit byte offsets (a token row is < 2^31 bytes)
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = wave / p.waves_per_token;
  const int w = (int)(wave - t * p.waves_per_token);
  const bool active = t < p.tokens;  // uniform over the wavefront
  const int heads = p.nq + p.nk + p.nv;
  const int qk_heads = p.nq + p.nk;
  const size_t row_elems = (size_t)heads * D;
  // a wavefront past the last token reads token 0's row (never used), so that
  // every load below is unconditional
  const uint8_t* row = static_cast<const uint8_t*>(p.qkv) + (size_t)(active ? t : 0) * row_elems * 2;
  const uint32_t oa_off = 8 * j;  // element offset of the lane's first-half vector inside a head
  const uint32_t lane_off = ((uint32_t)slot * D + oa_off) * 2;  // bytes, first half of the slot's head

  // gamma_q | gamma_k: thread i < D/4 loads 16-byte vector i first of all, so
  // that waiting for it (to fill LDS below) does not wait for the row loads
  // (the launcher gives every workgroup at least D/4 threads)
  const int gi = (int)threadIdx.x;
  const bool gfill = qk_heads > 0 && gi < D / 4 && (gi >= D / 8 ? p.nk > 0 : p.nq > 0);
  U4 gvec{};
  if (gfill)
    gvec = ld16(static_cast<const uint8_t*>(gi >= D / 8 ? p.gamma_k : p.gamma_q) +
                (size_t)(gi >= D / 8 ? gi - D / 8 : gi) * 16);

  int64_t pos = 0;
  if (active && qk_heads > 0) pos = p.positions[t];

  // The loads of all of the wavefront's head groups (at most PF, by the
  // launcher's choice of W) go out before anything waits on them, group 0's
  // first, then the token's cos|sin slice (after its position), then the other
  // groups': loads complete in issue order, so group 0 then waits only for
  // itself and cos|sin. Heads past the end re-read the last head (never
  // stored), and so do slots past the wavefront's last group.
  const int passes = (heads + HPP - 1) / HPP;
  const int W = p.waves_per_token;  // this wavefront takes passes w, w + W, ...
  const uint32_t last_off = ((uint32_t)(heads - 1) * D + oa_off) * 2;
  auto group_off = [&](int pass) {
    return min((uint32_t)pass * (HPP * D * 2) + lane_off, last_off);
  };
  U4 ra[PF], rb[PF];
  {
    const uint32_t o = group_off(w);
    ra[0] = ld16s<NT>(row + o);
    rb[0] = ld16s<NT>(row + o + HALF * 2);
  }

  // per-token constants: the lane's cos|sin values
  float c[8], s[8];
  if (active && qk_heads > 0) {
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
  }
#pragma unroll
  for (int u = 1; u < PF; ++u) {
    const uint32_t o = group_off(w + u * W);
    ra[u] = ld16s<NT>(row + o);
    rb[u] = ld16s<NT>(row + o + HALF * 2);
  }

  // gamma_q | gamma_k as binary32 in LDS, shared by the workgroup's
  // wavefronts; a lane reads elements [8j, 8j+8) and [D/2 + 8j, D/2 + 8j + 8)
  // of its head's gamma
  __shared__ float4 gam_lds[2 * D / 4];
  if (qk_heads > 0) {
    if (gfill) {
      float g[8];
      unpack8<DT>(gvec, g);
      gam_lds[2 * gi] = make_float4(g[0], g[1], g[2], g[3]);
      gam_lds[2 * gi + 1] = make_float4(g[4], g[5], g[6], g[7]);
    }
    __syncthreads();
  }
  if (!active) return;  // the whole wavefront, after the workgroup's barrier

  const float sc = *p.scale;
  const float inv_sc = recip_rn(sc);  // s is a positive normal <= 2^119
  const float sat = sat_bound(sc);  // the numerator clamp of div_rn_sat
  uint8_t* orow = p.out + (size_t)t * (STORE ? (size_t)p.nq * D : row_elems);
  uint8_t* kvrow = nullptr;  // KV store: the token's pool row, or none
  if constexpr (STORE) {
    if (p.num_slots > 0) {  // 0 also when there are no K/V heads (slots may then be NULL)
      const int64_t sl = p.slots[t];
      if (sl >= 0 && sl < p.num_slots) kvrow = p.kv + (size_t)sl * (size_t)(heads - p.nq) * D;
    }
  }
  const bool odd = (j & 1) != 0;
  // lanes 2m and 2m+1 each store 16 contiguous codes (see the swap below)
  const uint32_t st_off = odd ? HALF + 8 * (j - 1) : 8 * j;

  // one group of heads: the slot's head h = pass * HPP + slot, from its two
  // unpacked halves
  auto group = [&](int pass, float (&a)[8], float (&b)[8]) {
    const int h = pass * HPP + slot;
    float oa[8], ob[8];
    if (h < qk_heads) {  // uniform over the head's lanes
      const float4* gl = gam_lds + (h < p.nq ? 0 : D / 4);
      const float4 ga0 = gl[2 * j], ga1 = gl[2 * j + 1];
      const float4 gb0 = gl[2 * (LPH + j)], gb1 = gl[2 * (LPH + j) + 1];
      const float ga[8] = {ga0.x, ga0.y, ga0.z, ga0.w, ga1.x, ga1.y, ga1.z, ga1.w};
      const float gb[8] = {gb0.x, gb0.y, gb0.z, gb0.w, gb1.x, gb1.y, gb1.z, gb1.w};
      double acc = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc = __builtin_fma((double)a[i], (double)a[i], acc);
        acc = __builtin_fma((double)b[i], (double)b[i], acc);
      }
      const double S = lanes_sum<LPH>(acc);
      float ss = (float)S;
      if (near_f32_midpoint(S, D)) {
        // rare: the exact sum as a double-double, in the order a0 b0 a1 b1 ...
        // (this form, from the registers, measured 1.8 us faster at 4096
        // tokens than re-reading the elements, though it is seldom taken)
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
    const uint32_t r0 = dpp_u32<0xB1>(odd ? a0 : b0), r1 = dpp_u32<0xB1>(odd ? a1 : b1);
    uint8_t* dst = orow;
    uint32_t hd = (uint32_t)h;
    if constexpr (STORE) {
      if (h >= p.nq) {
        dst = kvrow;
        hd = (uint32_t)(h - p.nq);
      }
    }
    if (h < heads && dst) {
      U4 v;
      v.w[0] = odd ? r0 : a0;
      v.w[1] = odd ? r1 : a1;
      v.w[2] = odd ? b0 : r0;
      v.w[3] = odd ? b1 : r1;
      st16s<NT>(dst + (hd * D + st_off), v);
    }
  };

  const int mine = (passes - w + W - 1) / W;  // groups of this wavefront, <= PF (w < W <= passes)
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    if (u < mine) {  // uniform over the wavefront
      float a[8], b[8];
      unpack8<DT>(ra[u], a);
      unpack8<DT>(rb[u], b);
      group(w + u * W, a, b);
    }
  }
}

template <int DT, bool NT, bool STORE, int PF>
static const void* qk_fn(int lph) {
  switch (lph) {
    case 2: return (const void*)&qk_kernel<DT, 2, NT, STORE, PF>;
    case 4: return (const void*)&qk_kernel<DT, 4, NT, STORE, PF>;
    case 8: return (const void*)&qk_kernel<DT, 8, NT, STORE, PF>;
    case 16: return (const void*)&qk_kernel<DT, 16, NT, STORE, PF>;
    case 32: return (const void*)&qk_kernel<DT, 32, NT, STORE, PF>;
    default: return nullptr;
  }
}

// The tiling (wavefronts per token, head groups per wavefront, workgroup size,
// streaming hints) comes from pick_qk_tiling.
template <int DT, bool NT, bool STORE>
static hipError_t launch_qk_nt(const QKParams& p, const QKTiling& t, hipStream_t s) {
  void* args[] = {const_cast<QKParams*>(&p)};
  const int lph = p.head_dim / 16;
  const void* fn = t.groups == 4 ? qk_fn<DT, NT, STORE, 4>(lph)
                 : t.groups == 3 ? qk_fn<DT, NT, STORE, 3>(lph)
                 : t.groups == 2 ? qk_fn<DT, NT, STORE, 2>(lph)
                 : t.groups == 1 ? qk_fn<DT, NT, STORE, 1>(lph) : nullptr;
  if (!fn || p.waves_per_token != t.waves_per_token || t.block < p.head_dim / 4)
    return hipErrorInvalidConfiguration;
  return hipLaunchKernel(fn, dim3((unsigned)t.grid), dim3(t.block), args, 0, s);
}

template <int DT, bool STORE>
static hipError_t launch_qk_dt(const QKParams& p, const QKTiling& t, hipStream_t s) {
  return t.stream ? launch_qk_nt<DT, true, STORE>(p, t, s) : launch_qk_nt<DT, false, STORE>(p, t, s);
}

int launch_qk(int dtype, int store, const QKParams& p, const QKTiling& t, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.rotary_dim != p.head_dim || (store != kStoreNone && store != kStoreUniform))
    return (int)hipErrorInvalidValue;
  const bool kv = store == kStoreUniform;
  hipError_t e;
  if (kv) e = dtype == kBF16 ? launch_qk_dt<kBF16, true>(p, t, s) : launch_qk_dt<kF16, true>(p, t, s);
  else e = dtype == kBF16 ? launch_qk_dt<kBF16, false>(p, t, s) : launch_qk_dt<kF16, false>(p, t, s);
  return (int)e;
}

}  // namespace anq
