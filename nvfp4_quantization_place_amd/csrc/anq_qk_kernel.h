// Q/K per-head RMSNorm + NeoX RoPE + FP8 E4M3 of a fused QKV buffer, with its
// store epilogues (SGLang PR #32975 "fused norm + RoPE + uniform fp8 store";
// the Q/K RMSNorm and RoPE of TensorRT-LLM PR #17288, Description, whose Test
// Coverage guards the RoPE width). Included by anq_qk.hip (whole-head
// rotation) and anq_qk_part.hip (partial rotation, mixed pool), which
// instantiate it in two translation units that compile in parallel.
//
// gfx950 mapping: one or a few wavefronts per token. 64 lanes form 64/(D/16)
// head slots of D/16 lanes, and each lane holds two 8-element vectors a and b
// of its slot's head:
//   whole-head rotation (PART false): a = [8j, 8j+8), b = [D/2 + 8j, ...), so
//     every NeoX pair (k, k + D/2) lives in one lane;
//   partial rotation over the last R elements (PART true, N = D - R): lanes
//     j < R/16 hold a = [N + 8j, ...) and b = [N + R/2 + 8j, ...), the pairs
//     (N + k, N + k + R/2); lanes j >= R/16 (m = j - R/16) hold unrotated
//     elements a = [8m, ...) and b = [N/2 + 8m, ...), so each of the two
//     vector loads of a wavefront still covers two contiguous ranges of a
//     head (R = 16, a single rotated lane: a = [16m, ...), b = [16m + 8, ...)).
//     With R = D this is the whole-head layout.
// A wavefront takes at most four groups of heads of its token and issues all
// of their loads at once, with the token's cos|sin slice; the workgroup
// shares gamma_q and gamma_k as binary32 in LDS. A head's sum of squares
// meets through a DPP butterfly over its D/16 lanes. Q and K heads are
// normalised and rotated; V heads are only quantised.
//
// STORE: kStoreNone writes every head's E4M3 codes to out [tokens, heads*D];
// kStoreUniform writes the Q codes to a dense [tokens, nq*D] buffer and the
// token's K and V codes to its slot of a uniform FP8 pool (rows of (nk+nv)*D
// bytes); kStoreMixed writes the Q codes the same way and the token's pool row
// as, per K head, the unrotated part's E4M3 codes then the rotated part as
// bf16, then the V heads' codes (rows of nk*(D+R) + nv*D bytes). A slot
// outside [0, num_slots) stores nothing.
#pragma once

#include "anq_device.h"
#include "anq_internal.h"

namespace anq {

template <int DT, int LPH, bool NT, int STORE, int PF, bool PART>
__global__ void __launch_bounds__(1024) qk_kernel(QKParams p) {
  constexpr int D = LPH * 16;
  constexpr int HPP = 64 / LPH;  // heads per pass of a wavefront
  static_assert(!(STORE == kStoreMixed && !PART), "the mixed pool uses the partial-rotation layout");
  const int lane = threadIdx.x & 63;
  const int j = lane & (LPH - 1);
  const int slot = lane / LPH;
  // the rotated width R (a power of two, 16 <= R <= D), its lanes RL, and
  // the unrotated width N; compile-time constants without PART
  const int R = PART ? p.rotary_dim : D;
  const int RL = R >> 4;
  const int N = D - R;
  const bool rope_lane = !PART || j < RL;
  // element offsets of the lane's two vectors inside a head; with two or more
  // rotated lanes (RL even) the unrotated lanes split their part in halves as
  // the rotated ones do, so rotated and unrotated lanes alike pair up (j, j^1)
  // for the code stores below
  const bool halves = RL >= 2;
  const int m = j - RL;  // the unrotated lanes' index
  const uint32_t ea = rope_lane ? (uint32_t)(N + 8 * j) : (uint32_t)(halves ? 8 * m : 16 * m);
  const uint32_t eb = rope_lane ? (uint32_t)(N + R / 2 + 8 * j)
                                : (uint32_t)(halves ? N / 2 + 8 * m : 16 * m + 8);
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
  const uint32_t lane_off = ((uint32_t)slot * D + ea) * 2;  // bytes, the lane's a vector
  const uint32_t b_off = (eb - ea) * 2;                     // bytes from a to b

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
  const uint32_t last_off = ((uint32_t)(heads - 1) * D + ea) * 2;
  auto group_off = [&](int pass) {
    return min((uint32_t)pass * (HPP * D * 2) + lane_off, last_off);
  };
  U4 ra[PF], rb[PF];
  {
    const uint32_t o = group_off(w);
    ra[0] = ld16s<NT>(row + o);
    rb[0] = ld16s<NT>(row + o + b_off);
  }

  // per-token constants: the lane's cos|sin values (lanes of the unrotated
  // part read the last rotated lane's, unused)
  float c[8], s[8];
  if (active && qk_heads > 0) {
    pos = pos < 0 ? 0 : (pos >= p.max_pos ? p.max_pos - 1 : pos);  // never read outside the table
    const int jr = rope_lane ? j : RL - 1;
    const float* cs = p.cos_sin + (size_t)pos * R + 8 * jr;
    const float4 c0 = *reinterpret_cast<const float4*>(cs);
    const float4 c1 = *reinterpret_cast<const float4*>(cs + 4);
    const float4 s0 = *reinterpret_cast<const float4*>(cs + R / 2);
    const float4 s1 = *reinterpret_cast<const float4*>(cs + R / 2 + 4);
    c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
    c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
    s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
    s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
  }
#pragma unroll
  for (int u = 1; u < PF; ++u) {
    const uint32_t o = group_off(w + u * W);
    ra[u] = ld16s<NT>(row + o);
    rb[u] = ld16s<NT>(row + o + b_off);
  }

  // gamma_q | gamma_k as binary32 in LDS, shared by the workgroup's
  // wavefronts; a lane reads the elements of its a and b vectors
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
  uint8_t* orow = p.out + (size_t)t * (STORE != kStoreNone ? (size_t)p.nq * D : row_elems);
  // the pool row: uniform (nk+nv)*D bytes, mixed nk*(D+R) + nv*D
  const uint32_t k_bytes = STORE == kStoreMixed ? (uint32_t)(D + R) : (uint32_t)D;  // per K head
  uint8_t* kvrow = nullptr;  // the token's pool row, or none
  if constexpr (STORE != kStoreNone) {
    if (p.num_slots > 0) {  // 0 also when there are no K/V heads (slots may then be NULL)
      const int64_t sl = p.slots[t];
      const size_t row_bytes = (size_t)p.nk * k_bytes + (size_t)p.nv * D;
      if (sl >= 0 && sl < p.num_slots) kvrow = p.kv + (size_t)sl * row_bytes;
    }
  }
  // Code stores of 16 contiguous bytes per lane. Lanes pair up (j, j^1) and
  // swap one 8-byte half (see below): the even lane stores 16 consecutive
  // elements of the first half of its part (rotated or not), the odd lane the
  // same range of the second half. With a single rotated lane (R = 16) no lane
  // swaps: every lane already holds 16 consecutive elements.
  const bool odd = (j & 1) != 0;
  const bool swap = halves;
  const uint32_t half_off = rope_lane ? (uint32_t)(R / 2) : (uint32_t)(N / 2);  // eb - ea
  const uint32_t st_off = swap && odd ? ea - 8u + half_off : ea;

  // one group of heads: the slot's head h = pass * HPP + slot, from its two
  // unpacked vectors
  auto group = [&](int pass, float (&a)[8], float (&b)[8]) {
    const int h = pass * HPP + slot;
    float oa[8], ob[8];
    if (h < qk_heads) {  // uniform over the head's lanes
      const float4* gl = gam_lds + (h < p.nq ? 0 : D / 4);
      const float4 ga0 = gl[ea / 4], ga1 = gl[ea / 4 + 1];
      const float4 gb0 = gl[eb / 4], gb1 = gl[eb / 4 + 1];
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
        const float ra_ = (na * c[i]) - (nb * s[i]);
        const float rb_ = (nb * c[i]) + (na * s[i]);
        oa[i] = rope_lane ? ra_ : na;
        ob[i] = rope_lane ? rb_ : nb;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        oa[i] = a[i];
        ob[i] = b[i];
      }
    }
    // the mixed pool keeps a K head's rotated part in bf16, before the division
    U4 bfa{}, bfb{};
    const bool k_mixed = STORE == kStoreMixed && h >= p.nq && h < qk_heads;  // uniform per head
    if constexpr (STORE == kStoreMixed) {
      if (k_mixed) {
        bfa = pack8<kBF16>(oa);
        bfb = pack8<kBF16>(ob);
      }
    }
    float qa[8], qb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qa[i] = div_rn_sat(oa[i], sc, inv_sc, sat);
      qb[i] = div_rn_sat(ob[i], sc, inv_sc, sat);
    }
    const uint32_t a0 = e4m3x4_in_range(qa[0], qa[1], qa[2], qa[3]);
    const uint32_t a1 = e4m3x4_in_range(qa[4], qa[5], qa[6], qa[7]);
    const uint32_t b0 = e4m3x4_in_range(qb[0], qb[1], qb[2], qb[3]);
    const uint32_t b1 = e4m3x4_in_range(qb[4], qb[5], qb[6], qb[7]);
    // every lane takes part in the swap (it reads its partner's registers);
    // lanes that do not pair keep their own a and b codes
    const uint32_t r0 = dpp_u32<0xB1>(odd ? a0 : b0), r1 = dpp_u32<0xB1>(odd ? a1 : b1);
    U4 v;
    v.w[0] = swap && odd ? r0 : a0;
    v.w[1] = swap && odd ? r1 : a1;
    v.w[2] = swap && !odd ? r0 : b0;
    v.w[3] = swap && !odd ? r1 : b1;
    if (h >= heads) return;
    if constexpr (STORE == kStoreNone) {
      st16s<NT>(orow + ((uint32_t)h * D + st_off), v);
    } else {
      if (h < p.nq) {
        st16s<NT>(orow + ((uint32_t)h * D + st_off), v);
      } else if (kvrow) {
        if (STORE == kStoreMixed && k_mixed) {
          // a K head's D + R bytes need not fill whole 128-byte lines, and its
          // three stores are separate instructions: without the streaming
          // hint the L2 merges the shared lines before writing them back
          uint8_t* kh = kvrow + (uint32_t)(h - p.nq) * k_bytes;
          if (rope_lane) {  // the rotated part in bf16: elements N + 8j and N + R/2 + 8j
            st16s<false>(kh + (uint32_t)N + 16u * (uint32_t)j, bfa);
            st16s<false>(kh + (uint32_t)(N + R) + 16u * (uint32_t)j, bfb);
          } else {          // the unrotated part in E4M3: the lane's 16 codes
            st16s<false>(kh + st_off, v);
          }
        } else {  // V heads (and K heads of the uniform pool): codes
          const uint32_t base = STORE == kStoreMixed
                                    ? (uint32_t)p.nk * k_bytes + (uint32_t)(h - qk_heads) * D
                                    : (uint32_t)(h - p.nq) * D;
          st16s<NT>(kvrow + (base + st_off), v);
        }
      }
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

template <int DT, bool NT, int STORE, int PF, bool PART>
const void* qk_fn(int lph) {
  switch (lph) {
    case 2: return (const void*)&qk_kernel<DT, 2, NT, STORE, PF, PART>;
    case 4: return (const void*)&qk_kernel<DT, 4, NT, STORE, PF, PART>;
    case 8: return (const void*)&qk_kernel<DT, 8, NT, STORE, PF, PART>;
    case 16: return (const void*)&qk_kernel<DT, 16, NT, STORE, PF, PART>;
    case 32: return (const void*)&qk_kernel<DT, 32, NT, STORE, PF, PART>;
    default: return nullptr;
  }
}

// One launch in the tiling of pick_qk_tiling (wavefronts per token, head
// groups per wavefront, workgroup size, streaming hints).
template <int DT, bool NT, int STORE, bool PART>
hipError_t launch_qk_nt(const QKParams& p, const QKTiling& t, hipStream_t s) {
  void* args[] = {const_cast<QKParams*>(&p)};
  const int lph = p.head_dim / 16;
  const void* fn = t.groups == 4 ? qk_fn<DT, NT, STORE, 4, PART>(lph)
                 : t.groups == 3 ? qk_fn<DT, NT, STORE, 3, PART>(lph)
                 : t.groups == 2 ? qk_fn<DT, NT, STORE, 2, PART>(lph)
                 : t.groups == 1 ? qk_fn<DT, NT, STORE, 1, PART>(lph) : nullptr;
  if (!fn || p.waves_per_token != t.waves_per_token || t.block < p.head_dim / 4)
    return hipErrorInvalidConfiguration;
  return hipLaunchKernel(fn, dim3((unsigned)t.grid), dim3(t.block), args, 0, s);
}

template <int DT, int STORE, bool PART>
hipError_t launch_qk_store(const QKParams& p, const QKTiling& t, hipStream_t s) {
  return t.stream ? launch_qk_nt<DT, true, STORE, PART>(p, t, s)
                  : launch_qk_nt<DT, false, STORE, PART>(p, t, s);
}

// Launchers of the two translation units: whole-head rotation (anq_qk.hip,
// stores none and uniform) and partial rotation (anq_qk_part.hip, every
// store, the mixed pool at any width).
hipError_t launch_qk_whole(int dtype, int store, const QKParams& p, const QKTiling& t,
                           hipStream_t s);
hipError_t launch_qk_partial(int dtype, int store, const QKParams& p, const QKTiling& t,
                             hipStream_t s);

}  // namespace anq
