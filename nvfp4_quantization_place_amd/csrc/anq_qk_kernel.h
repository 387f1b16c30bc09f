// Q/K per-head RMSNorm + NeoX RoPE + FP8 E4M3 of a fused QKV buffer, with its
// store epilogues (SGLang PR #32975, the fused norm, RoPE and uniform FP8
// store; the Q/K RMSNorm and RoPE of TensorRT-LLM PR #17288, Description,
// whose Test Coverage guards the RoPE width). Included by anq_qk.hip
// (whole-head rotation) and anq_qk_part.hip (partial rotation), which
// instantiate it, each with every store, in two translation units that
// compile in parallel.
//
// gfx950 mapping: one or a few wavefronts per token. 64 lanes form 64/(D/16)
// head slots of D/16 lanes, and lane j of a slot holds two 8-element vectors
// of its head, a = [8j, 8j+8) and b = [D/2 + 8j, ...), so each of a
// wavefront's two vector loads reads whole contiguous halves of its heads.
//   whole-head rotation (PART false): every NeoX pair (k, k + D/2) lives in
//     one lane, as elements i of a and b;
//   partial rotation over the last R <= D/2 elements (PART true, N = D - R):
//     a is never rotated; the rotated part [N, D) is the b vectors of lanes
//     j >= D/16 - R/8, and the pair (N + k, N + k + R/2) is element i of b in
//     lanes j and j ^ R/16 of the same head, which exchange their normalised
//     b vectors through ds_bpermute.
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
// bf16 (with R = D the whole head in bf16), then the V heads' codes (rows of
// nk*(D+R) + nv*D bytes). A slot outside [0, num_slots) stores nothing.
#pragma once

#include "anq_device.h"
#include "anq_internal.h"

namespace anq {

template <int DT, int LPH, bool NT, int STORE, int PF, bool PART>
__global__ void __launch_bounds__(1024) qk_kernel(QKParams p) {
  constexpr int D = LPH * 16;
  constexpr int HPP = 64 / LPH;  // heads per pass of a wavefront
  const int lane = threadIdx.x & 63;
  const int j = lane & (LPH - 1);
  const int slot = lane / LPH;
  constexpr uint32_t kHalf = D / 2;
  const uint32_t ea = 8u * (uint32_t)j;  // element offsets of the lane's a and b in its head
  // the rotated width R (R = D without PART), and with PART: whether the
  // lane's b vector is rotated, and whether it holds the second element of
  // its pairs (partner lane = lane ^ RL)
  const int R = PART ? p.rotary_dim : D;
  const int RL = R >> 4;
  const bool rope_b = !PART || j >= LPH - 2 * RL;
  const bool upper = (j & RL) != 0;
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
  constexpr uint32_t b_off = kHalf * 2;                     // bytes from a to b

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

  // per-token constants: the lane's cos|sin values, those of frequency
  // 8j + i (whole head) or 8 (j mod RL) + i (partial)
  float c[8], s[8];
  if (active && qk_heads > 0) {
    pos = pos < 0 ? 0 : (pos >= p.max_pos ? p.max_pos - 1 : pos);  // never read outside the table
    const int kc = PART ? 8 * (j & (RL - 1)) : 8 * j;
    const float* cs = p.cos_sin + (size_t)pos * R + kc;
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
  // swap one 8-byte half (see below): the even lane stores the codes of
  // elements [8j, 8j + 16) (both a vectors), the odd lane those of
  // [D/2 + 8(j-1), D/2 + 8(j+1)) (both b vectors).
  const bool odd = (j & 1) != 0;
  const uint32_t st_off = odd ? ea - 8u + kHalf : ea;

  // one group of heads: the slot's head h = pass * HPP + slot, from its two
  // unpacked vectors, to the lane's 16 codes v and (K heads of the mixed
  // pool) its rotated values in bf16: b's in bfb, and with R = D a's in v
  // (such a head stores no codes), so a group holds 8 registers, not 12
  auto group = [&](int pass, float (&a)[8], float (&b)[8], U4& v, U4& bfb) {
    const int h = pass * HPP + slot;
    const bool qk = h < qk_heads;  // uniform over the head's lanes
    float oa[8], ob[8];
    if (qk) {
      const float4* gl = gam_lds + (h < p.nq ? 0 : D / 4);
      const float4 ga0 = gl[ea / 4], ga1 = gl[ea / 4 + 1];
      const float4 gb0 = gl[(kHalf + ea) / 4], gb1 = gl[(kHalf + ea) / 4 + 1];
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
        if constexpr (PART) {
          oa[i] = na;
          ob[i] = nb;
        } else {
          oa[i] = (na * c[i]) - (nb * s[i]);
          ob[i] = (nb * c[i]) + (na * s[i]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        oa[i] = a[i];
        ob[i] = b[i];
      }
    }
    if constexpr (PART) {
      // the partner of each rotated element is element i of b in lane ^ RL,
      // of the same head; the whole wavefront takes part in the exchange.
      // The first element of a pair takes x c - y s as x c + (-y) s (the
      // same binary32 result), the second x c + y s. Every lane computes the
      // rotation and selects it: a conditional assignment let the compiler
      // sink each product into a branch of its own, eight exec-mask branches
      // per group (same box, 4096 tokens, rotary 64: plain op 11.93 -> 11.66
      // us, mixed pool 12.53 -> 12.47).
      const int src = (lane ^ RL) << 2;
      const bool take = qk && rope_b;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float y = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(ob[i])));
        float rot = (ob[i] * c[i]) + ((upper ? y : -y) * s[i]);
        asm volatile("" : "+v"(rot));
        ob[i] = take ? rot : ob[i];
      }
    }
    // the mixed pool keeps a K head's rotated part in bf16, before the division
    const bool k_mixed = STORE == kStoreMixed && h >= p.nq && qk;  // uniform per head
    U4 bfa;
    if constexpr (STORE == kStoreMixed) {
      if (k_mixed) {
        if (!PART) bfa = pack8<kBF16>(oa);
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
    // every lane takes part in the swap (it reads its partner's registers)
    const uint32_t r0 = dpp_u32<0xB1>(odd ? a0 : b0), r1 = dpp_u32<0xB1>(odd ? a1 : b1);
    v.w[0] = odd ? r0 : a0;
    v.w[1] = odd ? r1 : a1;
    v.w[2] = odd ? b0 : r0;
    v.w[3] = odd ? b1 : r1;
    if constexpr (STORE == kStoreMixed && !PART) {
      if (k_mixed) v = bfa;
    }
  };

  // the stores of one group
  auto store = [&](int pass, const U4& v, const U4& bfb) {
    const int h = pass * HPP + slot;
    if (h >= heads) return;
    const bool k_mixed = STORE == kStoreMixed && h >= p.nq && h < qk_heads;
    if constexpr (STORE == kStoreNone) {
      st16s<NT>(orow + ((uint32_t)h * D + st_off), v);
    } else {
      if (h < p.nq) {
        st16s<NT>(orow + ((uint32_t)h * D + st_off), v);
      } else if (kvrow) {
        if (STORE == kStoreMixed && k_mixed) {
          // Element e of the rotated part is bf16 at byte N + 2 (e - N) of the
          // head. A K head's D + R bytes need not fill whole 128-byte lines and
          // its two stores are separate instructions, yet they take the
          // streaming hint like every other row store: workload 7's shape
          // (bf16, 4096 tokens, rotary 64, one GPU) 12.85 -> 12.15 us.
          uint8_t* kh = kvrow + (uint32_t)(h - p.nq) * k_bytes;
          if constexpr (PART) {
            // b of the rotated lanes in bf16; the unrotated codes come from
            // the even lanes (elements < D/2 <= N) and the odd lanes whose b
            // vectors are unrotated (the rotated part starts on a 16-element
            // boundary, so a pair of lanes is rotated or not together)
            if (rope_b) st16s<NT>(kh + (uint32_t)R + 16u * (uint32_t)j, bfb);
            if (!odd || !rope_b) st16s<NT>(kh + st_off, v);
          } else {  // R = D: the whole head in bf16 (a's half in v)
            st16s<NT>(kh + 16u * (uint32_t)j, v);
            st16s<NT>(kh + kHalf * 2 + 16u * (uint32_t)j, bfb);
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
  U4 v[PF], bfb[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    if (u < mine) {  // uniform over the wavefront
      float a[8], b[8];
      unpack8<DT>(ra[u], a);
      unpack8<DT>(rb[u], b);
      group(w + u * W, a, b, v[u], bfb[u]);
    }
  }
  // every store after every group: the wait for a group's loads then never
  // also waits for an earlier group's stores (one counter covers both)
#pragma unroll
  for (int u = 0; u < PF; ++u)
    if (u < mine) store(w + u * W, v[u], bfb[u]);
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

// Launchers of the two translation units: whole-head rotation (anq_qk.hip)
// and partial rotation (anq_qk_part.hip), each with every store.
hipError_t launch_qk_whole(int dtype, int store, const QKParams& p, const QKTiling& t,
                           hipStream_t s);
hipError_t launch_qk_partial(int dtype, int store, const QKParams& p, const QKTiling& t,
                             hipStream_t s);

}  // namespace anq
