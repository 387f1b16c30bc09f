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
//  * Small rows (up to 512 elements, and the gate-table variant's groups up to
//    1024) use 16, 32 or 64 lanes of one wavefront per row and reduce with
//    cross-lane shuffles; larger rows use one workgroup of up to 1024 lanes
//    per row and combine wavefront partials through LDS in a fixed order.
//  * A lane group that takes several rows takes them consecutively or, where
//    the host asks, interleaved across the grid (rows i, i + groups, ...).
//  * The sum of squares is accumulated in float64 (squares of fp16/bf16 values
//    are exact there) and rounded once to binary32. When that float64 total is
//    within its error bound of a binary32 rounding midpoint, the row is summed
//    again as a double-double, which settles the rounding of the exact sum.
//  * NVFP4: a 16-element block is two adjacent vectors held by lanes 2j and
//    2j+1; their amax meet through one lane swap.
#include <type_traits>

#include "anq_device.h"
#include "anq_gate_table.h"
#include "anq_internal.h"

namespace anq {

// ---------------------------------------------------------------- reducers

// G lanes of one wavefront, G in {16, 32, 64}: DPP butterfly (lanes_sum).
template <int G>
struct GroupReduce {
  __device__ __forceinline__ double sum(double v, int) const { return lanes_sum<G>(v); }
  __device__ __forceinline__ void sum_dd(double& hi, double& lo) const { lanes_sum_dd<G>(hi, lo); }
};

// One row per workgroup: a butterfly inside each wavefront, wavefront partials
// through LDS, then every 16-lane group of every wavefront reads the partials
// one per lane (zeros past the last wavefront) and runs the same butterfly over
// them. All groups add the same values in the same order, so all lanes of the
// workgroup hold identical bits. Partials of consecutive rows go to
// alternating LDS slots, so one barrier per row suffices: the slot a row reads
// is next written two rows later, after the following row's barrier.
struct BlockReduce {
  double* lds;  // 2 x 16 float64 partials, then 16 double-double partials
  __device__ __forceinline__ double sum(double v, int parity) const {
    v = GroupReduce<64>().sum(v, 0);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    double* slot = lds + 16 * parity;
    if (lane == 0) slot[w] = v;
    __syncthreads();
    const int i = lane & 15;
    return GroupReduce<16>().sum(i < nw ? slot[i] : 0.0, 0);
  }
  __device__ __forceinline__ void sum_dd(double& hi, double& lo) const {
    GroupReduce<64>().sum_dd(hi, lo);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    double* slot = lds + 32;
    __syncthreads();  // a previous double-double reduction may still be reading
    if (lane == 0) {
      slot[2 * w] = hi;
      slot[2 * w + 1] = lo;
    }
    __syncthreads();
    const int i = lane & 15;
    hi = i < nw ? slot[2 * i] : 0.0;
    lo = i < nw ? slot[2 * i + 1] : 0.0;
    GroupReduce<16>().sum_dd(hi, lo);
  }
};

// The bf16 gate table into the workgroup's LDS: 32 KiB copied from the
// library's constant table in 16-byte pieces.
__device__ __forceinline__ void fill_gate_tab(uint4* tab) {
  const uint4* src = reinterpret_cast<const uint4*>(kGateTabBits);
  for (int j = threadIdx.x; j < kGateTab / 4; j += blockDim.x) tab[j] = src[j];
}

// ---------------------------------------------------------------- the kernel

// Start of a row in a tensor. With one row per workgroup, or per 64-lane
// group (a whole wavefront), the row is the same in every lane of a
// wavefront, and its offset goes to scalar registers (SGPR base + 32-bit lane
// offsets instead of a 64-bit address computed per lane).
template <int G, class T>
__device__ __forceinline__ T* row_ptr(T* base, size_t off) {
  if constexpr (G == 0 || G == 64) return base + uniform_u64(off);
  return base + off;
}

// Rounded-once binary32 sum of squares of a row (see above). The rare
// double-double pass recomputes the lane's own row values one element at a
// time through `elem(k, i)` (re-reading memory, not registers), so it adds no
// registers to the common path.
template <int K, class Red, class Elem>
__device__ __forceinline__ float row_sum_squares_dd(int lane, int L, int V, const Red& red,
                                                    const Elem& elem) {
  double hi = 0.0, lo = 0.0;
#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    if (lane + k * L >= V) continue;  // a clamped copy past the row end
#pragma unroll 1
    for (int i = 0; i < 8; ++i) {
      const double d = (double)elem(k, i);
      dd_add(hi, lo, d * d, 0.0);
    }
  }
  red.sum_dd(hi, lo);
  return dd_to_f32(hi, lo);
}

template <int K, class Red, class Elem>
__device__ __forceinline__ float row_sum_squares(double acc, int32_t width, int parity,
                                                 int lane, int L, int V, const Red& red,
                                                 const Elem& elem) {
  const double S = red.sum(acc, parity);
  const float ss = (float)S;
  // float64 error of a sum of `width` non-negative terms is below width * 2^-53 * S
  if (near_f32_midpoint(S, width))  // uniform over the row
    return row_sum_squares_dd<K>(lane, L, V, red, elem);
  return ss;
}

// Each lane group (G lanes, or the whole workgroup when G == 0) walks its
// rows, rows_per_group consecutive ones or (interleaved) every groups-th one,
// and loads the next row's x and residual before it reduces and stores the
// current one, so load latency overlaps the previous row's work. With one row
// per lane group, or interleaved rows, the rows in flight across the GPU form
// one window of the tensor. Loads use clamped indices and are never predicated,
// so every load of a row is in flight at once; only the stores of vectors past
// the row end (hidden not a multiple of 8 * lanes) are skipped.
//
// Register budget, in wavefronts per SIMD: 7 (<= 72 VGPRs) for one vector per
// lane; 6 (<= 80) for the swizzled NVFP4 epilogue on 32-lane groups, which
// at 72 spilled three 64-bit values, one of them reloaded inside the row loop
// behind a wait for every load in flight (the next row's prefetch included);
// 4 (<= 128) for two or more vectors per lane and for the gated variants
// (their binary64 exp needs the registers). Of the instantiations the host
// can choose, only the gated one at eight vectors per lane spills (five
// values, reloaded on the rare paths only: the double-double sum, the
// division fallbacks).
template <int EPI, int K, int G>
constexpr int tail_waves_per_simd() {
  if (K != 1 || EPI == kEpiGatedNvfp4 || EPI == kEpiGatedNvfp4Lut) return 4;
  return EPI == kEpiNvfp4Swz && G == 32 ? 6 : 7;
}

// NT: 0 no streaming hints; 1 on the row loads and stores (x, residual, norm
// output); 2 also on the code and linear block-scale stores
template <int DT, int EPI, bool NORM, int K, int G, int NT, bool SL = (K >= 4)>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, G > 0 && EPI != kEpiGatedNvfp4Lut ? 256 : 1024),
                               amdgpu_waves_per_eu(tail_waves_per_simd<EPI, K, G>())))
tail_kernel(TailParams p) {
  __shared__ double lds[64];
  __shared__ float mult_tab[128];  // NVFP4: G / value(sf) for every block-scale code
  __shared__ double exp2_tab[64];  // gated: the table of the gate's exp
  const int32_t V = p.vec;
  int lane, L;
  int64_t group;
  if constexpr (G > 0) {
    lane = threadIdx.x & (G - 1);
    L = G;
    // a 64-lane group is a whole wavefront: its index (and so its rows) is
    // made wavefront-uniform here, so row arithmetic runs on the scalar unit
    const uint32_t gw = G == 64 ? __builtin_amdgcn_readfirstlane(threadIdx.x / G) : threadIdx.x / G;
    group = (int64_t)blockIdx.x * (blockDim.x / G) + gw;
  } else {
    lane = threadIdx.x;
    L = blockDim.x;
    group = blockIdx.x;
  }
  // consecutive: rows [group * rows_per_group, + rows_per_group); interleaved:
  // rows group, group + groups, ... (so the rows in flight across the GPU at
  // any time are one contiguous window of the tensor)
  const int64_t groups = G > 0 ? (int64_t)gridDim.x * (blockDim.x / G) : (int64_t)gridDim.x;
  int64_t row, row_end, step;
  if (p.interleave) {
    row = group;
    step = groups;
    row_end = p.tokens;
  } else {
    row = group * p.rows_per_group;
    step = 1;
    row_end = row + p.rows_per_group < p.tokens ? row + p.rows_per_group : p.tokens;
  }
  const int64_t last = p.tokens - 1;

  const uint8_t* x = static_cast<const uint8_t*>(p.x);
  uint8_t* res = static_cast<uint8_t*>(p.residual);
  const uint8_t* gam = static_cast<const uint8_t*>(p.gamma);
  uint8_t* nout = static_cast<uint8_t*>(p.norm_out);
  const size_t row_bytes = (size_t)p.hidden * 2;

  uint32_t voff[K];  // byte offset of each owned vector within a row (clamped)
  bool vok[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int v = lane + k * L;
    vok[k] = v < V;
    voff[k] = (uint32_t)(vok[k] ? v : V - 1) * 16u;
  }
  // the same offset for a run-time k (the rare double-double pass loops over
  // k without unrolling; indexing voff there would put the array in scratch)
  auto vec_off = [&](int k) { return (uint32_t)min(lane + k * L, V - 1) * 16u; };

  constexpr bool kLut = EPI == kEpiGatedNvfp4Lut;  // bf16 z, gate from the LDS table
  constexpr bool kGated = EPI == kEpiGatedNvfp4 || kLut;  // `res` is z: read only, never stored
  constexpr bool kNvfp4 = EPI == kEpiNvfp4 || EPI == kEpiNvfp4Swz || kGated;
  // The streamlined row (SL: 4 or 8 vectors per lane, and 2 when a workgroup
  // takes one row) keeps only what the next step needs in registers: the row's
  // vectors are loaded at the top of each row (no prefetch of the next one),
  // the residual is held packed in T (it is the stored value, so unpacking it
  // again is exact), and gamma is loaded after the sum of squares. Holding all
  // of it at once spilled: at bf16 [2048, 32768] and [1024, 65536] the kernel
  // streamed at 4.0 and 1.1 TB/s. The gated variants (groups wider than 16384)
  // take a row of the same shape: u is binary32 (no stored value), held across
  // the reduction at four vectors per lane and recomputed at eight. With the
  // prefetch they spilled 34 and 571 VGPRs.
  constexpr bool kWide = SL && !kGated;
  constexpr bool kWideGated = SL && kGated;
  constexpr bool kReload = kWide && K >= 8;

  U4 gv[K], xv[K], rv[K];
  if constexpr (!kWide && !kWideGated) {
    const size_t rb = (size_t)(row < last ? row : last) * row_bytes;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      gv[k] = ld16(gam + voff[k]);
      xv[k] = ld16s<(NT != 0)>(x + rb + voff[k]);
      rv[k] = ld16s<(NT != 0)>(res + rb + voff[k]);
    }
  }
  const float width_f = (float)p.hidden;  // row width (exact: <= 65536)
  const float inv_w = p.inv_w;            // RN(1 / width)
  float sc = 0.0f, inv_sc = 0.0f;  // FP8: s and RN(1/s); NVFP4: G
  if constexpr (EPI != kEpiNone) {
    sc = *p.scale;
    if constexpr (EPI == kEpiFp8) inv_sc = recip_rn(sc);  // s is a positive normal <= 2^119
  }
  // kLut: the bf16 gate table, kGateTab binary32 entries, in static shared
  // memory (its address is then a constant the LDS reads take as an offset)
  const float* gate_tab = nullptr;
  static_assert(!kLut || DT == kBF16, "the gate table covers bf16 z");
  if constexpr (kNvfp4) {
    fill_mult_tab(mult_tab, sc);
    if constexpr (kGated) fill_exp2_tab(exp2_tab);
    if constexpr (kLut) {
      __shared__ uint4 gate_tab4[kGateTab / 4];
      fill_gate_tab(gate_tab4);
      gate_tab = reinterpret_cast<const float*>(gate_tab4);
    }
    __syncthreads();
  }
  // gamma stays packed in registers (4 per vector) and is unpacked per row:
  // one extra conversion per element buys the registers that keep the
  // two-vector variants at 6 wavefronts per SIMD without spilling.

  typename std::conditional<(G > 0), GroupReduce<(G > 0 ? G : 64)>, BlockReduce>::type red;
  if constexpr (G == 0) red.lds = lds;

  // ss / width rounded once, then r = RN(1 / RN(sqrt(mean + eps))): the
  // Markstein-corrected quotient with RN(1/width) (three operations) inside the
  // range where it holds with margin, the IEEE division outside it (sums near
  // underflow or overflow; rare, and uniform over the row)
  auto row_r = [&](float ss) {
    float mean;
    if (ss >= 0x1p-100f && ss <= 0x1p120f) {
      const float q0 = ss * inv_w;
      const float t = __builtin_fmaf(q0, width_f, -ss);
      mean = __builtin_fmaf(-t, inv_w, q0);
    } else {
      mean = ss / width_f;
    }
    return recip_rn_ext(sqrtf(mean + p.eps));
  };

  // The epilogue of one of the lane's vectors of `row` (in the row, `ok`; at
  // byte offset `off`): the norm output and the codes.
  // Codes and linear block scales carry the streaming hint only with NT == 2
  // (the host's choice: plain epilogues below 32 MiB of x, where at large
  // calls their 8-, 4- and 1-byte stores fill whole lines only once merged in
  // the L2 and the hint measured 3-7% slower; the gate-table epilogue
  // wherever its rows are hinted). The swizzled scale words never take it.
  // (A run-time flag choosing between a hinted and a plain store compiled to
  // the plain store alone: the two stores were merged and the hint dropped.)
  auto emit = [&](int64_t row_, bool ok, uint32_t off, const float (&n)[8]) {
    if constexpr (NORM) {
      if (ok) st16s<(NT != 0)>(row_ptr<G>(nout, (size_t)row_ * row_bytes) + off, pack8<DT>(n));
    }
    if constexpr (EPI == kEpiFp8) {
      uint32_t lo, hi;
      fp8_codes8(n, sc, inv_sc, lo, hi);
      if (ok) st8s<NT == 2>(row_ptr<G>(p.q, (size_t)row_ * p.hidden) + off / 2, lo, hi);
    } else if constexpr (kNvfp4) {
      uint32_t w, sfc;
      nvfp4_half_block(n, sc, mult_tab, w, sfc);
      if constexpr (EPI == kEpiNvfp4Swz) {
        // Four consecutive blocks of a row are one 32-bit word of the swizzled
        // layout. Their codes sit in lanes 8j, 8j+2, 8j+4, 8j+6 (two lanes per
        // block, lane groups a multiple of 8 wide), so lane 8j gathers them
        // and stores the word; codes of vectors past the row end count as 0,
        // which also writes the padded columns of the last word.
        const uint32_t c8 = ok ? (sfc & 0xffu) : 0u;
        const uint32_t word = c8 | ((uint32_t)__shfl_down((int)c8, 2) << 8) |
                              ((uint32_t)__shfl_down((int)c8, 4) << 16) |
                              ((uint32_t)__shfl_down((int)c8, 6) << 24);
        if (ok && (lane & 7) == 0)
          st4s<false>(p.sf + sf_swizzled_offset(row_, (int32_t)(off / 32), p.sf_tiles), word);
      }
      if (ok) {
        st4s<NT == 2>(row_ptr<G>(p.q, (size_t)row_ * (p.hidden / 2)) + off / 4, w);
        if constexpr (EPI != kEpiNvfp4Swz) {
          if ((lane & 1) == 0)  // linear [rows, width/16] (the plain and the gated variants)
            st1s<NT == 2>(row_ptr<G>(p.sf, (size_t)row_ * (p.hidden / 16)) + off / 32,
                          (uint8_t)sfc);
        }
      }
    }
  };

  int parity = 0;
  // gated: the gamma slice of the row, row % gamma_period, kept as a running
  // counter (one modulo for the first row, none per row)
  int32_t gslice = kGated && p.gamma_period > 1 ? (int32_t)(row % p.gamma_period) : 0;
  const int32_t gstep = kGated && p.gamma_period > 1 ? (int32_t)(step % p.gamma_period) : 0;
  for (; row < row_end; row += step, parity ^= 1,
                        gslice = gslice + gstep >= p.gamma_period ? gslice + gstep - p.gamma_period : gslice + gstep) {
    uint8_t* rrow = row_ptr<G>(res, (size_t)row * row_bytes);
    // the rare double-double pass re-reads the lane's own just-stored residual
    // elements (the gated variant recomputes u from x and z below)
    auto stored_h = [&](int k, int i) {
      float f, unused;
      unpack2<DT>((uint32_t)*reinterpret_cast<const volatile uint16_t*>(rrow + vec_off(k) + 2 * i), f, unused);
      return f;
    };
    // gated: the same pass recomputes u from x and z
    auto gated_u = [&](int k, int i) {
      const uint8_t* xrow = row_ptr<G>(x, (size_t)row * row_bytes);
      float xf, zf, unused;
      unpack2<DT>((uint32_t)*reinterpret_cast<const volatile uint16_t*>(xrow + vec_off(k) + 2 * i), xf, unused);
      unpack2<DT>((uint32_t)*reinterpret_cast<const volatile uint16_t*>(rrow + vec_off(k) + 2 * i), zf, unused);
      return silu_gate(xf, zf, exp2_tab);
    };
    if constexpr (kWideGated) {
      static_assert(K == 4 || K == 8, "wide gated rows: four or eight vectors per lane");
      // Four vectors per lane hold u (32 VGPRs) across the reduction. Eight
      // would not fit beside the gate's arithmetic (nor, with the table gate,
      // beside their gamma and the loads in flight): they take the row in two
      // runs of four, in a loop the compiler keeps (unrolled, it overlapped
      // the runs and spilled), and recompute u after the reduction from x and
      // z read again (the lane's own lines, from the cache).
      constexpr bool kHold = K == 4;
      constexpr int kRunUnroll = kHold ? 4 : 1;  // the run loops: unrolled for one run, kept for two
      if constexpr (kHold) {
#pragma unroll
        for (int k = 0; k < K; ++k) asm volatile("" : "+v"(voff[k]));  // as in the wide row below
      }
      const uint8_t* xrow = row_ptr<G>(x, (size_t)row * row_bytes);
      const uint8_t* grow = p.gamma_period > 1 ? gam + (size_t)gslice * row_bytes : gam;
      // vector k's offset and whether it lies in the row: from the unrolled
      // arrays for one run, computed in the kept loop
      auto off_of = [&](int k) -> uint32_t {
        if constexpr (kHold) return voff[k];
        else return vec_off(k);
      };
      auto ok_of = [&](int k) -> bool {
        if constexpr (kHold) return vok[k];
        else return lane + k * L < V;
      };
      // u of the four vectors k0 .. k0 + 3, from x and z loaded together
      auto run_u = [&](int k0, float (&ur)[4][8], bool hint) {
        U4 xw[4], zw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t off = off_of(k0 + j);
          xw[j] = hint ? ld16s<(NT != 0)>(xrow + off) : ld16(xrow + off);
          zw[j] = hint ? ld16s<(NT != 0)>(rrow + off) : ld16(rrow + off);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float xf[8];
          unpack8<DT>(xw[j], xf);
          if constexpr (kLut) {
            gate_lut8(xf, zw[j], gate_tab, exp2_tab, ur[j]);  // binary32 u, looked up
          } else {
            float zf[8];
            unpack8<DT>(zw[j], zf);
            silu_gate8(xf, zf, exp2_tab, ur[j]);  // binary32 u
          }
        }
      };
      float u[4][8];
      double acc = 0.0;
#pragma unroll kRunUnroll
      for (int k0 = 0; k0 < K; k0 += 4) {
        run_u(k0, u, true);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          double a = 0.0;  // vectors past the row end hold a clamped copy: not counted
#pragma unroll
          for (int i = 0; i < 8; ++i) a = __builtin_fma((double)u[j][i], (double)u[j][i], a);
          acc += ok_of(k0 + j) ? a : 0.0;
        }
      }
      U4 gw[4];
      if constexpr (kHold) {
#pragma unroll
        for (int j = 0; j < 4; ++j) gw[j] = ld16(grow + voff[j]);  // lands during the reduction
      }
      const float r = row_r(row_sum_squares<K>(acc, p.hidden, parity, lane, L, V, red, gated_u));
#pragma unroll kRunUnroll
      for (int k0 = 0; k0 < K; k0 += 4) {
        if constexpr (!kHold) {
#pragma unroll
          for (int j = 0; j < 4; ++j) gw[j] = ld16(grow + off_of(k0 + j));
          run_u(k0, u, false);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float g[8], n[8];
          unpack8<DT>(gw[j], g);
#pragma unroll
          for (int i = 0; i < 8; ++i) n[i] = (u[j][i] * r) * g[i];
          emit(row, ok_of(k0 + j), off_of(k0 + j), n);
        }
      }
    } else if constexpr (kWide) {
      // Opaque per row (4 and 8 vectors per lane): otherwise the compiler
      // hoists a 64-bit address per vector and output stream (base + offset)
      // out of the row loop, which at 8 vectors per lane costs more registers
      // than the row itself. At 2 vectors the hoisted form measured faster.
      if constexpr (K >= 4) {
#pragma unroll
        for (int k = 0; k < K; ++k) asm volatile("" : "+v"(voff[k]));
      }
      const uint8_t* xrow = row_ptr<G>(x, (size_t)row * row_bytes);
      U4 hv[K];
      double acc = 0.0;
      {
        U4 xw[K], rw[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
          xw[k] = ld16s<(NT != 0)>(xrow + voff[k]);
          rw[k] = ld16s<(NT != 0)>(rrow + voff[k]);
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
          float xf[8], rf[8], s[8], h[8];
          unpack8<DT>(xw[k], xf);
          unpack8<DT>(rw[k], rf);
#pragma unroll
          for (int i = 0; i < 8; ++i) s[i] = xf[i] + rf[i];
          hv[k] = pack8<DT>(s);
          if (vok[k]) st16s<(NT != 0)>(rrow + voff[k], hv[k]);
          unpack8<DT>(hv[k], h);
          double a = 0.0;  // vectors past the row end hold a clamped copy: not counted
#pragma unroll
          for (int i = 0; i < 8; ++i) a = __builtin_fma((double)h[i], (double)h[i], a);
          acc += vok[k] ? a : 0.0;
        }
      }
      U4 gw[K];
#pragma unroll
      for (int k = 0; k < K; ++k) gw[k] = ld16(gam + voff[k]);  // lands during the reduction
      const float r = row_r(row_sum_squares<K>(acc, p.hidden, parity, lane, L, V, red, stored_h));
#pragma unroll
      for (int k = 0; k < K; ++k) {
        float h[8], g[8], n[8];
        // at 8 vectors per lane the residual is read back (the lane's own
        // just-stored vector, from the cache) instead of held across the sum
        unpack8<DT>(kReload ? ld16(rrow + voff[k]) : hv[k], h);
        unpack8<DT>(gw[k], g);
#pragma unroll
        for (int i = 0; i < 8; ++i) n[i] = (h[i] * r) * g[i];
        emit(row, vok[k], voff[k], n);
      }
    } else {
    if constexpr (kGated) {  // each group of a token has its own gamma slice
      if (p.gamma_period > 1) {
        const uint8_t* grow = gam + (size_t)gslice * row_bytes;
#pragma unroll
        for (int k = 0; k < K; ++k) gv[k] = ld16(grow + voff[k]);
      }
    }
    float h[K][8];
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float xf[8], rf[8];
      unpack8<DT>(xv[k], xf);
      unpack8<DT>(rv[k], rf);
      if constexpr (kLut) {
        gate_lut8(xf, rv[k], gate_tab, exp2_tab, h[k]);  // binary32 u, looked up
      } else if constexpr (kGated) {
        silu_gate8(xf, rf, exp2_tab, h[k]);  // binary32 u
      } else {
        float s[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] = xf[i] + rf[i];
        const U4 hv = pack8<DT>(s);
        if (vok[k]) st16s<(NT != 0)>(rrow + voff[k], hv);
        unpack8<DT>(hv, h[k]);
      }
      double a = 0.0;  // vectors past the row end hold a clamped copy: not counted
#pragma unroll
      for (int i = 0; i < 8; ++i) a = __builtin_fma((double)h[k][i], (double)h[k][i], a);
      acc += vok[k] ? a : 0.0;
    }
    // Prefetch this group's next row into the registers just freed; it lands
    // while this row is reduced, normalised and stored.
    if (row + step < row_end) {
      const uint8_t* xn = row_ptr<G>(x, (size_t)(row + step) * row_bytes);
      const uint8_t* rn = row_ptr<G>(res, (size_t)(row + step) * row_bytes);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        xv[k] = ld16s<(NT != 0)>(xn + voff[k]);
        rv[k] = ld16s<(NT != 0)>(rn + voff[k]);
      }
    }

    float ss;
    if constexpr (kGated) {
      ss = row_sum_squares<K>(acc, p.hidden, parity, lane, L, V, red, gated_u);
    } else {
      ss = row_sum_squares<K>(acc, p.hidden, parity, lane, L, V, red, stored_h);
    }
    const float r = row_r(ss);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float g[8], n[8];
      unpack8<DT>(gv[k], g);
#pragma unroll
      for (int i = 0; i < 8; ++i) n[i] = (h[k][i] * r) * g[i];
      emit(row, vok[k], voff[k], n);
    }
    }
  }
  if constexpr (EPI == kEpiNvfp4Swz) {  // lane groups share the padded rows
    zero_padded_scale_rows(p.sf, p.tokens, p.sf_tiles, group, groups, lane, L);
  }
}

// ---------------------------------------------------------------- dispatch

template <int DT, int EPI, bool NORM, int NT>
static hipError_t launch4(const TailParams& p, const Tiling& t, hipStream_t s) {
  void* args[] = {const_cast<TailParams*>(&p)};
  const void* fn = nullptr;
  // (group, vectors per lane) pairs without a kernel leave fn null: an error,
  // never a kernel that covers part of the row
  if (t.group == 16 && t.vec_per_lane == 1) fn = (const void*)&tail_kernel<DT, EPI, NORM, 1, 16, NT>;
  else if (t.group == 32 && t.vec_per_lane == 1) fn = (const void*)&tail_kernel<DT, EPI, NORM, 1, 32, NT>;
  else if (t.group == 64 && t.vec_per_lane == 1) fn = (const void*)&tail_kernel<DT, EPI, NORM, 1, 64, NT>;
  else if (t.group == 64 && t.vec_per_lane == 2) fn = (const void*)&tail_kernel<DT, EPI, NORM, 2, 64, NT>;
  else if (t.group == 0 && t.vec_per_lane == 1) fn = (const void*)&tail_kernel<DT, EPI, NORM, 1, 0, NT>;
  else if (t.group == 0 && t.vec_per_lane == 2) {
    // one row per workgroup: the streamlined row (no prefetch to keep); bf16
    // [1024, 12288] NVFP4 + norm 24.3 -> 21.9 us, [64, 16384] 6.2 -> 5.8. With
    // two or more rows the prefetching row is faster ([4096, 16384] 99.7
    // against 102.4 us).
    constexpr bool kGatedEpi = EPI == kEpiGatedNvfp4 || EPI == kEpiGatedNvfp4Lut;
    if constexpr (!kGatedEpi) {
      if (t.rows == 1) fn = (const void*)&tail_kernel<DT, EPI, NORM, 2, 0, NT, true>;
    }
    if (!fn) fn = (const void*)&tail_kernel<DT, EPI, NORM, 2, 0, NT>;
  }
  else if (t.group == 0 && t.vec_per_lane == 4) fn = (const void*)&tail_kernel<DT, EPI, NORM, 4, 0, NT>;
  else if (t.group == 0 && t.vec_per_lane == 8) fn = (const void*)&tail_kernel<DT, EPI, NORM, 8, 0, NT>;
  if (!fn) return hipErrorInvalidConfiguration;
  return hipLaunchKernel(fn, dim3((unsigned)t.grid), dim3((unsigned)t.block), args, 0, s);
}

template <int DT, int EPI, bool NORM>
static hipError_t launch3(const TailParams& p, const Tiling& t, hipStream_t s) {
  if (!t.stream) return launch4<DT, EPI, NORM, 0>(p, t, s);
  // the code-store hint exists for the plain FP8 and NVFP4 epilogues and the
  // gate-table one
  if constexpr (EPI == kEpiFp8 || EPI == kEpiNvfp4 || EPI == kEpiGatedNvfp4Lut) {
    if (t.stream_codes) return launch4<DT, EPI, NORM, 2>(p, t, s);
  }
  return launch4<DT, EPI, NORM, 1>(p, t, s);
}

template <int DT, int EPI>
static hipError_t launch2(bool norm, const TailParams& p, const Tiling& t, hipStream_t s) {
  return norm ? launch3<DT, EPI, true>(p, t, s) : launch3<DT, EPI, false>(p, t, s);
}

template <int DT>
static hipError_t launch1(int epi, bool norm, const TailParams& p, const Tiling& t, hipStream_t s) {
  if (epi == kEpiNone) return launch3<DT, kEpiNone, true>(p, t, s);  // add + RMSNorm only
  if (epi == kEpiNvfp4Swz) return launch2<DT, kEpiNvfp4Swz>(norm, p, t, s);
  if (epi == kEpiGatedNvfp4) return launch3<DT, kEpiGatedNvfp4, false>(p, t, s);  // no norm out
  if constexpr (DT == kBF16) {
    if (epi == kEpiGatedNvfp4Lut) return launch3<DT, kEpiGatedNvfp4Lut, false>(p, t, s);
  }
  if (epi == kEpiGatedNvfp4Lut) return hipErrorInvalidValue;  // the table covers bf16 z only
  return epi == kEpiFp8 ? launch2<DT, kEpiFp8>(norm, p, t, s) : launch2<DT, kEpiNvfp4>(norm, p, t, s);
}

int launch_tail(int dtype, int epi, bool norm, const TailParams& p_in, const Tiling& t,
                void* stream) {
  TailParams p = p_in;
  p.inv_w = 1.0f / (float)p.hidden;  // IEEE binary32 division on the host
  hipStream_t s = static_cast<hipStream_t>(stream);
  return (int)(dtype == kBF16 ? launch1<kBF16>(epi, norm, p, t, s)
                              : launch1<kF16>(epi, norm, p, t, s));
}

}  // namespace anq
