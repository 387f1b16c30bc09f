// Tiling choice of every launch: plain host C++, so that the front end and
// its choices can be built and checked on a machine without a GPU.
//
// Each pick_* returns ANQ_OK, ANQ_ERR_SHAPE (a grid past 2^31 - 1 workgroups)
// or ANQ_ERR_CONFIG. The ANQ_* environment variables below override a choice,
// for sweeps and A/B runs. An override is either taken exactly or refused: a
// value that is not a complete integer in range, or that names a tiling no
// kernel has, makes the call fail with ANQ_ERR_CONFIG before anything is
// enqueued (never a silent fallback to the default, and never a kernel that
// covers only part of a row). Every accepted choice gives identical results.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/addnormq.h"
#include "anq_internal.h"

namespace anq {

namespace {

// An integer tuning variable: unset or empty leaves *v as it is; a complete
// decimal integer in [lo, hi] is stored in *v; anything else is refused.
bool env_int(const char* name, int lo, int hi, int* v) {
  const char* s = getenv(name);
  if (!s || !*s) return true;
  char* end = nullptr;
  const long x = strtol(s, &end, 10);
  if (*end != '\0' || x < lo || x > hi) return false;
  *v = (int)x;
  return true;
}

// ANQ_STREAM: "0" or "1" when set.
bool env_stream(bool* stream) {
  int v = *stream ? 1 : 0;
  if (!env_int("ANQ_STREAM", 0, 1, &v)) return false;
  *stream = v == 1;
  return true;
}

bool env_interleave(bool* il) {
  int v = *il ? 1 : 0;
  if (!env_int("ANQ_ROW_ORDER", 0, 1, &v)) return false;
  *il = v == 1;
  return true;
}

bool env_stream_codes(bool* codes) {
  int v = *codes ? 1 : 0;
  if (!env_int("ANQ_STREAM_CODES", 0, 1, &v)) return false;
  *codes = v == 1;
  return true;
}

constexpr int64_t kMaxGrid = 0x7FFFFFFF;

// The tail kernels that exist: (group, vectors per lane) =
// (16, 1), (32, 1), (64, 1), (64, 2), and (0, 1 / 2 / 4 / 8) with at most
// 1024 lanes per workgroup; a lane group must cover the row.
bool tail_kernel_exists(int g, int k, int32_t vec) {
  if (g == 0) return (k == 1 || k == 2 || k == 4 || k == 8) && (vec + k - 1) / k <= 1024;
  if (g == 16 || g == 32) return k == 1 && g >= vec;
  if (g == 64) return (k == 1 || k == 2) && g * k >= vec;
  return false;
}

bool finish_grid(int64_t rows, int64_t groups_per_block, Tiling* t) {
  while ((rows + groups_per_block * t->rows - 1) / (groups_per_block * t->rows) > kMaxGrid)
    t->rows *= 2;
  t->grid = (rows + groups_per_block * t->rows - 1) / (groups_per_block * t->rows);
  return true;
}

}  // namespace

// Tiling by row width (vec = hidden / 8 vectors of 16 bytes), one vector per
// lane wherever a row fits in a workgroup:
//   vec <= 16, 32, 64 : 16, 32, 64 lanes of a wavefront per row
//   vec <= 1024       : a workgroup of vec lanes (rounded up to 64) per row
//   larger            : a workgroup of up to 1024 lanes, 2, 4 or 8 vectors each
// and rows per lane group chosen so that a small grid still fills the GPU.
// ANQ_TAIL_TILING="G:K" (G lanes per row, 0 = a workgroup; K vectors per lane),
// ANQ_ROWS_PER_GROUP (>= 1), ANQ_ROW_ORDER (0 consecutive / 1 interleaved),
// ANQ_STREAM and ANQ_STREAM_CODES (0 / 1) override the choice.
int pick_tail_tiling(int32_t vec, int64_t tokens, bool swizzled, Tiling* out) {
  Tiling t{};
  if (vec <= 64) {
    t.group = vec <= 16 ? 16 : (vec <= 32 ? 32 : 64);
    t.vec_per_lane = 1;
  } else {
    t.group = 0;
    t.vec_per_lane = vec <= 1024 ? 1 : (vec <= 2048 ? 2 : (vec <= 4096 ? 4 : 8));
    // rows of 4104 to 8184 elements, many of them: two vectors per lane and
    // one row per workgroup. bf16 NVFP4 + norm output, inputs from HBM, same
    // GPU: [8192, 7168] 85.8 -> 82.7 us, [4096, 7168] 47.6 -> 44.9, [16384,
    // 7168] 158.6 -> 157.4, [8192, 5120] 62.8 -> 61.1, [4096, 4608] 31.5 ->
    // 30.5, [8192, 6144] 71.6 -> 72.1 (the one loss). Not with the swizzled
    // scales: [8192, 7168] 84.1 -> 86.7 us.
    if (vec > 512 && vec < 1024 && tokens >= 2048 && !swizzled) t.vec_per_lane = 2;
  }
  if (const char* o = getenv("ANQ_TAIL_TILING")) {
    if (*o) {
      int g = -1, k = -1, n = 0;
      if (sscanf(o, "%d:%d%n", &g, &k, &n) != 2 || o[n] != '\0' || !tail_kernel_exists(g, k, vec))
        return ANQ_ERR_CONFIG;
      t.group = g;
      t.vec_per_lane = k;
    }
  }
  int64_t groups_per_block;
  if (t.group > 0) {
    t.block = 256;
    groups_per_block = 256 / t.group;
  } else {
    const int lanes = (vec + t.vec_per_lane - 1) / t.vec_per_lane;
    t.block = (lanes + 63) / 64 * 64;
    // 13 to 15 wavefronts of one vector per lane, 1024 rows or more: padded
    // to 16 (four per SIMD; the extra lanes own no vector). bf16 NVFP4 + norm,
    // 1024 tokens, one GPU: hidden 6656 13.6 -> 13.1 us, 7168 14.5 -> 13.8
    // (f16 14.4 -> 13.6, FP8 14.9 -> 14.4), 7680 14.5 -> 14.4; [1900, 7168]
    // 23.3 -> 22.8. At 512 tokens and fewer it measured 0.5-1.5% slower, and
    // 10 or 12 wavefronts padded to 16 measured 3-6% slower.
    if (t.vec_per_lane == 1 && t.block >= 13 * 64 && t.block < 1024 && tokens >= 1024)
      t.block = 1024;
    groups_per_block = 1;
  }
  // wide rows: two rows per workgroup once there are rows enough to spare, so
  // the second row's loads overlap the first row's reduction and stores (one
  // vector per lane; with two, one row per workgroup measured faster above)
  t.rows = (t.group == 0 && t.block >= 512 && tokens >= 4096 && t.vec_per_lane == 1) ? 2 : 1;
  if (!env_int("ANQ_ROWS_PER_GROUP", 1, 1 << 20, &t.rows)) return ANQ_ERR_CONFIG;
  // several rows per lane group: interleaved across the grid, so the rows in
  // flight stay one window of the tensor. bf16 with norm output, inputs from
  // HBM, one GPU, two rows per workgroup, consecutive -> interleaved: NVFP4
  // [8192, 8192] 93.1 -> 90.6-91.6 us, [16384, 4096] 92.4-92.8 -> 91.3,
  // [32768, 4096] 181.5 -> 178.2; FP8 [8192, 4096] 49.4-49.5 -> 49.0,
  // [4096, 8192] 48.8-49.0 -> 48.6-48.9
  t.interleave = t.rows > 1;
  // streaming hints from 1 MiB of x. With inputs coming from HBM they measured
  // 10-15% faster from 1 to 32 MiB of x on MI355X (fp16 [256, 8192] NVFP4 5.25
  // -> 4.65 us, [64, 8192] 4.08 -> 3.88) and 3% slower at 256 KiB; with inputs
  // already in cache, 0-5% slower.
  t.stream = (int64_t)vec * 16 * tokens >= ((int64_t)1 << 20);
  if (!env_stream(&t.stream)) return ANQ_ERR_CONFIG;
  // the hint on the code and linear scale stores too, for calls below 32 MiB
  // of x: there the kernel's end waits on what its stores left dirty in the
  // L2s. 20-call graphs from HBM, one GPU, off -> on: fp16 NVFP4 [64, 8192]
  // 4.29 -> 4.08 us, [256, 8192] 4.96 -> 4.88, [1024, 8192] 11.95 -> 12.09,
  // [2048, 8192] 21.2 -> 21.1; bf16 FP8 [256, 4096] 4.23 -> 3.93, [2048,
  // 4096] 12.47 -> 12.08, [4096, 4096] 21.33 -> 21.49; bf16 NVFP4 + norm
  // [1024, 7168] 14.37 -> 14.17, [2048, 7168] 24.16 -> 24.18, [4096, 7168]
  // 43.5 -> 44.1. At [65536, 1024] FP8 and [8192, 7168] NVFP4 it measured 7%
  // and 3% slower, and the swizzled scale words 28% slower at [64, 8192].
  t.stream_codes = t.stream && !swizzled && (int64_t)vec * 16 * tokens < ((int64_t)32 << 20);
  if (!env_stream_codes(&t.stream_codes)) return ANQ_ERR_CONFIG;
  if (!env_interleave(&t.interleave)) return ANQ_ERR_CONFIG;
  finish_grid(tokens, groups_per_block, &t);
  *out = t;
  return ANQ_OK;
}

// Tiling of the gated variant with the gate table (rows <= 1024 elements):
// lane groups of 16/32/64 lanes, one or two vectors per lane, in 512-lane
// workgroups (one 32 KiB table per 8 wavefronts), each lane group taking
// enough rows that about 512 workgroups cover the call (1024 once that still
// leaves 8 or more rows per group), so each workgroup copies its table once
// for many rows. The rows are interleaved: lane group i takes rows i, i +
// groups, ..., so the rows in flight across the GPU form one window that
// sweeps the tensor. bf16, inputs from HBM, one GPU, consecutive ->
// interleaved rows (512 workgroups): [2048, 8192] groups of 1024 22.0 -> 18.7
// us, [4096, 8192] 37.7 -> 33.0, [16384, 8192] 136.1 -> 119.9, [8192, 4096]
// groups of 128 36.1 -> 34.0; then 1024 workgroups at [8192, 8192] groups of
// 1024 66.1 -> 63.9, of 512 63.2 -> 59.9, [8192, 4096] groups of 128 34.3 ->
// 32.3. 256 and 1024 lanes per workgroup measured no better (320, 384, 768:
// 74-85 us).
// Wider rows (1040 to 65536 elements) take one workgroup per row, one vector
// per lane (two past 8192, four past 16384, eight past 32768), in about two
// waves of resident workgroups:
// 512 times the workgroups a CU holds (4 wavefronts per SIMD, four tables of
// LDS).
// bf16, one GPU, grid halved / as chosen / doubled: [8192, 8192] in one group
// 62.8 (as chosen) against 66.9 (doubled); in groups of 4096 63.9 / 62.9 /
// 63.5 us; [4096, 5120] in one group 24.3 (as chosen) against 31.6 (doubled).
// Two vectors per lane against the computed gate, one group per row: [2048,
// 16384] 58.7 -> 35.8 us, [4096, 12288] 93 -> 56. Four and eight: [256,
// 32768] 16.1 -> 12.3 us, [1024, 32768] 55.8 -> 40.0, [256, 65536] 43.3 ->
// 32.5, [1024, 65536] 159 -> 111, [32, 65536] 34.5 -> 19.8.
// ANQ_GATE_BLOCK (a multiple of 64, 64 to 1024; lane-group tilings only),
// ANQ_ROWS_PER_GROUP, ANQ_ROW_ORDER and ANQ_STREAM override.
int pick_gate_lut_tiling(int32_t vec, int64_t rows, Tiling* out) {
  Tiling t{};
  int block = 512;
  if (!env_int("ANQ_GATE_BLOCK", 64, 1024, &block) || block % 64 != 0) return ANQ_ERR_CONFIG;
  int64_t groups_per_block;
  int64_t r;
  if (vec <= 128) {
    t.group = vec <= 16 ? 16 : (vec <= 32 ? 32 : 64);
    t.vec_per_lane = vec <= 64 ? 1 : 2;
    t.block = block;
    groups_per_block = t.block / t.group;
    r = rows / (groups_per_block * 512);
    if (r >= 16) r /= 2;
  } else if (vec <= 8192) {
    t.group = 0;
    t.vec_per_lane = vec <= 1024 ? 1 : (vec <= 2048 ? 2 : (vec <= 4096 ? 4 : 8));
    t.block = ((vec + t.vec_per_lane - 1) / t.vec_per_lane + 63) / 64 * 64;
    groups_per_block = 1;
    const int waves = t.block / 64;
    const int per_cu = 16 / waves < 4 ? 16 / waves : 4;
    r = rows / (512 * (int64_t)per_cu);
  } else {
    return ANQ_ERR_UNSUPPORTED;  // past the widest row
  }
  t.rows = (int)(r < 1 ? 1 : (r > 64 ? 64 : r));
  t.interleave = true;
  if (!env_int("ANQ_ROWS_PER_GROUP", 1, 1 << 20, &t.rows)) return ANQ_ERR_CONFIG;
  // streaming hints from 1 MiB of x, as in the tail tiling (bf16 groups of
  // 1024, inputs from HBM: [2048, 1024] 6.33 -> 6.04 us, [2048, 8192] 25.6 ->
  // 24.1, [1024, 8192] 16.4 -> 16.9)
  t.stream = (int64_t)vec * 16 * rows >= ((int64_t)1 << 20);
  if (!env_stream(&t.stream)) return ANQ_ERR_CONFIG;
  // the hint on the code and linear scale stores too, wherever the rows take
  // it: bf16, one GPU, [4096, 5120] in one group 24.2 -> 22.8 us; no change
  // at [8192, 8192] and [2048, 8192] in groups of 1024 (63.0-63.7, 19.0 us)
  t.stream_codes = t.stream;
  if (!env_stream_codes(&t.stream_codes)) return ANQ_ERR_CONFIG;
  if (!env_interleave(&t.interleave)) return ANQ_ERR_CONFIG;
  finish_grid(rows, groups_per_block, &t);
  *out = t;
  return ANQ_OK;
}

// Wavefronts per token W: one once the call has enough tokens to fill the GPU
// (~2048 wavefronts), more for fewer tokens; and at least enough that no
// wavefront takes more than 4 head groups, all of whose loads it issues at
// once. Measured on MI355X (graph of 200 calls, bf16, 4096 tokens): 16+8+8
// heads of 128 (4 groups) 11.0 us with one wavefront per token, 12.4 with the
// cap at 3 or 2 (two wavefronts); 64+8+8 heads (10 groups) 25.3, 25.0 and 26.1
// us with the cap at 4, 3 and 2. 256-lane workgroups: 512 lanes measured 11.4
// us. Streaming hints at every size: 16+8+8 heads of 128 (bf16) measured
// faster with them from 64 to 4096 tokens, with inputs from HBM (64: 3.48 ->
// 3.31 us, 2048: 9.31 -> 7.49) and with inputs in cache alike (2048: 6.97 ->
// 6.62). ANQ_QK_WAVES (>= 1), ANQ_QK_GROUPS (the cap, 1-4), ANQ_QK_BLOCK (a
// multiple of 64, 64 to 1024) and ANQ_STREAM override.
int pick_qk_tiling(const QKParams& p, QKTiling* out) {
  QKTiling t{};
  const int hpp = 64 / (p.head_dim / 16);  // heads per pass of a wavefront
  const int passes = (p.nq + p.nk + p.nv + hpp - 1) / hpp;
  const int64_t want = p.tokens > 0 ? (2048 + p.tokens - 1) / p.tokens : 1;
  int W = (int)(want < passes ? want : passes);
  int cap = 4, block = 256;
  if (!env_int("ANQ_QK_WAVES", 1, 1 << 20, &W)) return ANQ_ERR_CONFIG;
  if (!env_int("ANQ_QK_GROUPS", 1, 4, &cap)) return ANQ_ERR_CONFIG;
  if (W < (passes + cap - 1) / cap) W = (passes + cap - 1) / cap;
  if (W > passes) W = passes;
  if (W < 1) W = 1;
  t.waves_per_token = W;
  t.groups = (passes + W - 1) / W;  // the most any wavefront takes (<= cap)
  if (!env_int("ANQ_QK_BLOCK", 64, 1024, &block) || block % 64 != 0) return ANQ_ERR_CONFIG;
  if (block < p.head_dim / 4) block = p.head_dim / 4;  // one gamma vector per thread (D <= 512)
  t.block = block;
  const int64_t wpb = block / 64;
  t.grid = (p.tokens * W + wpb - 1) / wpb;
  if (t.grid > kMaxGrid) return ANQ_ERR_SHAPE;
  t.stream = true;
  if (!env_stream(&t.stream)) return ANQ_ERR_CONFIG;
  *out = t;
  return ANQ_OK;
}

// One thread per 16-byte vector (and, with the swizzled scales, one per padded
// scale word), 256-thread workgroups; the streaming hint on the input once it
// is >= 32 MiB (ANQ_STREAM overrides).
int pick_quant_tiling(int epi, const QuantParams& p, QuantTiling* out) {
  QuantTiling t{};
  t.stream = p.vecs * 16 >= ((int64_t)32 << 20);
  if (!env_stream(&t.stream)) return ANQ_ERR_CONFIG;
  const int64_t threads = p.vecs + (epi == kEpiNvfp4Swz ? p.pad_rows * p.sf_tiles : 0);
  t.grid = (threads + 255) / 256;
  if (t.grid > kMaxGrid) return ANQ_ERR_SHAPE;
  *out = t;
  return ANQ_OK;
}

}  // namespace anq
