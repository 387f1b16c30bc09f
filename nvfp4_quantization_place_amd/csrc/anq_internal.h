// Launch interface between the C-ABI front end (anq_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace anq {

// kEpiNvfp4Swz: NVFP4 with the block scales in the 128x4-tiled GEMM layout
// (its own instantiation, so the linear-layout kernel carries none of its code).
// kEpiGatedNvfp4: the gated variant, n = RMSNorm(x * SiLU(z)) * gamma per row
// of `hidden` (a group), NVFP4 codes; `residual` then holds z (read only).
// kEpiGatedNvfp4Lut: the same with bf16 z and the gate from an 8192-entry LDS
// table (32 KiB of dynamic shared memory), for calls with many rows.
enum Epilogue {
  kEpiFp8 = 0, kEpiNvfp4 = 1, kEpiNone = 2, kEpiNvfp4Swz = 3, kEpiGatedNvfp4 = 4,
  kEpiGatedNvfp4Lut = 5
};

struct TailParams {
  const void* x;
  void* residual;
  const void* gamma;
  const float* scale;  // FP8: s; NVFP4: G
  void* norm_out;      // may be null
  uint8_t* q;
  uint8_t* sf;         // NVFP4 only
  float eps;
  float inv_w;         // RN(1 / hidden), set by launch_tail
  int64_t tokens;
  int32_t hidden;
  int32_t vec;         // hidden / 8: 16-byte vectors per row
  int32_t rows_per_group;  // consecutive rows each lane group processes
  int32_t sf_tiles;    // swizzled NVFP4 scales: 128x4 tiles per tile row
  int32_t gamma_period;  // gated: groups per token; row r uses gamma slice r % period
};

// How a row is spread over lanes: `group` lanes of one wavefront per row
// (16, 32 or 64; the workgroup holds 256 / group lane groups), or group == 0
// for one row at a time per workgroup of `block` lanes. Each lane owns vectors
// lane + k*lanes, k < vec_per_lane. Each lane group walks `rows` consecutive
// rows, loading the next while it finishes the current one.
struct Tiling {
  int group;
  int vec_per_lane;
  int block;
  int rows;
  bool stream;  // non-temporal loads and stores of the row streams
  int64_t grid;
};

Tiling pick_tail_tiling(int32_t vec, int64_t tokens);
Tiling pick_gate_lut_tiling(int32_t vec, int64_t rows);

hipError_t launch_tail(int dtype, int epi, bool norm_out, const TailParams& p, const Tiling& t,
                       hipStream_t stream);

struct QKParams {
  const void* qkv;
  const void* gamma_q;
  const void* gamma_k;
  const int64_t* positions;
  const float* cos_sin;
  const float* scale;
  uint8_t* out;            // [tokens, heads*D]; with a KV store: Q codes [tokens, nq*D]
  uint8_t* kv;             // KV store only: [num_slots, (nk+nv)*D] pool
  const int64_t* slots;    // KV store only: [tokens] slot of each token (< 0: no store)
  int64_t num_slots;
  int64_t max_pos;
  float eps;
  int64_t tokens;
  int32_t nq, nk, nv, head_dim;
  int32_t waves_per_token;  // set by the launcher
};

hipError_t launch_qk(int dtype, bool kv_store, const QKParams& p, hipStream_t stream);

// Standalone quantisation of an activation tensor [tokens, hidden] (the second
// kernel of the separated tail).
struct QuantParams {
  const void* in;
  const float* scale;  // FP8: s; NVFP4: G
  uint8_t* q;
  uint8_t* sf;         // NVFP4 only
  int64_t vecs;        // tokens * hidden / 8
  int64_t tokens;
  int32_t vec;         // hidden / 8
  int32_t sf_tiles;    // swizzled NVFP4 scales: 128x4 tiles per tile row
  int64_t pad_rows;    // swizzled: padded rows past tokens (threads past vecs zero them)
};

hipError_t launch_quant(int dtype, int epi, const QuantParams& p, hipStream_t stream);

// u = x * SiLU(z) for vecs * 8 elements (the gate of the gated RMSNorm).
hipError_t launch_gate(int dtype, const void* x, const void* z, float* u, int64_t vecs,
                       hipStream_t stream);

// Self-check of the device arithmetic: kSelfcheckCounts mismatch counts.
constexpr int kSelfcheckCounts = 4;
hipError_t launch_selfcheck(unsigned long long* counts, hipStream_t stream);

}  // namespace anq
