// Interface between the C-ABI front end (anq_api.cpp, host C++), the tiling
// choice (anq_tiling.cpp, host C++) and the kernels' launchers (the .hip files).
//
// Nothing here needs the HIP headers: streams travel as void* (a hipStream_t)
// and launch results as int (0 for hipSuccess, else the HIP error code), so the
// front end and the tiling compile as plain host C++. That is also how they are
// built with the host sanitizers, against stand-in launchers that record what
// would have been launched.
#pragma once

#include <stdint.h>

namespace anq {

constexpr int kF16 = 0;
constexpr int kBF16 = 1;

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
  int32_t interleave;   // 1: lane group i takes rows i, i + groups, ... instead
  int32_t sf_tiles;    // swizzled NVFP4 scales: 128x4 tiles per tile row
  int32_t gamma_period;  // gated: groups per token; row r uses gamma slice r % period
};

// How a row is spread over lanes: `group` lanes of one wavefront per row
// (16, 32 or 64; the workgroup holds block / group lane groups), or group == 0
// for one row at a time per workgroup of `block` lanes. Each lane owns vectors
// lane + k*lanes, k < vec_per_lane. Each lane group walks `rows` consecutive
// rows, or with `interleave` every (grid lane groups)-th row, loading the next
// while it finishes the current one.
struct Tiling {
  int group;
  int vec_per_lane;
  int block;
  int rows;
  bool interleave;    // rows in grid-stride order (rows then only sizes the grid)
  bool stream;        // non-temporal loads and stores of the row streams
  bool stream_codes;  // the same hint on the code and linear block-scale stores
                      // (plain FP8 and NVFP4 epilogues, gate-table epilogue)
  int64_t grid;
};

// The tiling of a call (anq_tiling.cpp): ANQ_OK, ANQ_ERR_SHAPE for a grid past
// 2^31 - 1 workgroups, or ANQ_ERR_CONFIG when an ANQ_* tuning variable in the
// environment names a tiling no kernel has.
int pick_tail_tiling(int32_t vec, int64_t tokens, bool swizzled_scales, Tiling* t);
int pick_gate_lut_tiling(int32_t vec, int64_t rows, Tiling* t);

int launch_tail(int dtype, int epi, bool norm_out, const TailParams& p, const Tiling& t,
                void* stream);

struct QKParams {
  const void* qkv;
  const void* gamma_q;
  const void* gamma_k;
  const int64_t* positions;
  const float* cos_sin;
  const float* scale;
  uint8_t* out;            // [tokens, heads*D]; with a KV store: Q codes [tokens, nq*D]
  uint8_t* kv;             // KV store only: the pool, num_slots rows
  const int64_t* slots;    // KV store only: [tokens] slot of each token (< 0: no store)
  int64_t num_slots;
  int64_t max_pos;
  float eps;
  int64_t tokens;
  int32_t nq, nk, nv, head_dim;
  int32_t rotary_dim;       // rotated width at the end of each Q/K head (== head_dim: all of it)
  int32_t waves_per_token;  // from the tiling
};

// Where the Q/K op's K and V codes go.
enum QKStore { kStoreNone = 0, kStoreUniform = 1, kStoreMixed = 2 };

struct QKTiling {
  int waves_per_token;  // wavefronts sharing a token's head groups
  int groups;           // the most head groups any wavefront takes (1..4)
  int block;            // workgroup lanes
  bool stream;
  int64_t grid;
};

int pick_qk_tiling(const QKParams& p, QKTiling* t);
int launch_qk(int dtype, int store, const QKParams& p, const QKTiling& t, void* stream);

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

struct QuantTiling {
  bool stream;
  int64_t grid;  // 256-thread workgroups, one thread per vector (and per padded scale word)
};

int pick_quant_tiling(int epi, const QuantParams& p, QuantTiling* t);
int launch_quant(int dtype, int epi, const QuantParams& p, const QuantTiling& t, void* stream);

// u = x * SiLU(z) for vecs * 8 elements (the gate of the gated RMSNorm).
int launch_gate(int dtype, const void* x, const void* z, float* u, int64_t vecs, void* stream);

// Self-check of the device arithmetic: kSelfcheckCounts mismatch counts.
constexpr int kSelfcheckCounts = 4;
int launch_selfcheck(unsigned long long* counts, void* stream);

// A streaming kernel that reads read_bytes and writes write_bytes, 16 bytes per
// lane access, in one pass: the practical ceiling of a given read/write mix.
int launch_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                  bool nt, void* stream);

}  // namespace anq
