// C-ABI front end: argument validation (host only, before any HIP call),
// tiling choice and launch. The contract of every entry point is stated in
// include/addnormq.h. Plain host C++: the launchers it calls are declared in
// anq_internal.h and defined next to their kernels.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/addnormq.h"
#include "anq_internal.h"

namespace {

struct Span {
  uintptr_t lo, hi;  // [lo, hi), empty when lo == hi
};

Span span(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlap(const Span& a, const Span& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// outputs[i] must not overlap any other buffer; inputs may overlap each other
bool any_alias(const Span* outs, int n_out, const Span* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j])) return true;
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j])) return true;
  }
  return false;
}

bool valid_dtype(int d) { return d == ANQ_F16 || d == ANQ_BF16; }

bool valid_eps(float eps) { return isfinite(eps) && eps >= 0.0f; }

// Common checks of the two row ops; fills the byte sizes on success.
int check_tail(const void* x, const void* residual, const void* gamma, const float* scale,
               float eps, int64_t tokens, int64_t hidden, int dtype, const void* q,
               const void* norm_out, int64_t* act_bytes) {
  // token-sized buffers may be NULL when there are no tokens (empty tensors)
  if (!gamma || !scale || (tokens != 0 && (!x || !residual || !q))) return ANQ_ERR_NULL;
  if (!valid_dtype(dtype)) return ANQ_ERR_DTYPE;
  if (tokens < 0 || hidden <= 0 || hidden % 16 != 0) return ANQ_ERR_SHAPE;
  if (hidden > ANQ_MAX_HIDDEN) return ANQ_ERR_UNSUPPORTED;
  if (tokens > INT64_MAX / (2 * hidden)) return ANQ_ERR_SHAPE;
  if (!valid_eps(eps)) return ANQ_ERR_VALUE;
  if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(gamma, 16) || !aligned(q, 16) ||
      (norm_out && !aligned(norm_out, 16)) || !aligned(scale, 4))
    return ANQ_ERR_ALIGN;
  *act_bytes = tokens * hidden * 2;
  return ANQ_OK;
}

int launch_status(int e) { return e == 0 ? ANQ_OK : ANQ_ERR_LAUNCH; }

}  // namespace

extern "C" int add_rmsnorm_quant_fp8(const void* x, void* residual, const void* gamma,
                                     const float* scale, float eps, int64_t tokens, int64_t hidden,
                                     anq_dtype dtype, uint8_t* q, void* norm_out, void* stream) {
  int64_t act = 0;
  int st = check_tail(x, residual, gamma, scale, eps, tokens, hidden, dtype, q, norm_out, &act);
  if (st != ANQ_OK) return st;
  const Span outs[3] = {span(residual, act), span(q, tokens * hidden), span(norm_out, norm_out ? act : 0)};
  const Span ins[3] = {span(x, act), span(gamma, hidden * 2), span(scale, 4)};
  if (any_alias(outs, 3, ins, 3)) return ANQ_ERR_ALIAS;
  if (tokens == 0) return ANQ_OK;

  anq::TailParams p{};
  p.x = x;
  p.residual = residual;
  p.gamma = gamma;
  p.scale = scale;
  p.norm_out = norm_out;
  p.q = q;
  p.sf = nullptr;
  p.eps = eps;
  p.tokens = tokens;
  p.hidden = (int32_t)hidden;
  p.vec = (int32_t)(hidden / 8);
  anq::Tiling t;
  if ((st = anq::pick_tail_tiling(p.vec, tokens, false, &t)) != ANQ_OK) return st;
  p.rows_per_group = t.rows;
  p.interleave = t.interleave ? 1 : 0;
  return launch_status(anq::launch_tail(dtype, anq::kEpiFp8, norm_out != nullptr, p, t, stream));
}

namespace {

int64_t sf_tiles_of(int64_t hidden) { return (hidden / 16 + 3) / 4; }

int64_t sf_bytes(int64_t tokens, int64_t hidden, bool swizzled) {
  if (!swizzled) return tokens * (hidden / 16);
  return ((tokens + 127) / 128) * 128 * sf_tiles_of(hidden) * 4;
}

int rmsnorm_nvfp4(const void* x, void* residual, const void* gamma, const float* global_scale,
                  float eps, int64_t tokens, int64_t hidden, int dtype, uint8_t* q, uint8_t* sf,
                  void* norm_out, bool swizzled, void* stream) {
  if (!sf && tokens != 0) return ANQ_ERR_NULL;
  int64_t act = 0;
  int st = check_tail(x, residual, gamma, global_scale, eps, tokens, hidden, dtype, q, norm_out,
                      &act);
  if (st != ANQ_OK) return st;
  if (swizzled && !aligned(sf, 4)) return ANQ_ERR_ALIGN;
  const Span outs[4] = {span(residual, act), span(q, tokens * (hidden / 2)),
                        span(sf, sf_bytes(tokens, hidden, swizzled)),
                        span(norm_out, norm_out ? act : 0)};
  const Span ins[3] = {span(x, act), span(gamma, hidden * 2), span(global_scale, 4)};
  if (any_alias(outs, 4, ins, 3)) return ANQ_ERR_ALIAS;
  if (tokens == 0) return ANQ_OK;

  anq::TailParams p{};
  p.x = x;
  p.residual = residual;
  p.gamma = gamma;
  p.scale = global_scale;
  p.norm_out = norm_out;
  p.q = q;
  p.sf = sf;
  p.eps = eps;
  p.tokens = tokens;
  p.hidden = (int32_t)hidden;
  p.vec = (int32_t)(hidden / 8);
  p.sf_tiles = swizzled ? (int32_t)sf_tiles_of(hidden) : 0;
  anq::Tiling t;
  if ((st = anq::pick_tail_tiling(p.vec, tokens, swizzled, &t)) != ANQ_OK) return st;
  p.rows_per_group = t.rows;
  p.interleave = t.interleave ? 1 : 0;
  return launch_status(anq::launch_tail(dtype, swizzled ? anq::kEpiNvfp4Swz : anq::kEpiNvfp4,
                                        norm_out != nullptr, p, t, stream));
}

}  // namespace

extern "C" int add_rmsnorm_quant_nvfp4(const void* x, void* residual, const void* gamma,
                                       const float* global_scale, float eps, int64_t tokens,
                                       int64_t hidden, anq_dtype dtype, uint8_t* q, uint8_t* sf,
                                       void* norm_out, void* stream) {
  return rmsnorm_nvfp4(x, residual, gamma, global_scale, eps, tokens, hidden, dtype, q, sf,
                       norm_out, false, stream);
}

extern "C" int add_rmsnorm_quant_nvfp4_swizzled(const void* x, void* residual, const void* gamma,
                                                const float* global_scale, float eps,
                                                int64_t tokens, int64_t hidden, anq_dtype dtype,
                                                uint8_t* q, uint8_t* sf, void* norm_out,
                                                void* stream) {
  return rmsnorm_nvfp4(x, residual, gamma, global_scale, eps, tokens, hidden, dtype, q, sf,
                       norm_out, true, stream);
}

extern "C" int gated_rmsnorm_quant_nvfp4(const void* x, const void* z, const void* gamma,
                                         const float* global_scale, float eps, int64_t tokens,
                                         int64_t hidden, int64_t group, anq_dtype dtype, uint8_t* q,
                                         uint8_t* sf, void* stream) {
  if (!gamma || !global_scale || (tokens != 0 && (!x || !z || !q || !sf))) return ANQ_ERR_NULL;
  if (!valid_dtype(dtype)) return ANQ_ERR_DTYPE;
  if (tokens < 0 || hidden <= 0 || group <= 0 || hidden % 16 != 0 || group % 16 != 0 ||
      hidden % group != 0)
    return ANQ_ERR_SHAPE;
  if (group > ANQ_MAX_HIDDEN) return ANQ_ERR_UNSUPPORTED;
  if (tokens > INT64_MAX / (2 * hidden) || hidden / group > INT32_MAX) return ANQ_ERR_SHAPE;
  if (!valid_eps(eps)) return ANQ_ERR_VALUE;
  if (!aligned(x, 16) || !aligned(z, 16) || !aligned(gamma, 16) || !aligned(q, 16) ||
      !aligned(global_scale, 4))
    return ANQ_ERR_ALIGN;
  const int64_t act = tokens * hidden * 2;
  const Span outs[2] = {span(q, tokens * (hidden / 2)), span(sf, tokens * (hidden / 16))};
  const Span ins[4] = {span(x, act), span(z, act), span(gamma, hidden * 2), span(global_scale, 4)};
  if (any_alias(outs, 2, ins, 4)) return ANQ_ERR_ALIAS;
  if (tokens == 0) return ANQ_OK;

  anq::TailParams p{};  // one row per group: [tokens * hidden / group, group]
  p.x = x;
  p.residual = const_cast<void*>(z);  // read only in the gated variant
  p.gamma = gamma;
  p.scale = global_scale;
  p.q = q;
  p.sf = sf;
  p.eps = eps;
  p.tokens = tokens * (hidden / group);
  p.hidden = (int32_t)group;
  p.vec = (int32_t)(group / 8);
  p.gamma_period = (int32_t)(hidden / group);
  // bf16 z and enough work to share a workgroup's table: the gate from the
  // lookup table (ANQ_GATE_LUT=0/1 overrides, for A/B
  // runs). Measured, one GPU: groups of at most 1024 gain 5-14% from 2048 group
  // rows up and lose below 1024 (the 32 KiB copy per workgroup is then not
  // amortised). Wider groups gain from 2^21 elements: bf16 [8192, 8192] in
  // groups of 8192, 4096, 2048 115 / 105 / 107 -> 63 / 63 / 66-68 us, [4096,
  // 5120] in one group 48 -> 24; [256, 8192] one group 6.8 -> 6.2; at 1.5 M
  // elements ([512, 3072], groups of 1536) the table lost, 6.3 -> 7.1. Groups
  // of 12288 and 16384: [4096, 12288] 93 -> 56 us, [2048, 16384] 58.7 -> 35.8;
  // of 32768 and 65536 (four and eight vectors per lane), from [32, 65536]:
  // 1.3-1.7x faster, e.g. [1024, 32768] 55.8 -> 40.0 us. Groups of 8192 and
  // more gain at any size, their rows being long beside the copy: [1, 65536]
  // 30.9 -> 15.0 us, [8, 32768] 11.1 -> 7.5, [4, 16384] 6.9 -> 5.5, [16, 8192]
  // 4.8 -> 4.1, [128, 8192] 6.1 -> 5.4.
  const bool lut_fits = dtype == ANQ_BF16;
  bool lut = lut_fits && (group >= 8192 || p.tokens >= 2048 ||
                          p.tokens * group >= ((int64_t)1 << 21));
  if (const char* e = getenv("ANQ_GATE_LUT")) {
    if (*e) {
      if (strcmp(e, "0") != 0 && strcmp(e, "1") != 0) return ANQ_ERR_CONFIG;
      lut = e[0] == '1' && lut_fits;  // the table covers bf16 z only
    }
  }
  anq::Tiling t;
  const int st = lut ? anq::pick_gate_lut_tiling(p.vec, p.tokens, &t)
                     : anq::pick_tail_tiling(p.vec, p.tokens, false, &t);
  if (st != ANQ_OK) return st;
  p.rows_per_group = t.rows;
  p.interleave = t.interleave ? 1 : 0;
  return launch_status(anq::launch_tail(dtype, lut ? anq::kEpiGatedNvfp4Lut : anq::kEpiGatedNvfp4,
                                        false, p, t, stream));
}

extern "C" int silu_gate_f32(const void* x, const void* z, int64_t n, anq_dtype dtype, float* u,
                             void* stream) {
  if (n != 0 && (!x || !z || !u)) return ANQ_ERR_NULL;
  if (!valid_dtype(dtype)) return ANQ_ERR_DTYPE;
  if (n < 0 || n % 8 != 0 || n > INT64_MAX / 4) return ANQ_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(z, 16) || !aligned(u, 16)) return ANQ_ERR_ALIGN;
  const Span outs[1] = {span(u, n * 4)};
  const Span ins[2] = {span(x, n * 2), span(z, n * 2)};
  if (any_alias(outs, 1, ins, 2)) return ANQ_ERR_ALIAS;
  if (n == 0) return ANQ_OK;
  if ((n / 8 + 255) / 256 > 0x7FFFFFFF) return ANQ_ERR_SHAPE;
  return launch_status(anq::launch_gate(dtype, x, z, u, n / 8, stream));
}

extern "C" int anq_selfcheck_arith(uint64_t* counts, void* stream) {
  if (!counts) return ANQ_ERR_NULL;
  if (!aligned(counts, 8)) return ANQ_ERR_ALIGN;
  static_assert(anq::kSelfcheckCounts == ANQ_SELFCHECK_COUNTS, "count array length");
  return launch_status(anq::launch_selfcheck(reinterpret_cast<unsigned long long*>(counts), stream));
}

namespace {

// Checks shared by the Q/K entry points. `store` is the epilogue (none,
// uniform pool, mixed pool); `out` is the dense code buffer (all heads, or the
// Q heads with a store).
int check_qk(const void* qkv, const void* gamma_q, const void* gamma_k, const int64_t* positions,
             const float* cos_sin, int64_t max_pos, const float* scale, float eps, int64_t tokens,
             int32_t nq, int32_t nk, int32_t nv, int32_t head_dim, int32_t rotary_dim, int dtype,
             const uint8_t* out, int store, const int64_t* slots, int64_t num_slots,
             const uint8_t* kv) {
  const bool kv_store = store != anq::kStoreNone;
  const bool need_out = !kv_store || nq > 0;
  const bool need_kv = kv_store && (int64_t)nk + nv > 0;
  if (!cos_sin || !scale ||
      (tokens != 0 && (!qkv || !positions || (need_out && !out) || (need_kv && (!slots || !kv)))))
    return ANQ_ERR_NULL;
  if (nq > 0 && !gamma_q) return ANQ_ERR_NULL;
  if (nk > 0 && !gamma_k) return ANQ_ERR_NULL;
  if (!valid_dtype(dtype)) return ANQ_ERR_DTYPE;
  if (nq < 0 || nk < 0 || nv < 0 || max_pos < 1 || (kv_store && num_slots < 0))
    return ANQ_ERR_VALUE;
  const int64_t heads = (int64_t)nq + nk + nv;  // in 64 bits: int32 counts may not sum in 32
  if (tokens < 0 || head_dim <= 0 || heads == 0 || heads > (1 << 20)) return ANQ_ERR_SHAPE;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
    return ANQ_ERR_UNSUPPORTED;
  // the rotated width: a power of two from 16 to head_dim (the last rotary_dim
  // elements of each Q/K head rotate); other widths keep a separated path
  if (rotary_dim < 16 || rotary_dim > head_dim || (rotary_dim & (rotary_dim - 1)) != 0)
    return ANQ_ERR_UNSUPPORTED;
  if (!valid_eps(eps)) return ANQ_ERR_VALUE;
  const int64_t cols = heads * head_dim;
  // bytes of one pool row: uniform (nk+nv)*D; mixed nk*(D+R) + nv*D
  const int64_t kv_cols = store == anq::kStoreMixed
                              ? (int64_t)nk * (head_dim + rotary_dim) + (int64_t)nv * head_dim
                              : ((int64_t)nk + nv) * head_dim;
  if (tokens > INT64_MAX / (2 * cols) || max_pos > INT64_MAX / (4 * (int64_t)rotary_dim) ||
      (kv_store && kv_cols > 0 && num_slots > INT64_MAX / kv_cols))
    return ANQ_ERR_SHAPE;
  if (!aligned(qkv, 16) || !aligned(out, 16) || !aligned(cos_sin, 16) || !aligned(positions, 8) ||
      !aligned(scale, 4) || (nq > 0 && !aligned(gamma_q, 16)) || (nk > 0 && !aligned(gamma_k, 16)) ||
      (kv_store && (!aligned(kv, 16) || !aligned(slots, 8))))
    return ANQ_ERR_ALIGN;
  const int64_t out_cols = kv_store ? (int64_t)nq * head_dim : cols;
  const int64_t kv_bytes = need_kv ? num_slots * kv_cols : 0;
  const Span outs[2] = {span(out, tokens * out_cols), span(kv, kv_bytes)};
  const Span ins[7] = {span(qkv, tokens * cols * 2), span(nq ? gamma_q : nullptr, nq ? head_dim * 2 : 0),
                       span(nk ? gamma_k : nullptr, nk ? head_dim * 2 : 0), span(positions, tokens * 8),
                       span(cos_sin, max_pos * rotary_dim * 4), span(scale, 4),
                       span(need_kv ? slots : nullptr, need_kv ? tokens * 8 : 0)};
  if (any_alias(outs, 2, ins, 7)) return ANQ_ERR_ALIAS;
  return ANQ_OK;
}

anq::QKParams qk_params(const void* qkv, const void* gamma_q, const void* gamma_k,
                        const int64_t* positions, const float* cos_sin, int64_t max_pos,
                        const float* scale, float eps, int64_t tokens, int32_t nq, int32_t nk,
                        int32_t nv, int32_t head_dim, int32_t rotary_dim, uint8_t* out) {
  anq::QKParams p{};
  p.qkv = qkv;
  p.gamma_q = gamma_q;
  p.gamma_k = gamma_k;
  p.positions = positions;
  p.cos_sin = cos_sin;
  p.max_pos = max_pos;
  p.scale = scale;
  p.out = out;
  p.eps = eps;
  p.tokens = tokens;
  p.nq = nq;
  p.nk = nk;
  p.nv = nv;
  p.head_dim = head_dim;
  p.rotary_dim = rotary_dim;
  return p;
}

int launch_qk_op(int dtype, int store, anq::QKParams& p, void* stream) {
  anq::QKTiling t;
  const int st = anq::pick_qk_tiling(p, &t);
  if (st != ANQ_OK) return st;
  p.waves_per_token = t.waves_per_token;
  return launch_status(anq::launch_qk(dtype, store, p, t, stream));
}

// The two KV-store entry points: Q codes dense, K and V to the pool.
int qk_store(const void* qkv, const void* gamma_q, const void* gamma_k, const int64_t* positions,
             const float* cos_sin, int64_t max_pos, const float* scale, float eps, int64_t tokens,
             int32_t nq, int32_t nk, int32_t nv, int32_t head_dim, int32_t rotary_dim, int dtype,
             const int64_t* slot_mapping, int64_t num_slots, uint8_t* q_out, uint8_t* kv_cache,
             int store, void* stream) {
  const int st = check_qk(qkv, gamma_q, gamma_k, positions, cos_sin, max_pos, scale, eps, tokens, nq,
                          nk, nv, head_dim, rotary_dim, dtype, q_out, store, slot_mapping, num_slots,
                          kv_cache);
  if (st != ANQ_OK || tokens == 0) return st;
  anq::QKParams p = qk_params(qkv, gamma_q, gamma_k, positions, cos_sin, max_pos, scale, eps, tokens,
                              nq, nk, nv, head_dim, rotary_dim, q_out);
  p.kv = kv_cache;
  p.slots = slot_mapping;
  p.num_slots = nk + nv > 0 ? num_slots : 0;
  return launch_qk_op(dtype, store, p, stream);
}

}  // namespace

extern "C" int qk_norm_rope_fp8(const void* qkv, const void* gamma_q, const void* gamma_k,
                                const int64_t* positions, const float* cos_sin, int64_t max_pos,
                                const float* scale, float eps, int64_t tokens, int32_t nq,
                                int32_t nk, int32_t nv, int32_t head_dim, int32_t rotary_dim,
                                anq_dtype dtype, uint8_t* out, void* stream) {
  const int st = check_qk(qkv, gamma_q, gamma_k, positions, cos_sin, max_pos, scale, eps, tokens, nq,
                          nk, nv, head_dim, rotary_dim, dtype, out, anq::kStoreNone, nullptr, 0,
                          nullptr);
  if (st != ANQ_OK || tokens == 0) return st;
  anq::QKParams p = qk_params(qkv, gamma_q, gamma_k, positions, cos_sin, max_pos, scale, eps,
                              tokens, nq, nk, nv, head_dim, rotary_dim, out);
  return launch_qk_op(dtype, anq::kStoreNone, p, stream);
}

extern "C" int qk_norm_rope_fp8_kv_store(const void* qkv, const void* gamma_q, const void* gamma_k,
                                         const int64_t* positions, const float* cos_sin,
                                         int64_t max_pos, const float* scale, float eps,
                                         int64_t tokens, int32_t nq, int32_t nk, int32_t nv,
                                         int32_t head_dim, int32_t rotary_dim, anq_dtype dtype,
                                         const int64_t* slot_mapping, int64_t num_slots,
                                         uint8_t* q_out, uint8_t* kv_cache, void* stream) {
  return qk_store(qkv, gamma_q, gamma_k, positions, cos_sin, max_pos, scale, eps, tokens, nq, nk,
                  nv, head_dim, rotary_dim, dtype, slot_mapping, num_slots, q_out, kv_cache,
                  anq::kStoreUniform, stream);
}

extern "C" int qk_norm_rope_kv_store_mixed(const void* qkv, const void* gamma_q,
                                           const void* gamma_k, const int64_t* positions,
                                           const float* cos_sin, int64_t max_pos,
                                           const float* scale, float eps, int64_t tokens,
                                           int32_t nq, int32_t nk, int32_t nv, int32_t head_dim,
                                           int32_t rotary_dim, anq_dtype dtype,
                                           const int64_t* slot_mapping, int64_t num_slots,
                                           uint8_t* q_out, uint8_t* kv_cache, void* stream) {
  return qk_store(qkv, gamma_q, gamma_k, positions, cos_sin, max_pos, scale, eps, tokens, nq, nk,
                  nv, head_dim, rotary_dim, dtype, slot_mapping, num_slots, q_out, kv_cache,
                  anq::kStoreMixed, stream);
}

extern "C" int add_rmsnorm(const void* x, void* residual, const void* gamma, float eps,
                           int64_t tokens, int64_t hidden, anq_dtype dtype, void* norm_out, void* stream) {
  if (!gamma || (tokens != 0 && (!x || !residual || !norm_out))) return ANQ_ERR_NULL;
  if (!valid_dtype(dtype)) return ANQ_ERR_DTYPE;
  if (tokens < 0 || hidden <= 0 || hidden % 16 != 0) return ANQ_ERR_SHAPE;
  if (hidden > ANQ_MAX_HIDDEN) return ANQ_ERR_UNSUPPORTED;
  if (tokens > INT64_MAX / (2 * hidden)) return ANQ_ERR_SHAPE;
  if (!valid_eps(eps)) return ANQ_ERR_VALUE;
  if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(gamma, 16) || !aligned(norm_out, 16))
    return ANQ_ERR_ALIGN;
  const int64_t act = tokens * hidden * 2;
  const Span outs[2] = {span(residual, act), span(norm_out, act)};
  const Span ins[2] = {span(x, act), span(gamma, hidden * 2)};
  if (any_alias(outs, 2, ins, 2)) return ANQ_ERR_ALIAS;
  if (tokens == 0) return ANQ_OK;

  anq::TailParams p{};
  p.x = x;
  p.residual = residual;
  p.gamma = gamma;
  p.scale = nullptr;
  p.norm_out = norm_out;
  p.q = nullptr;
  p.sf = nullptr;
  p.eps = eps;
  p.tokens = tokens;
  p.hidden = (int32_t)hidden;
  p.vec = (int32_t)(hidden / 8);
  anq::Tiling t;
  const int st = anq::pick_tail_tiling(p.vec, tokens, false, &t);
  if (st != ANQ_OK) return st;
  p.rows_per_group = t.rows;
  p.interleave = t.interleave ? 1 : 0;
  return launch_status(anq::launch_tail(dtype, anq::kEpiNone, true, p, t, stream));
}

namespace {

int quant_common(const void* in, const float* scale, int64_t tokens, int64_t hidden, int dtype,
                 uint8_t* q, uint8_t* sf, bool nvfp4, bool swizzled, void* stream) {
  if (!scale || (tokens != 0 && (!in || !q || (nvfp4 && !sf)))) return ANQ_ERR_NULL;
  if (!valid_dtype(dtype)) return ANQ_ERR_DTYPE;
  if (tokens < 0 || hidden <= 0 || hidden % 16 != 0) return ANQ_ERR_SHAPE;
  if (tokens > INT64_MAX / (2 * hidden) || hidden / 8 > INT32_MAX) return ANQ_ERR_SHAPE;
  if (!aligned(in, 16) || !aligned(q, 16) || !aligned(scale, 4) || (swizzled && !aligned(sf, 4)))
    return ANQ_ERR_ALIGN;
  const int64_t n = tokens * hidden;
  const Span outs[2] = {span(q, nvfp4 ? n / 2 : n), span(sf, nvfp4 ? sf_bytes(tokens, hidden, swizzled) : 0)};
  const Span ins[2] = {span(in, n * 2), span(scale, 4)};
  if (any_alias(outs, 2, ins, 2)) return ANQ_ERR_ALIAS;
  if (tokens == 0) return ANQ_OK;
  anq::QuantParams p{};
  p.in = in;
  p.scale = scale;
  p.q = q;
  p.sf = sf;
  p.vecs = n / 8;
  p.tokens = tokens;
  p.vec = (int32_t)(hidden / 8);
  p.sf_tiles = swizzled ? (int32_t)sf_tiles_of(hidden) : 0;
  p.pad_rows = swizzled ? ((tokens + 127) / 128) * 128 - tokens : 0;
  const int epi = !nvfp4 ? anq::kEpiFp8 : (swizzled ? anq::kEpiNvfp4Swz : anq::kEpiNvfp4);
  anq::QuantTiling t;
  const int st = anq::pick_quant_tiling(epi, p, &t);
  if (st != ANQ_OK) return st;
  return launch_status(anq::launch_quant(dtype, epi, p, t, stream));
}

}  // namespace

extern "C" int quant_fp8(const void* in, const float* scale, int64_t tokens, int64_t hidden,
                         anq_dtype dtype, uint8_t* q, void* stream) {
  return quant_common(in, scale, tokens, hidden, dtype, q, nullptr, false, false, stream);
}

extern "C" int quant_nvfp4(const void* in, const float* global_scale, int64_t tokens,
                           int64_t hidden, anq_dtype dtype, uint8_t* q, uint8_t* sf, void* stream) {
  return quant_common(in, global_scale, tokens, hidden, dtype, q, sf, true, false, stream);
}

extern "C" int quant_nvfp4_swizzled(const void* in, const float* global_scale, int64_t tokens,
                                    int64_t hidden, anq_dtype dtype, uint8_t* q, uint8_t* sf,
                                    void* stream) {
  return quant_common(in, global_scale, tokens, hidden, dtype, q, sf, true, true, stream);
}

extern "C" int anq_nvfp4_shape(int64_t tokens, int64_t hidden, int64_t* q_cols, int64_t* sf_cols) {
  if (!q_cols || !sf_cols) return ANQ_ERR_NULL;
  if (tokens < 0 || hidden <= 0 || hidden % 16 != 0) return ANQ_ERR_SHAPE;
  *q_cols = hidden / 2;
  *sf_cols = hidden / 16;
  return ANQ_OK;
}

extern "C" int anq_nvfp4_swizzled_sf_shape(int64_t tokens, int64_t hidden, int64_t* sf_rows,
                                           int64_t* sf_cols) {
  if (!sf_rows || !sf_cols) return ANQ_ERR_NULL;
  if (tokens < 0 || hidden <= 0 || hidden % 16 != 0) return ANQ_ERR_SHAPE;
  if (tokens > INT64_MAX - 127) return ANQ_ERR_SHAPE;
  *sf_rows = (tokens + 127) / 128 * 128;
  *sf_cols = sf_tiles_of(hidden) * 4;
  return ANQ_OK;
}

extern "C" int anq_stream_rw(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                             int nontemporal, void* stream) {
  if ((read_bytes != 0 && !src) || (write_bytes != 0 && !dst)) return ANQ_ERR_NULL;
  if (read_bytes < 0 || write_bytes < 0 || read_bytes % 16 != 0 || write_bytes % 16 != 0 ||
      (read_bytes > 0 && write_bytes == 0) || (write_bytes / 16 + 255) / 256 > 0x7FFFFFFF)
    return ANQ_ERR_SHAPE;
  if (nontemporal != 0 && nontemporal != 1) return ANQ_ERR_VALUE;
  if (!aligned(src, 16) || !aligned(dst, 16)) return ANQ_ERR_ALIGN;
  const Span outs[1] = {span(dst, write_bytes)};
  const Span ins[1] = {span(src, read_bytes)};
  if (any_alias(outs, 1, ins, 1)) return ANQ_ERR_ALIAS;
  if (write_bytes == 0) return ANQ_OK;
  return launch_status(anq::launch_stream(src, read_bytes, dst, write_bytes, nontemporal == 1,
                                          stream));
}

extern "C" const char* anq_status_string(int status) {
  switch (status) {
    case ANQ_OK: return "ok";
    case ANQ_ERR_NULL: return "a required pointer is NULL";
    case ANQ_ERR_SHAPE: return "bad shape: tokens < 0, hidden <= 0, hidden % 16 != 0 or size overflow";
    case ANQ_ERR_DTYPE: return "dtype must be ANQ_F16 or ANQ_BF16";
    case ANQ_ERR_ALIGN: return "misaligned pointer (16 bytes for tensors, 4 for scalars, 8 for positions)";
    case ANQ_ERR_ALIAS: return "output buffers overlap another buffer";
    case ANQ_ERR_UNSUPPORTED: return "unsupported case (hidden > 65536, head_dim not in {32..512}, rotary_dim not a power of two in [16, head_dim]): use a separated path";
    case ANQ_ERR_LAUNCH: return "HIP kernel launch failed";
    case ANQ_ERR_VALUE: return "bad scalar argument (eps < 0 or not finite, max_pos < 1, negative head count or num_slots)";
    case ANQ_ERR_CONFIG: return "an ANQ_* tuning variable in the environment names a tiling the library has no kernel for";
    default: return "unknown status";
  }
}
