/*
 * addnormq.h -- C ABI of the fused local tail of a transformer layer on
 * AMD Instinct MI355X (gfx950):
 *
 *   residual <- x + residual            (in place, rounded to the activation type)
 *   n        <- RMSNorm(residual) * gamma   (binary32)
 *   q        <- FP8 E4M3 (per-tensor scale) or NVFP4 (E2M1 + per-16 E4M3 scales)
 *   norm_out <- n rounded to the activation type   (optional)
 *
 * and of the Q/K per-head RMSNorm + NeoX RoPE + FP8 store (into dense codes, a
 * uniform FP8 KV pool, or a pool with FP8 unrotated and bf16 rotated parts).
 *
 * Sources of the operations (the pages these ops are built from):
 *  - TensorRT-LLM issue #17900, "[Performance]: Fuse local NVFP4 tail after
 *    NCCL fallback", Proposal: the residual add, RMSNorm and NVFP4 quantisation
 *    as one launch. The fused case it describes: the norm output is optional;
 *    activations are fp16 or bf16, all of one type; the scale is one fp32
 *    value; there is no bias; hidden is a multiple of 16. Anything else falls
 *    back to the unfused kernels.
 *  - TensorRT-LLM PR #17288, "Add NanoJet backend for AutoDeploy prefill-only
 *    FP8 inference", Description: RMSNorm with FP8 quantisation in the kernel
 *    epilogue; FP8 projection with an in-place residual add; Q/K RMSNorm and
 *    RoPE.  Test Coverage: head-layout and RoPE-width guards.
 *  - TensorRT-LLM PR #14361, "[perf] Add AutoDeploy NVFP4 RMSNorm quant
 *    fusion", Changes table: fused add + RMSNorm + NVFP4 ops (with and without
 *    the norm output) over a 2-D [tokens, hidden] view; review thread: one
 *    shared helper for the packed-FP4 / scale-factor shapes.
 *  - SGLang PR #32975, "perf: add fused norm + RoPE + uniform fp8 store for
 *    TRT-LLM DSv4 sparse attention": norm + RoPE + FP8 store into a uniform
 *    FP8 buffer.
 *
 * Numerics (every step is one IEEE binary32 operation, rounded to nearest
 * even, never fused):
 *   h_i   = RNE_T(x_i + res_i)                      written back to residual
 *   ss    = sum_i h_i^2, exact, rounded once to binary32
 *   r     = 1 / sqrt(ss / H + eps)                  four correctly rounded ops
 *   n_i   = (h_i * r) * gamma_i
 *   FP8   : q_i = E4M3(n_i / s)                     s = *scale (dequant scale)
 *   NVFP4 : per 16 consecutive elements of a row:
 *           sf = E4M3(G * (max|n_i| / 6)), S = value of sf,
 *           c_i = E2M1(n_i * (G / S))   (c_i = +-0 when S == 0), G = *global_scale
 * E4M3 is OCP E4M3FN (max 448, no infinities); E2M1 values {0,.5,1,1.5,2,3,4,6}
 * with the sign in bit 3. Both encoders round to nearest, ties to even, and
 * saturate; the sign of a code is the sign bit of its binary32 input.
 *
 * Layouts (all row-major, contiguous, no padding):
 *   x, residual, norm_out : [tokens, hidden] of T (T = fp16 or bf16, one dtype per call)
 *   gamma                 : [hidden] of T
 *   FP8 q                 : [tokens, hidden] bytes, one E4M3 code per element
 *   NVFP4 q               : [tokens, hidden/2] bytes; byte j of a row holds element 2j
 *                           in bits 0-3 and element 2j+1 in bits 4-7
 *   NVFP4 sf              : [tokens, hidden/16] bytes, E4M3 code of block b at column b
 *   qkv, out (Q/K op)     : [tokens, (nq+nk+nv)*head_dim]: Q heads, then K, then V
 *   cos_sin               : [max_pos, rotary_dim] binary32; columns k < rotary_dim/2
 *                           hold cos(angle_k), columns rotary_dim/2 + k sin(angle_k)
 *
 * Conventions shared by every entry point:
 *  - Pointers are device pointers unless stated; the caller owns every buffer.
 *    The library allocates nothing, keeps no state between calls and never
 *    synchronises the host.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *    runs asynchronously. Scales are read on the device when the kernel runs,
 *    so a producer kernel on the same stream may write them.
 *  - Arguments are validated on the host before any HIP call. A rejected call
 *    returns a nonzero status and enqueues nothing. The ANQ_* environment
 *    variables (ANQ_TAIL_TILING, ANQ_ROWS_PER_GROUP, ANQ_ROW_ORDER, ANQ_STREAM,
 *    ANQ_STREAM_CODES, ANQ_GATE_LUT, ANQ_GATE_BLOCK, ANQ_QK_WAVES, ANQ_QK_GROUPS,
 *    ANQ_QK_BLOCK) override the tiling for sweeps; a value the library has no kernel for is refused with
 *    ANQ_ERR_CONFIG, never replaced by a default. Every accepted tiling gives
 *    bit-identical results. tokens == 0 returns ANQ_OK
 *    and enqueues nothing; the token-sized buffers (x, z, residual, q, sf,
 *    norm_out, qkv, positions, out, slot_mapping) may then be NULL, as empty
 *    tensors are.
 *  - residual is the only in/out buffer. Every output must be disjoint from
 *    every other buffer of the call; x must be disjoint from residual; the
 *    read-only inputs may overlap each other. Violations return ANQ_ERR_ALIAS.
 *  - 16-byte alignment is required for x, residual, gamma, norm_out, q and
 *    qkv/out/cos_sin/q_out/kv_cache; 4 bytes for scalars and swizzled sf; 8 for
 *    positions and slot_mapping; linear sf has none.
 *  - Left to the caller (not checked): finite inputs, a positive normal
 *    binary32 scale (s or G, so that 1/s is finite; an FP8 s also at most
 *    2^119, so that 448 s is finite; an NVFP4 G below 2^119, so that every
 *    multiplier G / value(sf) is finite and no zero element meets an infinite
 *    one), 0 <= positions[t] < max_pos,
 *    distinct KV slots. Breaking them gives unspecified codes, never an
 *    out-of-bounds access: a position outside [0, max_pos) is clamped into it
 *    and a slot outside [0, num_slots) stores nothing.
 *  - Intermediate binary32 results that overflow (n, n / s, G * amax / 6,
 *    n * mult, reachable with bf16 gamma near its maximum) are infinities, and
 *    the encoders saturate them like any value past the top code.
 *  - With eps = 0, a row (or group) whose mean square is 0 has r = inf, and its
 *    zero elements give n = 0 * inf = NaN; the codes of such blocks are
 *    unspecified. Any eps > 0 keeps r finite.
 *  - Calls that share output buffers and overlap in time on different streams
 *    race; calls on one stream are ordered.
 */
#ifndef ADDNORMQ_H
#define ADDNORMQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Activation type T of a call. */
typedef enum { ANQ_F16 = 0, ANQ_BF16 = 1 } anq_dtype;

/* Status codes. ANQ_ERR_UNSUPPORTED is the answer that leaves a call to a separated path
 * for valid arguments outside what the fused kernels cover. */
enum {
  ANQ_OK = 0,
  ANQ_ERR_NULL = 1,        /* a required pointer is NULL */
  ANQ_ERR_SHAPE = 2,       /* tokens < 0, hidden <= 0, hidden % 16 != 0, bad group, bad head count, size overflow */
  ANQ_ERR_DTYPE = 3,       /* dtype is not ANQ_F16 / ANQ_BF16 */
  ANQ_ERR_ALIGN = 4,       /* a pointer breaks the alignment rule above */
  ANQ_ERR_ALIAS = 5,       /* buffers overlap where they must not */
  ANQ_ERR_UNSUPPORTED = 6, /* hidden > ANQ_MAX_HIDDEN, head_dim or rotary_dim not supported */
  ANQ_ERR_LAUNCH = 7,      /* the HIP launch failed (message via anq_status_string) */
  ANQ_ERR_VALUE = 8,       /* eps negative or not finite, max_pos < 1, negative head counts or num_slots */
  ANQ_ERR_CONFIG = 9       /* an ANQ_* tuning variable in the environment names no kernel of the library */
};

/* Largest hidden size the fused row kernels take (a row is held in registers). */
#define ANQ_MAX_HIDDEN 65536

/*
 * Residual add + RMSNorm + per-tensor FP8 E4M3 quantisation.
 * (TensorRT-LLM PR #17288, Description: the NanoJet backend quantises to FP8
 * in the epilogue of its RMSNorm and adds the residual in place.)
 *
 *   x        [tokens, hidden] T, read only
 *   residual [tokens, hidden] T, in/out: receives h = RNE_T(x + residual)
 *   gamma    [hidden] T
 *   scale    device pointer to one binary32 s; q = E4M3(n / s)
 *   eps      added to the mean square inside the square root (>= 0, finite)
 *   q        [tokens, hidden] uint8 E4M3 codes (output)
 *   norm_out [tokens, hidden] T (output) or NULL to skip it
 */
int add_rmsnorm_quant_fp8(const void* x, void* residual, const void* gamma, const float* scale,
                          float eps, int64_t tokens, int64_t hidden, anq_dtype dtype, uint8_t* q,
                          void* norm_out, void* stream);

/*
 * Residual add + RMSNorm + NVFP4 quantisation, with or without the
 * high-precision norm output (residualRmsNormFp4Quant-style local tail,
 * TensorRT-LLM issue #17900, Proposal).
 *
 *   global_scale  device pointer to one binary32 G (encode direction: the
 *                 block scale is E4M3(G * amax / 6), codes are E2M1(n * G / S))
 *   q             [tokens, hidden/2] uint8 packed E2M1 (output)
 *   sf            [tokens, hidden/16] uint8 E4M3 block scales (output)
 *   other arguments as for add_rmsnorm_quant_fp8.
 */
int add_rmsnorm_quant_nvfp4(const void* x, void* residual, const void* gamma,
                            const float* global_scale, float eps, int64_t tokens, int64_t hidden,
                            anq_dtype dtype, uint8_t* q, uint8_t* sf, void* norm_out, void* stream);

/*
 * Q/K per-head RMSNorm + NeoX RoPE + uniform FP8 E4M3 store of a fused QKV
 * buffer (SGLang PR #32975; Q/K RMSNorm and RoPE of TensorRT-LLM PR #17288,
 * Description; its Test Coverage guards the RoPE width).
 *
 * For token t and each of its nq Q heads and nk K heads (head_dim D each),
 * with R = rotary_dim and N = D - R:
 *   n = RMSNorm over all D elements with gamma_q (Q) or gamma_k (K), binary32;
 *   the first N elements keep o = n; the last R rotate as NeoX pairs
 *   (N + k, N + k + R/2), k < R/2, each product and sum rounded:
 *     o_{N+k}     = n_{N+k} * cos_k - n_{N+k+R/2} * sin_k,
 *     o_{N+k+R/2} = n_{N+k+R/2} * cos_k + n_{N+k} * sin_k,
 *   with cos_k = cos_sin[positions[t], k], sin_k = cos_sin[positions[t], R/2 + k];
 *   out = E4M3(o / s).  V heads: out = E4M3(v / s).
 * R = D rotates the whole head.
 *
 *   qkv        [tokens, (nq+nk+nv)*D] T, read only
 *   gamma_q,gamma_k [D] T
 *   positions  [tokens] int64 (device)
 *   cos_sin    [max_pos, R] binary32
 *   scale      device pointer to one binary32 s
 *   head_dim   one of 32, 64, 128, 256, 512
 *   rotary_dim a power of two from 16 to head_dim; other values (and other
 *              head_dim) return ANQ_ERR_UNSUPPORTED, the answer that
 *              leaves the call to a separated path
 *   nq, nk, nv >= 0, at least one head and at most 2^20 in all (ANQ_ERR_VALUE
 *              for a negative count, ANQ_ERR_SHAPE otherwise)
 *   out        [tokens, (nq+nk+nv)*D] uint8 E4M3 codes (output)
 */
int qk_norm_rope_fp8(const void* qkv, const void* gamma_q, const void* gamma_k,
                     const int64_t* positions, const float* cos_sin, int64_t max_pos,
                     const float* scale, float eps, int64_t tokens, int32_t nq, int32_t nk,
                     int32_t nv, int32_t head_dim, int32_t rotary_dim, anq_dtype dtype,
                     uint8_t* out, void* stream);

/*
 * The same op with the KV-cache store as its epilogue: the norm + RoPE + store
 * kernel of SGLang PR #32975, whose new epilogue writes a uniform FP8 pool
 * (every element of K and V an E4M3 code, no separate BF16 RoPE part).
 * The codes are those of qk_norm_rope_fp8; only where they go differs:
 *
 *   q_out        [tokens, nq*D] uint8: the Q heads' codes (may be NULL if nq == 0)
 *   kv_cache     [num_slots, (nk+nv)*D] uint8, in/out: the pool. Token t's K
 *                heads then V heads go to row slot_mapping[t]; every other
 *                row keeps its contents. A paged pool [blocks, block_size,
 *                (nk+nv)*D] is this layout with slot = block * block_size + offset.
 *   slot_mapping [tokens] int64 (device): the token's slot; a value outside
 *                [0, num_slots) (e.g. -1 for a padding token) stores nothing
 *   num_slots    rows of the pool (>= 0)
 * kv_cache and slot_mapping may be NULL if nk + nv == 0. Other arguments as
 * for qk_norm_rope_fp8. Two tokens with the same slot race.
 */
int qk_norm_rope_fp8_kv_store(const void* qkv, const void* gamma_q, const void* gamma_k,
                              const int64_t* positions, const float* cos_sin, int64_t max_pos,
                              const float* scale, float eps, int64_t tokens, int32_t nq,
                              int32_t nk, int32_t nv, int32_t head_dim, int32_t rotary_dim,
                              anq_dtype dtype, const int64_t* slot_mapping, int64_t num_slots,
                              uint8_t* q_out, uint8_t* kv_cache, void* stream);

/*
 * The same op with the mixed KV pool as its epilogue: FP8 for the part of a
 * K head that carries no position encoding, bf16 for the rotated part (the
 * FP8-nope / BF16-rope pool of the FlashMLA counterpart that the SGLang PR
 * #32975 discussion names). The pages give no layout; this is the one the
 * library writes, with R = rotary_dim and N = head_dim - R:
 *
 *   q_out        [tokens, nq*D] uint8: the Q heads' E4M3 codes, as qk_norm_rope_fp8's
 *   kv_cache     [num_slots, nk*(D+R) + nv*D] uint8, in/out. Row slot_mapping[t]
 *                receives token t's K heads, each as N bytes E4M3(o_i / s) of its
 *                first N elements followed by R bf16 values RNE_bf16(o_i) of its
 *                last R (2 bytes each, little endian; bf16 whatever T is), then
 *                its V heads, D bytes E4M3(v_i / s) each. Every other row keeps
 *                its contents.
 * The values o are those of qk_norm_rope_fp8 with the same rotary_dim; slots,
 * NULL rules, alignment and races as for qk_norm_rope_fp8_kv_store.
 */
int qk_norm_rope_kv_store_mixed(const void* qkv, const void* gamma_q, const void* gamma_k,
                                const int64_t* positions, const float* cos_sin, int64_t max_pos,
                                const float* scale, float eps, int64_t tokens, int32_t nq,
                                int32_t nk, int32_t nv, int32_t head_dim, int32_t rotary_dim,
                                anq_dtype dtype, const int64_t* slot_mapping, int64_t num_slots,
                                uint8_t* q_out, uint8_t* kv_cache, void* stream);

/*
 * The separated local tail, kept as the measured baseline of the fused ops and
 * as standalone ops. Without the fused kernel the tail launches a
 * residual/RMSNorm kernel and then a quantisation kernel (TensorRT-LLM issue
 * #17900, Proposal; Performance result: 0.103 ms separated vs 0.039 ms fused
 * at FP16 [64, 8192]). The quantiser then reads the norm output rounded to T,
 * so its codes can differ from the fused ops' (which quantise the binary32 n).
 *
 * add_rmsnorm: residual <- RNE_T(x + residual); norm_out <- RNE_T(n), with n
 *   as in the numerics above. norm_out is required. No scale, no codes.
 */
int add_rmsnorm(const void* x, void* residual, const void* gamma, float eps, int64_t tokens,
                int64_t hidden, anq_dtype dtype, void* norm_out, void* stream);

/*
 * quant_fp8: q_i = E4M3(in_i / s) for in [tokens, hidden] T (hidden % 16 == 0,
 *   hidden < 2^34: no ANQ_MAX_HIDDEN limit, the quantisers keep no row in
 *   registers), s = *scale; q [tokens, hidden] uint8.
 */
int quant_fp8(const void* in, const float* scale, int64_t tokens, int64_t hidden, anq_dtype dtype,
              uint8_t* q, void* stream);

/*
 * quant_nvfp4: the NVFP4 epilogue above applied to n_i = in_i (T converted to
 *   binary32, exact): q [tokens, hidden/2] packed E2M1, sf [tokens, hidden/16]
 *   E4M3, under G = *global_scale.
 */
int quant_nvfp4(const void* in, const float* global_scale, int64_t tokens, int64_t hidden,
                anq_dtype dtype, uint8_t* q, uint8_t* sf, void* stream);

/*
 * Gated RMSNorm + NVFP4: the gated variant among the fused NVFP4 norm ops
 * (TensorRT-LLM PR #14361, Changes table). The pages name the op but not the
 * gate; this is the Mamba-2 gated RMSNorm with the norm after the gate, over
 * groups of `group` consecutive elements of a row:
 *   E_i = exp(-z_i) rounded once to binary32 (correctly rounded);
 *   u_i = x_i * (z_i * (1 / (1 + E_i)))       each operation rounded, binary32;
 *   ss  = sum of u_i^2 over the group, exact, rounded once; r = 1 / sqrt(ss / group + eps);
 *   n_i = (u_i * r) * gamma_i;  then the NVFP4 epilogue above (q, sf linear).
 * No residual. x, z [tokens, hidden] T (read only; they may overlap each other);
 * gamma [hidden] T; hidden % group == 0, group % 16 == 0, group <= ANQ_MAX_HIDDEN
 * (group == hidden: one group per row). q [tokens, hidden/2], sf [tokens, hidden/16].
 */
int gated_rmsnorm_quant_nvfp4(const void* x, const void* z, const void* gamma,
                              const float* global_scale, float eps, int64_t tokens,
                              int64_t hidden, int64_t group, anq_dtype dtype, uint8_t* q, uint8_t* sf,
                              void* stream);

/*
 * The gate of gated_rmsnorm_quant_nvfp4 alone: u_i = x_i * SiLU(z_i) in the
 * binary32 steps stated there, for n elements (n % 8 == 0) of T; u [n]
 * binary32 (output). x, z and u 16-byte aligned.
 */
int silu_gate_f32(const void* x, const void* z, int64_t n, anq_dtype dtype, float* u, void* stream);

/*
 * NVFP4 with the block scales in the swizzled layout a block-scaled GEMM reads
 * (the fused ops feed "prequant GEMM" consumers, TensorRT-LLM PR #14361,
 * Changes table; its review thread names the sf_size packing math of that
 * layout). The pages do not spell the layout out; it is the 128x4-tiled
 * scale layout of NVFP4 GEMM operands:
 *   rows padded to R = roundup(tokens, 128), scale columns to C = roundup(hidden/16, 4);
 *   the scale of (row r, block column c) is at byte
 *     ((r / 128) * (C / 4) + c / 4) * 512 + (r % 32) * 16 + ((r / 32) % 4) * 4 + c % 4.
 * Every padding byte (rows >= tokens, columns >= hidden/16) is written as 0.
 * sf holds R * C bytes and must be 4-byte aligned. Codes, q, residual and
 * norm_out are exactly those of the linear-layout op.
 */
int add_rmsnorm_quant_nvfp4_swizzled(const void* x, void* residual, const void* gamma,
                                     const float* global_scale, float eps, int64_t tokens,
                                     int64_t hidden, anq_dtype dtype, uint8_t* q, uint8_t* sf,
                                     void* norm_out, void* stream);

/* quant_nvfp4 with the swizzled block-scale layout above. */
int quant_nvfp4_swizzled(const void* in, const float* global_scale, int64_t tokens,
                         int64_t hidden, anq_dtype dtype, uint8_t* q, uint8_t* sf, void* stream);

/*
 * Padded shape [sf_rows, sf_cols] of the swizzled block-scale buffer:
 * sf_rows = roundup(tokens, 128), sf_cols = roundup(hidden/16, 4).
 * Host only. Returns ANQ_OK, or ANQ_ERR_NULL / ANQ_ERR_SHAPE.
 */
int anq_nvfp4_swizzled_sf_shape(int64_t tokens, int64_t hidden, int64_t* sf_rows,
                                int64_t* sf_cols);

/*
 * The one place that states the NVFP4 output shapes (the review thread of
 * TensorRT-LLM PR #14361 asks for a single shared shape helper):
 *   q_cols = hidden / 2, sf_cols = hidden / 16, for tokens rows each.
 * Host only, no HIP call. Returns ANQ_OK, or ANQ_ERR_NULL / ANQ_ERR_SHAPE.
 */
int anq_nvfp4_shape(int64_t tokens, int64_t hidden, int64_t* q_cols, int64_t* sf_cols);

/*
 * The calibration stream (a measurement aid, not part of the method): one pass
 * that reads read_bytes of src and writes write_bytes of dst with the 16-byte
 * vector accesses of the fused kernels, the non-temporal hint on every access
 * when nontemporal == 1 (0: none). Timed with the read/write byte counts of a
 * call, it is the practical streaming ceiling of that mix on this GPU.
 * With n_in = read_bytes / 16 and n_out = write_bytes / 16 units of 16 bytes,
 * unit j < n_out of dst receives the XOR of source units j, j + n_out, ...
 * below n_in (each source unit is read once); where j >= n_in that XOR starts
 * from the unit (j as a little-endian 64-bit integer, then 8 zero bytes).
 * Both sizes are multiples of 16 (ANQ_ERR_SHAPE otherwise, also when bytes are
 * read but none written); src and dst 16-byte aligned and disjoint.
 */
int anq_stream_rw(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                  int nontemporal, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* anq_status_string(int status);

/*
 * Self-check of the device arithmetic that the exact results above rest on,
 * run on the current device. The kernels replace four IEEE operations by
 * cheaper forms; each count is the number of inputs where the form the
 * kernels use differs from the operation it stands for (all four are 0 where
 * the kernels are exact):
 *   counts[0] the reciprocal (hardware estimate + one FMA correction) against
 *             1 / b, every normal binary32 b below 2^120, and b = +0, +inf
 *   counts[1] the NVFP4 block-scale quotient against amax / 6, every
 *             non-negative binary32 amax (+inf included)
 *   counts[2] the E4M3 code of the FP8 quotient a / s against the code of the
 *             IEEE quotient, every binary32 a at seven scales s from 2^-126
 *             to 2^119
 *   counts[3] the E2M1 code of every binary32 at or beyond +-6 (infinities
 *             included) against the signed top code
 * counts: device memory, ANQ_SELFCHECK_COUNTS uint64 values, 8-byte aligned;
 * zeroed, then counted, on `stream` (read it after the stream completes).
 * About 3.4e10 comparisons. Returns ANQ_OK, ANQ_ERR_NULL, ANQ_ERR_ALIGN or
 * ANQ_ERR_LAUNCH.
 */
#define ANQ_SELFCHECK_COUNTS 4
int anq_selfcheck_arith(uint64_t* counts, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ADDNORMQ_H */
