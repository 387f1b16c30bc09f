// Stand-in launchers for the host-only build of the C ABI (anq_api.cpp and
// anq_tiling.cpp compiled with g++ and the host sanitizers). No kernel runs and
// no memory is touched: each launcher checks the launch geometry the front end
// chose against the work it must cover (the same covering rules the kernels'
// indexing relies on), records the launch, and reports success, or an error
// when the geometry does not cover the call. Test infrastructure only.
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../nvfp4_quantization_place_amd/csrc/anq_internal.h"

namespace {

char g_last[512];
int64_t g_calls = 0;
const int kBad = 98;  // a nonzero "launch" status: the front end maps it to ANQ_ERR_LAUNCH

int record(bool ok, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int record(bool ok, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last, sizeof g_last, fmt, ap);
  va_end(ap);
  ++g_calls;
  return ok ? 0 : kBad;
}

bool tail_kernel_exists(int g, int k) {
  if (g == 16 || g == 32) return k == 1;
  if (g == 64) return k == 1 || k == 2;
  return g == 0 && (k == 1 || k == 2 || k == 4 || k == 8);
}

}  // namespace

namespace anq {

int launch_tail(int dtype, int epi, bool norm_out, const TailParams& p, const Tiling& t,
                void* stream) {
  (void)stream;
  const int64_t lanes_per_row = t.group > 0 ? t.group : t.block;
  const int64_t groups_per_block = t.group > 0 ? t.block / t.group : 1;
  const bool ok = tail_kernel_exists(t.group, t.vec_per_lane) && t.block >= 64 &&
                  t.block <= 1024 && t.block % 64 == 0 &&
                  (t.group == 0 || (t.block == (epi == kEpiGatedNvfp4Lut ? t.block : 256) &&
                                    t.block % t.group == 0)) &&
                  lanes_per_row * t.vec_per_lane >= p.vec &&
                  (t.group > 0 || (int64_t)t.block - 64 < (p.vec + t.vec_per_lane - 1) / t.vec_per_lane ||
                   (t.block == 1024 && t.vec_per_lane == 1 && p.vec > 12 * 64)) &&
                  t.rows == p.rows_per_group && t.rows >= 1 && t.grid >= 1 &&
                  p.interleave == (t.interleave ? 1 : 0) &&
                  t.grid <= 0x7FFFFFFF && t.grid * groups_per_block * t.rows >= p.tokens &&
                  (t.grid - 1) * groups_per_block * t.rows < p.tokens &&
                  p.vec * 8 == p.hidden && p.tokens > 0;
  return record(ok,
                "kind=tail dtype=%d epi=%d norm=%d group=%d vec_per_lane=%d block=%d rows=%d "
                "interleave=%d stream=%d stream_codes=%d grid=%lld tokens=%lld hidden=%d ok=%d",
                dtype, epi, (int)norm_out, t.group, t.vec_per_lane, t.block, t.rows,
                (int)t.interleave, (int)t.stream, (int)t.stream_codes, (long long)t.grid, (long long)p.tokens,
                p.hidden, (int)ok);
}

int launch_qk(int dtype, int store, const QKParams& p, const QKTiling& t, void* stream) {
  (void)stream;
  const int hpp = 64 / (p.head_dim / 16);
  const int passes = (p.nq + p.nk + p.nv + hpp - 1) / hpp;
  const int64_t wpb = t.block / 64;
  const bool ok = t.block >= 64 && t.block <= 1024 && t.block % 64 == 0 &&
                  t.block >= p.head_dim / 4 && t.groups >= 1 && t.groups <= 4 &&
                  t.waves_per_token == p.waves_per_token && t.waves_per_token >= 1 &&
                  (int64_t)t.groups * t.waves_per_token >= passes &&
                  t.waves_per_token <= passes && t.grid >= 1 && t.grid <= 0x7FFFFFFF &&
                  t.grid * wpb >= p.tokens * t.waves_per_token &&
                  (t.grid - 1) * wpb < p.tokens * t.waves_per_token && p.tokens > 0 &&
                  p.rotary_dim >= 16 && p.rotary_dim <= p.head_dim &&
                  (p.rotary_dim & (p.rotary_dim - 1)) == 0;
  return record(ok,
                "kind=qk dtype=%d store=%d head_dim=%d rotary_dim=%d waves=%d groups=%d block=%d "
                "stream=%d grid=%lld tokens=%lld ok=%d",
                dtype, store, p.head_dim, p.rotary_dim, t.waves_per_token, t.groups, t.block,
                (int)t.stream, (long long)t.grid, (long long)p.tokens, (int)ok);
}

int launch_quant(int dtype, int epi, const QuantParams& p, const QuantTiling& t, void* stream) {
  (void)stream;
  const int64_t threads = p.vecs + (epi == kEpiNvfp4Swz ? p.pad_rows * p.sf_tiles : 0);
  const bool ok = t.grid >= 1 && t.grid <= 0x7FFFFFFF && t.grid * 256 >= threads &&
                  (t.grid - 1) * 256 < threads && p.vecs == p.tokens * p.vec;
  return record(ok, "kind=quant dtype=%d epi=%d stream=%d grid=%lld vecs=%lld ok=%d", dtype, epi,
                (int)t.stream, (long long)t.grid, (long long)p.vecs, (int)ok);
}

int launch_gate(int dtype, const void*, const void*, float*, int64_t vecs, void*) {
  return record(vecs > 0, "kind=gate dtype=%d vecs=%lld ok=%d", dtype, (long long)vecs,
                (int)(vecs > 0));
}

int launch_selfcheck(unsigned long long*, void*) { return record(true, "kind=selfcheck ok=1"); }

int launch_stream(const void*, int64_t read_bytes, void*, int64_t write_bytes, bool nt, void*) {
  const bool ok = write_bytes > 0 && read_bytes % 16 == 0 && write_bytes % 16 == 0;
  return record(ok, "kind=stream read=%lld write=%lld nt=%d ok=%d", (long long)read_bytes,
                (long long)write_bytes, (int)nt, (int)ok);
}

}  // namespace anq

// The last recorded launch ("" before the first) and the number of launches.
extern "C" const char* anq_hostcheck_last(void) { return g_last; }
extern "C" int64_t anq_hostcheck_calls(void) { return g_calls; }
