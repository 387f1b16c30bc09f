// The Q/K op's launches with the whole head rotated (rotary_dim == head_dim):
// the plain op and the uniform FP8 pool store. The kernel is in
// anq_qk_kernel.h; partial rotation and the mixed pool are instantiated in
// anq_qk_part.hip.
#include "anq_qk_kernel.h"

namespace anq {

hipError_t launch_qk_whole(int dtype, int store, const QKParams& p, const QKTiling& t,
                           hipStream_t s) {
  if (store == kStoreUniform)
    return dtype == kBF16 ? launch_qk_store<kBF16, kStoreUniform, false>(p, t, s)
                          : launch_qk_store<kF16, kStoreUniform, false>(p, t, s);
  if (store == kStoreNone)
    return dtype == kBF16 ? launch_qk_store<kBF16, kStoreNone, false>(p, t, s)
                          : launch_qk_store<kF16, kStoreNone, false>(p, t, s);
  return hipErrorInvalidValue;
}

// Whole-head rotation takes the layout whose pairs are compile-time; partial
// rotation and the mixed pool (whose K heads split at D - R) take the
// partial-rotation instances.
int launch_qk(int dtype, int store, const QKParams& p, const QKTiling& t, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.rotary_dim < 16 || p.rotary_dim > p.head_dim || (p.rotary_dim & (p.rotary_dim - 1)))
    return (int)hipErrorInvalidValue;
  if (p.rotary_dim != p.head_dim || store == kStoreMixed)
    return (int)launch_qk_partial(dtype, store, p, t, s);
  return (int)launch_qk_whole(dtype, store, p, t, s);
}

}  // namespace anq
