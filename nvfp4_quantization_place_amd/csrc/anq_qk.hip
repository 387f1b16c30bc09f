// The Q/K op's launches with the whole head rotated (rotary_dim == head_dim),
// with every store. The kernel is in anq_qk_kernel.h; partial rotation is
// instantiated in anq_qk_part.hip.
#include "anq_qk_kernel.h"

namespace anq {

hipError_t launch_qk_whole(int dtype, int store, const QKParams& p, const QKTiling& t,
                           hipStream_t s) {
  switch (store) {
    case kStoreNone:
      return dtype == kBF16 ? launch_qk_store<kBF16, kStoreNone, false>(p, t, s)
                            : launch_qk_store<kF16, kStoreNone, false>(p, t, s);
    case kStoreUniform:
      return dtype == kBF16 ? launch_qk_store<kBF16, kStoreUniform, false>(p, t, s)
                            : launch_qk_store<kF16, kStoreUniform, false>(p, t, s);
    case kStoreMixed:
      return dtype == kBF16 ? launch_qk_store<kBF16, kStoreMixed, false>(p, t, s)
                            : launch_qk_store<kF16, kStoreMixed, false>(p, t, s);
    default:
      return hipErrorInvalidValue;
  }
}

// Whole-head rotation keeps each NeoX pair in one lane; a partial width
// (a power of two R <= D/2) pairs lanes j and j ^ R/16.
int launch_qk(int dtype, int store, const QKParams& p, const QKTiling& t, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.rotary_dim < 16 || p.rotary_dim > p.head_dim || (p.rotary_dim & (p.rotary_dim - 1)))
    return (int)hipErrorInvalidValue;
  if (p.rotary_dim != p.head_dim) return (int)launch_qk_partial(dtype, store, p, t, s);
  return (int)launch_qk_whole(dtype, store, p, t, s);
}

}  // namespace anq
