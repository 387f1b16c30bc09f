// The Q/K op's launches with a partial rotary width (the last rotary_dim <=
// head_dim / 2 elements of each Q/K head rotate), with every store. The
// kernel is in anq_qk_kernel.h.
#include "anq_qk_kernel.h"

namespace anq {

hipError_t launch_qk_partial(int dtype, int store, const QKParams& p, const QKTiling& t,
                             hipStream_t s) {
  switch (store) {
    case kStoreNone:
      return dtype == kBF16 ? launch_qk_store<kBF16, kStoreNone, true>(p, t, s)
                            : launch_qk_store<kF16, kStoreNone, true>(p, t, s);
    case kStoreUniform:
      return dtype == kBF16 ? launch_qk_store<kBF16, kStoreUniform, true>(p, t, s)
                            : launch_qk_store<kF16, kStoreUniform, true>(p, t, s);
    case kStoreMixed:
      return dtype == kBF16 ? launch_qk_store<kBF16, kStoreMixed, true>(p, t, s)
                            : launch_qk_store<kF16, kStoreMixed, true>(p, t, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace anq
