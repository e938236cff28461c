// Stochastic-rounding instances of the Mamba2 decode kernels (bf16 state
// pool), compiled apart from the nearest-rounding ones to keep each object's
// build short.  Rounding rule and random bits: see replayssm.h.
#include "mamba2_kernel.hpp"

namespace rssm {

int dispatch_mamba2_sr(bool replay, const Mamba2Args& a, const rssm_dims& d, hipStream_t s) {
  return replay ? dispatch_mamba2<true, true, 16>(a, d, s) : dispatch_mamba2<false, true, 4>(a, d, s);
}

}  // namespace rssm
