// Replay instances of the Mamba2 decode kernel with 4 state vectors per
// lane (4 waves per 16 KB bf16 tile instead of 1): used when batch * heads
// is too small for one-wave tiles to fill the 256 compute units, e.g. one
// tensor-parallel rank's share of the heads.
#include "mamba2_kernel.hpp"

namespace rssm {

int dispatch_mamba2_small(const Mamba2Args& a, const rssm_dims& d, hipStream_t s) {
  return dispatch_mamba2<true, false, 4>(a, d, s);
}

}  // namespace rssm
