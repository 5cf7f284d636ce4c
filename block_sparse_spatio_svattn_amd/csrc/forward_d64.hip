// Instantiations of the attention forward for head_dim 64 (one wave = 32
// queries; block_q = 32 * waves).
#include "forward.hpp"

namespace svattn {

hipError_t launch_forward_d64(const FwdArgs& a, int block_q, int block_k, hipStream_t st) {
#define SVATTN_CASE(BQ, BK)                                                                   \
  if (block_q == BQ && block_k == BK)                                                       \
    return a.dense_bits ? launch_fwd_cfg<64, BK, BQ / 32, 1, true>(a, st)                   \
                        : launch_fwd_cfg<64, BK, BQ / 32, 1, false>(a, st);
  SVATTN_CASE(32, 32)
  SVATTN_CASE(32, 64)
  SVATTN_CASE(64, 32)
  SVATTN_CASE(64, 64)
  SVATTN_CASE(128, 32)
  SVATTN_CASE(128, 64)
  SVATTN_CASE(256, 32)
  SVATTN_CASE(256, 64)
#undef SVATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace svattn
