// Instantiations of the attention forward, head_dim 64, for an arbitrary bit mask (svattn_forward_dense_mask).
// One wave per 32 queries (block_q = 32 * waves), double-buffered K/V tiles.
#include "fwd2.hpp"

namespace svattn {

hipError_t launch_forward_d64_bits(const FwdArgs& a, int block_q, int block_k, hipStream_t st) {
#define SVATTN_CASE(BQ, BK) \
  if (block_q == BQ && block_k == BK) return fwd2::launch<64, BK, BQ / 32, 1, false, true>(a, st);
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
