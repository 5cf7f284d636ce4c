// Instantiations of the attention forward, head_dim 128, for tile maps and coordinate masks (svattn_forward).
// One wave per 32 queries (block_q = 32 * waves); the plain schedule, and for
// 256 x 32 tiles the two-group schedule.
#include "fwd2.hpp"

namespace svattn {

hipError_t launch_forward_d128_map(const FwdArgs& a, int block_q, int block_k, bool two_group, hipStream_t st) {
  // The two-group schedule needs eight waves (block_q 256).  256 x 64 tiles
  // take the plain schedule even for dense launches: with two tiles per
  // barrier it ran the 75,600-token dense launch 2% faster (25.98 against
  // 26.55 ms, same run).
  if (two_group && block_q == 256 && block_k == 32) return fwd2::launch<128, 32, 8, 1, true, false>(a, st);
#define SVATTN_CASE(BQ, BK) \
  if (block_q == BQ && block_k == BK) return fwd2::launch<128, BK, BQ / 32, 1, false, false>(a, st);
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
