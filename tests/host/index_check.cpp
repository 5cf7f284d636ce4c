// Host build of the library's token-order and tile-classification helpers
// (internal.hpp, tilemap.hip) for the CPU tests: prints, for one geometry and
// token order, perm[t'] and inv[t] of the order, and optionally the tile
// classes of one mask, so the tests can compare them with the oracle.
//
//   index_check F H W order                      -> two lines: perm, inv
//   index_check F H W order kind w r bq bk       -> n_qt lines of n_kt class digits
#include "tilemap.hip"

#include <algorithm>
#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc != 5 && argc != 10) return 2;
  const svattn_geom sg{atoi(argv[1]), atoi(argv[2]), atoi(argv[3])};
  const int order = atoi(argv[4]);
  const svattn::Geo g = svattn::make_geo(sg);
  if (argc == 5) {
    for (int t = 0; t < g.N; ++t) printf("%d ", order == SVATTN_FRAME_MAJOR ? t : svattn::tm_to_fm(g, order, t));
    printf("\n");
    for (int t = 0; t < g.N; ++t) printf("%d ", order == SVATTN_FRAME_MAJOR ? t : svattn::fm_to_tm(g, order, t));
    printf("\n");
    return 0;
  }
  const svattn_mask m{atoi(argv[5]), order, atoi(argv[6]), atoi(argv[7])};
  const int bq = atoi(argv[8]), bk = atoi(argv[9]);
  for (int r0 = 0; r0 < g.N; r0 += bq) {
    for (int c0 = 0; c0 < g.N; c0 += bk)
      printf("%d", (int)svattn::classify(g, m, r0, std::min(g.N, r0 + bq), c0, std::min(g.N, c0 + bk)));
    printf("\n");
  }
  return 0;
}
