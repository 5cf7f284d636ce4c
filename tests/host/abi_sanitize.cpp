// Host-only check of the C ABI layer (csrc/api.hip) under AddressSanitizer
// and UndefinedBehaviorSanitizer.  The kernel launchers are replaced by the
// stubs below, which check the launch descriptors the ABI layer builds and
// return success, so every validation and descriptor-building path of the
// host code runs, on any machine, without a GPU and without launching a
// kernel.  The one HIP call the ABI layer makes itself (the work-counter
// clear, with a workspace) is exercised only when no GPU is visible, where it
// must fail with SVATTN_ERR_HIP.
//
// Exit status 0 when every expectation holds; a sanitizer report aborts.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "internal.hpp"

namespace svattn {
namespace {
int g_fwd_launches = 0, g_map_launches = 0, g_perm_launches = 0, g_route_launches = 0;

void check_fwd(const FwdArgs& a, int block_q, int block_k) {
  if (a.n_slots < 1 || a.n_slots > kMaxHeadsPerLaunch || a.n_split < 1 || a.n_split > 32 ||
      a.n_items != a.n_slots * a.n_sel * a.n_split) {
    fprintf(stderr, "bad launch table: slots %d items %d sel %d splits %d\n", a.n_slots, a.n_items, a.n_sel,
            a.n_split);
    abort();
  }
  // key splits and partial outputs only for selected whole q-tiles
  if ((a.n_split > 1 || a.partial) && (!a.use_sel || !a.compact || !a.partial)) abort();
  // rank-by-rank tail: persistent whole-row launches only, over trailing heads of one map
  if (a.tail_m < 0 || a.tail_m == 1 || a.tail_m > kTailHeads || a.tail_m > a.n_slots) abort();
  if (a.tail_m > 1) {
    if (!a.queue || a.use_sel || a.n_split != 1 || a.dense_bits) abort();
    const HeadDesc& last = a.heads[a.n_slots - 1];
    for (int i = a.n_slots - a.tail_m; i < a.n_slots; ++i)
      if (a.heads[i].row_ptr != last.row_ptr || a.heads[i].qt_order != last.qt_order) abort();
  }
  if (block_q < 32 || block_k < 32 || a.n_qt < 1 || a.n_kt < 1) abort();
  for (int i = 0; i < a.n_slots; ++i) {
    const HeadDesc& h = a.heads[i];
    if (!h.q || !h.k || !h.v || !h.o) abort();
    if (h.gather && h.order == SVATTN_FRAME_MAJOR) abort();  // only temporal-major heads gather
  }
  ++g_fwd_launches;
}
}  // namespace

hipError_t launch_forward_d64_map(const FwdArgs& a, int bq, int bk, bool, hipStream_t) {
  check_fwd(a, bq, bk);
  return hipSuccess;
}
hipError_t launch_forward_d128_map(const FwdArgs& a, int bq, int bk, bool, hipStream_t) {
  check_fwd(a, bq, bk);
  return hipSuccess;
}
hipError_t launch_forward_d64_bits(const FwdArgs& a, int bq, int bk, hipStream_t) {
  check_fwd(a, bq, bk);
  return hipSuccess;
}
hipError_t launch_forward_d128_bits(const FwdArgs& a, int bq, int bk, hipStream_t) {
  check_fwd(a, bq, bk);
  return hipSuccess;
}
hipError_t launch_tile_map(const Geo& g, const svattn_mask&, const svattn_tile_map& m, uint32_t, hipStream_t) {
  if (g.N < 1 || (int64_t)m.n_qt * m.n_kt >= (1ll << 31)) abort();
  ++g_map_launches;
  return hipSuccess;
}
hipError_t launch_perm_index(const Geo& g, int, int32_t* perm, int32_t*, hipStream_t) {
  if (g.N < 1 || !perm) abort();
  ++g_perm_launches;
  return hipSuccess;
}
hipError_t launch_permute(const Geo& g, int, int heads, int head_dim, const void* src, void* dst, bool,
                          hipStream_t) {
  if (g.N < 1 || heads < 1 || (head_dim != 64 && head_dim != 128) || !src || !dst) abort();
  ++g_perm_launches;
  return hipSuccess;
}
hipError_t launch_route(const float* const o[3], const float* const lse[3], int heads, int n_sel, int n_split,
                        int block_q, int head_dim, float* perr, float* err, int32_t* choice, hipStream_t) {
  if (heads < 1 || n_sel < 1 || n_split < 1 || block_q % route_rows_per_block(head_dim) || !perr || !err ||
      !choice)
    abort();
  for (int m = 0; m < 3; ++m)
    if (!o[m] || !lse[m]) abort();
  ++g_route_launches;
  return hipSuccess;
}
}  // namespace svattn

namespace {
int g_fail = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, got, want, svattn_last_error());
    ++g_fail;
  }
}

// Device-pointer stand-ins: 16-byte aligned, far apart, never dereferenced.
void* fake(uintptr_t i) { return (void*)(uintptr_t)(0x100000000ull * (i + 1)); }

svattn_tile_map map_of(const svattn_geom& g, int bq, int bk) {
  int32_t n_qt = 0, n_kt = 0;
  if (svattn_tile_map_dims(&g, bq, bk, &n_qt, &n_kt) != SVATTN_OK) abort();
  return svattn_tile_map{bq, bk, n_qt, n_kt, (uint8_t*)fake(40), (int32_t*)fake(41), (int32_t*)fake(42),
                         (uint8_t*)fake(43), (int32_t*)fake(44)};
}
}  // namespace

int main() {
  int devices = 0;
  if (hipGetDeviceCount(&devices) != hipSuccess) devices = 0;

  // ---- invalid arguments: rejected before any HIP call ----
  const svattn_geom g{5, 24, 40};
  int32_t a = 0, b = 0;
  expect(svattn_tile_map_dims(nullptr, 256, 64, &a, &b), SVATTN_ERR_INVALID_ARG, "dims: NULL geom");
  expect(svattn_tile_map_dims(&g, 48, 64, &a, &b), SVATTN_ERR_UNSUPPORTED, "dims: block_q 48");
  const svattn_geom huge{2, 2048, 2048};
  expect(svattn_tile_map_dims(&huge, 256, 64, &a, &b), SVATTN_ERR_UNSUPPORTED, "dims: N = 2^23");
  const svattn_geom zero{0, 4, 4};
  expect(svattn_tile_map_dims(&zero, 256, 64, &a, &b), SVATTN_ERR_INVALID_ARG, "dims: zero frames");

  svattn_tile_map m = map_of(g, 256, 64);
  const svattn_mask sp{SVATTN_SPATIAL, SVATTN_FRAME_MAJOR, 1, 0};
  const svattn_mask tp{SVATTN_TEMPORAL, SVATTN_TEMPORAL_MAJOR_BLOCKED, 0, 2};
  const svattn_mask bad_kind{7, 0, 0, 0};
  expect(svattn_build_tile_map(&g, &bad_kind, &m, nullptr), SVATTN_ERR_INVALID_ARG, "map: bad kind");
  svattn_tile_map m_bad = m;
  m_bad.n_qt += 1;
  expect(svattn_build_tile_map(&g, &sp, &m_bad, nullptr), SVATTN_ERR_INVALID_ARG, "map: wrong dims");
  expect(svattn_build_tile_map_ex(&g, &sp, &m, 3u, nullptr), SVATTN_ERR_INVALID_ARG, "map: both flags");
  const svattn_geom big{4, 1024, 2000};
  svattn_tile_map m_big = map_of(big, 32, 32);
  expect(svattn_build_tile_map(&big, &sp, &m_big, nullptr), SVATTN_ERR_UNSUPPORTED, "map: 2^31 blocks");

  expect(svattn_permute_tokens(&g, 2, 96, fake(0), fake(1), nullptr), SVATTN_ERR_UNSUPPORTED, "permute: d96");
  expect(svattn_unpermute(&g, 2, 64, fake(0), (char*)fake(0) + 64, nullptr), SVATTN_ERR_INVALID_ARG,
         "unpermute: overlap");
  expect(svattn_permutation_index_order(&g, 4, (int32_t*)fake(0), nullptr, nullptr), SVATTN_ERR_INVALID_ARG,
         "perm index: order 4");

  const int H = 20;  // more heads than one launch takes
  std::vector<svattn_mask> masks(H);
  std::vector<const svattn_tile_map*> maps(H, &m);
  std::vector<float> scales(H, 0.088f);
  for (int h = 0; h < H; ++h) masks[h] = h % 2 ? tp : sp;
  expect(svattn_forward(&g, H, 128, masks.data(), maps.data(), scales.data(), fake(0), fake(1), fake(2),
                        (char*)fake(0) + 4096, nullptr, nullptr, nullptr),
         SVATTN_ERR_INVALID_ARG, "forward: o overlaps q");
  std::vector<float> bad_scales = scales;
  bad_scales[7] = -1.f;
  expect(svattn_forward(&g, H, 128, masks.data(), maps.data(), bad_scales.data(), fake(0), fake(1), fake(2),
                        fake(3), nullptr, nullptr, nullptr),
         SVATTN_ERR_INVALID_ARG, "forward: negative scale");
  std::vector<const svattn_tile_map*> big_maps(1, &m_big);
  expect(svattn_forward(&big, 1, 128, &sp, big_maps.data(), scales.data(), fake(0), fake(1), fake(2), fake(3),
                        nullptr, nullptr, nullptr),
         SVATTN_ERR_UNSUPPORTED, "forward: 2^31-block map");
  expect(svattn_forward_dense_mask(2, 1 << 23, 128, (const uint32_t*)fake(9), 0, scales.data(), fake(0),
                                   fake(1), fake(2), fake(3), nullptr, 256, 64, nullptr),
         SVATTN_ERR_INVALID_ARG, "dense mask: n_tokens = 2^23");
  size_t rb = 0;
  expect(svattn_route_scratch_bytes(2, 128, 256, 33, &rb), SVATTN_ERR_INVALID_ARG, "route: 33 q-tiles");

  // ---- valid arguments: the stubs stand in for the kernels ----
  if (devices == 0) {
    expect(svattn_build_tile_map(&g, &tp, &m, nullptr), SVATTN_OK, "map: valid");
    expect(svattn_permutation_index_order(&g, SVATTN_TEMPORAL_MAJOR_BLOCKED, (int32_t*)fake(0), (int32_t*)fake(1),
                                          nullptr),
           SVATTN_OK, "perm index: valid");
    expect(svattn_permute_tokens_order(&g, SVATTN_TEMPORAL_MAJOR_BLOCKED, H, 128, fake(0), fake(1), nullptr),
           SVATTN_OK, "permute: valid");
    const svattn_mask ts{SVATTN_TEMPORAL, SVATTN_TEMPORAL_MAJOR_STRIPS, 0, 2};
    expect(svattn_build_tile_map(&g, &ts, &m, nullptr), SVATTN_OK, "map: valid, strip order");
    expect(svattn_permute_tokens_order(&g, SVATTN_TEMPORAL_MAJOR_STRIPS, H, 128, fake(0), fake(1), nullptr),
           SVATTN_OK, "permute: valid, strip order");
    const int before = svattn::g_fwd_launches;
    expect(svattn_forward(&g, H, 128, masks.data(), maps.data(), scales.data(), fake(0), fake(1), fake(2), fake(3),
                          (float*)fake(4), nullptr, nullptr),
           SVATTN_OK, "forward: valid, 20 heads");
    if (svattn::g_fwd_launches - before != 2) {
      fprintf(stderr, "FAIL forward: 20 heads took %d launches, expected 2\n", svattn::g_fwd_launches - before);
      ++g_fail;
    }
    std::vector<const void*> qp(H), kp(H), vp(H);
    std::vector<void*> op(H);
    std::vector<float*> lp(H, nullptr);
    for (int h = 0; h < H; ++h) {
      qp[h] = fake(10 + h);
      kp[h] = fake(40 + h);
      vp[h] = fake(70 + h);
      op[h] = fake(100 + h);
    }
    expect(svattn_forward_ptrs(&g, H, 128, masks.data(), maps.data(), scales.data(), qp.data(), kp.data(),
                               vp.data(), op.data(), lp.data(), nullptr, nullptr),
           SVATTN_OK, "forward_ptrs: valid");
    expect(svattn_forward_fused(&g, H, 128, masks.data(), maps.data(), scales.data(), fake(0), fake(1), fake(2),
                                fake(3), nullptr, nullptr, nullptr),
           SVATTN_OK, "forward_fused: valid");
    svattn_tile_map m128 = map_of(g, 256, 128);
    std::vector<const svattn_tile_map*> maps128(H, &m128);
    expect(svattn_forward(&g, H, 64, masks.data(), maps128.data(), scales.data(), fake(0), fake(1), fake(2),
                          fake(3), nullptr, nullptr, nullptr),
           SVATTN_OK, "forward: valid, 128-key maps, d64");
    expect(svattn_forward_dense_mask(3, 4800, 128, (const uint32_t*)fake(9), 1, scales.data(), fake(0), fake(1),
                                     fake(2), fake(3), nullptr, 128, 32, nullptr),
           SVATTN_OK, "dense mask: valid");
    const svattn_mask spf{SVATTN_SPATIAL, SVATTN_FRAME_MAJOR, 1, 0};
    const svattn_mask tpf{SVATTN_TEMPORAL, SVATTN_FRAME_MAJOR, 0, 2};
    const int32_t qts[2] = {1, 5};
    expect(svattn_route_scratch_bytes(2, 128, 256, 2, &rb), SVATTN_OK, "route scratch: valid");
    // routing keeps its work counter in the scratch and clears it itself: no device, so a HIP error
    expect(svattn_route_heads(&g, 2, 128, &spf, &tpf, &m, &m, &m, scales.data(), qts, 2, fake(0), fake(1), fake(2),
                              fake(6), rb, (float*)fake(7), (int32_t*)fake(8), nullptr),
           SVATTN_ERR_HIP, "route: valid, no device");
    // with a workspace the ABI layer clears the work counter itself: no device, so a HIP error
    expect(svattn_forward(&g, 2, 128, masks.data(), maps.data(), scales.data(), fake(0), fake(1), fake(2), fake(3),
                          nullptr, fake(11), nullptr),
           SVATTN_ERR_HIP, "forward: workspace, no device");
    printf("valid-argument paths: %d forward launches, %d map, %d permutation, %d routing\n",
           svattn::g_fwd_launches, svattn::g_map_launches, svattn::g_perm_launches, svattn::g_route_launches);
  } else {
    printf("a GPU is visible: valid-argument paths skipped (stand-in pointers must not reach a launch)\n");
  }
  printf("%s (%d failures)\n", g_fail ? "FAILED" : "OK", g_fail);
  return g_fail ? 1 : 0;
}
