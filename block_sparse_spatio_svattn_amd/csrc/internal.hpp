// Internal declarations shared by the HIP kernels and the C ABI layer of
// libsvattn.so.  Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "svattn.h"

namespace svattn {

// Unsigned division by a runtime constant d (1 <= d < 2^31) for dividends
// n < 2^31: q = (mulhi(n, m) + n) >> s with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1 (round-up multiplier method of
// Granlund & Montgomery, "Division by invariant integers using
// multiplication", 1994).
struct FastDiv {
  uint32_t d, m, s;
  FastDiv() : d(1), m(0), s(0) {}
  explicit FastDiv(uint32_t div) : d(div) {
    s = 0;
    while ((1ull << s) < div) ++s;
    m = (uint32_t)((((1ull << s) - div) << 32) / div + 1);
  }
  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t t = __umulhi(n, m);
#else
    uint32_t t = (uint32_t)(((uint64_t)n * m) >> 32);
#endif
    return (t + n) >> s;
  }
  __host__ __device__ __forceinline__ uint32_t mod(uint32_t n) const { return n - div(n) * d; }
};

// Token geometry with precomputed divisors.
struct Geo {
  int32_t F, H, W, P, N;
  FastDiv divP, divW, divF1;  // by P, W and max(F-1, 1)
};

inline Geo make_geo(const svattn_geom& g) {
  Geo o;
  o.F = g.frames;
  o.H = g.height;
  o.W = g.width;
  o.P = g.height * g.width;
  o.N = g.frames * o.P;
  o.divP = FastDiv((uint32_t)o.P);
  o.divW = FastDiv((uint32_t)o.W);
  o.divF1 = FastDiv((uint32_t)(o.F > 1 ? o.F - 1 : 1));
  return o;
}

// Patch index of a token position in a given order (frame-major or
// anchor-first temporal-major).
__device__ __forceinline__ int patch_of(const Geo& g, int order, int t) {
  if (order == SVATTN_FRAME_MAJOR) return (int)g.divP.mod((uint32_t)t);
  return t < g.P ? t : (int)g.divF1.div((uint32_t)(t - g.P));
}

// Frame-major token stored at temporal-major position tp (perm[tp]).
__host__ __device__ __forceinline__ int tm_to_fm(const Geo& g, int tp) {
  if (tp < g.P) return tp;
  uint32_t u = (uint32_t)(tp - g.P);
  uint32_t p = g.divF1.div(u);
  uint32_t f = 1 + (u - p * g.divF1.d);
  return (int)(f * (uint32_t)g.P + p);
}

// Temporal-major position of frame-major token t (inv[t]).
__host__ __device__ __forceinline__ int fm_to_tm(const Geo& g, int t) {
  uint32_t f = g.divP.div((uint32_t)t);
  uint32_t p = (uint32_t)t - f * (uint32_t)g.P;
  if (f == 0) return (int)p;
  return (int)((uint32_t)g.P + p * (uint32_t)(g.F - 1) + (f - 1));
}

// ---- launchers (defined in the .hip files; return hipError_t) ----
hipError_t launch_tile_map(const Geo& g, const svattn_mask& m, const svattn_tile_map& map,
                           uint32_t flags, hipStream_t st);
hipError_t launch_perm_index(const Geo& g, int32_t* perm, int32_t* inv, hipStream_t st);
hipError_t launch_permute(const Geo& g, int heads, int head_dim, const void* src, void* dst,
                          bool to_temporal_major, hipStream_t st);

// Forward: per-head descriptor passed by value in the kernel arguments.
struct HeadDesc {
  const void* q;         // [N, D] bf16 of this head, in the head's token order
  const void* k;
  const void* v;
  void* o;
  float* lse;            // [N] fp32 or nullptr
  const int32_t* row_ptr;
  const int32_t* col;
  const uint8_t* col_cls;
  const int32_t* qt_order;  // visiting order of q-tiles, or nullptr for index order
  const int32_t* perm;      // row of q/k/v/o holding layout position t' (gathered head), or nullptr
  const uint32_t* bits;  // dense-mask mode: [N][ceil(N/32)] words of this head
  float scale_log2;      // scale * log2(e)
  float scale;
  int32_t kind, order, window, radius;
};

constexpr int kMaxHeadsPerLaunch = 16;
constexpr int kMaxDevices = 64;
constexpr int kMaxSelectedTiles = 32;  // q-tiles of a selected-rows launch (kernel arguments)
constexpr float kLog2eHost = 1.4426950408889634f;

struct FwdArgs {
  Geo g;
  int32_t n_qt, n_kt;
  int32_t n_items;        // heads_in_launch * n_qt
  int32_t n_slots;        // heads in this launch
  int32_t chunk;          // consecutive work items kept on one XCD (static schedule)
  uint32_t* queue;        // zeroed work counter (persistent schedule), or nullptr
  int32_t n_sel;          // work items per head: n_qt, or the number of selected q-tiles
  int32_t use_sel;        // 1: compute only q-tiles qt_sel[0 .. n_sel), the same for every head
  int32_t compact;        // 1: O / lse rows of selected q-tile i at i * block_q + row (with use_sel)
  int32_t qt_sel[kMaxSelectedTiles];
  int32_t dense_bits;     // 1: visit every k-tile and mask from bits
  int32_t words_per_row;  // ceil(N/32) for the bit mask
  HeadDesc heads[kMaxHeadsPerLaunch];
};

hipError_t launch_forward(const FwdArgs& a, int head_dim, int block_q, int block_k, hipStream_t st);
static_assert(sizeof(FwdArgs) <= 4096, "forward arguments must fit the kernel argument segment");
hipError_t launch_route(const void* o_dense, const void* o_spatial, const void* o_temporal, int heads,
                        int64_t per_head, int64_t valid, float* err, int32_t* choice, hipStream_t st);

}  // namespace svattn
