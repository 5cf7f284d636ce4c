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
  // Blocked patch order (B = SVATTN_PATCH_BLOCK): NBR x NBC blocks; the last
  // block row has HL rows, the last block column WL columns.
  int32_t NBR, NBC, HL, WL;
  FastDiv divBW, divBHL, divWL;  // by B*W, B*HL and WL
  // Snake-strip patch order (S = SVATTN_PATCH_STRIP): NS column strips, the
  // last one WS columns wide.
  int32_t NS, WS;
  FastDiv divSH;  // by S*H
};

constexpr int kPatchBlock = SVATTN_PATCH_BLOCK;
static_assert(kPatchBlock == 4, "block arithmetic below uses shifts by 2 and 4");
constexpr int kPatchStrip = SVATTN_PATCH_STRIP;
static_assert(kPatchStrip == 2, "strip arithmetic below uses shifts by 1");

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
  o.NBR = (o.H + kPatchBlock - 1) / kPatchBlock;
  o.NBC = (o.W + kPatchBlock - 1) / kPatchBlock;
  o.HL = o.H - (o.NBR - 1) * kPatchBlock;
  o.WL = o.W - (o.NBC - 1) * kPatchBlock;
  o.divBW = FastDiv((uint32_t)(kPatchBlock * o.W));
  o.divBHL = FastDiv((uint32_t)(kPatchBlock * o.HL));
  o.divWL = FastDiv((uint32_t)o.WL);
  o.NS = (o.W + kPatchStrip - 1) / kPatchStrip;
  o.WS = o.W - (o.NS - 1) * kPatchStrip;
  o.divSH = FastDiv((uint32_t)(kPatchStrip * o.H));
  return o;
}

// Patch row and column of the patch with rank r in the blocked order: block
// row tr holds ranks [tr*B*W, (tr+1)*B*W); inside it, block column tc holds
// B*h ranks (h = B, or HL in the last block row), listed row by row with w =
// B columns (WL in the last block column).
__host__ __device__ __forceinline__ void blocked_yx(const Geo& g, int r, int& y, int& x) {
  const uint32_t tr = g.divBW.div((uint32_t)r);
  const uint32_t rem = (uint32_t)r - tr * (uint32_t)(kPatchBlock * g.W);
  const bool last_r = (int)tr == g.NBR - 1;
  const uint32_t tc = last_r ? g.divBHL.div(rem) : rem >> 4;
  const uint32_t rem2 = rem - tc * (last_r ? (uint32_t)(kPatchBlock * g.HL) : 16u);
  const bool last_c = (int)tc == g.NBC - 1;
  const uint32_t iy = last_c ? g.divWL.div(rem2) : rem2 >> 2;
  const uint32_t ix = rem2 - iy * (last_c ? (uint32_t)g.WL : 4u);
  y = (int)(tr * kPatchBlock + iy);
  x = (int)(tc * kPatchBlock + ix);
}

// Raster patch index of rank r in the blocked order.
__host__ __device__ __forceinline__ int blocked_patch(const Geo& g, int r) {
  int y, x;
  blocked_yx(g, r, y, x);
  return y * g.W + x;
}

// Rank in the blocked order of raster patch p.
__host__ __device__ __forceinline__ int blocked_rank(const Geo& g, int p) {
  const int y = (int)g.divW.div((uint32_t)p), x = p - y * g.W;
  const int tr = y >> 2, tc = x >> 2;
  const int h = tr == g.NBR - 1 ? g.HL : kPatchBlock;
  const int w = tc == g.NBC - 1 ? g.WL : kPatchBlock;
  return tr * kPatchBlock * g.W + tc * kPatchBlock * h + (y - tr * kPatchBlock) * w + (x - tc * kPatchBlock);
}

// Patch row and column of the patch with rank r in the snake-strip order:
// strip s holds ranks [s*S*H, (s+1)*S*H) (fewer in a narrower last strip),
// listed row by row with w = S columns (WS in the last strip); rows run down
// in even strips and up in odd ones.
__host__ __device__ __forceinline__ void strips_yx(const Geo& g, int r, int& y, int& x) {
  const uint32_t s = g.divSH.div((uint32_t)r);
  const uint32_t rem = (uint32_t)r - s * (uint32_t)(kPatchStrip * g.H);
  const bool one = (int)s == g.NS - 1 && g.WS == 1;  // a last strip one column wide
  const uint32_t iy = one ? rem : rem >> 1;
  const uint32_t ix = rem - (one ? iy : iy << 1);
  y = (s & 1u) ? g.H - 1 - (int)iy : (int)iy;
  x = (int)(s * kPatchStrip + ix);
}

// Rank in the snake-strip order of raster patch p.
__host__ __device__ __forceinline__ int strips_rank(const Geo& g, int p) {
  const int y = (int)g.divW.div((uint32_t)p), x = p - y * g.W;
  const int s = x >> 1;
  const int w = s == g.NS - 1 ? g.WS : kPatchStrip;
  const int iy = (s & 1) ? g.H - 1 - y : y;
  return s * kPatchStrip * g.H + iy * w + (x - s * kPatchStrip);
}

// Raster patch index of rank r in the patch sequence of a temporal-major
// order, and its inverse.
__host__ __device__ __forceinline__ int order_patch(const Geo& g, int order, int r) {
  if (order == SVATTN_TEMPORAL_MAJOR_BLOCKED) return blocked_patch(g, r);
  if (order == SVATTN_TEMPORAL_MAJOR_STRIPS) {
    int y, x;
    strips_yx(g, r, y, x);
    return y * g.W + x;
  }
  return r;
}
__host__ __device__ __forceinline__ int order_rank(const Geo& g, int order, int p) {
  if (order == SVATTN_TEMPORAL_MAJOR_BLOCKED) return blocked_rank(g, p);
  if (order == SVATTN_TEMPORAL_MAJOR_STRIPS) return strips_rank(g, p);
  return p;
}

// The three temporal-major orders.
__host__ __device__ __forceinline__ bool is_temporal_major(int order) {
  return order == SVATTN_TEMPORAL_MAJOR || order == SVATTN_TEMPORAL_MAJOR_BLOCKED ||
         order == SVATTN_TEMPORAL_MAJOR_STRIPS;
}

// Rank (in the order's patch sequence) of the patch at position t of a
// temporal-major order.
__host__ __device__ __forceinline__ int tm_rank(const Geo& g, int t) {
  return t < g.P ? t : (int)g.divF1.div((uint32_t)(t - g.P));
}

// Patch index of a token position in a given order (frame-major, or one of
// the anchor-first temporal-major orders).
__host__ __device__ __forceinline__ int patch_of(const Geo& g, int order, int t) {
  if (order == SVATTN_FRAME_MAJOR) return (int)g.divP.mod((uint32_t)t);
  return order_patch(g, order, tm_rank(g, t));
}

// Frame-major token stored at position tp of a temporal-major order (perm[tp]).
__host__ __device__ __forceinline__ int tm_to_fm(const Geo& g, int order, int tp) {
  uint32_t f = 0, r = (uint32_t)tp;
  if (tp >= g.P) {
    const uint32_t u = (uint32_t)(tp - g.P);
    r = g.divF1.div(u);
    f = 1 + (u - r * g.divF1.d);
  }
  const uint32_t p = (uint32_t)order_patch(g, order, (int)r);
  return (int)(f * (uint32_t)g.P + p);
}

// Position in a temporal-major order of frame-major token t (inv[t]).
__host__ __device__ __forceinline__ int fm_to_tm(const Geo& g, int order, int t) {
  const uint32_t f = g.divP.div((uint32_t)t);
  const uint32_t p = (uint32_t)t - f * (uint32_t)g.P;
  const uint32_t r = (uint32_t)order_rank(g, order, (int)p);
  if (f == 0) return (int)r;
  return (int)((uint32_t)g.P + r * (uint32_t)(g.F - 1) + (f - 1));
}

// ---- launchers (defined in the .hip files; return hipError_t) ----
hipError_t launch_tile_map(const Geo& g, const svattn_mask& m, const svattn_tile_map& map,
                           uint32_t flags, hipStream_t st);
hipError_t launch_perm_index(const Geo& g, int order, int32_t* perm, int32_t* inv, hipStream_t st);
hipError_t launch_permute(const Geo& g, int order, int heads, int head_dim, const void* src, void* dst,
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
  int32_t gather;           // 1: q/k/v/o are frame-major, position t' of `order` is row tm_to_fm(t')
  const uint32_t* bits;  // dense-mask mode: [N][ceil(N/32)] words of this head
  float scale_log2;      // scale * log2(e)
  float scale;
  int32_t kind, order, window, radius;
};

constexpr int kMaxHeadsPerLaunch = 16;
// Size of the library-held work-counter area of svattn_forward_noalloc (one
// copy per device): the forward needs SVATTN_FORWARD_WORKSPACE_BYTES.
constexpr int kNoallocScratchBytes = 256;
static_assert(kNoallocScratchBytes >= SVATTN_FORWARD_WORKSPACE_BYTES, "forward workspace must fit the scratch area");
constexpr int kMaxDevices = 64;
constexpr int kMaxSelectedTiles = 32;  // q-tiles of a selected-rows launch (kernel arguments)
constexpr int kTailHeads = 3;          // most head slots dealt rank by rank at the end of a launch
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
  // Key splits per (head, q-tile) work item (1: whole rows; more only with use_sel and partial): split s
  // takes the map entries whose keys lie in 128-key units [s U / n_split, (s + 1) U / n_split), U =
  // ceil(N / 128), so a split covers the same keys whatever the map's block_k.
  int32_t n_split;
  // > 1 (persistent whole-row launches whose heads all share one tile map): the last tail_m head slots are
  // dealt rank by rank at the end of the work order (rank-0 q-tiles of all of them, then rank 1, ...)
  int32_t tail_m;
  // 1: O is fp32, normalised over the split's keys alone, with lse of the split (-inf when it keeps no
  // key); rows of (selected q-tile i, split s) at (i * n_split + s) * block_q + row
  int32_t partial;
  int32_t qt_sel[kMaxSelectedTiles];
  int32_t sub;            // map entries hold 1 << sub compute tiles (a 128-key map on the 64-key kernel: 1)
  int32_t dense_bits;     // 1: visit every k-tile and mask from bits
  int32_t words_per_row;  // ceil(N/32) for the bit mask
  HeadDesc heads[kMaxHeadsPerLaunch];
};

hipError_t launch_forward(const FwdArgs& a, int head_dim, int block_q, int block_k, hipStream_t st);
static_assert(sizeof(FwdArgs) <= 4096, "forward arguments must fit the kernel argument segment");
// Head routing from split partial outputs: o[m], lse[m] (m = dense, spatial, temporal) are
// [heads][n_sel][n_split][block_q] rows of head_dim fp32 / one fp32, as the partial forward writes
// them; perr holds heads * n_sel * block_q / route_rows_per_block(head_dim) pairs of fp32.
constexpr int kRouteMergeThreads = 256, kRouteColsPerThread = 4;  // merge workgroup: 4 columns per thread
inline int route_rows_per_block(int head_dim) { return kRouteMergeThreads / (head_dim / kRouteColsPerThread); }
hipError_t launch_route(const float* const o[3], const float* const lse[3], int heads, int n_sel, int n_split,
                        int block_q, int head_dim, float* perr, float* err, int32_t* choice, hipStream_t st);

}  // namespace svattn
