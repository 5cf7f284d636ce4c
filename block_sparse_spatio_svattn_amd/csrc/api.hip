// C ABI of libsvattn.so: argument validation, per-head launch tables and
// dispatch.  Every check runs before the first HIP call, so invalid calls
// return a status without touching the GPU.  No allocation, no host sync.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "internal.hpp"

namespace svattn {
hipError_t launch_forward_d64_map(const FwdArgs& a, int block_q, int block_k, bool two_group, hipStream_t st);
hipError_t launch_forward_d128_map(const FwdArgs& a, int block_q, int block_k, bool two_group, hipStream_t st);
hipError_t launch_forward_d64_bits(const FwdArgs& a, int block_q, int block_k, hipStream_t st);
hipError_t launch_forward_d128_bits(const FwdArgs& a, int block_q, int block_k, hipStream_t st);
}  // namespace svattn

using namespace svattn;

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SVATTN_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// N < 2^23: the kernels form row byte offsets N * head_dim * 2 (< 2^31 at
// head_dim 128) and tile indices in 32-bit arithmetic.
constexpr int64_t kMaxTokens = (1 << 23) - 1;

int check_geom(const svattn_geom* g, int64_t* n_out) {
  if (!g) return fail(SVATTN_ERR_INVALID_ARG, "geom is NULL");
  if (g->frames < 1 || g->height < 1 || g->width < 1)
    return fail(SVATTN_ERR_INVALID_ARG, "geometry %d x %d x %d: every extent must be >= 1", g->frames,
                g->height, g->width);
  const int64_t n = (int64_t)g->frames * g->height * g->width;
  if (n > kMaxTokens) return fail(SVATTN_ERR_UNSUPPORTED, "N = %lld tokens exceeds the limit %lld (N < 2^23)",
                                  (long long)n, (long long)kMaxTokens);
  *n_out = n;
  return SVATTN_OK;
}

int check_mask(const svattn_mask* m) {
  if (!m) return fail(SVATTN_ERR_INVALID_ARG, "mask is NULL");
  if (m->kind < SVATTN_SPATIAL || m->kind > SVATTN_DENSE)
    return fail(SVATTN_ERR_INVALID_ARG, "mask kind %d is not SPATIAL/TEMPORAL/DENSE", m->kind);
  if (m->order != SVATTN_FRAME_MAJOR && !is_temporal_major(m->order))
    return fail(SVATTN_ERR_INVALID_ARG,
                "token order %d is not FRAME_MAJOR / TEMPORAL_MAJOR / TEMPORAL_MAJOR_BLOCKED / TEMPORAL_MAJOR_STRIPS",
                m->order);
  if (m->window < 0 || m->radius < 0)
    return fail(SVATTN_ERR_INVALID_ARG, "window %d / radius %d must be >= 0", m->window, m->radius);
  if (m->kind == SVATTN_SPATIAL && m->order != SVATTN_FRAME_MAJOR)
    return fail(SVATTN_ERR_UNSUPPORTED, "spatial heads run in frame-major order only");
  return SVATTN_OK;
}

bool map_bq_ok(int b) { return b == 32 || b == 64 || b == 128 || b == 256; }
bool map_bk_ok(int b) { return b == 32 || b == 64 || b == 128; }
bool fwd_bk_ok(int b) { return b == 32 || b == 64; }                 // bit-mask entry
bool fwd_map_bk_ok(int b) { return b == 32 || b == 64 || b == 128; }  // tile maps (128: two 64-key halves)

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Kept query-key pairs of a head (closed form), used only to order heads
// longest-first.
double head_cost(const svattn_geom& g, const svattn_mask& m) {
  const double F = g.frames, P = (double)g.height * g.width, N = F * P;
  if (m.kind == SVATTN_DENSE) return N * N;
  if (m.kind == SVATTN_SPATIAL) {
    const int w = m.window;
    if (w >= g.frames - 1) return N * N;
    return P * P * (F * (2 * w + 1) - (double)w * (w + 1) + std::max(0, g.frames - 1 - w));
  }
  auto sw = [](int L, int r) { return r >= L - 1 ? (double)L * L : (double)L * (2 * r + 1) - (double)r * (r + 1); };
  double c = F * (F - 1) * sw(g.height, m.radius) * sw(g.width, m.radius) + F * P * P;
  if (m.order == SVATTN_FRAME_MAJOR) c *= 1.5;  // frame-major temporal heads visit more tiles
  return c;
}

int check_map_buffers(const svattn_tile_map* map, const char* who) {
  if (!map->cls || !map->row_ptr || !map->col || !map->col_cls)
    return fail(SVATTN_ERR_INVALID_ARG, "%s: tile map buffer is NULL", who);
  return SVATTN_OK;
}

// Schedule choice: launches whose heads are all dense may take the two-group
// schedule (one wave's MFMA work beside its SIMD partner's softmax); with
// boundary tiles the masked softmax phase becomes its long pole and the plain
// schedule wins.  The head_dim 128 launchers decide per tile shape (256 x 64
// takes the plain schedule, two tiles per barrier, in every case).

// Clears the work counter of the persistent schedule.  A kernel rather than a
// memset, so that a captured graph replays it correctly.
__global__ void clear_queue_kernel(uint32_t* q) {
  if (threadIdx.x < 8) q[threadIdx.x] = 0u;  // the eight per-XCD work counters
}

// Work counter area of svattn_forward_noalloc, for callers that cannot
// allocate a workspace.  One copy per GPU, held until the process ends.  In
// host code this name only stands in for the symbol: kernels get the device
// address that noalloc_scratch() looks up once per device.
static __device__ __align__(256) uint32_t scratch[kNoallocScratchBytes / 4];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call per device, then cached).
int noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SVATTN_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(SVATTN_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SVATTN_OK;
}

hipError_t dispatch_forward(const FwdArgs& a, int head_dim, int bq, int bk, hipStream_t st) {
  if (a.dense_bits)
    return head_dim == 128 ? launch_forward_d128_bits(a, bq, bk, st) : launch_forward_d64_bits(a, bq, bk, st);
  bool all_dense = true;
  for (int i = 0; i < a.n_slots; ++i)
    all_dense = all_dense && a.heads[i].kind == SVATTN_DENSE && !a.heads[i].gather;  // gathered: plain schedule
  return head_dim == 128 ? launch_forward_d128_map(a, bq, bk, all_dense, st)
                         : launch_forward_d64_map(a, bq, bk, all_dense, st);
}

}  // namespace

extern "C" {

int svattn_version(void) { return SVATTN_VERSION; }

const char* svattn_status_string(int s) {
  switch (s) {
    case SVATTN_OK: return "SVATTN_OK";
    case SVATTN_ERR_INVALID_ARG: return "SVATTN_ERR_INVALID_ARG";
    case SVATTN_ERR_UNSUPPORTED: return "SVATTN_ERR_UNSUPPORTED";
    case SVATTN_ERR_HIP: return "SVATTN_ERR_HIP";
    default: return "SVATTN_ERR_UNKNOWN";
  }
}

const char* svattn_last_error(void) { return g_err; }

int svattn_tile_map_dims(const svattn_geom* geom, int32_t block_q, int32_t block_k, int32_t* n_qt,
                         int32_t* n_kt) {
  int64_t n;
  int s = check_geom(geom, &n);
  if (s) return s;
  if (!n_qt || !n_kt) return fail(SVATTN_ERR_INVALID_ARG, "n_qt / n_kt output is NULL");
  if (!map_bq_ok(block_q) || !map_bk_ok(block_k))
    return fail(SVATTN_ERR_UNSUPPORTED, "tile %d x %d: block_q in {32,64,128,256}, block_k in {32,64,128}",
                block_q, block_k);
  *n_qt = (int32_t)cdiv(n, block_q);
  *n_kt = (int32_t)cdiv(n, block_k);
  return SVATTN_OK;
}

int svattn_build_tile_map_ex(const svattn_geom* geom, const svattn_mask* mask, svattn_tile_map* map,
                             uint32_t flags, void* stream) {
  int64_t n;
  int s = check_geom(geom, &n);
  if (s) return s;
  if ((s = check_mask(mask))) return s;
  if (!map) return fail(SVATTN_ERR_INVALID_ARG, "map is NULL");
  if (flags & ~(SVATTN_MAP_ALL_BOUNDARY | SVATTN_MAP_TILE_ALIGNED))
    return fail(SVATTN_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if ((flags & SVATTN_MAP_ALL_BOUNDARY) && (flags & SVATTN_MAP_TILE_ALIGNED))
    return fail(SVATTN_ERR_INVALID_ARG, "ALL_BOUNDARY and TILE_ALIGNED exclude each other");
  if (!map_bq_ok(map->block_q) || !map_bk_ok(map->block_k))
    return fail(SVATTN_ERR_UNSUPPORTED, "tile %d x %d: block_q in {32,64,128,256}, block_k in {32,64,128}",
                map->block_q, map->block_k);
  if (map->n_qt != cdiv(n, map->block_q) || map->n_kt != cdiv(n, map->block_k))
    return fail(SVATTN_ERR_INVALID_ARG, "map dims %d x %d do not match ceil(N/block) = %lld x %lld", map->n_qt,
                map->n_kt, (long long)cdiv(n, map->block_q), (long long)cdiv(n, map->block_k));
  if ((int64_t)map->n_qt * map->n_kt >= (1ll << 31))
    return fail(SVATTN_ERR_UNSUPPORTED, "tile map of %d x %d blocks is too large", map->n_qt, map->n_kt);
  if ((s = check_map_buffers(map, "svattn_build_tile_map"))) return s;
  if (!aligned(map->row_ptr, 4) || !aligned(map->col, 4) || !aligned(map->qt_order, 4))
    return fail(SVATTN_ERR_INVALID_ARG, "row_ptr / col / qt_order must be 4-byte aligned");
  const Geo g = make_geo(*geom);
  hipError_t e = launch_tile_map(g, *mask, *map, flags, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tile map launch");
  return SVATTN_OK;
}

int svattn_build_tile_map(const svattn_geom* geom, const svattn_mask* mask, svattn_tile_map* map,
                          void* stream) {
  return svattn_build_tile_map_ex(geom, mask, map, 0u, stream);
}

int svattn_permutation_index(const svattn_geom* geom, int32_t* perm, int32_t* inv, void* stream) {
  return svattn_permutation_index_order(geom, SVATTN_TEMPORAL_MAJOR, perm, inv, stream);
}

int svattn_permutation_index_order(const svattn_geom* geom, int32_t order, int32_t* perm, int32_t* inv,
                                   void* stream) {
  int64_t n;
  int s = check_geom(geom, &n);
  if (s) return s;
  if (order != SVATTN_FRAME_MAJOR && !is_temporal_major(order))
    return fail(SVATTN_ERR_INVALID_ARG,
                "token order %d is not FRAME_MAJOR / TEMPORAL_MAJOR / TEMPORAL_MAJOR_BLOCKED / TEMPORAL_MAJOR_STRIPS",
                order);
  if (!perm) return fail(SVATTN_ERR_INVALID_ARG, "perm is NULL");
  if (!aligned(perm, 4) || (inv && !aligned(inv, 4)))
    return fail(SVATTN_ERR_INVALID_ARG, "perm / inv must be 4-byte aligned");
  if (inv && overlap(perm, n * 4, inv, n * 4)) return fail(SVATTN_ERR_INVALID_ARG, "perm and inv overlap");
  hipError_t e = launch_perm_index(make_geo(*geom), order, perm, inv, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "permutation index launch");
  return SVATTN_OK;
}

static int permute_common(const svattn_geom* geom, int32_t order, int32_t heads, int32_t head_dim,
                          const void* src, void* dst, bool to_tm, void* stream) {
  int64_t n;
  int s = check_geom(geom, &n);
  if (s) return s;
  if (!is_temporal_major(order))
    return fail(SVATTN_ERR_INVALID_ARG,
                "token order %d is not TEMPORAL_MAJOR / TEMPORAL_MAJOR_BLOCKED / TEMPORAL_MAJOR_STRIPS", order);
  if (heads < 1) return fail(SVATTN_ERR_INVALID_ARG, "heads = %d must be >= 1", heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(SVATTN_ERR_UNSUPPORTED, "head_dim %d: supported 64, 128", head_dim);
  if (!src || !dst) return fail(SVATTN_ERR_INVALID_ARG, "src / dst is NULL");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(SVATTN_ERR_INVALID_ARG, "src / dst must be 16-byte aligned");
  const int64_t chunks = (int64_t)heads * n * (head_dim / 8);
  if (chunks >= (1ll << 31)) return fail(SVATTN_ERR_UNSUPPORTED, "tensor too large (%lld rows)", (long long)(heads * n));
  const size_t bytes = (size_t)heads * n * head_dim * 2;
  if (overlap(src, bytes, dst, bytes)) return fail(SVATTN_ERR_INVALID_ARG, "src and dst overlap (no in-place)");
  hipError_t e = launch_permute(make_geo(*geom), order, heads, head_dim, src, dst, to_tm, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "permute launch");
  return SVATTN_OK;
}

int svattn_permute_tokens(const svattn_geom* geom, int32_t heads, int32_t head_dim, const void* src, void* dst,
                          void* stream) {
  return permute_common(geom, SVATTN_TEMPORAL_MAJOR, heads, head_dim, src, dst, true, stream);
}

int svattn_unpermute(const svattn_geom* geom, int32_t heads, int32_t head_dim, const void* src, void* dst,
                     void* stream) {
  return permute_common(geom, SVATTN_TEMPORAL_MAJOR, heads, head_dim, src, dst, false, stream);
}

int svattn_permute_tokens_order(const svattn_geom* geom, int32_t order, int32_t heads, int32_t head_dim,
                                const void* src, void* dst, void* stream) {
  return permute_common(geom, order, heads, head_dim, src, dst, true, stream);
}

int svattn_unpermute_order(const svattn_geom* geom, int32_t order, int32_t heads, int32_t head_dim,
                           const void* src, void* dst, void* stream) {
  return permute_common(geom, order, heads, head_dim, src, dst, false, stream);
}

static int check_common(int32_t heads, int32_t head_dim, const float* scales) {
  if (heads < 1) return fail(SVATTN_ERR_INVALID_ARG, "heads = %d must be >= 1", heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(SVATTN_ERR_UNSUPPORTED, "head_dim %d: supported 64, 128", head_dim);
  if (!scales) return fail(SVATTN_ERR_INVALID_ARG, "scales is NULL");
  for (int h = 0; h < heads; ++h)
    if (!(scales[h] > 0.f) || !isfinite(scales[h]))
      return fail(SVATTN_ERR_INVALID_ARG, "scales[%d] = %g must be finite and > 0", h, (double)scales[h]);
  return SVATTN_OK;
}

// Per-head tensor pointers: q/k/v/o [N, head_dim] bf16 each, lse [N] fp32 or NULL.
struct HeadPtrs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
};

static int check_ptrs(const std::vector<HeadPtrs>& p, int64_t n, int32_t head_dim) {
  const size_t bytes = (size_t)n * head_dim * 2, lb = (size_t)n * 4;
  for (size_t h = 0; h < p.size(); ++h) {
    if (!p[h].q || !p[h].k || !p[h].v || !p[h].o)
      return fail(SVATTN_ERR_INVALID_ARG, "head %zu: q / k / v / o is NULL", h);
    if (!aligned(p[h].q, 16) || !aligned(p[h].k, 16) || !aligned(p[h].v, 16) || !aligned(p[h].o, 16))
      return fail(SVATTN_ERR_INVALID_ARG, "head %zu: q / k / v / o must be 16-byte aligned", h);
    if (p[h].lse && !aligned(p[h].lse, 4)) return fail(SVATTN_ERR_INVALID_ARG, "head %zu: lse must be 4-byte aligned", h);
  }
  // outputs must not overlap any input or each other
  for (size_t h = 0; h < p.size(); ++h) {
    for (size_t j = 0; j < p.size(); ++j) {
      if (overlap(p[h].o, bytes, p[j].q, bytes) || overlap(p[h].o, bytes, p[j].k, bytes) ||
          overlap(p[h].o, bytes, p[j].v, bytes))
        return fail(SVATTN_ERR_INVALID_ARG, "o of head %zu overlaps q, k or v of head %zu", h, j);
      if (j != h && overlap(p[h].o, bytes, p[j].o, bytes))
        return fail(SVATTN_ERR_INVALID_ARG, "o of heads %zu and %zu overlap", h, j);
      if (p[h].lse) {
        if (overlap(p[h].lse, lb, p[j].q, bytes) || overlap(p[h].lse, lb, p[j].k, bytes) ||
            overlap(p[h].lse, lb, p[j].v, bytes) || overlap(p[h].lse, lb, p[j].o, bytes))
          return fail(SVATTN_ERR_INVALID_ARG, "lse of head %zu overlaps a tensor of head %zu", h, j);
        if (j != h && p[j].lse && overlap(p[h].lse, lb, p[j].lse, lb))
          return fail(SVATTN_ERR_INVALID_ARG, "lse of heads %zu and %zu overlap", h, j);
      }
    }
  }
  return SVATTN_OK;
}

// The forward workspace: NULL, or SVATTN_FORWARD_WORKSPACE_BYTES of device
// memory, 4-byte aligned, overlapping no tensor of the call.
static int check_workspace(const std::vector<HeadPtrs>& p, int64_t n, int32_t head_dim, const void* ws) {
  if (!ws) return SVATTN_OK;
  if (!aligned(ws, 4)) return fail(SVATTN_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
  const size_t bytes = (size_t)n * head_dim * 2, lb = (size_t)n * 4, wb = SVATTN_FORWARD_WORKSPACE_BYTES;
  for (size_t h = 0; h < p.size(); ++h) {
    if (overlap(ws, wb, p[h].q, bytes) || overlap(ws, wb, p[h].k, bytes) || overlap(ws, wb, p[h].v, bytes) ||
        overlap(ws, wb, p[h].o, bytes) || (p[h].lse && overlap(ws, wb, p[h].lse, lb)))
      return fail(SVATTN_ERR_INVALID_ARG, "workspace overlaps a tensor of head %zu", h);
  }
  return SVATTN_OK;
}

static std::vector<HeadPtrs> contiguous_ptrs(int64_t n, int32_t heads, int32_t head_dim, const void* q,
                                             const void* k, const void* v, void* o, float* lse) {
  std::vector<HeadPtrs> p(heads);
  const size_t hb = (size_t)n * head_dim * 2;
  for (int h = 0; h < heads; ++h) {
    p[h].q = q ? (const char*)q + h * hb : nullptr;
    p[h].k = k ? (const char*)k + h * hb : nullptr;
    p[h].v = v ? (const char*)v + h * hb : nullptr;
    p[h].o = o ? (char*)o + h * hb : nullptr;
    p[h].lse = lse ? lse + (size_t)h * n : nullptr;
  }
  return p;
}

static int run_launches(FwdArgs base, const std::vector<HeadDesc>& descs, int head_dim, int bq, int bk,
                        hipStream_t st) {
  // 128-key tile maps run on the 64-key kernel, two halves per map entry
  // (base.n_kt stays the map's k-tile count).
  if (bk == 128) {
    base.sub = 1;
    bk = 64;
  }
  for (size_t h0 = 0; h0 < descs.size(); h0 += kMaxHeadsPerLaunch) {
    FwdArgs a = base;
    const int nh = (int)std::min<size_t>(kMaxHeadsPerLaunch, descs.size() - h0);
    for (int i = 0; i < nh; ++i) a.heads[i] = descs[h0 + i];
    a.n_slots = nh;
    if (a.n_split < 1) a.n_split = 1;
    a.n_items = nh * a.n_sel * a.n_split;
    // Heads run one after another (each longest row first), which keeps one head's K/V in an XCD's L2 at a
    // time.  When every head of the launch shares one map, the last head's longest rows would start only in
    // the last stretch of the launch and leave most workgroups idle at its end, so the last kTailHeads heads
    // are dealt rank by rank instead.  (Heads come heaviest mask first, so in a launch of several maps the
    // last map's rows are the shortest and already fill the end.)
    a.tail_m = 0;
    if (a.queue && !a.use_sel && a.n_split == 1 && !a.dense_bits && nh >= 2) {
      bool one_map = true;
      for (int i = 0; i + 1 < nh; ++i)
        one_map = one_map && a.heads[i].row_ptr == a.heads[nh - 1].row_ptr &&
                  a.heads[i].qt_order == a.heads[nh - 1].qt_order;
      if (one_map) a.tail_m = std::min(nh, kTailHeads);
    }
    if (a.queue) {
      // launches on one stream run in order, so one counter serves them all
      hipLaunchKernelGGL(clear_queue_kernel, dim3(1), dim3(64), 0, st, a.queue);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return hip_fail(e, "work counter clear");
    }
    hipError_t e = dispatch_forward(a, head_dim, bq, bk, st);
    if (e != hipSuccess) return hip_fail(e, "forward launch");
  }
  return SVATTN_OK;
}

// use_scratch: the work counter lives in the library's per-device `scratch`
// (svattn_forward_noalloc) instead of the caller's workspace; it is looked up
// after every argument check, so validation still precedes any HIP call.
static int forward_impl(const svattn_geom* geom, int64_t n, int32_t heads, int32_t head_dim,
                        const svattn_mask* masks, const svattn_tile_map* const* maps, const float* scales,
                        const std::vector<HeadPtrs>& ptrs, void* workspace, void* stream,
                        bool gather = false, bool use_scratch = false) {
  int s;
  if (!masks || !maps) return fail(SVATTN_ERR_INVALID_ARG, "masks / maps is NULL");
  int bq = 0, bk = 0;
  for (int h = 0; h < heads; ++h) {
    if ((s = check_mask(&masks[h]))) return fail(s, "head %d: %s", h, svattn_last_error());
    const svattn_tile_map* m = maps[h];
    if (!m) return fail(SVATTN_ERR_INVALID_ARG, "maps[%d] is NULL", h);
    if (h == 0) {
      bq = m->block_q;
      bk = m->block_k;
    } else if (m->block_q != bq || m->block_k != bk) {
      return fail(SVATTN_ERR_INVALID_ARG, "maps[%d] tile %d x %d differs from maps[0] %d x %d", h, m->block_q,
                  m->block_k, bq, bk);
    }
    if (!map_bq_ok(bq) || !fwd_map_bk_ok(bk))
      return fail(SVATTN_ERR_UNSUPPORTED, "forward tile %d x %d: block_q in {32,64,128,256}, block_k in {32,64,128}",
                  bq, bk);
    if (m->n_qt != cdiv(n, bq) || m->n_kt != cdiv(n, bk))
      return fail(SVATTN_ERR_INVALID_ARG, "maps[%d] dims %d x %d do not match the geometry", h, m->n_qt, m->n_kt);
    if ((int64_t)m->n_qt * m->n_kt >= (1ll << 31))
      return fail(SVATTN_ERR_UNSUPPORTED, "maps[%d]: tile map of %d x %d blocks is too large", h, m->n_qt, m->n_kt);
    if (!m->row_ptr || !m->col || !m->col_cls) return fail(SVATTN_ERR_INVALID_ARG, "maps[%d] buffer is NULL", h);
    if (!aligned(m->row_ptr, 4) || !aligned(m->col, 4) || !aligned(m->col_cls, 4))
      return fail(SVATTN_ERR_INVALID_ARG, "maps[%d]: row_ptr, col and col_cls must be 4-byte aligned", h);
    if (m->qt_order && !aligned(m->qt_order, 4))
      return fail(SVATTN_ERR_INVALID_ARG, "maps[%d]: qt_order must be 4-byte aligned", h);
  }
  if ((s = check_ptrs(ptrs, n, head_dim))) return s;
  if ((s = check_workspace(ptrs, n, head_dim, workspace))) return s;

  std::vector<HeadDesc> descs(heads);
  std::vector<double> cost(heads);
  std::vector<int> order(heads);
  for (int h = 0; h < heads; ++h) {
    HeadDesc& d = descs[h];
    memset(&d, 0, sizeof(d));
    d.q = ptrs[h].q;
    d.k = ptrs[h].k;
    d.v = ptrs[h].v;
    d.o = ptrs[h].o;
    d.lse = ptrs[h].lse;
    d.row_ptr = maps[h]->row_ptr;
    d.col = maps[h]->col;
    d.col_cls = maps[h]->col_cls;
    d.qt_order = maps[h]->qt_order;
    d.gather = gather && masks[h].order != SVATTN_FRAME_MAJOR;
    d.scale = scales[h];
    d.scale_log2 = scales[h] * kLog2eHost;
    d.kind = masks[h].kind;
    d.order = masks[h].order;
    d.window = masks[h].window;
    d.radius = masks[h].radius;
    cost[h] = head_cost(*geom, masks[h]);
    order[h] = h;
  }
  // Longest heads first so the tail of the grid is short work.
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return cost[x] > cost[y]; });
  std::vector<HeadDesc> sorted(heads);
  for (int i = 0; i < heads; ++i) sorted[i] = descs[order[i]];

  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.g = make_geo(*geom);
  a.n_qt = (int32_t)cdiv(n, bq);
  a.n_sel = a.n_qt;
  a.n_kt = (int32_t)cdiv(n, bk);
  a.chunk = 32;
  a.dense_bits = 0;
  a.queue = (uint32_t*)workspace;
  if (use_scratch) {
    void* p = nullptr;
    if ((s = noalloc_scratch(&p))) return s;
    a.queue = (uint32_t*)p;
  }
  return run_launches(a, sorted, head_dim, bq, bk, (hipStream_t)stream);
}

int svattn_forward(const svattn_geom* geom, int32_t heads, int32_t head_dim, const svattn_mask* masks,
                   const svattn_tile_map* const* maps, const float* scales, const void* q, const void* k,
                   const void* v, void* o, float* lse, void* workspace, void* stream) {
  int64_t n;
  int s = check_geom(geom, &n);
  if (s) return s;
  if ((s = check_common(heads, head_dim, scales))) return s;
  if (!q || !k || !v || !o) return fail(SVATTN_ERR_INVALID_ARG, "q / k / v / o is NULL");
  return forward_impl(geom, n, heads, head_dim, masks, maps, scales,
                      contiguous_ptrs(n, heads, head_dim, q, k, v, o, lse), workspace, stream);
}

int svattn_forward_noalloc(const svattn_geom* geom, int32_t heads, int32_t head_dim, const svattn_mask* masks,
                           const svattn_tile_map* const* maps, const float* scales, const void* q, const void* k,
                           const void* v, void* o, float* lse, void* stream) {
  int64_t n;
  int s = check_geom(geom, &n);
  if (s) return s;
  if ((s = check_common(heads, head_dim, scales))) return s;
  if (!q || !k || !v || !o) return fail(SVATTN_ERR_INVALID_ARG, "q / k / v / o is NULL");
  return forward_impl(geom, n, heads, head_dim, masks, maps, scales,
                      contiguous_ptrs(n, heads, head_dim, q, k, v, o, lse), nullptr, stream, false, true);
}

int svattn_forward_ptrs(const svattn_geom* geom, int32_t heads, int32_t head_dim, const svattn_mask* masks,
                        const svattn_tile_map* const* maps, const float* scales, const void* const* q,
                        const void* const* k, const void* const* v, void* const* o, float* const* lse,
                        void* workspace, void* stream) {
  int64_t n;
  int s = check_geom(geom, &n);
  if (s) return s;
  if ((s = check_common(heads, head_dim, scales))) return s;
  if (!q || !k || !v || !o) return fail(SVATTN_ERR_INVALID_ARG, "q / k / v / o pointer array is NULL");
  std::vector<HeadPtrs> p(heads);
  for (int h = 0; h < heads; ++h) p[h] = HeadPtrs{q[h], k[h], v[h], o[h], lse ? lse[h] : nullptr};
  return forward_impl(geom, n, heads, head_dim, masks, maps, scales, p, workspace, stream);
}

int svattn_forward_fused(const svattn_geom* geom, int32_t heads, int32_t head_dim, const svattn_mask* masks,
                         const svattn_tile_map* const* maps, const float* scales, const void* q, const void* k,
                         const void* v, void* o, float* lse, void* workspace, void* stream) {
  int64_t n;
  int s = check_geom(geom, &n);
  if (s) return s;
  if ((s = check_common(heads, head_dim, scales))) return s;
  if (!q || !k || !v || !o) return fail(SVATTN_ERR_INVALID_ARG, "q / k / v / o is NULL");
  return forward_impl(geom, n, heads, head_dim, masks, maps, scales,
                      contiguous_ptrs(n, heads, head_dim, q, k, v, o, lse), workspace, stream, true);
}

// Key splits per (head, q-tile) of a routing launch: enough work items (three
// masks * heads * q-tiles * splits) for about four per compute unit of a
// 256-unit chip, at most 32.
static int route_splits(int32_t heads, int32_t n_qtiles) {
  const int64_t per = 3ll * heads * n_qtiles;
  return (int)std::min<int64_t>(32, std::max<int64_t>(1, (1024 + per - 1) / per));
}

// Routing scratch: the forward's work counter, then per mask (dense, spatial,
// temporal) the split partial outputs (fp32 rows) and their lse, then the
// per-workgroup deviation sums.
struct RouteLayout {
  int n_split;
  size_t o_bytes, lse_bytes, perr_off, total;  // o_bytes, lse_bytes: one mask
};

static int route_dims(int32_t heads, int32_t head_dim, int32_t block_q, int32_t n_qtiles, RouteLayout* lay) {
  if (heads < 1 || heads > (1 << 16)) return fail(SVATTN_ERR_INVALID_ARG, "heads = %d", heads);
  if (head_dim != 64 && head_dim != 128) return fail(SVATTN_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
  if (!map_bq_ok(block_q)) return fail(SVATTN_ERR_UNSUPPORTED, "block_q %d not in {32, 64, 128, 256}", block_q);
  if (n_qtiles < 1 || n_qtiles > kMaxSelectedTiles)
    return fail(SVATTN_ERR_INVALID_ARG, "n_qtiles = %d must be in [1, %d]", n_qtiles, kMaxSelectedTiles);
  lay->n_split = route_splits(heads, n_qtiles);
  const size_t rows = (size_t)heads * n_qtiles * lay->n_split * block_q;
  lay->o_bytes = rows * head_dim * 4;
  lay->lse_bytes = rows * 4;
  lay->perr_off = SVATTN_FORWARD_WORKSPACE_BYTES + 3 * (lay->o_bytes + lay->lse_bytes);
  const size_t blocks = (size_t)heads * n_qtiles * (block_q / route_rows_per_block(head_dim));
  lay->total = lay->perr_off + blocks * 2 * 4;
  return SVATTN_OK;
}

int svattn_route_scratch_bytes(int32_t heads, int32_t head_dim, int32_t block_q, int32_t n_qtiles,
                               size_t* bytes) {
  RouteLayout lay;
  int s = route_dims(heads, head_dim, block_q, n_qtiles, &lay);
  if (s) return s;
  if (!bytes) return fail(SVATTN_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = lay.total;
  return SVATTN_OK;
}

int svattn_route_heads(const svattn_geom* geom, int32_t heads, int32_t head_dim, const svattn_mask* spatial,
                       const svattn_mask* temporal, const svattn_tile_map* dense_map,
                       const svattn_tile_map* spatial_map, const svattn_tile_map* temporal_map, const float* scales,
                       const int32_t* qtiles, int32_t n_qtiles, const void* q, const void* k, const void* v,
                       void* scratch, size_t scratch_bytes, float* err, int32_t* choice, void* stream) {
  int64_t n;
  int s = check_geom(geom, &n);
  if (s) return s;
  if ((s = check_common(heads, head_dim, scales))) return s;
  if (!spatial || !temporal) return fail(SVATTN_ERR_INVALID_ARG, "spatial / temporal mask is NULL");
  if ((s = check_mask(spatial)) || (s = check_mask(temporal))) return s;
  if (spatial->kind != SVATTN_SPATIAL || temporal->kind != SVATTN_TEMPORAL ||
      spatial->order != SVATTN_FRAME_MAJOR || temporal->order != SVATTN_FRAME_MAJOR)
    return fail(SVATTN_ERR_INVALID_ARG, "routing compares a SPATIAL and a TEMPORAL mask, both FRAME_MAJOR");
  const svattn_tile_map* maps3[3] = {dense_map, spatial_map, temporal_map};
  for (int m = 0; m < 3; ++m) {
    const svattn_tile_map* mp = maps3[m];
    if (!mp || !mp->row_ptr || !mp->col || !mp->col_cls) return fail(SVATTN_ERR_INVALID_ARG, "map %d incomplete", m);
    if (mp->block_q != dense_map->block_q || mp->block_k != dense_map->block_k)
      return fail(SVATTN_ERR_INVALID_ARG, "routing maps must share one tile shape");
    if (!map_bq_ok(mp->block_q) || !fwd_map_bk_ok(mp->block_k))
      return fail(SVATTN_ERR_UNSUPPORTED, "forward tile %d x %d", mp->block_q, mp->block_k);
    if (mp->n_qt != cdiv(n, mp->block_q) || mp->n_kt != cdiv(n, mp->block_k))
      return fail(SVATTN_ERR_INVALID_ARG, "map %d dims do not match the geometry", m);
    if ((int64_t)mp->n_qt * mp->n_kt >= (1ll << 31))
      return fail(SVATTN_ERR_UNSUPPORTED, "map %d: tile map of %d x %d blocks is too large", m, mp->n_qt, mp->n_kt);
    if (!aligned(mp->row_ptr, 4) || !aligned(mp->col, 4) || !aligned(mp->col_cls, 4))
      return fail(SVATTN_ERR_INVALID_ARG, "map %d: row_ptr, col and col_cls must be 4-byte aligned", m);
  }
  const int bq = dense_map->block_q, bk = dense_map->block_k;
  RouteLayout lay;
  if ((s = route_dims(heads, head_dim, bq, n_qtiles, &lay))) return s;
  if (!qtiles) return fail(SVATTN_ERR_INVALID_ARG, "qtiles is NULL");
  for (int i = 0; i < n_qtiles; ++i) {
    if (qtiles[i] < 0 || (int64_t)(qtiles[i] + 1) * bq > n)
      return fail(SVATTN_ERR_INVALID_ARG, "qtiles[%d] = %d is not a whole q-tile of %lld tokens", i, qtiles[i],
                  (long long)n);
    for (int j = 0; j < i; ++j)
      if (qtiles[j] == qtiles[i]) return fail(SVATTN_ERR_INVALID_ARG, "qtiles[%d] repeats q-tile %d", i, qtiles[i]);
  }
  if (!q || !k || !v || !scratch || !err || !choice) return fail(SVATTN_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(scratch, 16) || !aligned(err, 4) ||
      !aligned(choice, 4))
    return fail(SVATTN_ERR_INVALID_ARG, "q / k / v / scratch need 16-byte, err / choice 4-byte alignment");
  if (scratch_bytes < lay.total)
    return fail(SVATTN_ERR_INVALID_ARG, "scratch of %zu bytes, %zu needed", scratch_bytes, lay.total);
  const size_t tb = (size_t)heads * n * head_dim * 2, eb = (size_t)heads * 8, cb = (size_t)heads * 4;
  const void* ins[3] = {q, k, v};
  for (const void* in : ins)
    if (overlap(scratch, lay.total, in, tb) || overlap(err, eb, in, tb) || overlap(choice, cb, in, tb))
      return fail(SVATTN_ERR_INVALID_ARG, "scratch / err / choice overlap q, k or v");
  if (overlap(err, eb, scratch, lay.total) || overlap(choice, cb, scratch, lay.total) || overlap(err, eb, choice, cb))
    return fail(SVATTN_ERR_INVALID_ARG, "scratch, err and choice must not overlap");

  // One forward over the sampled q-tiles of all three masks: work items are
  // (mask, head, q-tile, key split), the dense and temporal ones (long rows)
  // first, taken from a shared counter.
  char* sc = (char*)scratch;
  const float* o_part[3];
  const float* lse_part[3];
  FwdArgs base;
  memset(&base, 0, sizeof(base));
  base.g = make_geo(*geom);
  base.n_qt = (int32_t)cdiv(n, bq);
  base.n_kt = (int32_t)cdiv(n, bk);
  base.chunk = 32;
  base.queue = (uint32_t*)sc;
  base.use_sel = 1;
  base.compact = 1;
  base.partial = 1;
  base.n_split = lay.n_split;
  base.n_sel = n_qtiles;
  for (int i = 0; i < n_qtiles; ++i) base.qt_sel[i] = qtiles[i];
  const svattn_mask dense{SVATTN_DENSE, SVATTN_FRAME_MAJOR, 0, 0};
  const svattn_mask* masks3[3] = {&dense, spatial, temporal};
  const size_t rows_h = (size_t)n_qtiles * lay.n_split * bq;  // partial rows of one head
  std::vector<HeadDesc> descs;
  descs.reserve(3 * (size_t)heads);
  for (int m : {0, 2, 1}) {
    float* o_m = (float*)(sc + SVATTN_FORWARD_WORKSPACE_BYTES + m * lay.o_bytes);
    float* l_m = (float*)(sc + SVATTN_FORWARD_WORKSPACE_BYTES + 3 * lay.o_bytes + m * lay.lse_bytes);
    o_part[m] = o_m;
    lse_part[m] = l_m;
    for (int h = 0; h < heads; ++h) {
      HeadDesc d;
      memset(&d, 0, sizeof(d));
      const size_t hb = (size_t)n * head_dim * 2;
      d.q = (const char*)q + h * hb;
      d.k = (const char*)k + h * hb;
      d.v = (const char*)v + h * hb;
      d.o = o_m + h * rows_h * head_dim;
      d.lse = l_m + h * rows_h;
      d.row_ptr = maps3[m]->row_ptr;
      d.col = maps3[m]->col;
      d.col_cls = maps3[m]->col_cls;
      d.scale = scales[h];
      d.scale_log2 = scales[h] * kLog2eHost;
      d.kind = masks3[m]->kind;
      d.order = SVATTN_FRAME_MAJOR;
      d.window = masks3[m]->window;
      d.radius = masks3[m]->radius;
      descs.push_back(d);
    }
  }
  if ((s = run_launches(base, descs, head_dim, bq, bk, (hipStream_t)stream))) return s;
  hipError_t e = launch_route(o_part, lse_part, heads, n_qtiles, lay.n_split, bq, head_dim,
                              (float*)(sc + lay.perr_off), err, choice, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "routing launch");
  return SVATTN_OK;
}

int svattn_forward_dense_mask(int32_t heads, int32_t n_tokens, int32_t head_dim, const uint32_t* mask_bits,
                              int32_t per_head, const float* scales, const void* q, const void* k, const void* v,
                              void* o, float* lse, int32_t block_q, int32_t block_k, void* stream) {
  if (n_tokens < 1 || n_tokens > kMaxTokens)
    return fail(SVATTN_ERR_INVALID_ARG, "n_tokens = %d must be in [1, %lld]", n_tokens, (long long)kMaxTokens);
  const int64_t n = n_tokens;
  int s = check_common(heads, head_dim, scales);
  if (s) return s;
  if (!q || !k || !v || !o) return fail(SVATTN_ERR_INVALID_ARG, "q / k / v / o is NULL");
  if (!mask_bits) return fail(SVATTN_ERR_INVALID_ARG, "mask_bits is NULL");
  if (!aligned(mask_bits, 4)) return fail(SVATTN_ERR_INVALID_ARG, "mask_bits must be 4-byte aligned");
  if (!map_bq_ok(block_q) || !fwd_bk_ok(block_k))
    return fail(SVATTN_ERR_UNSUPPORTED, "forward tile %d x %d: block_q in {32,64,128,256}, block_k in {32,64}",
                block_q, block_k);
  const std::vector<HeadPtrs> ptrs = contiguous_ptrs(n, heads, head_dim, q, k, v, o, lse);
  if ((s = check_ptrs(ptrs, n, head_dim))) return s;
  const int64_t wpr = cdiv(n, 32);
  const size_t mb = (size_t)(per_head ? heads : 1) * n * wpr * 4, hb = (size_t)heads * n * head_dim * 2;
  if (overlap(mask_bits, mb, o, hb)) return fail(SVATTN_ERR_INVALID_ARG, "mask_bits overlaps o");
  std::vector<HeadDesc> descs(heads);
  for (int h = 0; h < heads; ++h) {
    HeadDesc& d = descs[h];
    memset(&d, 0, sizeof(d));
    d.q = ptrs[h].q;
    d.k = ptrs[h].k;
    d.v = ptrs[h].v;
    d.o = ptrs[h].o;
    d.lse = ptrs[h].lse;
    d.bits = mask_bits + (per_head ? (size_t)h * n * wpr : 0);
    d.scale = scales[h];
    d.scale_log2 = scales[h] * kLog2eHost;
    d.kind = SVATTN_DENSE;
  }
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  svattn_geom g1 = {1, 1, n_tokens};
  a.g = make_geo(g1);
  a.n_qt = (int32_t)cdiv(n, block_q);
  a.n_sel = a.n_qt;
  a.n_kt = (int32_t)cdiv(n, block_k);
  a.chunk = 32;
  a.dense_bits = 1;
  a.words_per_row = (int32_t)wpr;
  return run_launches(a, descs, head_dim, block_q, block_k, (hipStream_t)stream);
}

}  // extern "C"
