// Tile classifier and CSR compaction.
//
// A (q-tile, k-tile) block is EMPTY when no pair in it is kept, FULL when every
// in-range pair is kept, BOUNDARY otherwise; the attention kernel skips EMPTY
// blocks, runs FULL blocks without a mask and evaluates the coordinate mask
// only on BOUNDARY blocks ("Accelerating Spatio-Temporal Attention for Video
// Diffusion on TPUs", aihirek.info, section "A TPU-kernel kialakítása
// döntőnek bizonyult", paragraphs 2-3).
//
// Classes are exact and computed from coordinates, one thread per block, with
// no per-pair work: the rows of a block cover a set of patches that is the
// union of at most two contiguous ranges of the order's patch sequence (a
// frame-major range can wrap once around a frame boundary; an anchor-first
// temporal-major range can straddle the frame-0 prefix).  A range of raster
// patch indices is at most three grid rectangles, a range of the blocked
// patch order at most seven (the tail of its first block, whole blocks to the
// end of that block row, whole block rows, whole blocks from the start of the
// last block row, the head of its last block), a range of the snake-strip
// order at most seven (the tail of its first strip, whole strips, the head of
// its last strip; a strip's rows reversed when it runs upwards).  Between two rectangles the
// smallest Chebyshev distance is max(gap_y, gap_x) and the largest is
// max(span_y, span_x).  Key positions below P (frame 0, the anchor) are kept
// for every query in every order.

#include "internal.hpp"

namespace svattn {
namespace {

struct Rect {
  int y0, y1, x0, x1;
};

// Contiguous patch-index ranges [lo, hi] covered by positions [a, b), b > a.
__host__ __device__ int patch_ranges(const Geo& g, int order, int a, int b, int2 out[2]) {
  if (order == SVATTN_FRAME_MAJOR) {
    if (b - a >= g.P) {
      out[0] = make_int2(0, g.P - 1);
      return 1;
    }
    uint32_t fa = g.divP.div((uint32_t)a), fb = g.divP.div((uint32_t)(b - 1));
    int pa = a - (int)fa * g.P, pb = (b - 1) - (int)fb * g.P;
    if (fa == fb) {
      out[0] = make_int2(pa, pb);
      return 1;
    }
    out[0] = make_int2(pa, g.P - 1);
    out[1] = make_int2(0, pb);
    return 2;
  }
  int n = 0;
  if (a < g.P) out[n++] = make_int2(a, min(b, g.P) - 1);
  if (b > g.P) {
    int s = max(a, g.P);
    out[n++] = make_int2((int)g.divF1.div((uint32_t)(s - g.P)), (int)g.divF1.div((uint32_t)(b - 1 - g.P)));
  }
  return n;
}

__host__ __device__ int rects_of(const Geo& g, int2 r, Rect* out) {
  int ylo = (int)g.divW.div((uint32_t)r.x), yhi = (int)g.divW.div((uint32_t)r.y);
  int xlo = r.x - ylo * g.W, xhi = r.y - yhi * g.W;
  if (ylo == yhi) {
    out[0] = Rect{ylo, ylo, xlo, xhi};
    return 1;
  }
  out[0] = Rect{ylo, ylo, xlo, g.W - 1};
  out[1] = Rect{yhi, yhi, 0, xhi};
  if (yhi > ylo + 1) {
    out[2] = Rect{ylo + 1, yhi - 1, 0, g.W - 1};
    return 3;
  }
  return 2;
}

// Position of rank r of the blocked patch order: block (tr, tc) of h x w
// patches, index i = row * w + column inside it.
struct BlockPos {
  int tr, tc, h, w, i;
};
__host__ __device__ BlockPos block_pos(const Geo& g, int r) {
  int y, x;
  blocked_yx(g, r, y, x);
  BlockPos b;
  b.tr = y / kPatchBlock;
  b.tc = x / kPatchBlock;
  b.h = b.tr == g.NBR - 1 ? g.HL : kPatchBlock;
  b.w = b.tc == g.NBC - 1 ? g.WL : kPatchBlock;
  b.i = (y - b.tr * kPatchBlock) * b.w + (x - b.tc * kPatchBlock);
  return b;
}

// Rectangles of in-block indices [i0, i1] of block b (raster inside the block).
__host__ __device__ int block_part(const BlockPos& b, int i0, int i1, Rect* out) {
  const int y0 = b.tr * kPatchBlock, x0 = b.tc * kPatchBlock;
  const int ya = i0 / b.w, xa = i0 - ya * b.w, yb = i1 / b.w, xb = i1 - yb * b.w;
  if (ya == yb) {
    out[0] = Rect{y0 + ya, y0 + ya, x0 + xa, x0 + xb};
    return 1;
  }
  int n = 0;
  out[n++] = Rect{y0 + ya, y0 + ya, x0 + xa, x0 + b.w - 1};
  out[n++] = Rect{y0 + yb, y0 + yb, x0, x0 + xb};
  if (yb > ya + 1) out[n++] = Rect{y0 + ya + 1, y0 + yb - 1, x0, x0 + b.w - 1};
  return n;
}

// Rectangles of ranks [r.x, r.y] of the blocked patch order.
__host__ __device__ int blocked_rects(const Geo& g, int2 r, Rect* out) {
  const BlockPos a = block_pos(g, r.x), b = block_pos(g, r.y);
  if (a.tr == b.tr && a.tc == b.tc) return block_part(a, a.i, b.i, out);
  int n = 0;
  n += block_part(a, a.i, a.h * a.w - 1, out + n);  // tail of the first block
  n += block_part(b, 0, b.i, out + n);              // head of the last block
  if (a.tr == b.tr) {
    if (b.tc > a.tc + 1)
      out[n++] = Rect{a.tr * kPatchBlock, a.tr * kPatchBlock + a.h - 1, (a.tc + 1) * kPatchBlock, b.tc * kPatchBlock - 1};
    return n;
  }
  if (a.tc + 1 < g.NBC)  // rest of the first block row
    out[n++] = Rect{a.tr * kPatchBlock, a.tr * kPatchBlock + a.h - 1, (a.tc + 1) * kPatchBlock, g.W - 1};
  if (b.tr > a.tr + 1)  // whole block rows between
    out[n++] = Rect{(a.tr + 1) * kPatchBlock, b.tr * kPatchBlock - 1, 0, g.W - 1};
  if (b.tc > 0)  // start of the last block row
    out[n++] = Rect{b.tr * kPatchBlock, b.tr * kPatchBlock + b.h - 1, 0, b.tc * kPatchBlock - 1};
  return n;
}

// Rectangles of in-strip indices [i0, i1] of strip s of the snake-strip
// order: rows of w patches, index i at walking row i / w, column i % w; the
// walking row is the grid row in an even strip and H-1 minus it in an odd one.
__host__ __device__ int strip_part(const Geo& g, int s, int i0, int i1, Rect* out) {
  const int w = s == g.NS - 1 ? g.WS : kPatchStrip, x0 = s * kPatchStrip;
  const int ya = i0 / w, xa = i0 - ya * w, yb = i1 / w, xb = i1 - yb * w;
  int n = 0;
  if (ya == yb) {
    out[n++] = Rect{ya, ya, x0 + xa, x0 + xb};
  } else {
    out[n++] = Rect{ya, ya, x0 + xa, x0 + w - 1};
    out[n++] = Rect{yb, yb, x0, x0 + xb};
    if (yb > ya + 1) out[n++] = Rect{ya + 1, yb - 1, x0, x0 + w - 1};
  }
  if (s & 1)
    for (int i = 0; i < n; ++i) out[i] = Rect{g.H - 1 - out[i].y1, g.H - 1 - out[i].y0, out[i].x0, out[i].x1};
  return n;
}

// Rectangles of ranks [r.x, r.y] of the snake-strip patch order.
__host__ __device__ int strips_rects(const Geo& g, int2 r, Rect* out) {
  const int sh = kPatchStrip * g.H;
  const int sa = (int)g.divSH.div((uint32_t)r.x), sb = (int)g.divSH.div((uint32_t)r.y);
  const int ia = r.x - sa * sh, ib = r.y - sb * sh;
  if (sa == sb) return strip_part(g, sa, ia, ib, out);
  const int wa = sa == g.NS - 1 ? g.WS : kPatchStrip;
  int n = 0;
  n += strip_part(g, sa, ia, wa * g.H - 1, out + n);  // tail of the first strip
  n += strip_part(g, sb, 0, ib, out + n);             // head of the last strip
  if (sb > sa + 1)                                    // whole strips between
    out[n++] = Rect{0, g.H - 1, (sa + 1) * kPatchStrip, sb * kPatchStrip - 1};
  return n;
}

constexpr int kMaxRects = 2 * 9;  // two ranges of at most 3 + 3 + 3 rectangles

__host__ __device__ int rect_set(const Geo& g, int order, int a, int b, Rect out[kMaxRects]) {
  int2 rg[2];
  int nr = patch_ranges(g, order, a, b, rg);
  int n = 0;
  for (int i = 0; i < nr; ++i)
    n += order == SVATTN_TEMPORAL_MAJOR_BLOCKED  ? blocked_rects(g, rg[i], out + n)
         : order == SVATTN_TEMPORAL_MAJOR_STRIPS ? strips_rects(g, rg[i], out + n)
                                                 : rects_of(g, rg[i], out + n);
  return n;
}

// Class of the block rows [r0, r1) x columns [c0, c1) (both clipped to N).
__host__ __device__ uint8_t classify(const Geo& g, const svattn_mask& m, int r0, int r1, int c0, int c1) {
  const bool anchor = c0 < g.P;  // some key of the block is in frame 0
  const int n0 = max(c0, g.P);   // first key outside frame 0
  if (n0 >= c1 || m.kind == SVATTN_DENSE) return SVATTN_TILE_FULL;
  bool near_any, near_all;
  if (m.kind == SVATTN_SPATIAL) {  // frame-major only: frames of a range are an interval
    int a = (int)g.divP.div((uint32_t)r0), b = (int)g.divP.div((uint32_t)(r1 - 1));
    int c = (int)g.divP.div((uint32_t)n0), d = (int)g.divP.div((uint32_t)(c1 - 1));
    near_any = max(0, max(a - d, c - b)) <= m.window;
    near_all = max(b - c, d - a) <= m.window;
  } else {
    Rect R[kMaxRects], C[kMaxRects];
    int nr = rect_set(g, m.order, r0, r1, R);
    int nc = rect_set(g, m.order, n0, c1, C);
    int dmin = 1 << 30, dmax = 0;
    for (int i = 0; i < nr; ++i) {
      for (int j = 0; j < nc; ++j) {
        int gy = max(0, max(R[i].y0 - C[j].y1, C[j].y0 - R[i].y1));
        int gx = max(0, max(R[i].x0 - C[j].x1, C[j].x0 - R[i].x1));
        dmin = min(dmin, max(gy, gx));
        int sy = max(R[i].y1 - C[j].y0, C[j].y1 - R[i].y0);
        int sx = max(R[i].x1 - C[j].x0, C[j].x1 - R[i].x0);
        dmax = max(dmax, max(sy, sx));
      }
    }
    near_any = dmin <= m.radius;
    near_all = dmax <= m.radius;
  }
  if (near_all) return SVATTN_TILE_FULL;
  return (near_any || anchor) ? SVATTN_TILE_BOUNDARY : SVATTN_TILE_EMPTY;
}

constexpr int kThreads = 256;

__device__ int block_sum(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int t = 0;
  for (int w = 0; w < kThreads / 64; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Pass 1: classes of one q-tile row; row_ptr[qt+1] = number of non-empty blocks.
__global__ __launch_bounds__(kThreads) void classify_kernel(Geo g, svattn_mask m, svattn_tile_map map,
                                                            uint32_t flags) {
  __shared__ int red[kThreads / 64];
  const int qt = blockIdx.x;
  const int r0 = qt * map.block_q, r1 = min(g.N, r0 + map.block_q);
  int count = 0;
  for (int kt = threadIdx.x; kt < map.n_kt; kt += kThreads) {
    const int c0 = kt * map.block_k, c1 = min(g.N, c0 + map.block_k);
    uint8_t c = classify(g, m, r0, r1, c0, c1);
    if ((flags & SVATTN_MAP_ALL_BOUNDARY) && c != SVATTN_TILE_EMPTY) c = SVATTN_TILE_BOUNDARY;
    if ((flags & SVATTN_MAP_TILE_ALIGNED) && c != SVATTN_TILE_EMPTY) c = SVATTN_TILE_FULL;
    map.cls[(size_t)qt * map.n_kt + kt] = c;
    count += (c != SVATTN_TILE_EMPTY);
  }
  count = block_sum(count, red);
  if (threadIdx.x == 0) {
    map.row_ptr[qt + 1] = count;
    if (qt == 0) map.row_ptr[0] = 0;
  }
}

// Pass 2: in-place inclusive scan of row_ptr[1..n] by one workgroup.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void scan_kernel(int32_t* row_ptr, int n) {
  __shared__ int part[kScanThreads];
  const int t = threadIdx.x;
  const int seg = (n + kScanThreads - 1) / kScanThreads;
  const int lo = 1 + t * seg, hi = min(n + 1, lo + seg);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += row_ptr[i];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {  // Hillis-Steele inclusive scan
    int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = t > 0 ? part[t - 1] : 0;
  for (int i = lo; i < hi; ++i) {
    run += row_ptr[i];
    row_ptr[i] = run;
  }
}

// Pass 3: ascending list of non-empty k-tiles of each q-tile row.
__global__ __launch_bounds__(kThreads) void compact_kernel(svattn_tile_map map) {
  __shared__ int wave_cnt[kThreads / 64];
  const int qt = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int base = map.row_ptr[qt];
  const uint8_t* row = map.cls + (size_t)qt * map.n_kt;
  for (int k0 = 0; k0 < map.n_kt; k0 += kThreads) {
    const int kt = k0 + threadIdx.x;
    const uint8_t c = kt < map.n_kt ? row[kt] : SVATTN_TILE_EMPTY;
    const bool nz = c != SVATTN_TILE_EMPTY;
    const uint64_t bal = __ballot(nz);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = base, total = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      if (w < wave) off += wave_cnt[w];
      total += wave_cnt[w];
    }
    if (nz) {
      map.col[off + before] = kt;
      map.col_cls[off + before] = c;
    }
    base += total;
    __syncthreads();
  }
}

// Pass 4 (when qt_order is requested): rank of each q-tile under the order
// (longer row first, then smaller index), a strict total order, so
// qt_order[rank] = qt is a permutation.  One thread per q-tile compares its
// row length with every other row's, read through LDS in chunks.
__global__ __launch_bounds__(kThreads) void order_kernel(svattn_tile_map map) {
  __shared__ int len[kThreads];
  const int qt = blockIdx.x * kThreads + threadIdx.x;
  const int mine = qt < map.n_qt ? map.row_ptr[qt + 1] - map.row_ptr[qt] : 0;
  int rank = 0;
  for (int j0 = 0; j0 < map.n_qt; j0 += kThreads) {
    const int j = j0 + threadIdx.x;
    len[threadIdx.x] = j < map.n_qt ? map.row_ptr[j + 1] - map.row_ptr[j] : -1;
    __syncthreads();
    const int lim = min(kThreads, map.n_qt - j0);
    for (int i = 0; i < lim; ++i) {
      const int l = len[i];
      rank += (l > mine) | ((l == mine) & (j0 + i < qt));
    }
    __syncthreads();
  }
  if (qt < map.n_qt) map.qt_order[rank] = qt;
}

}  // namespace

hipError_t launch_tile_map(const Geo& g, const svattn_mask& m, const svattn_tile_map& map, uint32_t flags,
                           hipStream_t st) {
  hipLaunchKernelGGL(classify_kernel, dim3(map.n_qt), dim3(kThreads), 0, st, g, m, map, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, st, map.row_ptr, map.n_qt);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_kernel, dim3(map.n_qt), dim3(kThreads), 0, st, map);
  e = hipGetLastError();
  if (e != hipSuccess || !map.qt_order) return e;
  hipLaunchKernelGGL(order_kernel, dim3((map.n_qt + kThreads - 1) / kThreads), dim3(kThreads), 0, st, map);
  return hipGetLastError();
}

}  // namespace svattn
