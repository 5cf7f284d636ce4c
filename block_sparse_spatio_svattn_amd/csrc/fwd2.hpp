// Block-sparse flash-attention forward for gfx950 (CDNA4), bf16 MFMA,
// software-pipelined.
//
// What it computes ("Accelerating Spatio-Temporal Attention for Video
// Diffusion on TPUs", aihirek.info): softmax attention restricted to the kept
// query-key pairs of a spatial or temporal head with a first-frame anchor
// (section "A Sparse VideoGen a figyelmi fejeket osztályozza", paragraphs 2-3),
// visiting only the non-empty tiles of the tile map, with a mask-free path for
// full tiles and coordinate masking only on boundary tiles and on the ragged
// last k-tile (section "A TPU-kernel kialakítása döntőnek bizonyult",
// paragraphs 2-3).
//
// Work decomposition.  One workgroup owns one (head, q-tile) of
// BQ = NW * QG * 32 queries; each of its NW waves owns QG groups of 32
// queries and keeps their Q fragments in registers.  The workgroup walks the
// q-tile's list of non-empty k-tiles.  K and V tiles (BK keys each) go from
// HBM straight into an LDS ring of STAGES stages with global_load_lds_dwordx4
// (each lane's 16 bytes land at the wave's LDS base + 16 * lane), so no
// registers hold staged tiles.
//
// Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16 MFMA:
// lane l holds query l % 32 and 16 of the 32 keys of a key block, so a
// query's running max and sum stay inside the lane pair (l, l ^ 32).  The
// same registers, rounded to bf16, are the B operand of O^T += V^T P^T.  The A
// operand V^T is read from the row-major V tile with ds_read_b64_tr_b16: in
// each 16-lane group, lane j receives element j % 4 of the 8-byte rows read by
// lanes 4t + (j % 16) / 4, t = 0..3, i.e. four consecutive keys of one
// dimension.  Two such reads give the eight keys a lane's P fragment holds.
//
// LDS layout.  K and V tiles are row-major (one key per row, D bf16).  K rows
// are padded to 2D + 16 bytes, so the 16-byte reads of 16 consecutive keys
// start 4 banks apart (the DMA fills the padding slots with a harmless copy
// of a valid chunk).  V rows are unpadded and their 16-byte chunks are XOR
// swizzled by the row (vswz): a transpose read covers rows 4a..4a+3, and the
// swizzle gives each of those rows its own banks.
//
// Schedules.  The plain schedule (PP = false) runs every wave through
// S, mask, softmax and P V of a tile (of two tiles, for the d128 256 x 64
// launch), then one barrier; K/V of the next tile(s) stream into the other
// half of an LDS ring meanwhile.  The two-group
// schedule (PP = true, 8 waves) offsets waves 4-7 by half a tile so that on
// each SIMD one wave's MFMA work overlaps the other wave's softmax; it keeps a
// ring of three K/V stages (see the loop).
//
// Softmax.  exp2 with the scale folded into one FMA; masked scores are -inf.
// The running max only moves when a new score exceeds it by more than 8 in
// log2 units, so most tiles skip rescaling the accumulator, and a tile whose
// exponentials all stay within 2^8 of the running max needs no max reduction
// at all; the result differs only by rounding.  P is rounded to bf16 for the
// P V product; the row sum (and so lse) accumulates the fp32 values.
#pragma once

#include <type_traits>

#include "internal.hpp"

namespace svattn {
namespace fwd2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

template <int D, int BK, int NW, int QG>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int BQ = NW * QG * 32;
  static constexpr int CPR = D / 8;                       // 16-byte chunks per row
  static constexpr int RBK = D * 2 + 16;                  // K row stride in LDS (bytes)
  static constexpr int RBV = D * 2;                       // V row stride in LDS (bytes)
  static constexpr int K_PIECES = (BK * RBK + 1023) / 1024;  // 1 KB DMA pieces
  static constexpr int V_PIECES = (BK * RBV + 1023) / 1024;
  static constexpr int K_BYTES = K_PIECES * 1024;         // K region of a stage
  static constexpr int STAGE_BYTES = (K_PIECES + V_PIECES) * 1024;
  static constexpr int KB = BK / 32;                      // 32-key blocks per tile
  static constexpr int DS = D / 16;                       // 16-dim MFMA steps of Q K^T
  static constexpr int DB = D / 32;                       // 32-dim blocks of O
};

// Fragments of K (KPF) and of V (VPF) read from LDS ahead of the MFMA that
// consumes them.  Without the explicit prefetch (and the fences that hold
// it), the scheduler placed each read right before its MFMA and waited for
// it there, so every MFMA of the plain schedule waited out one LDS latency.
#ifndef SVATTN_KPF
#define SVATTN_KPF 6
#endif
#ifndef SVATTN_VPF
#define SVATTN_VPF 4
#endif
constexpr int KPF = SVATTN_KPF;
constexpr int VPF = SVATTN_VPF;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr uint32_t kXcdBlock = 32;          // consecutive work items dealt to one XCD
constexpr float kSumBound = 256.0f;         // 2^kRescaleThreshold
constexpr float kNegBig = -1.0e30f;        // initial running max (finite)

// XOR applied to the chunk index of V row r (an involution for a fixed row).
// Rows 4a..4a+3 map a 64-byte run of chunks to four distinct quarters of a
// 256-byte bank window and a 32-byte run to four distinct quarters of a
// 128-byte window (with 128-byte rows, D = 64, the row parity already picks
// the half of the 256-byte window).
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? 4 * (r & 3) + 2 * ((r >> 1) & 1) : 2 * (r & 3);
}

__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Load through the constant address space: a wave-uniform address becomes a
// scalar load even after the tile copies' inline asm, which the compiler must
// treat as a possible memory write.  Used only for the tile map, which no
// kernel writes while the forward runs.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Packed patch coordinates (y << 16 | x) of a key position, or a far-away
// value for positions >= N.
__device__ __forceinline__ int key_coord(const Geo& g, int order, int key) {
  if (key >= g.N) return 0x7fff7fff;
  const int p = patch_of(g, order, key);
  const int y = (int)g.divW.div((uint32_t)p);
  return (y << 16) | (p - y * g.W);
}

// Bits [lo, hi) of a 64-bit word (lo and hi clamped to [0, 64]).
__device__ __forceinline__ uint64_t bit_range(int lo, int hi) {
  lo = min(max(lo, 0), 64);
  hi = min(max(hi, lo), 64);
  const uint64_t below_hi = hi >= 64 ? ~0ull : ((1ull << hi) - 1ull);
  const uint64_t below_lo = lo >= 64 ? ~0ull : ((1ull << lo) - 1ull);
  return below_hi & ~below_lo;
}

template <int D, int BK, int NW, int QG, bool PP, bool BITS, bool PST, bool GTH>
// At least two waves per SIMD: workgroups of fewer than eight waves would
// otherwise be compiled for the whole register file and run one wave per SIMD.
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void fwd2_kernel(const FwdArgs a) {
  using C = Cfg<D, BK, NW, QG>;
  static_assert(BK % 32 == 0 && (D == 64 || D == 128), "tile shape");
  static_assert(!PP || NW == 8, "the two-group schedule pairs waves w and w + 4 on one SIMD");
  static_assert(!GTH || (!PP && !BITS), "gathered heads run the plain schedule over tile maps");
  // Tiles per barrier of the plain schedule: the d128, 256 x 64 launch runs
  // two tiles between barriers (four LDS stages, 132 KB), the others one.
  constexpr int TPB = (!PP && !BITS && D == 128 && BK == 64 && NW == 8) ? 2 : 1;
  constexpr int STAGES = PP ? 3 : 2 * TPB;
  __shared__ __attribute__((aligned(16))) char smem[STAGES * C::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) int kcs[STAGES][BK];
  // Gathered heads, plain schedule: the frame-major rows of the keys of the
  // tiles 2 TPB list steps ahead, one slot per tile, written by one wave.
  __shared__ int grow[GTH && !PP ? 2 * TPB : 1][BK];

  __shared__ int ticket;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // Persistent schedule: one work counter per XCD (workgroup b runs on XCD
  // b % 8).  Counter x deals items in blocks of kXcdBlock consecutive items,
  // block j of XCD x being items [(8 j + x) kXcdBlock, ...), so each XCD's
  // L2 serves neighbouring items of the longest-first order, and every XCD
  // starts on the longest ones.  An XCD whose counter runs dry takes items
  // from the next XCD's counter (thread 0's state; at most eight counters
  // are found dry, so every workgroup ends).
  int xq = blockIdx.x & 7, xdry = 0;
  auto next_item = [&]() __attribute__((always_inline)) -> int {
    while (xdry < 8) {
      const uint32_t t = atomicAdd(a.queue + xq, 1u);
      const int it = (int)(((t / kXcdBlock) * 8u + (uint32_t)xq) * kXcdBlock + t % kXcdBlock);
      if (it < a.n_items) return it;
      xq = (xq + 1) & 7;
      ++xdry;
    }
    return a.n_items;
  };

  // ---- work items ----
  // Static schedule (no queue): one item per workgroup, XCD-aware (workgroup
  // b runs on XCD b % 8).  Persistent schedule: as many workgroups as fit on
  // the chip at once, each taking the next item from a counter until the
  // items run out.  A chip hands the workgroups of a grid to its shader
  // engines in a fixed rotation, so with items of unequal length a static
  // grid leaves compute units idle while work waits for another engine; a
  // shared counter keeps every resident workgroup busy to the end.
  int item;
  if constexpr (!PST) {
    const int b = blockIdx.x;
    const int xcd = b & 7, s = b >> 3;
    item = ((s / a.chunk) * 8 + xcd) * a.chunk + (s % a.chunk);
  } else {
    if (tid == 0) ticket = next_item();
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(ticket);
  }
  while (item < a.n_items) {
  const int per_slot = a.n_sel * a.n_split;
  const int tail0 = a.n_items - a.tail_m * a.n_sel;  // first item of the rank-by-rank tail (tail_m > 1)
  int slot, sel, split;  // head slot, rank of the q-tile among the head's work items, key split
  if (a.tail_m > 1 && item >= tail0) {
    const int r = item - tail0;
    sel = r / a.tail_m;
    slot = a.n_slots - a.tail_m + (r - sel * a.tail_m);
    split = 0;
  } else {
    slot = item / per_slot;
    const int rest = item - slot * per_slot;
    sel = a.n_split == 1 ? rest : rest / a.n_split;
    split = rest - sel * a.n_split;
  }
  const HeadDesc& hd = a.heads[slot];
  const int qt = a.use_sel ? a.qt_sel[sel] : (BITS || !hd.qt_order) ? sel : ld_const(hd.qt_order + sel);
  const Geo g = a.g;
  const int N = g.N;

  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave index as a scalar
  const __bf16* __restrict__ Q = (const __bf16*)hd.q;
  const __bf16* __restrict__ K = (const __bf16*)hd.k;
  const __bf16* __restrict__ V = (const __bf16*)hd.v;
  const int q0 = qt * C::BQ + wave * (QG * 32);
  const int kind = hd.kind, order = hd.order;

  // ---- Q fragments (B operand of S^T = K Q^T); rows past N are clamped ----
  bf16x8 qf[QG][C::DS];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    const int qi = min(q0 + gq * 32 + l32, N - 1);
    const int qr = (GTH && hd.gather) ? tm_to_fm(g, order, qi) : qi;  // gathered head: the row of position qi
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) qf[gq][ds] = *(const bf16x8*)(Q + (size_t)qr * D + ds * 16 + hh * 8);
  }
  // Wait for Q here: the compiler then knows no load of its own is pending
  // in the loop, where the vector-memory counter belongs to the tile copies.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // ---- per-query mask parameters ----
  // spatial: kept non-anchor keys are [mq_a, mq_a + mq_b); temporal: patch (y, x)
  int mq_a[QG], mq_b[QG];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    const int qi = min(q0 + gq * 32 + l32, N - 1);
    if (kind == SVATTN_SPATIAL) {
      const int f = (int)g.divP.div((uint32_t)qi);
      const int flo = max(0, f - hd.window), fhi = min(g.F, f + hd.window + 1);
      mq_a[gq] = flo * g.P;
      mq_b[gq] = (fhi - flo) * g.P;
    } else {
      const int p = patch_of(g, order, qi);
      const int y = (int)g.divW.div((uint32_t)p);
      mq_a[gq] = y;
      mq_b[gq] = p - y * g.W;
    }
  }

  // ---- lane-constant LDS offsets ----
  // K (A operand of S^T): row kb*32 + l32, bytes 32*ds + 16*hh.
  const int koff = l32 * C::RBK + hh * 16;
  // V (transpose reads): 16-lane group G = lane / 16, i = lane % 16 reads row
  // 4*(G / 2) + i / 4 (+ 8 for the second read; rows are 4k + i / 4, so the
  // swizzle only depends on i), 8 bytes at dims 32*db + 16*(G % 2) + 4*(i % 4).
  const int G = lane >> 4, gi = lane & 15;
  const int vsw = vswz<D>(gi >> 2);
  int voff[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    const int chunk = 4 * db + 2 * (G & 1) + ((gi & 3) >> 1);
    voff[db] = (4 * (G >> 1) + (gi >> 2)) * C::RBV + ((chunk ^ vsw) << 4) + ((gi & 1) << 3);
  }

  floatx16 acc[QG][C::DB];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[gq][db] = floatx16{};
  float m_run[QG], l_run[QG];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    m_run[gq] = kNegBig;
    l_run[gq] = 0.f;
  }
  const float c = hd.scale_log2;
  // Keys of a tile fall into runs that share a patch (temporal heads, either
  // temporal-major order: runs of F-1 keys) or a patch row (temporal heads,
  // frame-major: runs of W keys); a lane decides a whole run at once when runs
  // are at least 16 keys long, else it reads per-key coordinates from LDS.
  const bool runs_ok = order != SVATTN_FRAME_MAJOR ? g.F - 1 >= 16 : g.W >= 16;
  const bool need_kc = kind == SVATTN_TEMPORAL && !runs_ok;

  // Tile list: the map's CSR row; with a bit mask, every k-tile.  A map of
  // (BK << sub)-key tiles is walked as 1 << sub tiles of BK keys per entry,
  // each masked exactly on its own; the last entry's second half is dropped
  // when it lies wholly past the last token.
  const int sub = BITS ? 0 : a.sub;
  int e0 = BITS ? 0 : ld_const(hd.row_ptr + qt);
  int len = BITS ? 0 : ld_const(hd.row_ptr + qt + 1) - e0;
  if (!BITS && a.n_split > 1) {
    // Entries of this split: the row's columns are ascending, so two binary
    // searches find those in [c0, c1), the split's 128-key units in map
    // k-tiles.
    const int units = (N + 127) >> 7, per = 128 / (BK << sub);
    const int c0 = (split * units / a.n_split) * per, c1 = ((split + 1) * units / a.n_split) * per;
    auto lower = [&](int v) __attribute__((always_inline)) -> int {
      int lo = 0, hi = len;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (ld_const(hd.col + e0 + mid) < v) lo = mid + 1;
        else hi = mid;
      }
      return lo;
    };
    const int lo = lower(c0), hi = lower(c1);
    e0 += lo;
    len = hi - lo;
  }
  const int32_t* __restrict__ col = hd.col + e0;
  const int n = [&]() __attribute__((always_inline)) -> int {
    if constexpr (BITS) return a.n_kt;
    const int nn = len << sub;
    return (sub && len > 0 && ld_const(col + len - 1) * (BK << sub) + BK >= N) ? nn - 1 : nn;
  }();

  const int cap = a.n_qt * a.n_kt;  // capacity of col / col_cls (map entries)
  const uint8_t* __restrict__ col_cls = hd.col_cls;
  // First key of list entry j.
  auto tile_key0 = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (BITS) return j * BK;
    else return ld_const(col + (j >> sub)) * (BK << sub) + (j & ((1 << sub) - 1)) * BK;
  };
  // Bit-mask rows of this lane's queries (bit j % 32 of word j / 32: pair kept).
  const uint32_t* bits_row[QG];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq)
    bits_row[gq] = BITS ? hd.bits + (size_t)min(q0 + gq * 32 + l32, N - 1) * a.words_per_row : nullptr;

  // Class of list entry e0 + j, read with a scalar load of its aligned
  // 4-byte word (col_cls is 4-byte aligned); a byte read serves the last
  // partial word of the buffer.
  auto tile_class = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (BITS) return SVATTN_TILE_BOUNDARY;
    const int e = e0 + (j >> sub);
    if ((e | 3) < cap) {
      const uint32_t w = ld_const((const uint32_t*)(col_cls + (e & ~3)));
      return (int)((w >> ((e & 3) * 8)) & 0xffu);
    }
    return __builtin_amdgcn_readfirstlane((int)col_cls[e]);
  };

  // First key and class of list entry t (zeros past the end of the list).
  auto fetch = [&](int t, int& key0, int& cls) __attribute__((always_inline)) {
    if (t < n) {
      key0 = tile_key0(t);
      cls = tile_class(t);
    }
  };

  // HBM -> LDS copies of K and V tiles.  A stage is K_PIECES + V_PIECES 1 KB
  // pieces; lane L of a piece fills byte 16 L of it, i.e. one 16-byte chunk
  // slot of a row, and fetches that chunk of the key's row (K padding slots
  // fetch the tile's first chunk).  Copier wave c copies K pieces c, c + NCW,
  // ... with its first KOPS copies and V pieces c, c + NCW, ... with the
  // rest, so whether a copy reads K or V is fixed at compile time.  A copy
  // blocks its wave until the vector-memory queue takes it, so the copies go
  // where a wave has no LDS reads in flight and, in the two-group schedule,
  // trickle through the softmax of the group without MFMA work.  They are
  // inline asm, so the compiler adds no wait for them before the LDS reads of
  // other stages; explicit waits precede the barriers.
  constexpr int NCW = PP ? NW / 2 : NW;       // copier waves: group B, or all
  constexpr int KOPS = (C::K_PIECES + NCW - 1) / NCW;
  constexpr int VOPS = (C::V_PIECES + NCW - 1) / NCW;
  constexpr int OPC = KOPS + VOPS;            // copies per copier wave
  const int cw = PP ? wave_u - NW / 2 : wave_u;  // index among the copiers
  // Piece (within K or V) and byte offset, from the tile's first row, of the
  // chunk each of this lane's copies fetches.  A copy then needs no vector
  // arithmetic: the tile's first row is a scalar base and the lane offset is
  // precomputed (the rows past N of a ragged tile are clamped at issue).
  auto op_piece = [&](int i) __attribute__((always_inline)) { return cw + (i < KOPS ? i : i - KOPS) * NCW; };
  int dma_off[OPC];
#pragma unroll
  for (int i = 0; i < OPC; ++i) {
    const bool is_k = i < KOPS;
    const int byte = op_piece(i) * 1024 + lane * 16;
    const int rb = is_k ? C::RBK : C::RBV;
    const int row = byte / rb, slot = (byte - row * rb) >> 4;
    const bool real = row < BK && slot < C::CPR;
    dma_off[i] = real ? (row * D + (is_k ? slot : (slot ^ vswz<D>(row))) * 8) * 2 : 0;
  }
  // Gathered heads: the tensors are frame-major and the head runs in a
  // temporal-major order; the row holding position t' is a closed form of
  // the geometry (tm_to_fm), so a gathered copy waits on no load.  Lane j of
  // a wave works out the row of the tile's key j once per tile, and each copy
  // takes the row of its key from that lane (a cross-lane read): one closed
  // form per lane and tile instead of one per copy.
  // The offsets are worked out when the tile's turn in the list comes, one
  // step before its copies go out, so the cross-lane reads land while the
  // wave computes scores.  (In the plain schedule only an item's first TPB
  // tiles are done this way; later tiles take their rows from a ring in LDS
  // that one wave fills per tile, see the main loop.)
  static_assert(BK <= 64, "one lane per key of a tile");
  const bool gathered = GTH && hd.gather;
  uint32_t goff[GTH ? OPC : 1];  // this lane's copy offsets for the next gathered tile
  auto gather_offsets = [&](int key0) __attribute__((always_inline)) {
    if constexpr (GTH) {
      const int rows = tm_to_fm(g, order, min(key0 + lane, N - 1));
#pragma unroll
      for (int i = 0; i < OPC; ++i) {
        const uint32_t off = (uint32_t)dma_off[i];
        const int row = __builtin_amdgcn_ds_bpermute((int)(off / (D * 2)) << 2, rows);
        goff[i] = (uint32_t)row * (uint32_t)(D * 2) + off % (D * 2);
      }
    }
  };
  // Copy i of this wave for the tile starting at key0, into stage st (ragged:
  // the tile runs past the last token).
  auto issue_op = [&](int i, int key0, int st, bool ragged) __attribute__((always_inline)) {
    const bool is_k = i < KOPS;
    const int pc = op_piece(i);
    if (cw < 0) return;
    if ((is_k && C::K_PIECES % NCW != 0 && i == KOPS - 1 && pc >= C::K_PIECES) ||
        (!is_k && C::V_PIECES % NCW != 0 && i == OPC - 1 && pc >= C::V_PIECES))
      return;
    // The tile's first row (or, gathered, the head's first row) as a scalar
    // base address (uniform by construction; readfirstlane makes that
    // explicit for the asm's SGPR operand).
    const uint64_t b64 = (uint64_t)((const char*)(is_k ? K : V) + (gathered ? 0 : (size_t)key0 * (D * 2)));
    const uint64_t base = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b64 >> 32)) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b64);
    uint32_t off = (uint32_t)dma_off[i];
    if (gathered) {  // the row holding the key's position (the last one past N), same chunk
      if constexpr (GTH) off = goff[i];
    } else if (ragged) {  // rows past N read row N-1 (their keys are masked)
      const int row = (int)(off / (D * 2));
      off = (uint32_t)((min(key0 + row, N - 1) - key0) * (D * 2) + (off - row * (D * 2)));
    }
    const uint32_t dst = lds_base + st * C::STAGE_BYTES + ((is_k ? 0 : C::K_PIECES) + pc) * 1024;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(dst), "v"(off), "s"(base) : "m0");
  };
  // Key coordinates of temporal heads for the tile starting at key0 (the
  // first BK threads of the copier waves).
  auto issue_kc = [&](int key0, int st) __attribute__((always_inline)) {
    const int t = tid - (PP ? NW / 2 : 0) * 64;
    if (need_kc && t >= 0 && t < BK) kcs[st][t] = fwd2::key_coord(g, order, key0 + t);
  };
  // All copies of a tile at once (one branch for a ragged tile).
  auto issue = [&](int key0, int st) __attribute__((always_inline)) {
    if (key0 + BK > N) {
#pragma unroll
      for (int i = 0; i < OPC; ++i) issue_op(i, key0, st, true);
    } else {
#pragma unroll
      for (int i = 0; i < OPC; ++i) issue_op(i, key0, st, false);
    }
    issue_kc(key0, st);
  };
  // All of this wave's copies have landed in LDS (the barrier that follows
  // makes every wave's copies visible).
  auto wait_tiles = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // S^T = K Q^T for the tile in stage st.  K fragments are read KPF MFMAs
  // ahead of their use; a scheduling fence after each MFMA keeps that order.
  auto qk = [&](int st, floatx16 (&S)[C::KB][QG], auto&& after_mfma) __attribute__((always_inline)) {
    const char* Ks = smem + st * C::STAGE_BYTES;
    constexpr int NR = C::DS * C::KB;
    auto ld = [&](int r) __attribute__((always_inline)) {
      const int ds = r / C::KB, kb = r % C::KB;
      return *(const bf16x8*)(Ks + kb * 32 * C::RBK + koff + ds * 32);
    };
    constexpr int PF = KPF < NR ? KPF : NR;  // prefetch depth, at most the fragment count
    bf16x8 kf[NR];
#pragma unroll
    for (int r = 0; r < PF; ++r) kf[r] = ld(r);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int ds = r / C::KB, kb = r % C::KB;
      if (r + PF < NR) kf[r + PF] = ld(r + PF);
#pragma unroll
      for (int gq = 0; gq < QG; ++gq)
        S[kb][gq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[r], qf[gq][ds], ds == 0 ? floatx16{} : S[kb][gq], 0, 0, 0);
      after_mfma(r);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Coordinate mask of the tile in stage st (boundary and ragged tiles only).
  // Key kk of the tile (kk = 32 kb + 8 (i / 4) + 4 hh + i % 4 for accumulator
  // element i) is an anchor key iff kk < P - key0, which can hold only on the
  // tile that reaches into the first P positions.  Each lane builds a 64-bit
  // keep mask of its query over the tile's keys from ranges and runs, then
  // applies it with one bit extract and one bit select per score.
  auto apply_keep = [&](int gq, uint64_t m, floatx16 (&S)[C::KB][QG]) __attribute__((always_inline)) {
    const uint32_t ninf = 0xff800000u;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      const uint32_t w = (uint32_t)(m >> (32 * kb)) >> (4 * hh);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int pos = 8 * (i / 4) + (i % 4);
        const uint32_t t = (uint32_t)((int)(w << (31 - pos)) >> 31);  // all ones iff kept
        // score = t ? score : -inf, written over the score in place (the
        // output is tied to the input), so masked and unmasked tiles leave
        // the scores in the same registers and nothing is copied where the
        // two paths meet.  (A bit cast straight from a vector element reads
        // element 0 with this compiler, so the score goes through a scalar.)
        float sf = S[kb][gq][i];
        asm("v_bfi_b32 %0, %1, %0, %2" : "+v"(sf) : "v"(t), "s"(ninf));
        S[kb][gq][i] = sf;
      }
    }
  };
  constexpr int MAXR = BK / 16 + 1;  // runs of >= 16 keys in one tile
  // Mask plan of the tile starting at key0 (in stage st), from coordinates or
  // mask bits only, so it runs before the tile's scores exist.  Returns, the
  // same for the whole wave: 1 if no score needs masking (not a boundary or
  // ragged tile, or every pair kept), 2 if every score of the wave's queries
  // is masked (the tile changes nothing for them: S, softmax and P V are
  // skipped), 0 if the per-lane keep masks in keep[] (bit kk: key key0 + kk of
  // the lane's query is kept) must be applied.
  auto plan = [&](int st, int key0, int cls, uint64_t (&keep)[QG]) __attribute__((always_inline)) -> int {
    if (!(cls == SVATTN_TILE_BOUNDARY || key0 + BK > N)) return 1;
    const int lim_anchor = g.P - key0;    // kk < lim_anchor: frame-0 key
    const int lim_n = N - key0;           // kk >= lim_n: past the last token
    // A full tile that runs past the last token keeps every in-range pair:
    // only the key range applies (with tile-aligned maps it keeps pairs the
    // coordinate mask would drop).
    const int mkind = cls == SVATTN_TILE_BOUNDARY ? kind : SVATTN_DENSE;
    {
      const uint64_t in_range = bit_range(0, lim_n);
      const uint64_t anchor = bit_range(0, lim_anchor);
      if constexpr (BITS) {
        // the lane's row of the bit mask: one 32-bit word per 32 keys
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
          const uint32_t w0 = bits_row[gq][key0 >> 5];
          const uint32_t w1 = (BK > 32 && lim_n > 32) ? bits_row[gq][(key0 >> 5) + 1] : 0u;
          keep[gq] = ((uint64_t)w1 << 32) | w0;
        }
      } else if (mkind == SVATTN_TEMPORAL && !runs_ok) {
        // short key runs: the lane's own keys tested one by one against the
        // per-key patch coordinates the copier waves wrote to LDS
        const uint32_t r = (uint32_t)hd.radius, r2 = 2u * r;
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) keep[gq] = anchor;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int kk0 = kb * 32 + 8 * i4 + 4 * hh;
            const int4 kc4 = *(const int4*)&kcs[st][kk0];
            const int kcv[4] = {kc4.x, kc4.y, kc4.z, kc4.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int yk = kcv[j] >> 16, xk = kcv[j] & 0xffff;
#pragma unroll
              for (int gq = 0; gq < QG; ++gq) {
                const bool ok = ((uint32_t)(yk - mq_a[gq]) + r <= r2) & ((uint32_t)(xk - mq_b[gq]) + r <= r2);
                keep[gq] |= (uint64_t)ok << (kk0 + j);
              }
            }
          }
        }
      } else if (mkind == SVATTN_SPATIAL) {
        // kept non-anchor keys: [mq_a, mq_a + mq_b)
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) keep[gq] = bit_range(mq_a[gq] - key0, mq_a[gq] + mq_b[gq] - key0) | anchor;
      } else if (mkind == SVATTN_TEMPORAL) {
        const int r = hd.radius;
        const uint32_t r2 = 2u * (uint32_t)r;
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) keep[gq] = anchor;
        const int s0 = max(key0, g.P) - key0;  // first non-anchor key of the tile
        const int e0 = min(BK, lim_n);         // past the last key of the tile
        if (s0 < e0) {
          if (order != SVATTN_FRAME_MAJOR) {
            // run: the F-1 frames of one patch.  Lane i works out run i of
            // the tile (its patch's rank in the order's patch sequence, the
            // patch's row and column, and its key range as a 64-bit mask);
            // the wave then reads each run's values back as scalars and
            // every lane tests its own query against them.  The run
            // arithmetic is the same for every wave, and in vector lanes it
            // does not queue on the compute unit's one scalar unit.
            const int F1 = g.F - 1;
            const int p0 = (int)g.divF1.div((uint32_t)(s0 + key0 - g.P));  // the first run's patch rank
            const int pr = p0 + (lane < MAXR ? lane : 0);
            const int rs = max(g.P + pr * F1 - key0, s0);
            const int re = min(g.P + (pr + 1) * F1 - key0, e0);  // empty when re <= rs (past the last patch)
            int ry, rx;
            if (order == SVATTN_TEMPORAL_MAJOR_BLOCKED) {
              blocked_yx(g, pr, ry, rx);
            } else if (order == SVATTN_TEMPORAL_MAJOR_STRIPS) {
              strips_yx(g, pr, ry, rx);
            } else {
              ry = (int)g.divW.div((uint32_t)pr);
              rx = pr - ry * g.W;
            }
            // bits [rs, re) of the tile's 64 keys, as two 32-bit halves
            auto below32 = [](int b) __attribute__((always_inline)) -> uint32_t {
              return b <= 0 ? 0u : b >= 32 ? 0xffffffffu : (1u << b) - 1u;
            };
            const uint32_t rlo = below32(re) & ~below32(rs);
            const uint32_t rhi = below32(re - 32) & ~below32(rs - 32);
            uint32_t klo[QG], khi[QG];
#pragma unroll
            for (int gq = 0; gq < QG; ++gq) {
              klo[gq] = 0u;
              khi[gq] = 0u;
            }
#pragma unroll
            for (int i = 0; i < MAXR; ++i) {
              const int y = __builtin_amdgcn_readlane(ry, i);
              const int x = __builtin_amdgcn_readlane(rx, i);
              const uint32_t blo = (uint32_t)__builtin_amdgcn_readlane((int)rlo, i);
              const uint32_t bhi = (uint32_t)__builtin_amdgcn_readlane((int)rhi, i);
#pragma unroll
              for (int gq = 0; gq < QG; ++gq) {
                const bool k = ((uint32_t)(y - mq_a[gq] + r) <= r2) & ((uint32_t)(x - mq_b[gq] + r) <= r2);
                klo[gq] |= k ? blo : 0u;
                khi[gq] |= k ? bhi : 0u;
              }
            }
#pragma unroll
            for (int gq = 0; gq < QG; ++gq) keep[gq] |= ((uint64_t)khi[gq] << 32) | klo[gq];
          } else {
            // run: one patch row of one frame; x advances with the key.  The
            // first run's row and column are divided out once; every later
            // run starts a new row at column 0 (the row after the last one
            // of a frame is row 0 of the next frame).
            int rs = s0;
            const int pp = (int)g.divP.mod((uint32_t)(key0 + rs));
            int y = (int)g.divW.div((uint32_t)pp), x0 = pp - y * g.W;
#pragma unroll
            for (int i = 0; i < MAXR; ++i) {
              const int re = min(rs + (g.W - x0), e0);
#pragma unroll
              for (int gq = 0; gq < QG; ++gq) {
                const bool ky = (uint32_t)(y - mq_a[gq] + r) <= r2;
                const int lo = rs + (mq_b[gq] - r - x0), hi = rs + (mq_b[gq] + r + 1 - x0);
                keep[gq] |= ky ? bit_range(max(lo, rs), min(hi, re)) : 0ull;
              }
              rs = max(re, rs);
              x0 = 0;
              y = y + 1 == g.H ? 0 : y + 1;
            }
          }
        }
      } else {
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) keep[gq] = ~0ull;  // dense: only the key range
      }
      bool none = true, all = true;
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) {
        keep[gq] &= in_range;
        none &= keep[gq] == 0ull;
        all &= keep[gq] == ~0ull;
      }
      if (__all(none)) return 2;
      if (__all(all)) return 1;
      return 0;
    }
  };


  // plan + apply in one step (the two-group schedule): masked scores become
  // -inf before the softmax.
  auto mask = [&](int st, int key0, int cls, floatx16 (&S)[C::KB][QG]) __attribute__((always_inline)) -> int {
    uint64_t keep[QG];
    const int m = plan(st, key0, cls, keep);
    if (m != 1) {
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) apply_keep(gq, m == 2 ? 0ull : keep[gq], S);
    }
    return m;
  };

  // Online softmax of one tile's scores; P (bf16) is the B operand of P V.
  // The exponentials are first taken against the running max as it stands.
  // If every lane's partial row sum stays within 2^8 (so no exponential
  // exceeds 2^8), the tile's max cannot have passed the running max by more
  // than the rescale threshold, and the values stand as computed: the usual
  // case, with no max reduction.  Otherwise (the first tile of a row, whose
  // running max is still the initial value, or a tile with larger scores)
  // the exact tile max is taken, the accumulator is rescaled if the max moves,
  // and the exponentials are taken again.
  auto softmax = [&](floatx16 (&S)[C::KB][QG], bf16x8 (&P)[2 * C::KB][QG], auto&& after_chunk) __attribute__((always_inline)) {
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
      auto exps = [&](auto&& hook) __attribute__((always_inline)) -> float {
        const float mc = m_run[gq] * c;
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            bf16x8 p;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][gq][h * 8 + j], c, -mc));
              ls += e;
              p[j] = (__bf16)e;
            }
            P[kb * 2 + h][gq] = p;
            hook((gq * C::KB + kb) * 2 + h);
          }
        }
        return ls;
      };
      float ls = exps(after_chunk);
      if (__any(!(ls <= kSumBound))) {  // also true for inf and NaN
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[kb][gq][i]);
        mx = max_xor32(mx);
        const float m_new = fmaxf(m_run[gq], mx);
        const bool need = (m_new - m_run[gq]) * c > kRescaleThreshold;
        if (__any(need)) {
          const float alpha = need ? __builtin_amdgcn_exp2f((m_run[gq] - m_new) * c) : 1.0f;
          if (need) m_run[gq] = m_new;
          l_run[gq] *= alpha;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) acc[gq][db] *= alpha;
        }
        ls = exps([](int) {});
      }
      l_run[gq] += ls;
    }
  };

  // O^T += V^T P^T for the tile in stage st.  V^T fragments (two transpose
  // reads each) are read VPF MFMAs ahead of their use, fenced like qk.
  auto pv = [&](int st, const bf16x8 (&P)[2 * C::KB][QG], auto&& after_mfma) __attribute__((always_inline)) {
    const char* Vs = smem + st * C::STAGE_BYTES + C::K_BYTES;
    constexpr int NR = 2 * C::KB * C::DB;
    auto ld = [&](int r) __attribute__((always_inline)) {
      const int ks = r / C::DB, db = r % C::DB;
      const char* base = Vs + ks * 16 * C::RBV + voff[db];
      const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(base));
      const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(base + 8 * C::RBV));
      const short4v both[2] = {lo, hi};
      bf16x8 va;
      __builtin_memcpy(&va, both, sizeof(va));
      return va;
    };
    constexpr int PF = VPF < NR ? VPF : NR;
    bf16x8 vf[NR];
#pragma unroll
    for (int r = 0; r < PF; ++r) vf[r] = ld(r);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int ks = r / C::DB, db = r % C::DB;
      if (r + PF < NR) vf[r + PF] = ld(r + PF);
#pragma unroll
      for (int gq = 0; gq < QG; ++gq)
        acc[gq][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[r], P[ks][gq], acc[gq][db], 0, 0, 0);
      after_mfma(r);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  floatx16 S[C::KB][QG];
  bf16x8 P[2 * C::KB][QG];

  constexpr int NCH = 2 * C::KB * QG;  // softmax chunks per tile
  // The copier's pieces spread over the softmax chunks of one tile.
  auto dma_in_softmax = [&](int chunk, bool dma, int key0, int st) __attribute__((always_inline)) {
    if (!dma) return;
#pragma unroll
    for (int i = 0; i < OPC; ++i)
      if ((i * NCH) / OPC == chunk) issue_op(i, key0, st, key0 + BK > N);
  };
  auto next_stage = [&](int st) __attribute__((always_inline)) { return st == STAGES - 1 ? 0 : st + 1; };

  int key_c = 0, cls_c = 0, key_n = 0, cls_n = 0;
  fetch(0, key_c, cls_c);
  fetch(1, key_n, cls_n);

  if constexpr (PP) {
    // Two wave groups, A = waves 0-3 and B = waves 4-7; waves w and w + 4
    // share a SIMD.  Step j has two barrier-separated phases.  Group A runs
    // its MFMA work (P V of tile j-1, then S = K Q^T of tile j) in the first
    // phase and its VALU work (mask and softmax of tile j) in the second;
    // group B runs the softmax of tile j-1 in the first phase and P V of tile
    // j-1 plus S of tile j in the second.  So in every phase one wave of each
    // SIMD feeds the matrix cores while the other runs the exponentials.
    // Tile t lives in LDS stage t % 3: K of tile j is read during step j, V of
    // tile j during step j+1, and group B copies tile j+1 during its softmax
    // in step j into the stage of tile j-2, whose last reader finished in step
    // j-1.  Each group has its own loop (a compile-time flag) so that the
    // compiler sees which of S and P is live.
    if (n > 0) issue(key_c, 0);
    if (n > 1) issue(key_n, 1);
    wait_tiles();
    __syncthreads();
    const bool grp_b = wave_u >= 4;
    auto mfma_work = [&](int j, int sj, int sp) __attribute__((always_inline)) {
      __builtin_amdgcn_s_setprio(1);
      if (j >= 1) pv(sp, P, [](int) {});
      if (j < n) qk(sj, S, [](int) {});
      __builtin_amdgcn_s_setprio(0);
    };
    // key_c / cls_c: tile j; key_n / cls_n: tile j+1; key_p / cls_p: tile j-1
    auto run = [&](auto group_b) __attribute__((always_inline)) {
      constexpr bool B = decltype(group_b)::value;
      int sj = 0;  // stage of tile j
      int key_p = 0, cls_p = 0;
      for (int j = 0; j <= n; ++j) {
        const int sp = sj == 0 ? STAGES - 1 : sj - 1, sn = next_stage(sj);
        int key_nn = 0, cls_nn = 0;
        fetch(j + 2, key_nn, cls_nn);
        if constexpr (!B) {
          mfma_work(j, sj, sp);
          __syncthreads();
          if (j < n) {
            (void)mask(sj, key_c, cls_c, S);
            softmax(S, P, [](int) {});
          }
        } else {
          if (j >= 1) {
            const bool dma = j + 1 < n;
            if (dma) issue_kc(key_n, sn);
            (void)mask(sp, key_p, cls_p, S);
            softmax(S, P, [&](int ch) { dma_in_softmax(ch, dma, key_n, sn); });
          }
          __syncthreads();
          mfma_work(j, sj, sp);
        }
        wait_tiles();
        __syncthreads();
        key_p = key_c; cls_p = cls_c;
        key_c = key_n; cls_c = cls_n;
        key_n = key_nn; cls_n = cls_nn;
        sj = sn;
      }
    };
    if (grp_b) run(std::true_type{});
    else run(std::false_type{});
  } else {
    // Tiles go in groups of TPB between two barriers, over a ring of 2 TPB
    // stages: group g reads stages (g % 2) TPB + u, u < TPB.  Every wave
    // runs S, mask and softmax of a tile, then the copies of the tile TPB
    // places later (into the other half of the ring, whose readers finished
    // before the last barrier; the wave has no LDS reads in flight here),
    // then P V; one barrier ends the group.
    // Tile list window: wk/wc[0] is the current tile, [TPB] the one whose
    // copies go out with it, [LA] fetched ahead (gathered heads also use
    // [2 TPB], the tile whose rows go into the row ring).
    //
    // Gathered heads: the rows of a tile's keys are a closed form that every
    // wave would otherwise work out for every tile; here the rows of tile
    // t + 2 TPB are worked out once, by wave t % NW while the group of tile t
    // runs, into slot (t + 2 TPB) % 2 TPB of `grow`, and read back by every
    // wave with its copies' offsets one group later (a barrier in between).
    // A slot is rewritten 2 TPB tiles after it was written, always in a later
    // group than its readers.  The first 2 TPB tiles: the first TPB work out
    // their own offsets, the next TPB go into the ring before the first
    // barrier.
    constexpr int LA = GTH ? 2 * TPB + 1 : TPB + 1;
    int wk[LA + 1], wc[LA + 1];
#pragma unroll
    for (int i = 0; i <= LA; ++i) {
      wk[i] = 0;
      wc[i] = 0;
    }
#pragma unroll
    for (int i = 0; i < LA; ++i) fetch(i, wk[i], wc[i]);
    auto ring_write = [&](int t, int key0) __attribute__((always_inline)) {
      if constexpr (GTH) {
        if (wave_u == t % NW && lane < BK) grow[t % (2 * TPB)][lane] = tm_to_fm(g, order, min(key0 + lane, N - 1));
      }
    };
    auto ring_offsets = [&](int t) __attribute__((always_inline)) {
      if constexpr (GTH) {
#pragma unroll
        for (int i = 0; i < OPC; ++i) {
          const uint32_t off = (uint32_t)dma_off[i];
          // (the clamp keeps a copy inside the tensor whatever the slot holds)
          const uint32_t row = min((uint32_t)grow[t % (2 * TPB)][off / (D * 2)], (uint32_t)(N - 1));
          goff[i] = row * (uint32_t)(D * 2) + off % (D * 2);
        }
      }
    };
    if (n > 0) {
      if (gathered) gather_offsets(wk[0]);
      issue(wk[0], 0);
    }
    if constexpr (TPB == 2)
      if (n > 1) {
        if (gathered) gather_offsets(wk[1]);
        issue(wk[1], 1);
      }
    if (gathered) {
#pragma unroll
      for (int t = TPB; t < 2 * TPB; ++t)
        if (t < n) ring_write(t, wk[t]);
    }
    wait_tiles();
    __syncthreads();
    int grp = 0;  // first stage of the current group
    for (int j = 0; j < n; j += TPB) {
#pragma unroll
      for (int u = 0; u < TPB; ++u) {
        const int t = j + u;
        if (u == 0 || t < n) {
          const int st = grp + u;
          fetch(t + LA, wk[LA], wc[LA]);
          if (gathered) {
            if (t + TPB < n) ring_offsets(t + TPB);
            if (t + 2 * TPB < n) ring_write(t + 2 * TPB, wk[2 * TPB]);
          }
          // a wave whose queries keep no key of this tile skips S, softmax and P V
          uint64_t keep[QG];
          const int ms = plan(st, wk[0], wc[0], keep);
          if (ms != 2) {
            qk(st, S, [](int) {});
            if (ms == 0) {
#pragma unroll
              for (int gq = 0; gq < QG; ++gq) apply_keep(gq, keep[gq], S);
            }
            softmax(S, P, [](int) {});
          }
          __builtin_amdgcn_sched_barrier(0);
          if (t + TPB < n) issue(wk[TPB], (grp ^ TPB) + u);
          __builtin_amdgcn_sched_barrier(0);
          if (ms != 2) pv(st, P, [](int) {});
#pragma unroll
          for (int i = 0; i < LA; ++i) {
            wk[i] = wk[i + 1];
            wc[i] = wc[i + 1];
          }
        }
      }
      wait_tiles();
      __syncthreads();
      grp ^= TPB;
    }
  }

  // ---- epilogue: O = acc / l, lse = m*scale + ln l ----
  __bf16* __restrict__ O = (__bf16*)hd.o;
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    const int qp = q0 + gq * 32 + l32;
    const float l = sum_xor32(l_run[gq]);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    if (!BITS && !GTH && a.partial) {
      // split partial (selected whole q-tiles only, so qp < N): fp32 rows
      const int pr = (sel * a.n_split + split) * C::BQ + (qp - qt * C::BQ);
      float* __restrict__ Op = (float*)hd.o + (size_t)pr * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          floatx4 ov;
#pragma unroll
          for (int j = 0; j < 4; ++j) ov[j] = acc[gq][db][i4 * 4 + j] * inv;
          *(floatx4*)(Op + db * 32 + 8 * i4 + 4 * hh) = ov;
        }
      }
      if (hh == 0) hd.lse[pr] = l > 0.f ? m_run[gq] * hd.scale + __logf(l) : -INFINITY;
      continue;
    }
    if (qp < N) {
      // gathered head: scatter to the row of position qp; compact output: rank-major rows
      const int qi = (GTH && hd.gather) ? tm_to_fm(g, order, qp) : a.compact ? sel * C::BQ + (qp - qt * C::BQ) : qp;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = db * 32 + 8 * i4 + 4 * hh;
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 ov;
#pragma unroll
          for (int j = 0; j < 4; ++j) ov[j] = (__bf16)(acc[gq][db][i4 * 4 + j] * inv);
          *(bf16x4*)(O + (size_t)qi * D + d0) = ov;
        }
      }
      if (hd.lse && hh == 0) hd.lse[qi] = l > 0.f ? m_run[gq] * hd.scale + __logf(l) : -INFINITY;
    }
  }

  if constexpr (!PST) break;
  __syncthreads();  // every wave has read the previous ticket
  if (tid == 0) ticket = next_item();
  __syncthreads();
  item = __builtin_amdgcn_readfirstlane(ticket);
  }  // items
}

// Workgroups of this kernel resident on the current device at once (cached
// per device).
template <int D, int BK, int NW, int QG, bool PP, bool BITS, bool PST, bool GTH>
hipError_t resident_workgroups(int* out) {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fwd2_kernel<D, BK, NW, QG, PP, BITS, PST, GTH>, NW * 64, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    v = per_cu * cus > 0 ? per_cu * cus : 1;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  *out = v;
  return hipSuccess;
}

// Persistent schedule when a queue is given (plain schedule over a tile map
// only: the two-group schedule serves launches of equal-length rows, where a
// static grid already balances), else the static grid.  Launches with
// gathered heads use their own instantiation, so the others carry no code for
// it.
template <int D, int BK, int NW, int QG, bool PP, bool BITS, bool GTH>
hipError_t launch_sched(const FwdArgs& a, hipStream_t st) {
  if constexpr (!PP && !BITS) {
    if (a.queue) {
      int resident = 0;
      hipError_t e = resident_workgroups<D, BK, NW, QG, PP, BITS, true, GTH>(&resident);
      if (e != hipSuccess) return e;
      const int grid = resident < a.n_items ? resident : a.n_items;
      hipLaunchKernelGGL((fwd2_kernel<D, BK, NW, QG, PP, BITS, true, GTH>), dim3(grid), dim3(NW * 64), 0, st, a);
      return hipGetLastError();
    }
  }
  const int per_round = 8 * a.chunk;
  const int grid = ((a.n_items + per_round - 1) / per_round) * per_round;
  hipLaunchKernelGGL((fwd2_kernel<D, BK, NW, QG, PP, BITS, false, GTH>), dim3(grid), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

template <int D, int BK, int NW, int QG, bool PP, bool BITS = false>
hipError_t launch(const FwdArgs& a, hipStream_t st) {
  if constexpr (!PP && !BITS) {
    bool gather = false;
    for (int i = 0; i < a.n_slots; ++i) gather = gather || a.heads[i].gather;
    if (gather) return launch_sched<D, BK, NW, QG, PP, BITS, true>(a, st);
  }
  return launch_sched<D, BK, NW, QG, PP, BITS, false>(a, st);
}

}  // namespace fwd2
}  // namespace svattn
