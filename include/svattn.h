/*
 * svattn.h -- C ABI of the MI355X (gfx950) block-sparse spatio-temporal
 * attention library (libsvattn.so).
 *
 * The method: Sparse-VideoGen-style self-attention for video diffusion, where
 * every head is either spatial (keys in the query's own and nearby frames) or
 * temporal (keys at nearby patch positions in every frame), and both kinds
 * always keep every key of the first frame as an anchor ("Accelerating
 * Spatio-Temporal Attention for Video Diffusion on TPUs", Google for
 * Developers, as retold on aihirek.info, section "A Sparse VideoGen a figyelmi
 * fejeket osztályozza", paragraphs 2-3).  The kernel work is tiled: tiles with
 * no kept pair are skipped, fully kept tiles run without any mask, and only
 * boundary tiles evaluate the coordinate mask (same page, section "A
 * TPU-kernel kialakítása döntőnek bizonyult", paragraphs 2-3).  Temporal heads
 * may be run in a temporal-major token order (ainews.tenesys.com, list "Co się
 * zmieniło?", item 5).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  Buffers must stay valid until the
 *     work queued on `stream` has completed.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     GPU work is queued asynchronously on it; no entry point synchronises the
 *     host.
 *   - Tokens: a video latent of F frames x H x W patches, P = H*W patches per
 *     frame, N = F*P tokens.  Frame-major token t = f*P + y*W + x.
 *     Temporal-major position t' (anchor-first): t' < P holds frame 0, patch
 *     t'; otherwise u = t'-P holds patch u / (F-1) of frame 1 + u % (F-1).
 *   - Q, K, V, O: bf16, contiguous [heads, N, head_dim], 16-byte aligned.
 *   - Every argument is validated before any HIP call; a failed check returns
 *     a non-zero status and queues no work.  Nothing throws across the ABI.
 *     svattn_last_error() gives a thread-local message for the last failure.
 */
#ifndef SVATTN_H
#define SVATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define SVATTN_API __attribute__((visibility("default")))
#else
#define SVATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define SVATTN_VERSION 10400 /* major*10000 + minor*100 + patch */

/* Status codes. */
#define SVATTN_OK 0
#define SVATTN_ERR_INVALID_ARG 1  /* null pointer, bad size, misalignment, aliasing */
#define SVATTN_ERR_UNSUPPORTED 2  /* valid but not implemented (head_dim, tile size, kind/order) */
#define SVATTN_ERR_HIP 3          /* HIP runtime or launch failure, including "no device" */

/* Head kinds. */
#define SVATTN_SPATIAL 0   /* keep iff |f_q - f_k| <= window, or f_k == 0 */
#define SVATTN_TEMPORAL 1  /* keep iff max(|y_q-y_k|, |x_q-x_k|) <= radius, or f_k == 0 */
#define SVATTN_DENSE 2     /* keep every pair (the dense comparator) */

/* Token order a head's Q/K/V/O are stored in. */
#define SVATTN_FRAME_MAJOR 0
#define SVATTN_TEMPORAL_MAJOR 1   /* anchor-first; only for TEMPORAL and DENSE heads */
/* Anchor-first temporal-major over patches listed block by block: the patch
 * grid is cut into SVATTN_PATCH_BLOCK x SVATTN_PATCH_BLOCK blocks (the last
 * block row and column may be smaller), blocks in raster order, patches
 * inside a block in raster order.  Frame 0 comes first in that patch order,
 * then each patch (same order) brings its frames 1..F-1.  A library layout,
 * not one the pages give (they fix only that a patch's frames are adjacent):
 * consecutive positions then cover compact patch regions, so a temporal
 * head's tiles are fewer and less often BOUNDARY.  TEMPORAL and DENSE heads. */
#define SVATTN_TEMPORAL_MAJOR_BLOCKED 2
#define SVATTN_PATCH_BLOCK 4
/* Anchor-first temporal-major over patches listed in snake strips: the patch
 * grid is cut into column strips SVATTN_PATCH_STRIP patches wide (the last
 * strip narrower when W is odd), strips left to right, strip 0, 2, 4, ...
 * walked from patch row 0 down and strip 1, 3, ... from row H-1 up, each row
 * of a strip left to right.  Frame 0 comes first in that patch order, then
 * each patch (same order) brings its frames 1..F-1.  Also a library layout:
 * a q-tile then covers a patch region about two columns wide, and
 * consecutive patches are always grid neighbours, so a temporal head visits
 * fewer tiles, and fewer BOUNDARY ones, than with 4x4 blocks (the boundary
 * of a radius-r mask on a grid wider than tall runs mostly along columns).
 * TEMPORAL and DENSE heads. */
#define SVATTN_TEMPORAL_MAJOR_STRIPS 3
#define SVATTN_PATCH_STRIP 2

/* Tile classes stored in svattn_tile_map.cls / col_cls. */
#define SVATTN_TILE_EMPTY 0
#define SVATTN_TILE_BOUNDARY 1
#define SVATTN_TILE_FULL 2

/* Size of the optional workspace of svattn_forward / svattn_forward_ptrs. */
#define SVATTN_FORWARD_WORKSPACE_BYTES 256

/* Flags for svattn_build_tile_map_ex. */
#define SVATTN_MAP_ALL_BOUNDARY 1u  /* mark every non-empty tile BOUNDARY (the naive
                                       traversal that masks every visited tile) */
#define SVATTN_MAP_TILE_ALIGNED 2u  /* mark every non-empty tile FULL: the mask snapped to
                                       the tiles (ainews.tenesys.com, "W skrócie" and item 4
                                       of its list; oossa.com, body paragraph 1), read as:
                                       every pair of a tile that holds a kept pair is kept.
                                       The result then depends on block_q x block_k. */

typedef struct {
  int32_t frames, height, width; /* F, H, W >= 1; N = F*H*W < 2^23 (= 2^31 / 256), else
                                    SVATTN_ERR_UNSUPPORTED */
} svattn_geom;

typedef struct {
  int32_t kind;   /* SVATTN_SPATIAL / SVATTN_TEMPORAL / SVATTN_DENSE */
  int32_t order;  /* SVATTN_FRAME_MAJOR / SVATTN_TEMPORAL_MAJOR / SVATTN_TEMPORAL_MAJOR_BLOCKED /
                     SVATTN_TEMPORAL_MAJOR_STRIPS */
  int32_t window; /* spatial frame window w >= 0 (inclusive) */
  int32_t radius; /* temporal Chebyshev patch radius r >= 0 (inclusive) */
} svattn_mask;

/*
 * Tile map of one head layout: tile classes and, per q-tile, the ascending
 * list of non-empty k-tiles (CSR).  Classes count only in-range pairs: EMPTY
 * if no pair is kept, FULL if every in-range pair is kept, BOUNDARY otherwise.
 * All four arrays are caller-owned device buffers:
 *   cls     uint8 [n_qt * n_kt]   class of block (qt, kt) at qt*n_kt + kt
 *   row_ptr int32 [n_qt + 1]      row_ptr[0] = 0, nnz = row_ptr[n_qt]
 *   col     int32 [n_qt * n_kt]   capacity; entries [row_ptr[qt], row_ptr[qt+1])
 *   col_cls uint8 [n_qt * n_kt]   class of each listed block (BOUNDARY or FULL)
 *   qt_order int32 [n_qt]         optional (NULL: not built, q-tiles run in index
 *                                 order): the q-tile indices sorted by decreasing
 *                                 row length row_ptr[qt+1] - row_ptr[qt], equal
 *                                 lengths by increasing index.  The forward runs
 *                                 long rows first so short rows fill the end of
 *                                 the launch; results do not depend on it.
 * n_qt = ceil(N / block_q), n_kt = ceil(N / block_k) (svattn_tile_map_dims).
 */
typedef struct {
  int32_t block_q, block_k, n_qt, n_kt;
  uint8_t* cls;
  int32_t* row_ptr;
  int32_t* col;
  uint8_t* col_cls;
  int32_t* qt_order;
} svattn_tile_map;

/* Host only.  n_qt / n_kt for a geometry and tile shape.
 * block_q in {32, 64, 128, 256}, block_k in {32, 64, 128}. */
SVATTN_API int svattn_tile_map_dims(const svattn_geom* geom, int32_t block_q, int32_t block_k,
                         int32_t* n_qt, int32_t* n_kt);

/*
 * Tile classifier (the empty / full / boundary split of the aihirek.info page,
 * section "A TPU-kernel kialakítása döntőnek bizonyult", paragraphs 2-3).
 * Fills map->cls, row_ptr, col, col_cls (and qt_order if not NULL) for `mask`
 * in `mask->order`.  Exact:
 * classes are derived from the token coordinates of each block, not sampled.
 * map->block_q/block_k/n_qt/n_kt must be set (n_qt/n_kt as from
 * svattn_tile_map_dims).  The map depends only on (geom, mask, tile shape) and
 * can be reused across calls.  Spatial heads must be FRAME_MAJOR.  flags: 0,
 * SVATTN_MAP_ALL_BOUNDARY or SVATTN_MAP_TILE_ALIGNED (not both).
 */
SVATTN_API int svattn_build_tile_map(const svattn_geom* geom, const svattn_mask* mask,
                          svattn_tile_map* map, void* stream);
SVATTN_API int svattn_build_tile_map_ex(const svattn_geom* geom, const svattn_mask* mask,
                             svattn_tile_map* map, uint32_t flags, void* stream);

/*
 * Permutation index of the temporal-major order (ainews.tenesys.com, "Co się
 * zmieniło?", item 5).  perm[t'] = frame-major token at temporal-major
 * position t'; inv[t] = position of token t (inv may be NULL).  int32 [N].
 */
SVATTN_API int svattn_permutation_index(const svattn_geom* geom, int32_t* perm, int32_t* inv, void* stream);
/* The same for any token order: SVATTN_TEMPORAL_MAJOR (as above),
 * SVATTN_TEMPORAL_MAJOR_BLOCKED, SVATTN_TEMPORAL_MAJOR_STRIPS, or
 * SVATTN_FRAME_MAJOR (the identity).
 * SVATTN_ERR_INVALID_ARG for another order. */
SVATTN_API int svattn_permutation_index_order(const svattn_geom* geom, int32_t order, int32_t* perm,
                                              int32_t* inv, void* stream);

/*
 * Token reordering for temporal heads (ainews.tenesys.com, "Co się
 * zmieniło?", item 5: temporal heads run fastest when the tokens of one
 * patch position across frames sit next to each other, so the frame-major
 * sequence is reordered to temporal-major before attention and back after).
 * Reorder rows of a [heads, N, head_dim] bf16 tensor frame-major ->
 * temporal-major (permute) or back (unpermute): dst[h, t', :] = src[h,
 * perm[t'], :] and its inverse, perm as from svattn_permutation_index.
 *   src, dst  caller-owned device buffers [heads, N, head_dim] bf16, 16-byte
 *             aligned; they must not overlap (no in-place):
 *             SVATTN_ERR_INVALID_ARG otherwise, or for heads < 1
 *   head_dim  64 or 128 (SVATTN_ERR_UNSUPPORTED otherwise); heads * N *
 *             head_dim / 8 < 2^31
 * Bit-exact row moves, queued on `stream`.
 */
SVATTN_API int svattn_permute_tokens(const svattn_geom* geom, int32_t heads, int32_t head_dim,
                          const void* src, void* dst, void* stream);
SVATTN_API int svattn_unpermute(const svattn_geom* geom, int32_t heads, int32_t head_dim,
                     const void* src, void* dst, void* stream);
/* The same between frame-major and the temporal-major order `order`
 * (SVATTN_TEMPORAL_MAJOR, SVATTN_TEMPORAL_MAJOR_BLOCKED or
 * SVATTN_TEMPORAL_MAJOR_STRIPS; another order is SVATTN_ERR_INVALID_ARG): dst[h, t', :] = src[h, perm[t'], :] with perm from
 * svattn_permutation_index_order, and its inverse. */
SVATTN_API int svattn_permute_tokens_order(const svattn_geom* geom, int32_t order, int32_t heads,
                                           int32_t head_dim, const void* src, void* dst, void* stream);
SVATTN_API int svattn_unpermute_order(const svattn_geom* geom, int32_t order, int32_t heads, int32_t head_dim,
                                      const void* src, void* dst, void* stream);

/*
 * Block-sparse attention forward (aihirek.info, sections "A Sparse VideoGen a
 * figyelmi fejeket osztályozza" and "A TPU-kernel kialakítása döntőnek
 * bizonyult"): for every head h and query i,
 *   O[h,i,:] = sum_j softmax_j(scales[h] * Q[h,i,:].K[h,j,:] over kept j) V[h,j,:]
 * visiting only the k-tiles listed in maps[h]; FULL tiles run without a mask,
 * BOUNDARY tiles (and the ragged last k-tile) evaluate the coordinate mask.
 *   masks  host array [heads]: kind/order/window/radius of each head; Q/K/V/O
 *          of head h are in masks[h].order
 *   maps   host array [heads] of pointers to maps built for (geom, masks[h]);
 *          heads may share a map; all maps share one (block_q, block_k) with
 *          block_q in {32, 64, 128, 256} and block_k in {32, 64, 128} (each
 *          128-key tile runs as two 64-key halves, each masked exactly); row_ptr,
 *          col and col_cls must be 4-byte aligned (col_cls is read as aligned
 *          4-byte words, never past byte n_qt * n_kt - 1)
 *   scales host array [heads], finite fp32 softmax scales > 0
 *   lse    optional device fp32 [heads, N]: natural-log sum of exp of kept
 *          scaled scores (NULL to skip)
 * bf16 in, fp32 accumulation and softmax, bf16 out (round to nearest even).
 *   workspace  NULL, or caller-owned device memory of at least
 *          SVATTN_FORWARD_WORKSPACE_BYTES, 4-byte aligned, overlapping no
 *          tensor of the call.  With it the forward runs a persistent
 *          schedule: as many workgroups as the GPU holds at once take q-tiles
 *          from a counter in the workspace, in the maps' qt_order (longest rows
 *          first), so rows of unequal length keep every compute unit busy to
 *          the end.  The library clears the counter on `stream` before each
 *          launch; calls that can run at the same time (other streams) need
 *          distinct workspaces.  Its contents after the call are unspecified.
 * head_dim in {64, 128}.  o (and lse) must not overlap q, k or v.  Maps with
 * n_qt * n_kt >= 2^31 blocks are SVATTN_ERR_UNSUPPORTED.  The result
 * does not depend on the order of heads, on which heads share a map, on
 * qt_order or on the workspace: the output is bit-identical either way.
 */
SVATTN_API int svattn_forward(const svattn_geom* geom, int32_t heads, int32_t head_dim,
                              const svattn_mask* masks, const svattn_tile_map* const* maps,
                              const float* scales, const void* q, const void* k, const void* v,
                              void* o, float* lse, void* workspace, void* stream);

/*
 * svattn_forward with the persistent schedule and no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The work counter
 * lives in a 256-byte area the library holds in device memory, one copy per
 * GPU for the life of the process; the call allocates nothing.  The area's
 * device address is looked up on the first call on each device (a HIP call
 * made after every argument check).  Its size does not depend on the
 * arguments, so no size is rejected for it; the other limits are those of
 * svattn_forward.  Every call on one GPU shares that area: calls that can
 * overlap on one GPU (different streams, or graph replays that overlap) race
 * on it and must not be issued; calls queued on one stream are safe (the
 * counter is cleared by a kernel before each launch).  Arguments, layouts,
 * errors and results as for svattn_forward (bit-identical to it with a
 * workspace).
 */
SVATTN_API int svattn_forward_noalloc(const svattn_geom* geom, int32_t heads, int32_t head_dim,
                                      const svattn_mask* masks, const svattn_tile_map* const* maps,
                                      const float* scales, const void* q, const void* k, const void* v,
                                      void* o, float* lse, void* stream);

/*
 * Same as svattn_forward, with a separate device pointer per head instead of
 * one [heads, N, head_dim] tensor: q[h], k[h], v[h], o[h] are [N, head_dim]
 * bf16 (16-byte aligned), lse is NULL or a host array whose entries are NULL
 * or fp32 [N].  Lets frame-major heads read the model's tensors in place
 * while temporal heads read permuted copies.  No o[h] may overlap any input
 * or another head's output.
 */
SVATTN_API int svattn_forward_ptrs(const svattn_geom* geom, int32_t heads, int32_t head_dim,
                                   const svattn_mask* masks, const svattn_tile_map* const* maps,
                                   const float* scales, const void* const* q, const void* const* k,
                                   const void* const* v, void* const* o, float* const* lse,
                                   void* workspace, void* stream);

/*
 * Forward with the temporal-major permutation fused in (ainews.tenesys.com,
 * "Co się zmieniło?", item 5, without the separate reordering passes): Q, K,
 * V, O (and lse) of every head stay in frame-major order ([heads, N,
 * head_dim] as for svattn_forward), and a head whose mask has a
 * temporal-major order (TEMPORAL_MAJOR, TEMPORAL_MAJOR_BLOCKED or
 * TEMPORAL_MAJOR_STRIPS, its map built for that order; heads may mix them) is
 * computed in that order: the
 * kernel reads the row holding each position, which is a closed form of the
 * geometry (the permutation svattn_permutation_index_order writes), and
 * writes its O and lse rows back the same way.  The result equals
 * svattn_permute_tokens_order, then svattn_forward, then
 * svattn_unpermute_order, bit for bit.  Arguments, errors and workspace as
 * for svattn_forward.
 */
SVATTN_API int svattn_forward_fused(const svattn_geom* geom, int32_t heads, int32_t head_dim,
                                    const svattn_mask* masks, const svattn_tile_map* const* maps,
                                    const float* scales, const void* q, const void* k, const void* v, void* o,
                                    float* lse, void* workspace, void* stream);

/*
 * Head routing (aihirek.info, section "A Sparse VideoGen a figyelmi fejeket
 * osztályozza", paragraph 3): for a few query rows, each head's dense,
 * spatial and temporal attention outputs are computed, and the sparse mask
 * whose output deviates least from the dense one is chosen.  The pages fix
 * neither the rows nor the deviation; here the rows are the selected whole
 * q-tiles of the frame-major order (block_q rows each) and the deviation is
 * the mean squared difference of the bf16 outputs over those rows and all
 * head_dim columns; a tie goes to the spatial mask.  Each output row is
 * computed as several key splits merged by their log-sum-exp (the same
 * softmax up to fp32 rounding), then rounded to bf16.  Results are
 * deterministic.
 *   spatial, temporal  the two candidate masks, FRAME_MAJOR (window / radius
 *          as for svattn_forward; the same for every head)
 *   dense_map, spatial_map, temporal_map  tile maps of the frame-major order
 *          for a DENSE mask and for spatial / temporal, one tile shape
 *          (block_q in {32, 64, 128, 256}, block_k in {32, 64, 128})
 *   scales host fp32 [heads]
 *   qtiles host int32 [n_qtiles], 1 <= n_qtiles <= 32: distinct q-tiles, each
 *          wholly inside the sequence ((qtile + 1) * block_q <= N)
 *   q, k, v frame-major [heads, N, head_dim] bf16 (16-byte aligned)
 *   scratch device memory of svattn_route_scratch_bytes() bytes (16-byte
 *          aligned), caller-owned, needs no clearing; holds a work counter,
 *          the three outputs of the sampled rows as key splits (fp32 rows
 *          normalised over each split's keys, with their lse; the split
 *          count depends on heads and n_qtiles only) and the per-workgroup
 *          sums of the merge.  Two calls sharing a scratch must not overlap
 *          in time.
 *   err    device fp32 [heads, 2]: deviation of the spatial and the temporal
 *          output;  choice  device int32 [heads]: SVATTN_SPATIAL or
 *          SVATTN_TEMPORAL
 * Scratch, err and choice must not overlap each other or q, k, v.
 */
SVATTN_API int svattn_route_scratch_bytes(int32_t heads, int32_t head_dim, int32_t block_q, int32_t n_qtiles,
                                          size_t* bytes);
SVATTN_API int svattn_route_heads(const svattn_geom* geom, int32_t heads, int32_t head_dim,
                                  const svattn_mask* spatial, const svattn_mask* temporal,
                                  const svattn_tile_map* dense_map, const svattn_tile_map* spatial_map,
                                  const svattn_tile_map* temporal_map, const float* scales, const int32_t* qtiles,
                                  int32_t n_qtiles, const void* q, const void* k, const void* v, void* scratch,
                                  size_t scratch_bytes, float* err, int32_t* choice, void* stream);

/*
 * Reference forward for an arbitrary mask given as bits: masked softmax
 * attention over an explicit per-pair keep matrix (aihirek.info, section "A
 * Sparse VideoGen a figyelmi fejeket osztályozza", paragraph 1: attention
 * restricted to the kept query-key pairs; here the pairs are listed rather
 * than derived from coordinates).  For checking and debugging: it visits
 * every tile and masks every pair, so it runs at dense cost.
 *   n_tokens  1 <= n_tokens < 2^23 (SVATTN_ERR_INVALID_ARG otherwise)
 *   mask_bits device uint32 [per_head ? heads : 1][n_tokens][ceil(n_tokens/32)],
 *             caller-owned, 4-byte aligned, not overlapping o:
 *             bit (j % 32) of word j / 32 of row i is 1 iff pair (i, j) is kept
 *   A query row with no kept key gets O = 0 and lse = -inf.
 * block_q in {32, 64, 128, 256}, block_k in {32, 64} (SVATTN_ERR_UNSUPPORTED
 * otherwise); q, k, v, o, lse, scales, head_dim and stream as for
 * svattn_forward (single token order: rows are in whatever order the bits
 * use).
 */
SVATTN_API int svattn_forward_dense_mask(int32_t heads, int32_t n_tokens, int32_t head_dim,
                              const uint32_t* mask_bits, int32_t per_head, const float* scales,
                              const void* q, const void* k, const void* v, void* o, float* lse,
                              int32_t block_q, int32_t block_k, void* stream);

/* Static description of a status code. */
SVATTN_API const char* svattn_status_string(int status);
/* Thread-local detail of the last non-zero status returned on this thread. */
SVATTN_API const char* svattn_last_error(void);
/* SVATTN_VERSION of the loaded library. */
SVATTN_API int svattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SVATTN_H */
