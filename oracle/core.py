"""fp64 CPU oracle: coordinates, masks, permutation, tile maps, attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every function below is
a direct, unblocked statement of its definition; row blocking in
``attend_head`` only bounds memory and does not change any arithmetic.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Geometry:
    frames: int
    height: int
    width: int

    @property
    def patches(self) -> int:
        return self.height * self.width

    @property
    def n(self) -> int:
        return self.frames * self.patches


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Token coordinates and orders (tenesys page, list item 5: frame-major vs
# temporal-major token layouts; the flattening itself is a reading).
# ---------------------------------------------------------------------------

def frame_major_coords(g: Geometry):
    """Frame-major token t -> (frame, patch row y, patch column x)."""
    f = np.repeat(np.arange(g.frames), g.patches)
    y = np.tile(np.repeat(np.arange(g.height), g.width), g.frames)
    x = np.tile(np.arange(g.width), g.frames * g.height)
    return f, y, x


def temporal_major_perm(g: Geometry) -> np.ndarray:
    """perm[t'] = frame-major token stored at temporal-major position t'.

    Anchor-first temporal-major order: the whole first frame stays in front in
    patch order, then every patch brings its frames 1..F-1 together.  Built by
    listing the tokens in that order, not from a position formula.
    """
    order = list(range(g.patches))          # frame 0, patch order
    for p in range(g.patches):
        for f in range(1, g.frames):
            order.append(f * g.patches + p)
    return np.asarray(order, dtype=np.int64)


PATCH_BLOCK = 4


def blocked_patch_order(g: Geometry) -> np.ndarray:
    """Raster patch indices listed in blocked order.

    Not from the pages (they fix only that a temporal head's frames of one
    patch sit together): the library may also list the patches of a
    temporal-major layout block by block, so that a run of consecutive
    positions covers a compact patch region instead of a strip of one patch
    row.  The grid is cut into PATCH_BLOCK x PATCH_BLOCK blocks (the last block
    row and column may be smaller), blocks in raster order, patches inside a
    block in raster order.  Built by sorting the patches on (block row, block
    column, row in block, column in block), not from a rank formula.
    """
    b = PATCH_BLOCK
    y, x = np.divmod(np.arange(g.patches), g.width)
    return np.lexsort((x % b, y % b, x // b, y // b)).astype(np.int64)  # last key is the primary one


def temporal_major_blocked_perm(g: Geometry) -> np.ndarray:
    """perm[t'] for the anchor-first temporal-major layout over patches in
    blocked order: frame 0 in blocked patch order, then for each patch in that
    order its frames 1..F-1."""
    seq = blocked_patch_order(g)
    order = [int(p) for p in seq]
    for p in seq:
        for f in range(1, g.frames):
            order.append(f * g.patches + int(p))
    return np.asarray(order, dtype=np.int64)


PATCH_STRIP = 2


def strip_patch_order(g: Geometry) -> np.ndarray:
    """Raster patch indices listed in snake strips.

    Not from the pages either (a library layout, like the blocked order): the
    grid is cut into column strips PATCH_STRIP patches wide (the last one
    narrower when the width does not divide), the strips are listed left to
    right, an even-numbered strip is walked from the top patch row down and an
    odd-numbered one from the bottom row up, and each patch row of a strip is
    listed left to right.  Consecutive patches are then always grid neighbours,
    also from one strip to the next.  Built by sorting the patches on (strip,
    row in the strip's walking direction, column), not from a rank formula.
    """
    y, x = np.divmod(np.arange(g.patches), g.width)
    strip = x // PATCH_STRIP
    walk = np.where(strip % 2 == 1, g.height - 1 - y, y)
    return np.lexsort((x, walk, strip)).astype(np.int64)  # last key is the primary one


def temporal_major_strips_perm(g: Geometry) -> np.ndarray:
    """perm[t'] for the anchor-first temporal-major layout over patches in
    snake-strip order: frame 0 in that patch order, then for each patch in it
    its frames 1..F-1."""
    seq = strip_patch_order(g)
    order = [int(p) for p in seq]
    for p in seq:
        for f in range(1, g.frames):
            order.append(f * g.patches + int(p))
    return np.asarray(order, dtype=np.int64)


def layout_tokens(g: Geometry, order: str) -> np.ndarray:
    """Frame-major token id held at each position of a head's token order
    ("fm", "tm", "tmb" for temporal-major over blocked patches, or "tms" for
    temporal-major over snake strips)."""
    if order == "fm":
        return np.arange(g.n, dtype=np.int64)
    if order == "tm":
        return temporal_major_perm(g)
    if order == "tmb":
        return temporal_major_blocked_perm(g)
    if order == "tms":
        return temporal_major_strips_perm(g)
    raise ValueError(order)


# ---------------------------------------------------------------------------
# Masks (aihirek page, section on SVG head classes, paragraphs 2 and 3).
# ---------------------------------------------------------------------------

def keep_matrix(g: Geometry, kind: str, window: int, radius: int,
                rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """Boolean keep[i, j] for frame-major query tokens ``rows`` and key tokens ``cols``."""
    f, y, x = frame_major_coords(g)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    anchor = (f[cols] == 0)[None, :]
    if kind == "dense":
        return np.ones((rows.size, cols.size), dtype=bool)
    if kind == "spatial":
        near = np.abs(f[rows][:, None] - f[cols][None, :]) <= window
    elif kind == "temporal":
        dy = np.abs(y[rows][:, None] - y[cols][None, :])
        dx = np.abs(x[rows][:, None] - x[cols][None, :])
        near = np.maximum(dy, dx) <= radius
    else:
        raise ValueError(kind)
    return near | anchor


def kept_counts_per_row(g: Geometry, kind: str, window: int, radius: int,
                        rows: np.ndarray, block: int = 512) -> np.ndarray:
    """Number of kept keys for each query token in ``rows`` (brute force)."""
    cols = np.arange(g.n)
    out = np.empty(len(rows), dtype=np.int64)
    for s in range(0, len(rows), block):
        out[s:s + block] = keep_matrix(g, kind, window, radius, rows[s:s + block], cols).sum(1)
    return out


def kept_count(g: Geometry, kind: str, window: int, radius: int) -> int:
    """Total kept query-key pairs of one head (brute force over every pair)."""
    return int(kept_counts_per_row(g, kind, window, radius, np.arange(g.n)).sum())


# ---------------------------------------------------------------------------
# Tile map (aihirek page, section on the TPU kernel, paragraphs 2-3: skip empty
# tiles, mask-free full tiles, coordinate masks on boundary tiles).
# Classes: 0 empty, 1 boundary, 2 full; counted over in-range pairs only.
# ---------------------------------------------------------------------------

def tile_counts(g: Geometry, kind: str, window: int, radius: int, order: str,
                block_q: int, block_k: int, qtiles: Optional[Sequence[int]] = None):
    """Kept in-range pairs of every (q-tile, k-tile) block, by brute force.

    Returns counts [len(qtiles), n_kt] int64 and the in-range block sizes.
    """
    toks = layout_tokens(g, order)
    n = g.n
    n_qt = -(-n // block_q)
    n_kt = -(-n // block_k)
    qtiles = range(n_qt) if qtiles is None else qtiles
    col_lo = np.arange(n_kt) * block_k
    col_size = np.minimum(n, col_lo + block_k) - col_lo      # in-range keys per k-tile
    counts = np.zeros((len(qtiles), n_kt), dtype=np.int64)
    sizes = np.zeros((len(qtiles), n_kt), dtype=np.int64)
    for i, qt in enumerate(qtiles):
        r0, r1 = qt * block_q, min(n, (qt + 1) * block_q)
        keep = keep_matrix(g, kind, window, radius, toks[r0:r1], toks)
        padded = np.zeros((r1 - r0, n_kt * block_k), dtype=bool)
        padded[:, :n] = keep
        counts[i] = padded.reshape(r1 - r0, n_kt, block_k).sum(axis=(0, 2))
        sizes[i] = (r1 - r0) * col_size
    return counts, sizes


def tile_map(g: Geometry, kind: str, window: int, radius: int, order: str,
             block_q: int, block_k: int, qtiles: Optional[Sequence[int]] = None):
    """Brute-force tile classes and the per-q-tile list of non-empty k-tiles.

    Returns (cls [n_qt, n_kt] uint8, row_ptr [n_qt+1] int32, col [nnz] int32,
    col_cls [nnz] uint8), columns ascending within each row.  With ``qtiles``
    only those q-tile rows are built (cls has len(qtiles) rows, row_ptr counts
    only those rows).
    """
    counts, sizes = tile_counts(g, kind, window, radius, order, block_q, block_k, qtiles)
    cls = np.where(counts == 0, 0, np.where(counts == sizes, 2, 1)).astype(np.uint8)
    n_rows, n_kt = cls.shape
    row_ptr = [0]
    col, col_cls = [], []
    for qt in range(n_rows):
        for kt in range(n_kt):
            if cls[qt, kt] != 0:
                col.append(kt)
                col_cls.append(cls[qt, kt])
        row_ptr.append(len(col))
    return (cls, np.asarray(row_ptr, dtype=np.int32), np.asarray(col, dtype=np.int32),
            np.asarray(col_cls, dtype=np.uint8))


def qtile_order(row_ptr: np.ndarray) -> np.ndarray:
    """Visiting order of the q-tiles of a tile map: indices sorted by decreasing
    row length row_ptr[qt+1] - row_ptr[qt], equal lengths by increasing index.

    The pages leave the order in which query tiles are processed open (each
    q-tile's output is independent of the others); this order is the library's
    longest-first schedule, stated here so the map can be checked exactly.
    """
    lengths = np.diff(np.asarray(row_ptr, dtype=np.int64))
    return np.argsort(-lengths, kind="stable").astype(np.int32)


def tile_aligned_keep(g: Geometry, kind: str, window: int, radius: int, order: str,
                      block_q: int, block_k: int, rows: np.ndarray) -> np.ndarray:
    """Mask snapped to the tiles of a head's layout (the final tile-aligned
    traversal of the tenesys page, "W skrócie" and item 4 of its list; oossa
    page, body paragraph 1).  The pages give no rule; the reading here: a tile
    of block_q x block_k layout positions that holds at least one kept pair is
    kept whole, any other tile is dropped, so no pair of the exact mask is lost.

    Returns keep[i, j] for frame-major query tokens ``rows`` and all frame-major
    key tokens.
    """
    toks = layout_tokens(g, order)
    pos = np.empty(g.n, dtype=np.int64)
    pos[toks] = np.arange(g.n)                       # layout position of each token
    rows = np.asarray(rows)
    q_tile = pos[rows] // block_q
    tiles = np.unique(q_tile)
    counts, _ = tile_counts(g, kind, window, radius, order, block_q, block_k, qtiles=tiles)
    nonempty = counts > 0                            # [len(tiles), n_kt]
    row_of = np.searchsorted(tiles, q_tile)
    k_tile = pos // block_k                          # k-tile of each key token
    return nonempty[row_of][:, k_tile]


# ---------------------------------------------------------------------------
# Attention (aihirek page, SVG section paragraph 1: softmax attention over the
# kept pairs).  O = softmax(S + M) V with S = Q K^T * scale, M = 0 or -inf.
# ---------------------------------------------------------------------------

def attend_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                keep: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 masked softmax attention for a block of query rows.

    q [r, d], k [n, d], v [n, d] float64; keep [r, n] bool.  Returns
    (O [r, d], lse [r]) with lse the natural-log sum of exp of kept scores.
    """
    s = (q @ k.T) * scale
    s = np.where(keep, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ v) / l
    return o, (m + np.log(l))[:, 0]


def attend_head(qb: np.ndarray, kb: np.ndarray, vb: np.ndarray, scale: float,
                g: Geometry, kind: str, window: int, radius: int,
                rows: Optional[np.ndarray] = None, block: int = 256,
                tile_aligned: Optional[Tuple[str, int, int]] = None):
    """Attention of one head in frame-major order.

    qb, kb, vb: bf16 bit patterns [N, d].  ``rows``: frame-major query tokens to
    compute (default all).  ``tile_aligned`` = (order, block_q, block_k) uses the
    tile-snapped mask of ``tile_aligned_keep`` instead of the exact one.
    Returns (O [len(rows), d] float64, lse float64).
    """
    k = bf16_to_f64(kb)
    v = bf16_to_f64(vb)
    rows = np.arange(g.n) if rows is None else np.asarray(rows)
    cols = np.arange(g.n)
    o = np.empty((len(rows), qb.shape[1]))
    lse = np.empty(len(rows))
    sc = float(np.float32(scale))
    for s in range(0, len(rows), block):
        rr = rows[s:s + block]
        if tile_aligned is None:
            keep = keep_matrix(g, kind, window, radius, rr, cols)
        else:
            keep = tile_aligned_keep(g, kind, window, radius, *tile_aligned, rr)
        o[s:s + block], lse[s:s + block] = attend_rows(bf16_to_f64(qb[rr]), k, v, sc, keep)
    return o, lse


def unpermute_rows(x_tm: np.ndarray, g: Geometry, order: str = "tm") -> np.ndarray:
    """Rows stored in a head's token order (default temporal-major) ->
    frame-major order."""
    perm = layout_tokens(g, order)
    out = np.empty_like(x_tm)
    out[perm] = x_tm
    return out


# ---------------------------------------------------------------------------
# Head routing (aihirek page, SVG section paragraph 3): for a few queries,
# the dense, spatial and temporal outputs; the sparse mask whose output
# deviates least from the dense one is chosen.
# ---------------------------------------------------------------------------

def route_head(qb: np.ndarray, kb: np.ndarray, vb: np.ndarray, scale: float, g: Geometry,
               window: int, radius: int, rows: np.ndarray) -> Tuple[float, float, str]:
    """Deviation of the spatial and temporal outputs from the dense output over
    frame-major query tokens ``rows``: the mean over rows and columns of the
    squared difference (the pages name no measure; this is the plain one).
    Returns (err_spatial, err_temporal, choice), a tie going to "spatial".
    """
    od, _ = attend_head(qb, kb, vb, scale, g, "dense", 0, 0, rows=rows)
    osp, _ = attend_head(qb, kb, vb, scale, g, "spatial", window, 0, rows=rows)
    ot, _ = attend_head(qb, kb, vb, scale, g, "temporal", 0, radius, rows=rows)
    es = float(np.mean((osp - od) ** 2))
    et = float(np.mean((ot - od) ** 2))
    return es, et, ("temporal" if et < es else "spatial")
