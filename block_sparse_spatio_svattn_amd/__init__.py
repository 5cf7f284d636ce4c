"""Python binding of libsvattn.so: MI355X (gfx950) block-sparse spatio-temporal attention.

The library computes Sparse-VideoGen-style self-attention for video diffusion
("Accelerating Spatio-Temporal Attention for Video Diffusion on TPUs", Google
for Developers): spatial heads attend to keys in nearby frames, temporal heads
to keys at nearby patch positions in every frame, and every head keeps the
first frame as an anchor.  All compute runs in the HIP kernels of
libsvattn.so; this module only marshals arguments.  PyTorch supplies device
memory and the current stream, nothing else.  If the library is missing or a
tensor is not on the GPU, calls raise instead of falling back to anything.

Build the library with ``python -m block_sparse_spatio_svattn_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "SPATIAL", "TEMPORAL", "DENSE", "FRAME_MAJOR", "TEMPORAL_MAJOR", "TEMPORAL_MAJOR_BLOCKED", "PATCH_BLOCK",
    "TEMPORAL_MAJOR_STRIPS", "PATCH_STRIP",
    "TILE_EMPTY", "TILE_BOUNDARY", "TILE_FULL", "MAP_ALL_BOUNDARY", "MAP_TILE_ALIGNED", "FORWARD_WORKSPACE_BYTES",
    "new_workspace", "forward_fused", "route_heads", "route_scratch_bytes",
    "SvattnError", "Geom", "Mask", "TileMap", "lib", "version",
    "tile_map_dims", "build_tile_map", "permutation_index", "permute_tokens",
    "unpermute", "forward", "forward_ptrs", "forward_dense_mask",
]

SPATIAL, TEMPORAL, DENSE = 0, 1, 2
FRAME_MAJOR, TEMPORAL_MAJOR, TEMPORAL_MAJOR_BLOCKED, TEMPORAL_MAJOR_STRIPS = 0, 1, 2, 3
PATCH_BLOCK = 4  # SVATTN_PATCH_BLOCK: patches per block side in TEMPORAL_MAJOR_BLOCKED
PATCH_STRIP = 2  # SVATTN_PATCH_STRIP: patch columns per strip in TEMPORAL_MAJOR_STRIPS
TILE_EMPTY, TILE_BOUNDARY, TILE_FULL = 0, 1, 2
MAP_ALL_BOUNDARY = 1
MAP_TILE_ALIGNED = 2
FORWARD_WORKSPACE_BYTES = 256  # SVATTN_FORWARD_WORKSPACE_BYTES

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsvattn.so")

_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


class SvattnError(RuntimeError):
    """A libsvattn call returned a non-zero status."""


class Geom(ctypes.Structure):
    _fields_ = [("frames", _i32), ("height", _i32), ("width", _i32)]

    @property
    def n(self) -> int:
        return self.frames * self.height * self.width

    @property
    def patches(self) -> int:
        return self.height * self.width

    def __repr__(self):
        return f"Geom({self.frames}, {self.height}, {self.width})"


class Mask(ctypes.Structure):
    _fields_ = [("kind", _i32), ("order", _i32), ("window", _i32), ("radius", _i32)]

    def __repr__(self):
        return f"Mask(kind={self.kind}, order={self.order}, window={self.window}, radius={self.radius})"


class _TileMapC(ctypes.Structure):
    _fields_ = [("block_q", _i32), ("block_k", _i32), ("n_qt", _i32), ("n_kt", _i32),
                ("cls", _vp), ("row_ptr", _vp), ("col", _vp), ("col_cls", _vp), ("qt_order", _vp)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libsvattn.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise SvattnError(f"{LIB_PATH} is missing; build it with "
                          "`python -m block_sparse_spatio_svattn_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.svattn_version.restype = ctypes.c_int
    L.svattn_status_string.restype = ctypes.c_char_p
    L.svattn_status_string.argtypes = [ctypes.c_int]
    L.svattn_last_error.restype = ctypes.c_char_p
    L.svattn_tile_map_dims.argtypes = [P(Geom), _i32, _i32, P(_i32), P(_i32)]
    L.svattn_build_tile_map.argtypes = [P(Geom), P(Mask), P(_TileMapC), _vp]
    L.svattn_build_tile_map_ex.argtypes = [P(Geom), P(Mask), P(_TileMapC), ctypes.c_uint32, _vp]
    L.svattn_permutation_index.argtypes = [P(Geom), _vp, _vp, _vp]
    L.svattn_permute_tokens.argtypes = [P(Geom), _i32, _i32, _vp, _vp, _vp]
    L.svattn_unpermute.argtypes = [P(Geom), _i32, _i32, _vp, _vp, _vp]
    L.svattn_permutation_index_order.argtypes = [P(Geom), _i32, _vp, _vp, _vp]
    L.svattn_permute_tokens_order.argtypes = [P(Geom), _i32, _i32, _i32, _vp, _vp, _vp]
    L.svattn_unpermute_order.argtypes = [P(Geom), _i32, _i32, _i32, _vp, _vp, _vp]
    L.svattn_forward.argtypes = [P(Geom), _i32, _i32, P(Mask), P(P(_TileMapC)), P(ctypes.c_float),
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.svattn_forward_noalloc.argtypes = [P(Geom), _i32, _i32, P(Mask), P(P(_TileMapC)), P(ctypes.c_float),
                                         _vp, _vp, _vp, _vp, _vp, _vp]
    L.svattn_forward_ptrs.argtypes = [P(Geom), _i32, _i32, P(Mask), P(P(_TileMapC)), P(ctypes.c_float),
                                      P(_vp), P(_vp), P(_vp), P(_vp), P(_vp), _vp, _vp]
    L.svattn_forward_fused.argtypes = [P(Geom), _i32, _i32, P(Mask), P(P(_TileMapC)), P(ctypes.c_float),
                                       _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.svattn_route_scratch_bytes.argtypes = [_i32, _i32, _i32, _i32, P(ctypes.c_size_t)]
    L.svattn_route_heads.argtypes = [P(Geom), _i32, _i32, P(Mask), P(Mask), P(_TileMapC), P(_TileMapC),
                                     P(_TileMapC), P(ctypes.c_float), P(_i32), _i32, _vp, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp, _vp, _vp]
    L.svattn_forward_dense_mask.argtypes = [_i32, _i32, _i32, _vp, _i32, P(ctypes.c_float),
                                            _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp]
    for f in ("svattn_tile_map_dims", "svattn_build_tile_map", "svattn_build_tile_map_ex",
              "svattn_permutation_index", "svattn_permute_tokens", "svattn_unpermute",
              "svattn_permutation_index_order", "svattn_permute_tokens_order", "svattn_unpermute_order",
              "svattn_forward", "svattn_forward_ptrs", "svattn_forward_fused", "svattn_forward_dense_mask",
              "svattn_forward_noalloc",
              "svattn_route_scratch_bytes", "svattn_route_heads"):
        getattr(L, f).restype = ctypes.c_int
    _LIB = L
    return L


def version() -> int:
    return lib().svattn_version()


def _check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        raise SvattnError(f"{what}: {L.svattn_status_string(status).decode()}: "
                          f"{L.svattn_last_error().decode()}")


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> ctypes.c_void_p:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise SvattnError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise SvattnError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise SvattnError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def tile_map_dims(geom: Geom, block_q: int, block_k: int):
    a, b = _i32(), _i32()
    _check(lib().svattn_tile_map_dims(ctypes.byref(geom), block_q, block_k, ctypes.byref(a),
                                      ctypes.byref(b)), "svattn_tile_map_dims")
    return a.value, b.value


class TileMap:
    """Device buffers of one tile map (classes, CSR list of non-empty k-tiles and
    the longest-row-first q-tile order)."""

    def __init__(self, geom: Geom, block_q: int, block_k: int, device="cuda"):
        self.geom = geom
        self.block_q, self.block_k = block_q, block_k
        self.n_qt, self.n_kt = tile_map_dims(geom, block_q, block_k)
        cap = self.n_qt * self.n_kt
        self.cls = torch.empty(cap, dtype=torch.uint8, device=device)
        self.row_ptr = torch.empty(self.n_qt + 1, dtype=torch.int32, device=device)
        self.col = torch.empty(cap, dtype=torch.int32, device=device)
        self.col_cls = torch.empty(cap, dtype=torch.uint8, device=device)
        self.qt_order = torch.empty(self.n_qt, dtype=torch.int32, device=device)
        self.c = _TileMapC(block_q, block_k, self.n_qt, self.n_kt,
                           _dev(self.cls, "cls"), _dev(self.row_ptr, "row_ptr"),
                           _dev(self.col, "col"), _dev(self.col_cls, "col_cls"),
                           _dev(self.qt_order, "qt_order"))

    def rebuild(self, mask: Mask, flags: int = 0, stream=None) -> "TileMap":
        """Run the tile classifier into this map's buffers (no allocation)."""
        _check(lib().svattn_build_tile_map_ex(ctypes.byref(self.geom), ctypes.byref(mask), ctypes.byref(self.c),
                                              flags, _stream(stream)), "svattn_build_tile_map")
        return self

    def nnz(self) -> int:
        return int(self.row_ptr[-1].item())

    def csr(self):
        nnz = self.nnz()
        return self.row_ptr, self.col[:nnz], self.col_cls[:nnz]


def build_tile_map(geom: Geom, mask: Mask, block_q: int, block_k: int, device="cuda",
                   flags: int = 0, stream=None) -> TileMap:
    return TileMap(geom, block_q, block_k, device).rebuild(mask, flags, stream)


def permutation_index(geom: Geom, device="cuda", stream=None, order: int = TEMPORAL_MAJOR):
    """perm[t'] = frame-major token at position t' of `order`, and its inverse."""
    perm = torch.empty(geom.n, dtype=torch.int32, device=device)
    inv = torch.empty(geom.n, dtype=torch.int32, device=device)
    if order == TEMPORAL_MAJOR:
        st = lib().svattn_permutation_index(ctypes.byref(geom), _dev(perm, "perm"), _dev(inv, "inv"), _stream(stream))
    else:
        st = lib().svattn_permutation_index_order(ctypes.byref(geom), order, _dev(perm, "perm"), _dev(inv, "inv"),
                                                  _stream(stream))
    _check(st, "svattn_permutation_index")
    return perm, inv


def _permute(geom, x, out, stream, order, to_tm, what):
    if x.dim() != 3 or x.shape[1] != geom.n:
        raise SvattnError(f"{what}: expected [heads, {geom.n}, d], got {tuple(x.shape)}")
    out = torch.empty_like(x) if out is None else out
    if out.shape != x.shape:
        raise SvattnError(f"{what}: out shape {tuple(out.shape)} != {tuple(x.shape)}")
    args = (x.shape[0], x.shape[2], _dev(x, "src", torch.bfloat16), _dev(out, "dst", torch.bfloat16), _stream(stream))
    L = lib()
    if order == TEMPORAL_MAJOR:
        st = (L.svattn_permute_tokens if to_tm else L.svattn_unpermute)(ctypes.byref(geom), *args)
    else:
        st = (L.svattn_permute_tokens_order if to_tm else L.svattn_unpermute_order)(ctypes.byref(geom), order, *args)
    _check(st, what)
    return out


def permute_tokens(geom: Geom, x: torch.Tensor, out=None, stream=None, order: int = TEMPORAL_MAJOR) -> torch.Tensor:
    """Frame-major -> temporal-major rows (anchor-first; `order` TEMPORAL_MAJOR,
    TEMPORAL_MAJOR_BLOCKED or TEMPORAL_MAJOR_STRIPS) of a [heads, N, d] bf16 tensor."""
    return _permute(geom, x, out, stream, order, True, "svattn_permute_tokens")


def unpermute(geom: Geom, x: torch.Tensor, out=None, stream=None, order: int = TEMPORAL_MAJOR) -> torch.Tensor:
    """Temporal-major (`order`) -> frame-major rows of a [heads, N, d] bf16 tensor."""
    return _permute(geom, x, out, stream, order, False, "svattn_unpermute")


def _qkvo(q, k, v, out, n):
    if q.dim() != 3 or q.shape[1] != n or k.shape != q.shape or v.shape != q.shape:
        raise SvattnError(f"q/k/v must all be [heads, {n}, d]; got {tuple(q.shape)}, "
                          f"{tuple(k.shape)}, {tuple(v.shape)}")
    out = torch.empty_like(q) if out is None else out
    if out.shape != q.shape:
        raise SvattnError("out shape mismatch")
    return out


def _scales(scales, heads):
    s = [float(x) for x in scales]
    if len(s) != heads:
        raise SvattnError(f"{len(s)} scales for {heads} heads")
    return (ctypes.c_float * heads)(*s)


def new_workspace(device="cuda") -> torch.Tensor:
    """Device buffer for the persistent schedule of forward / forward_ptrs."""
    return torch.empty(FORWARD_WORKSPACE_BYTES, dtype=torch.uint8, device=device)


def _ws(workspace):
    if workspace is None:
        return None
    if workspace.numel() * workspace.element_size() < FORWARD_WORKSPACE_BYTES:
        raise SvattnError(f"workspace must hold at least {FORWARD_WORKSPACE_BYTES} bytes")
    return _dev(workspace, "workspace")


def forward(geom: Geom, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            masks: Sequence[Mask], maps: Sequence[TileMap], scales: Sequence[float],
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Block-sparse attention forward over [heads, N, d] bf16 tensors.

    Head h's tensors are in masks[h].order; maps[h] must be built for
    (geom, masks[h]).  ``lse`` (fp32 [heads, N]) is filled if given.  With a
    ``workspace`` (new_workspace()) the persistent schedule runs.
    """
    heads = q.shape[0]
    out = _qkvo(q, k, v, out, geom.n)
    if len(masks) != heads or len(maps) != heads:
        raise SvattnError("need one mask and one map per head")
    marr = (Mask * heads)(*[Mask(m.kind, m.order, m.window, m.radius) for m in masks])
    P = ctypes.POINTER(_TileMapC)
    parr = (P * heads)(*[ctypes.pointer(m.c) for m in maps])
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    _check(lib().svattn_forward(ctypes.byref(geom), heads, q.shape[2], marr, parr, _scales(scales, heads),
                                _dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16),
                                _dev(v, "v", torch.bfloat16), _dev(out, "o", torch.bfloat16),
                                lse_p, _ws(workspace), _stream(stream)), "svattn_forward")
    return out


def forward_fused(geom: Geom, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  masks: Sequence[Mask], maps: Sequence[TileMap], scales: Sequence[float],
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Forward over frame-major [heads, N, d] tensors with the temporal-major
    permutation fused in: a head whose mask order is temporal-major is
    computed in that order, the kernel reading and writing the rows of its
    positions in place (no permuted copies)."""
    heads = q.shape[0]
    out = _qkvo(q, k, v, out, geom.n)
    if len(masks) != heads or len(maps) != heads:
        raise SvattnError("need one mask and one map per head")
    marr = (Mask * heads)(*[Mask(m.kind, m.order, m.window, m.radius) for m in masks])
    P = ctypes.POINTER(_TileMapC)
    parr = (P * heads)(*[ctypes.pointer(m.c) for m in maps])
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    _check(lib().svattn_forward_fused(ctypes.byref(geom), heads, q.shape[2], marr, parr, _scales(scales, heads),
                                      _dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16),
                                      _dev(v, "v", torch.bfloat16), _dev(out, "o", torch.bfloat16),
                                      lse_p, _ws(workspace), _stream(stream)), "svattn_forward_fused")
    return out


def forward_noalloc(geom: Geom, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    masks: Sequence[Mask], maps: Sequence[TileMap], scales: Sequence[float],
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """svattn_forward_noalloc: the persistent forward with the library's own
    per-device work counter (no workspace).  Calls on one GPU must not overlap."""
    heads = q.shape[0]
    out = _qkvo(q, k, v, out, geom.n)
    if len(masks) != heads or len(maps) != heads:
        raise SvattnError("need one mask and one map per head")
    marr = (Mask * heads)(*[Mask(m.kind, m.order, m.window, m.radius) for m in masks])
    P = ctypes.POINTER(_TileMapC)
    parr = (P * heads)(*[ctypes.pointer(m.c) for m in maps])
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    _check(lib().svattn_forward_noalloc(ctypes.byref(geom), heads, q.shape[-1], marr, parr, _scales(scales, heads),
                                        _dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16),
                                        _dev(v, "v", torch.bfloat16), _dev(out, "o", torch.bfloat16),
                                        lse_p, _stream(stream)), "svattn_forward_noalloc")
    return out


def route_scratch_bytes(heads: int, head_dim: int, block_q: int, n_qtiles: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().svattn_route_scratch_bytes(heads, head_dim, block_q, n_qtiles, ctypes.byref(b)),
           "svattn_route_scratch_bytes")
    return b.value


def route_heads(geom: Geom, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, spatial: Mask, temporal: Mask,
                dense_map: TileMap, spatial_map: TileMap, temporal_map: TileMap, scales: Sequence[float],
                qtiles: Sequence[int], scratch: Optional[torch.Tensor] = None, stream=None):
    """SVG head routing over the selected frame-major q-tiles.  Returns
    (err fp32 [heads, 2] = deviation of the spatial / temporal output from the
    dense one, choice int32 [heads] = SPATIAL or TEMPORAL), on the device."""
    heads, d = q.shape[0], q.shape[2]
    _qkvo(q, k, v, None, geom.n)
    qt = [int(x) for x in qtiles]
    need = route_scratch_bytes(heads, d, dense_map.block_q, len(qt))
    if scratch is None:
        scratch = torch.empty(need, dtype=torch.uint8, device=q.device)
    err = torch.empty(heads, 2, dtype=torch.float32, device=q.device)
    choice = torch.empty(heads, dtype=torch.int32, device=q.device)
    _check(lib().svattn_route_heads(ctypes.byref(geom), heads, d, ctypes.byref(spatial), ctypes.byref(temporal),
                                    ctypes.byref(dense_map.c), ctypes.byref(spatial_map.c),
                                    ctypes.byref(temporal_map.c), _scales(scales, heads), (_i32 * len(qt))(*qt),
                                    len(qt), _dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16),
                                    _dev(v, "v", torch.bfloat16), _dev(scratch, "scratch"),
                                    scratch.numel() * scratch.element_size(), _dev(err, "err", torch.float32),
                                    _dev(choice, "choice", torch.int32), _stream(stream)), "svattn_route_heads")
    return err, choice


def forward_ptrs(geom: Geom, qs: Sequence[torch.Tensor], ks: Sequence[torch.Tensor],
                 vs: Sequence[torch.Tensor], os_: Sequence[torch.Tensor], masks: Sequence[Mask],
                 maps: Sequence[TileMap], scales: Sequence[float],
                 lses: Optional[Sequence[Optional[torch.Tensor]]] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Forward with one [N, d] bf16 tensor per head (outputs written into ``os_``)."""
    heads = len(qs)
    if not (len(ks) == len(vs) == len(os_) == len(masks) == len(maps) == heads):
        raise SvattnError("need one q/k/v/o/mask/map per head")
    n, d = geom.n, qs[0].shape[-1]
    for name, ts in (("q", qs), ("k", ks), ("v", vs), ("o", os_)):
        for t in ts:
            if tuple(t.shape) != (n, d):
                raise SvattnError(f"{name}: expected [{n}, {d}], got {tuple(t.shape)}")
    arr = lambda ts, nm, dt: (_vp * heads)(*[_dev(t, nm, dt).value for t in ts])
    marr = (Mask * heads)(*[Mask(m.kind, m.order, m.window, m.radius) for m in masks])
    P = ctypes.POINTER(_TileMapC)
    parr = (P * heads)(*[ctypes.pointer(m.c) for m in maps])
    lse_arr = None
    if lses is not None:
        lse_arr = (_vp * heads)(*[(_dev(t, "lse", torch.float32).value if t is not None else None)
                                   for t in lses])
    _check(lib().svattn_forward_ptrs(ctypes.byref(geom), heads, d, marr, parr, _scales(scales, heads),
                                     arr(qs, "q", torch.bfloat16), arr(ks, "k", torch.bfloat16),
                                     arr(vs, "v", torch.bfloat16), arr(os_, "o", torch.bfloat16),
                                     lse_arr, _ws(workspace), _stream(stream)), "svattn_forward_ptrs")


def forward_dense_mask(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask_bits: torch.Tensor,
                       scales: Sequence[float], per_head: bool = True, block_q: int = 128,
                       block_k: int = 64, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Reference forward for an arbitrary bit mask ([heads or 1, N, ceil(N/32)] int32/uint32 words)."""
    heads, n = q.shape[0], q.shape[1]
    out = _qkvo(q, k, v, out, n)
    words = (n + 31) // 32
    rows = heads if per_head else 1
    if tuple(mask_bits.shape) != (rows, n, words) or mask_bits.dtype not in (torch.int32, torch.uint32):
        raise SvattnError(f"mask_bits must be int32 [{rows}, {n}, {words}]")
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    _check(lib().svattn_forward_dense_mask(heads, n, q.shape[2], _dev(mask_bits, "mask_bits"), int(per_head),
                                           _scales(scales, heads), _dev(q, "q", torch.bfloat16),
                                           _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16),
                                           _dev(out, "o", torch.bfloat16), lse_p, block_q, block_k,
                                           _stream(stream)), "svattn_forward_dense_mask")
    return out
