"""One attention layer of spatial and temporal heads on frame-major tensors.

Builds each distinct head mask's tile map once (maps depend only on the
geometry, the mask and the tile shape, so they are reused across denoising
steps), permutes the temporal-major heads' Q/K/V into scratch buffers, runs
one forward over all heads with per-head pointers (frame-major heads read and
write the caller's tensors in place) and unpermutes the temporal heads'
outputs back.  Every step is a libsvattn kernel; this class holds buffers
and launches.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import (FRAME_MAJOR, Geom, Mask, SvattnError, TileMap, build_tile_map, new_workspace, forward_fused,
               forward_ptrs, permute_tokens, unpermute)


def _runs(idx: List[int], key=lambda h: 0) -> List[Tuple[int, int]]:
    """Maximal runs [a, b) of consecutive integers of a sorted list that share key(h)."""
    out = []
    for h in idx:
        if out and out[-1][1] == h and key(h) == key(out[-1][0]):
            out[-1] = (out[-1][0], h + 1)
        else:
            out.append((h, h + 1))
    return out


class SparseVideoAttention:
    def __init__(self, geom: Geom, masks: Sequence[Mask], head_dim: int, block_q: int = 256,
                 block_k: int = 64, device="cuda", map_flags: int = 0, persistent: bool = True,
                 fused: bool = False):
        self.geom = geom
        self.masks = [Mask(m.kind, m.order, m.window, m.radius) for m in masks]
        self.head_dim = head_dim
        self.block_q, self.block_k = block_q, block_k
        self.device = device
        cache: Dict[tuple, TileMap] = {}
        self.maps: List[TileMap] = []
        for m in self.masks:
            key = (m.kind, m.order, m.window, m.radius)
            if key not in cache:
                cache[key] = build_tile_map(geom, m, block_q, block_k, device=device, flags=map_flags)
            self.maps.append(cache[key])
        # heads stored in a temporal-major order (raster, blocked or strip patches)
        self.tm_heads = [h for h, m in enumerate(self.masks) if m.order != FRAME_MAJOR]
        self.tm_runs = _runs(self.tm_heads, key=lambda h: self.masks[h].order)
        self._slot = {h: i for i, h in enumerate(self.tm_heads)}
        self._buf = None
        # work counter of the persistent schedule (None: static grid)
        self.workspace = new_workspace(device) if persistent else None
        # fused: temporal-major heads read and write the rows of their
        # positions in the frame-major tensors instead of permuted copies
        self.fused = fused

    def _buffers(self):
        if self._buf is None:
            shape = (len(self.tm_heads), self.geom.n, self.head_dim)
            self._buf = [torch.empty(shape, dtype=torch.bfloat16, device=self.device) for _ in range(4)]
        return self._buf

    def permute_inputs(self, q, k, v, stream=None):
        """Temporal-major copies of the temporal heads' Q, K, V (into scratch)."""
        if not self.tm_heads:
            return
        qt, kt, vt, _ = self._buffers()
        for a, b in self.tm_runs:
            s = self._slot[a]
            for src, dst in ((q, qt), (k, kt), (v, vt)):
                permute_tokens(self.geom, src[a:b], out=dst[s:s + (b - a)], stream=stream,
                               order=self.masks[a].order)

    def attend(self, q, k, v, out, scales, stream=None, lses=None):
        """Forward over all heads; temporal heads read/write the scratch buffers.
        ``lses``: optional per-head fp32 [N] tensors (or None entries) that get
        each head's lse in that head's token order (layout positions)."""
        if self.tm_heads:
            qt, kt, vt, ot = self._buffers()
        qs, ks, vs, os_ = [], [], [], []
        for h, m in enumerate(self.masks):
            if m.order != FRAME_MAJOR:
                s = self._slot[h]
                qs.append(qt[s]); ks.append(kt[s]); vs.append(vt[s]); os_.append(ot[s])
            else:
                qs.append(q[h]); ks.append(k[h]); vs.append(v[h]); os_.append(out[h])
        forward_ptrs(self.geom, qs, ks, vs, os_, self.masks, self.maps, scales, lses=lses,
                     workspace=self.workspace, stream=stream)

    def unpermute_output(self, out, stream=None):
        if not self.tm_heads:
            return
        ot = self._buffers()[3]
        for a, b in self.tm_runs:
            s = self._slot[a]
            unpermute(self.geom, ot[s:s + (b - a)], out=out[a:b], stream=stream, order=self.masks[a].order)

    def __call__(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scales: Sequence[float],
                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """q, k, v: frame-major bf16 [heads, N, head_dim]; returns frame-major O."""
        H = len(self.masks)
        if q.shape != (H, self.geom.n, self.head_dim) or k.shape != q.shape or v.shape != q.shape:
            raise SvattnError(f"expected q/k/v of shape {(H, self.geom.n, self.head_dim)}")
        out = torch.empty_like(q) if out is None else out
        if self.fused:
            forward_fused(self.geom, q, k, v, self.masks, self.maps, scales, out=out,
                          workspace=self.workspace, stream=stream)
            return out
        self.permute_inputs(q, k, v, stream)
        self.attend(q, k, v, out, scales, stream)
        self.unpermute_output(out, stream)
        return out
