"""Host-side work accounting for the benchmark: kept query-key pairs of a head
(closed form) and the effective FLOP count 4 * head_dim * kept pairs.

Kept pairs.  Spatial head, window w <= F-1: a query in frame f keeps the
frames of [max(0, f-w), min(F-1, f+w)] plus frame 0 when f-w > 0, so the
frame pairs number F(2w+1) - w(w+1) + max(0, F-1-w), each worth P*P token
pairs.  Temporal head, radius r: frame-0 keys count for everyone (F*P*P),
and keys in frames 1..F-1 at patch distance <= r contribute
F(F-1) * S_H(r) * S_W(r) with S_L(r) = L(2r+1) - r(r+1) for r <= L-1, else L^2.
"""
from __future__ import annotations

from . import DENSE, SPATIAL, Geom, Mask

# MI355X dense bf16 MFMA peak (vendor figure, TFLOP/s) and HBM3E bandwidth (GB/s).
BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0


def _window_sum(L: int, r: int) -> int:
    return L * L if r >= L - 1 else L * (2 * r + 1) - r * (r + 1)


def kept_pairs(g: Geom, m: Mask) -> int:
    F, P = g.frames, g.height * g.width
    N = F * P
    if m.kind == DENSE:
        return N * N
    if m.kind == SPATIAL:
        w = m.window
        if w >= F - 1:
            return N * N
        return P * P * (F * (2 * w + 1) - w * (w + 1) + max(0, F - 1 - w))
    return F * (F - 1) * _window_sum(g.height, m.radius) * _window_sum(g.width, m.radius) + F * P * P


def effective_flops(g: Geom, masks, head_dim: int) -> float:
    """4 * d FLOP per kept pair (2d for Q.K, 2d for P.V), summed over heads."""
    return float(sum(4 * head_dim * kept_pairs(g, m) for m in masks))
