"""Seeded synthetic inputs for spatio-temporal block-sparse attention.

This module is the only code shared by the CPU oracle and the HIP path's
harness (tests, bench, smoke).  It holds workload *definitions* (geometry,
head kinds, mask parameters, seeds) and the random draws, and none of the
attention method's arithmetic: no masks, no coordinates, no permutation, no
softmax.

Workloads follow the measurement setup of "Accelerating Spatio-Temporal
Attention for Video Diffusion on TPUs" (Google for Developers), as reported
by the aihirek.info page, section "A TPU-kernel kialakítása döntőnek
bizonyult" (75,600 tokens, 10 heads, head dim 128, synthetic bf16 inputs,
about 38.87% of query-key pairs kept), plus smaller and larger shapes of the
same family.  The pages give no mask parameters; the spatial window w and
temporal radius r below are chosen so the kept fraction matches the pages'
density (see the readings listed in the design notes).

Random recipe (fixed, so both sides see identical bytes):
  rng = numpy.random.Generator(PCG64(seed))
  if the workload has per-head random softmax-scale multipliers:
      s = rng.uniform(0.5, 2.0, heads)            (drawn first)
  Q[h] for h in 0..heads-1, then K[h] ..., then V[h] ...,
      each rng.standard_normal((N, d), dtype=float32)
  every fp32 draw is rounded to bf16 with round-to-nearest-even.
  scale[h] = float32(s[h] / sqrt(d))   (s[h] = 1 when not randomised)
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional, Tuple

import numpy as np

SPATIAL = "spatial"
TEMPORAL = "temporal"
DENSE = "dense"

FRAME_MAJOR = "fm"
TEMPORAL_MAJOR = "tm"
TEMPORAL_MAJOR_BLOCKED = "tmb"  # temporal-major over 4x4 patch blocks (a library layout)
TEMPORAL_MAJOR_STRIPS = "tms"   # temporal-major over snake strips two patches wide (a library layout)


@dataclasses.dataclass(frozen=True)
class Head:
    kind: str            # "spatial" | "temporal" | "dense"
    window: int = 0      # spatial: |f_q - f_k| <= window
    radius: int = 0      # temporal: Chebyshev patch distance <= radius
    order: str = FRAME_MAJOR  # token order the head is run in


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    frames: int
    height: int
    width: int
    head_dim: int
    heads: Tuple[Head, ...]
    tiles: Tuple[Tuple[int, int], ...]
    random_scale: bool = False
    sample_rows: Optional[int] = None   # rows per head checked against the oracle
    sample_seed: Optional[int] = None
    description: str = ""

    @property
    def n_tokens(self) -> int:
        return self.frames * self.height * self.width

    @property
    def n_heads(self) -> int:
        return len(self.heads)

    def with_heads(self, heads) -> "Workload":
        return dataclasses.replace(self, heads=tuple(heads))


def _mix(n_sp, w, n_tp, r, order=TEMPORAL_MAJOR):
    return tuple([Head(SPATIAL, window=w, order=FRAME_MAJOR)] * n_sp +
                 [Head(TEMPORAL, radius=r, order=order)] * n_tp)


WORKLOADS = {
    "tiny": Workload(
        name="tiny", seed=0, frames=4, height=8, width=8, head_dim=64,
        heads=(Head(SPATIAL, window=1), Head(TEMPORAL, radius=1, order=TEMPORAL_MAJOR)),
        tiles=((32, 32),),
        description="4 frames x 8x8 patches = 256 tokens, h0 spatial w=1, h1 temporal r=1, d=64"),
    "small": Workload(
        name="small", seed=1, frames=5, height=24, width=40, head_dim=128,
        heads=_mix(2, 1, 2, 2),
        tiles=((64, 64), (64, 128), (128, 64), (128, 128)),
        description="5 frames x 24x40 = 4,800 tokens, 2 spatial w=1 + 2 temporal r=2, d=128"),
    "headline": Workload(
        name="headline", seed=2, frames=21, height=45, width=80, head_dim=128,
        heads=_mix(5, 1, 5, 31),
        tiles=((256, 64),), random_scale=True, sample_rows=256, sample_seed=12,
        description="21 latent frames x 45x80 = 75,600 tokens, 5 spatial w=1 + 5 temporal r=31, "
                    "d=128, per-head softmax-scale multiplier in [0.5, 2]"),
    "perm_study": Workload(
        name="perm_study", seed=3, frames=21, height=45, width=80, head_dim=128,
        heads=tuple([Head(TEMPORAL, radius=22, order=TEMPORAL_MAJOR)] * 10),
        tiles=((256, 64),), sample_rows=128, sample_seed=13,
        description="75,600 tokens, 10 temporal heads r=22, frame-major vs temporal-major"),
    "headline_alt": Workload(
        name="headline_alt", seed=6, frames=21, height=45, width=80, head_dim=128,
        heads=_mix(5, 7, 5, 11),
        tiles=((256, 64),), random_scale=True, sample_rows=256, sample_seed=14,
        description="the headline's 75,600 tokens with the other mask fit of its density: 5 spatial w=7 + "
                    "5 temporal r=11 (38.887% kept), d=128, per-head softmax-scale multiplier in [0.5, 2]"),
    "headline_d64": Workload(
        name="headline_d64", seed=7, frames=21, height=45, width=80, head_dim=64,
        heads=_mix(2, 1, 2, 31),
        tiles=((256, 64),), random_scale=True, sample_rows=256, sample_seed=15,
        description="the headline's 75,600 tokens and masks at head_dim 64: 2 spatial w=1 + 2 temporal r=31 "
                    "(a parity workload for the d64 kernels at full size)"),
    "p1440": Workload(
        name="p1440", seed=4, frames=21, height=90, width=160, head_dim=128,
        heads=_mix(5, 1, 5, 62),
        tiles=((256, 64),), sample_rows=2048, sample_seed=5,
        description="21 frames x 90x160 = 302,400 tokens, 5 spatial w=1 + 5 temporal r=62, d=128"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 with round-to-nearest-even; returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Inputs:
    q: np.ndarray        # uint16 [heads, N, d] bf16 bit patterns
    k: np.ndarray
    v: np.ndarray
    scales: np.ndarray   # float32 [heads]: softmax scale passed to both sides
    multipliers: np.ndarray  # float64 [heads]: the drawn s_h (1.0 when fixed)

    def sha256(self) -> dict:
        return {n: hashlib.sha256(getattr(self, n).tobytes()).hexdigest()
                for n in ("q", "k", "v", "scales")}


def make_inputs(wl: Workload, heads: Optional[int] = None) -> Inputs:
    """Draw Q, K, V and per-head scales for a workload (recipe in the module docstring)."""
    H = wl.n_heads if heads is None else heads
    N, d = wl.n_tokens, wl.head_dim
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    if wl.random_scale:
        s = rng.uniform(0.5, 2.0, H)
    else:
        s = np.ones(H)
    out = []
    for _ in range(3):
        t = np.empty((H, N, d), dtype=np.uint16)
        for h in range(H):
            t[h] = f32_to_bf16_bits(rng.standard_normal((N, d), dtype=np.float32))
        out.append(t)
    scales = (s / np.sqrt(d)).astype(np.float32)
    return Inputs(q=out[0], k=out[1], v=out[2], scales=scales, multipliers=s)


def sample_rows(wl: Workload, n_rows: Optional[int] = None) -> np.ndarray:
    """Seeded sorted query rows (frame-major token ids) per head: int64 [heads, n_rows]."""
    n = wl.sample_rows if n_rows is None else n_rows
    rng = np.random.Generator(np.random.PCG64(wl.sample_seed if wl.sample_seed is not None else 99))
    return np.stack([np.sort(rng.choice(wl.n_tokens, size=n, replace=False))
                     for _ in range(wl.n_heads)])


def random_bits(shape, seed: int, density: float = 0.5) -> np.ndarray:
    """Seeded boolean array (for arbitrary-mask tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.random(shape) < density


def random_bf16(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """Seeded N(0, std^2) draws rounded to bf16 bit patterns."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))
