"""Helpers shared by the GPU tests: moving bf16 bit patterns to and from the
device, masks for workload heads, and the error metrics of the parity bar."""
import numpy as np
import torch

import svattn_synth as synth

# Parity bar for bf16 outputs against the fp64 oracle.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def sv_mask(head: synth.Head, order=None):
    import block_sparse_spatio_svattn_amd as sv
    kind = {synth.SPATIAL: sv.SPATIAL, synth.TEMPORAL: sv.TEMPORAL, synth.DENSE: sv.DENSE}[head.kind]
    o = head.order if order is None else order
    orders = {synth.FRAME_MAJOR: sv.FRAME_MAJOR, synth.TEMPORAL_MAJOR: sv.TEMPORAL_MAJOR,
              synth.TEMPORAL_MAJOR_BLOCKED: sv.TEMPORAL_MAJOR_BLOCKED,
              synth.TEMPORAL_MAJOR_STRIPS: sv.TEMPORAL_MAJOR_STRIPS}
    return sv.Mask(kind, orders[o], head.window, head.radius)


def errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got.astype(np.float64) - ref)
    return float(d.max()), float(d.mean())


def assert_close(got, ref, what=""):
    mx, mean = errors(got, ref)
    print(f"{what}: max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert np.isfinite(got).all(), what
    assert mx <= MAX_ABS and mean <= MEAN_ABS, (what, mx, mean)
