"""The hot path under HIP graph capture.

Every launch of a step goes to the caller's stream and nothing allocates,
synchronises or memsets (the work counters are cleared by a kernel), so a
whole step can be captured once and replayed.  Each test captures a step,
replays the graph several times with eager work and synchronisations in
between, and requires every replay to give the eager result bit for bit.
"""
import numpy as np
import pytest
import torch

import svattn_synth as synth
from _util import bits_of, sv_mask, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import block_sparse_spatio_svattn_amd as m
    return m


def _capture(fn):
    """Warm up on a side stream (default priority), then capture fn() into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


@pytest.mark.parametrize("fused", [False, True])
def test_layer_step_replays_bit_identical(sv, fused):
    """permute -> persistent forward (work-counter clear kernel included) ->
    unpermute, or the fused forward, on the 4,800-token workload with the
    temporal heads in the strip temporal-major order."""
    from block_sparse_spatio_svattn_amd.layer import SparseVideoAttention
    wl = synth.WORKLOADS["small"]
    inp = synth.make_inputs(wl)
    g = sv.Geom(wl.frames, wl.height, wl.width)
    masks = [sv_mask(h, "tms" if h.kind == synth.TEMPORAL else "fm") for h in wl.heads]
    layer = SparseVideoAttention(g, masks, wl.head_dim, 256, 64, fused=fused)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    ref = layer(q, k, v, scales).clone()
    out = torch.empty_like(q)
    graph = _capture(lambda: layer(q, k, v, scales, out=out))
    # eager work on other data between replays, through the same layer buffers
    q2, k2, v2 = q.flip(1).contiguous(), k.flip(1).contiguous(), v.flip(1).contiguous()
    other_ref = layer(q2, k2, v2, scales).clone()
    for r in range(4):
        out.zero_()
        other = layer(q2, k2, v2, scales)
        torch.cuda.synchronize()
        assert (bits_of(other) == bits_of(other_ref)).all(), f"eager call after replay {r}"
        graph.replay()
        torch.cuda.synchronize()
        assert (bits_of(out) == bits_of(ref)).all(), f"replay {r}"


def test_noalloc_forward_replays_bit_identical(sv):
    """The allocation-free entry (its work counters in the library's own
    device array) captured and replayed, frame-major heads."""
    wl = synth.WORKLOADS["small"]
    inp = synth.make_inputs(wl)
    g = sv.Geom(wl.frames, wl.height, wl.width)
    masks = [sv_mask(h, "fm") for h in wl.heads]
    maps = [sv.build_tile_map(g, m, 128, 64) for m in masks]
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    ref = sv.forward(g, q, k, v, masks, maps, scales, workspace=sv.new_workspace()).clone()
    out = torch.empty_like(q)
    lse = torch.empty(wl.n_heads, wl.n_tokens, dtype=torch.float32, device="cuda")
    sv.forward_noalloc(g, q, k, v, masks, maps, scales, out=out, lse=lse)  # first call looks up the array
    torch.cuda.synchronize()
    lse_ref = lse.clone()
    graph = _capture(lambda: sv.forward_noalloc(g, q, k, v, masks, maps, scales, out=out, lse=lse))
    for r in range(4):
        out.zero_()
        lse.zero_()
        eager = sv.forward_noalloc(g, q, k, v, masks, maps, scales)  # eager use of the same counters
        torch.cuda.synchronize()
        assert (bits_of(eager) == bits_of(ref)).all(), f"eager call after replay {r}"
        graph.replay()
        torch.cuda.synchronize()
        assert (bits_of(out) == bits_of(ref)).all(), f"replay {r}"
        assert torch.equal(lse, lse_ref), f"replay {r} lse"
    assert np.isfinite(lse.cpu().numpy()).all()
