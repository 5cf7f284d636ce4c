"""svattn_forward_noalloc (the forward with the library's own per-device work
counter) against svattn_forward with a caller workspace, through the C ABI:
two calls in a row, the second on a smaller input, each bit-identical (O and
lse) to the workspace entry point on the same input, and within the parity
bar of the fp64 oracle on the small one."""
import numpy as np
import pytest
import torch

import oracle
import svattn_synth as synth
from _util import assert_close, f64_of, sv_mask, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import block_sparse_spatio_svattn_amd as m
    return m


def _case(sv, wl, orders):
    g = sv.Geom(wl.frames, wl.height, wl.width)
    masks = [sv_mask(h, o) for h, o in zip(wl.heads, orders)]
    maps = {}
    for m in masks:
        key = (m.kind, m.order, m.window, m.radius)
        if key not in maps:
            maps[key] = sv.build_tile_map(g, m, 256, 64)
    mp = [maps[(m.kind, m.order, m.window, m.radius)] for m in masks]
    inp = synth.make_inputs(wl)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    return g, masks, mp, inp, q, k, v, [float(s) for s in inp.scales]


def _both(sv, g, masks, mp, q, k, v, scales):
    H, N = q.shape[0], q.shape[1]
    o_na = torch.empty_like(q)
    l_na = torch.empty(H, N, dtype=torch.float32, device="cuda")
    sv.forward_noalloc(g, q, k, v, masks, mp, scales, out=o_na, lse=l_na)
    o_ws = torch.empty_like(q)
    l_ws = torch.empty(H, N, dtype=torch.float32, device="cuda")
    sv.forward(g, q, k, v, masks, mp, scales, out=o_ws, lse=l_ws, workspace=sv.new_workspace())
    torch.cuda.synchronize()
    assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16))
    assert torch.equal(l_na.view(torch.int32), l_ws.view(torch.int32))
    return o_na


def test_noalloc_matches_workspace_entry_two_calls(sv):
    big = synth.WORKLOADS["headline"]
    orders = ["tms" if h.kind == synth.TEMPORAL else "fm" for h in big.heads]
    print("call 1: 75,600 tokens x 10 heads", flush=True)
    g, masks, mp, _, q, k, v, scales = _case(sv, big, orders)
    _both(sv, g, masks, mp, q, k, v, scales)
    del q, k, v

    small = synth.WORKLOADS["small"]
    orders = ["fm"] * small.n_heads                      # layout = frame-major: comparable with the oracle
    print("call 2: 4,800 tokens x 4 heads", flush=True)
    g, masks, mp, inp, q, k, v, scales = _case(sv, small, orders)
    o = _both(sv, g, masks, mp, q, k, v, scales)
    og = oracle.Geometry(small.frames, small.height, small.width)
    for h, head in enumerate(small.heads):
        ref, _ = oracle.attend_head(inp.q[h], inp.k[h], inp.v[h], scales[h], og, head.kind, head.window,
                                    head.radius)
        assert_close(f64_of(o[h]), ref, f"noalloc small h{h}")
