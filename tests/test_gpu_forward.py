"""GPU parity of the attention forward against the fp64 oracle.

Bar (bf16 output vs fp64 oracle): max-abs <= 2e-2 and mean-abs <= 2e-3 over
the compared outputs.  Small shapes compare every output; the full-size
workloads compare seeded sampled query rows, in the launch configuration the
benchmark times (block 256 x 64, temporal heads temporal-major through the
permute -> forward -> unpermute path).
"""
import numpy as np
import pytest
import torch

import oracle
import svattn_synth as synth
from _util import assert_close, bits_of, f64_of, sv_mask, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import block_sparse_spatio_svattn_amd as m
    return m


def _oracle_rows(wl, inp, rows_per_head):
    g = oracle.Geometry(wl.frames, wl.height, wl.width)
    out = []
    for h, head in enumerate(wl.heads):
        o, lse = oracle.attend_head(inp.q[h], inp.k[h], inp.v[h], float(inp.scales[h]), g, head.kind,
                                    head.window, head.radius, rows=rows_per_head[h])
        out.append((o, lse))
    return out


def _run_layer(sv, wl, inp, bq, bk, orders=None, flags=0):
    from block_sparse_spatio_svattn_amd.layer import SparseVideoAttention
    g = sv.Geom(wl.frames, wl.height, wl.width)
    masks = [sv_mask(h, None if orders is None else orders[i]) for i, h in enumerate(wl.heads)]
    layer = SparseVideoAttention(g, masks, wl.head_dim, bq, bk, map_flags=flags)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    o = layer(q, k, v, [float(s) for s in inp.scales])
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("bq,bk", [(32, 32), (64, 32), (32, 64), (256, 64), (128, 64)])
@pytest.mark.parametrize("order", ["fm", "tm", "tmb", "tms"])
def test_tiny_all_rows(sv, bq, bk, order):
    wl = synth.WORKLOADS["tiny"]
    inp = synth.make_inputs(wl)
    o = _run_layer(sv, wl, inp, bq, bk, orders=["fm", order])
    ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * wl.n_heads)
    for h in range(wl.n_heads):
        assert_close(f64_of(o[h]), ref[h][0], f"tiny h{h} {order} {bq}x{bk}")


@pytest.mark.parametrize("bq,bk", [(64, 64), (128, 64), (256, 64), (256, 32), (128, 32)])
def test_small_all_rows(sv, bq, bk):
    wl = synth.WORKLOADS["small"]
    inp = synth.make_inputs(wl)
    o = _run_layer(sv, wl, inp, bq, bk)
    ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * wl.n_heads)
    for h in range(wl.n_heads):
        assert_close(f64_of(o[h]), ref[h][0], f"small h{h} {bq}x{bk}")


@pytest.mark.parametrize("bq,bk", [(64, 64), (256, 64), (128, 32)])
@pytest.mark.parametrize("order", ["tmb", "tms"])
def test_small_blocked_order_all_rows(sv, bq, bk, order):
    """Temporal heads in the temporal-major order over 4x4 patch blocks or
    snake strips (24 x 40 patches: whole blocks and strips), every output row."""
    wl = synth.WORKLOADS["small"]
    inp = synth.make_inputs(wl)
    orders = [order if h.kind == synth.TEMPORAL else h.order for h in wl.heads]
    o = _run_layer(sv, wl, inp, bq, bk, orders=orders)
    ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * wl.n_heads)
    for h in range(wl.n_heads):
        assert_close(f64_of(o[h]), ref[h][0], f"small {order} h{h} {bq}x{bk}")


def test_small_lse_and_direct_entry(sv):
    """svattn_forward on layout tensors (frame-major heads only) incl. lse."""
    wl = synth.WORKLOADS["small"]
    inp = synth.make_inputs(wl)
    g = sv.Geom(wl.frames, wl.height, wl.width)
    masks = [sv_mask(h, "fm") for h in wl.heads]
    maps = [sv.build_tile_map(g, m, 256, 64) for m in masks]
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    lse = torch.empty(wl.n_heads, wl.n_tokens, dtype=torch.float32, device="cuda")
    o = sv.forward(g, q, k, v, masks, maps, [float(s) for s in inp.scales], lse=lse)
    torch.cuda.synchronize()
    ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * wl.n_heads)
    for h in range(wl.n_heads):
        assert_close(f64_of(o[h]), ref[h][0], f"small direct h{h}")
        dl = np.abs(lse[h].cpu().numpy().astype(np.float64) - ref[h][1]).max()
        assert dl < 1e-3, dl


@pytest.mark.parametrize("wl_name", ["headline", "perm_study", "p1440"])
def test_full_size_sampled_rows(sv, wl_name):
    wl = synth.WORKLOADS[wl_name]
    inp = synth.make_inputs(wl)
    rows = synth.sample_rows(wl, min(wl.sample_rows, 256))
    print(f"{wl_name}: N={wl.n_tokens} heads={wl.n_heads} rows/head={rows.shape[1]}", flush=True)
    o = _run_layer(sv, wl, inp, 256, 64)
    ref = _oracle_rows(wl, inp, rows)
    got = np.stack([f64_of(o[h][torch.from_numpy(rows[h]).cuda()]) for h in range(wl.n_heads)])
    assert_close(got, np.stack([r[0] for r in ref]), f"{wl_name} sampled rows")


@pytest.mark.parametrize("wl_name", ["headline", "p1440"])
@pytest.mark.parametrize("order", ["tmb", "tms"])
def test_full_size_sampled_rows_blocked_order(sv, wl_name, order):
    """The full-size workloads with their temporal heads in the blocked or
    strip temporal-major order, in the benchmark's launch configuration."""
    wl = synth.WORKLOADS[wl_name]
    inp = synth.make_inputs(wl)
    rows = synth.sample_rows(wl, min(wl.sample_rows, 256))
    orders = [order if h.kind == synth.TEMPORAL else h.order for h in wl.heads]
    o = _run_layer(sv, wl, inp, 256, 64, orders=orders)
    ref = _oracle_rows(wl, inp, rows)
    got = np.stack([f64_of(o[h][torch.from_numpy(rows[h]).cuda()]) for h in range(wl.n_heads)])
    assert_close(got, np.stack([r[0] for r in ref]), f"{wl_name} {order} order sampled rows")


def test_perm_study_frame_major_order(sv):
    wl = synth.WORKLOADS["perm_study"]
    inp = synth.make_inputs(wl)
    rows = synth.sample_rows(wl, 64)
    o = _run_layer(sv, wl, inp, 256, 64, orders=["fm"] * wl.n_heads)
    ref = _oracle_rows(wl, inp, rows)
    got = np.stack([f64_of(o[h][torch.from_numpy(rows[h]).cuda()]) for h in range(wl.n_heads)])
    assert_close(got, np.stack([r[0] for r in ref]), "perm_study frame-major")


@pytest.mark.slow
def test_p1440_2048_rows(sv):
    wl = synth.WORKLOADS["p1440"]
    inp = synth.make_inputs(wl)
    rows = synth.sample_rows(wl)
    o = _run_layer(sv, wl, inp, 256, 64)
    ref = _oracle_rows(wl, inp, rows)
    got = np.stack([f64_of(o[h][torch.from_numpy(rows[h]).cuda()]) for h in range(wl.n_heads)])
    assert_close(got, np.stack([r[0] for r in ref]), "p1440 2048 rows/head")


def test_dense_kind_and_all_boundary_bit_identical(sv):
    """DENSE heads equal the oracle's dense attention; a map with every tile
    marked BOUNDARY gives bit-identical outputs to the normal map."""
    wl = synth.WORKLOADS["small"]
    inp = synth.make_inputs(wl)
    o1 = _run_layer(sv, wl, inp, 256, 64)
    o2 = _run_layer(sv, wl, inp, 256, 64, flags=sv.MAP_ALL_BOUNDARY)
    assert (bits_of(o1) == bits_of(o2)).all()
    dwl = wl.with_heads([synth.Head("dense")] * 2)
    dinp = synth.make_inputs(dwl)
    od = _run_layer(sv, dwl, dinp, 256, 64)
    ref = _oracle_rows(dwl, dinp, [np.arange(dwl.n_tokens)] * 2)
    for h in range(2):
        assert_close(f64_of(od[h]), ref[h][0], f"dense h{h}")


def test_deterministic_and_head_order_invariant(sv):
    wl = synth.WORKLOADS["small"]
    inp = synth.make_inputs(wl)
    o1 = bits_of(_run_layer(sv, wl, inp, 256, 64))
    o2 = bits_of(_run_layer(sv, wl, inp, 256, 64))
    assert (o1 == o2).all()
    rev = wl.with_heads(list(reversed(wl.heads)))
    rinp = synth.Inputs(q=inp.q[::-1].copy(), k=inp.k[::-1].copy(), v=inp.v[::-1].copy(),
                        scales=inp.scales[::-1].copy(), multipliers=inp.multipliers[::-1].copy())
    o3 = bits_of(_run_layer(sv, rev, rinp, 256, 64))
    assert (o3[::-1] == o1).all()


@pytest.mark.parametrize("geom,heads,bq,bk", [
    ((3, 5, 7), [synth.Head("temporal", radius=1, order="tm"), synth.Head("spatial", window=0)], 64, 32),
    ((3, 5, 7), [synth.Head("temporal", radius=0, order="fm"), synth.Head("spatial", window=1)], 32, 64),
    ((1, 8, 8), [synth.Head("temporal", radius=1, order="tm"), synth.Head("spatial", window=0)], 32, 32),
    ((2, 3, 5), [synth.Head("temporal", radius=3, order="tm"), synth.Head("dense")], 256, 64),
    ((9, 1, 3), [synth.Head("temporal", radius=0, order="tm"), synth.Head("spatial", window=2)], 64, 64),
])
def test_edge_geometries(sv, geom, heads, bq, bk):
    """Ragged tails (N not a multiple of either tile), a single frame (every key is
    an anchor), N smaller than one tile, zero windows, and dense heads."""
    F, H, W = geom
    wl = synth.Workload(name="edge", seed=77, frames=F, height=H, width=W, head_dim=64,
                        heads=tuple(heads), tiles=((bq, bk),))
    inp = synth.make_inputs(wl)
    o = _run_layer(sv, wl, inp, bq, bk)
    ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * wl.n_heads)
    for h in range(wl.n_heads):
        assert_close(f64_of(o[h]), ref[h][0], f"edge {geom} h{h}")


@pytest.mark.parametrize("geom,heads", [
    ((2, 3, 5), [synth.Head("dense"), synth.Head("temporal", radius=3, order="tm")]),
    ((5, 9, 11), [synth.Head("spatial", window=0), synth.Head("temporal", radius=1, order="tm")]),
    ((17, 6, 8), [synth.Head("temporal", radius=2, order="tmb"), synth.Head("spatial", window=1)]),
    ((17, 6, 9), [synth.Head("temporal", radius=2, order="tms"), synth.Head("spatial", window=1)]),
])
def test_d128_two_tiles_per_barrier(sv, geom, heads):
    """The head_dim 128, 256 x 64 launch runs two list entries between barriers.
    These geometries give lists of 1, 3, 5, 7, 8, 12 and 13 entries (so groups
    whose second entry is missing), ragged k- and q-tiles, patch runs shorter
    than 16 keys (per-score test) and runs of exactly 16 in the blocked and
    strip orders (with an odd grid width: a last strip one patch wide); every
    output row is checked against the oracle."""
    F, H, W = geom
    wl = synth.Workload(name="tpb", seed=79, frames=F, height=H, width=W, head_dim=128,
                        heads=tuple(heads), tiles=((256, 64),))
    inp = synth.make_inputs(wl)
    o = _run_layer(sv, wl, inp, 256, 64)
    ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * wl.n_heads)
    for h in range(wl.n_heads):
        assert_close(f64_of(o[h]), ref[h][0], f"two tiles per barrier {geom} h{h}")


@pytest.mark.parametrize("bq", [256, 128, 64])
def test_small_128_key_tiles(sv, bq):
    """Tile maps of 128-key tiles run as two 64-key halves per map entry.  At
    4,800 tokens the last 128-key tile's second half lies wholly past the last
    token and is dropped.  Every output row matches the oracle, and the output
    is bit-identical to the one from the 64-key map (the same tiles, halves
    without kept pairs skipped, in the same order)."""
    wl = synth.WORKLOADS["small"]
    assert wl.n_tokens % 128 == 64
    inp = synth.make_inputs(wl)
    o128 = _run_layer(sv, wl, inp, bq, 128)
    o64 = _run_layer(sv, wl, inp, bq, 64)
    assert (bits_of(o128) == bits_of(o64)).all()
    ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * wl.n_heads)
    for h in range(wl.n_heads):
        assert_close(f64_of(o128[h]), ref[h][0], f"small {bq}x128 h{h}")


def test_tiny_128_key_tiles_all_orders(sv):
    """128-key tiles on the 256-token workload in every temporal order, against
    the oracle."""
    wl = synth.WORKLOADS["tiny"]
    inp = synth.make_inputs(wl)
    for order in ("fm", "tm", "tmb", "tms"):
        o = _run_layer(sv, wl, inp, 256, 128, orders=["fm", order])
        ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * wl.n_heads)
        for h in range(wl.n_heads):
            assert_close(f64_of(o[h]), ref[h][0], f"tiny {order} 256x128 h{h}")


def _bits_from_keep(keep):
    n = keep.shape[-1]
    words = (n + 31) // 32
    pad = np.zeros(keep.shape[:-1] + (words * 32,), dtype=bool)
    pad[..., :n] = keep
    b = pad.reshape(keep.shape[:-1] + (words, 32)).astype(np.uint64)
    w = (b << np.arange(32, dtype=np.uint64)).sum(-1).astype(np.uint32)
    return torch.from_numpy(w.view(np.int32)).cuda()


@pytest.mark.parametrize("n,d,bq,bk", [(200, 64, 64, 32), (333, 128, 128, 64), (96, 128, 32, 64)])
def test_dense_mask_entry_random_bits(sv, n, d, bq, bk):
    heads = 2
    q = synth.random_bf16((heads, n, d), 5)
    k = synth.random_bf16((heads, n, d), 6)
    v = synth.random_bf16((heads, n, d), 7)
    keep = synth.random_bits((heads, n, n), 8, density=0.3)
    keep[0, 3, :] = False          # a row with no kept key: O = 0, lse = -inf
    keep[1, :, 0] = True
    scales = [0.1, 0.2]
    lse = torch.empty(heads, n, dtype=torch.float32, device="cuda")
    o = sv.forward_dense_mask(to_dev(q), to_dev(k), to_dev(v), _bits_from_keep(keep), scales,
                              per_head=True, block_q=bq, block_k=bk, lse=lse)
    torch.cuda.synchronize()
    for h in range(heads):
        live = keep[h].any(1)
        ref, rl = oracle.attend_rows(oracle.bf16_to_f64(q[h][live]), oracle.bf16_to_f64(k[h]),
                                     oracle.bf16_to_f64(v[h]), float(np.float32(scales[h])), keep[h][live])
        got = f64_of(o[h])
        assert_close(got[live], ref, f"dense-mask h{h}")
        assert (got[~live] == 0).all()
        lh = lse[h].cpu().numpy()
        assert np.isneginf(lh[~live]).all()
        assert np.abs(lh[live] - rl).max() < 1e-3


def test_dense_mask_entry_matches_coordinate_masks(sv):
    """The bit-mask reference path with the oracle's spatial/temporal masks agrees
    with the coordinate-mask path (both within the parity bar of the oracle)."""
    wl = synth.WORKLOADS["tiny"]
    inp = synth.make_inputs(wl)
    g = oracle.Geometry(wl.frames, wl.height, wl.width)
    keep = np.stack([oracle.keep_matrix(g, h.kind, h.window, h.radius, np.arange(g.n), np.arange(g.n))
                     for h in wl.heads])
    o = sv.forward_dense_mask(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), _bits_from_keep(keep),
                              [float(s) for s in inp.scales], per_head=True, block_q=64, block_k=32)
    o2 = _run_layer(sv, wl, inp, 64, 32, orders=["fm", "fm"])
    torch.cuda.synchronize()
    ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * 2)
    for h in range(2):
        assert_close(f64_of(o[h]), ref[h][0], f"bits h{h}")
        assert (bits_of(o[h]) == bits_of(o2[h])).all()


@pytest.mark.parametrize("geom,d,bk", [((5, 24, 40), 128, 64), ((5, 24, 40), 128, 32), ((3, 5, 7), 64, 64),
                                       ((2, 9, 11), 64, 32), ((4, 8, 8), 128, 32)])
def test_two_group_schedule_matches_plain_schedule(sv, geom, d, bk):
    """A launch whose heads are all dense runs the two-group schedule (block_q
    256; d128 256 x 64 launches take the plain schedule, two tiles per
    barrier); the same dense head next to a spatial head runs the plain
    schedule.  Both do the same arithmetic in the same order, so the dense
    head's output is bit-identical, and it matches the oracle.  Covers ragged
    q- and k-tiles."""
    F, H, W = geom
    heads_pp = [synth.Head("dense"), synth.Head("dense")]
    heads_plain = [synth.Head("dense"), synth.Head("spatial", window=0)]
    wl = synth.Workload(name="sched", seed=91, frames=F, height=H, width=W, head_dim=d,
                        heads=tuple(heads_pp), tiles=((256, bk),))
    inp = synth.make_inputs(wl)
    o_pp = _run_layer(sv, wl, inp, 256, bk)
    o_plain = _run_layer(sv, wl.with_heads(heads_plain), inp, 256, bk)
    assert (bits_of(o_pp[0]) == bits_of(o_plain[0])).all()
    ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * 2)
    for h in range(2):
        assert_close(f64_of(o_pp[h]), ref[h][0], f"two-group dense h{h} {geom}")


@pytest.mark.parametrize("bq,bk", [(256, 64), (64, 32), (128, 64)])
def test_schedules_give_identical_results(sv, bq, bk):
    """The persistent schedule (workspace given) and the static grid, with and
    without the longest-row-first q-tile order, only change which workgroup
    runs a q-tile: every output bit is the same in all four runs."""
    from block_sparse_spatio_svattn_amd.layer import SparseVideoAttention
    wl = synth.WORKLOADS["small"]
    inp = synth.make_inputs(wl)
    g = sv.Geom(wl.frames, wl.height, wl.width)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    outs = []
    for persistent in (True, False):
        layer = SparseVideoAttention(g, [sv_mask(h) for h in wl.heads], wl.head_dim, bq, bk,
                                     persistent=persistent)
        outs.append(layer(q, k, v, scales))
        for m in layer.maps:
            m.c.qt_order = None
        outs.append(layer(q, k, v, scales))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert (bits_of(o) == bits_of(outs[0])).all()
    ref = _oracle_rows(wl, inp, [np.arange(0, wl.n_tokens, 7)] * wl.n_heads)
    for h in range(wl.n_heads):
        assert_close(f64_of(outs[0][h][::7]), ref[h][0], f"persistent h{h} {bq}x{bk}")


def test_persistent_schedule_over_several_launches(sv):
    """20 heads take two launches (16 heads each at most) that share one work
    counter, cleared before each launch; both launches match the static grid
    bit for bit and the oracle on every row.  Ragged q- and k-tiles."""
    from block_sparse_spatio_svattn_amd.layer import SparseVideoAttention
    kinds = [synth.Head("temporal", radius=1, order="tm"), synth.Head("spatial", window=1),
             synth.Head("dense"), synth.Head("temporal", radius=2, order="fm")]
    heads = tuple(kinds[i % 4] for i in range(20))
    wl = synth.Workload(name="many", seed=17, frames=3, height=5, width=7, head_dim=64,
                        heads=heads, tiles=((64, 32),))
    inp = synth.make_inputs(wl)
    g = sv.Geom(wl.frames, wl.height, wl.width)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    masks = [sv_mask(h) for h in heads]
    o_p = SparseVideoAttention(g, masks, 64, 64, 32, persistent=True)(q, k, v, scales)
    o_s = SparseVideoAttention(g, masks, 64, 64, 32, persistent=False)(q, k, v, scales)
    torch.cuda.synchronize()
    assert (bits_of(o_p) == bits_of(o_s)).all()
    ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * wl.n_heads)
    for h in range(wl.n_heads):
        assert_close(f64_of(o_p[h]), ref[h][0], f"many h{h}")


@pytest.mark.parametrize("n_heads,d,bq,bk", [(2, 128, 256, 64), (5, 128, 256, 64), (20, 64, 64, 32), (3, 128, 128, 64)])
def test_one_map_launch_rank_by_rank_tail(sv, n_heads, d, bq, bk):
    """Heads that all share one tile map: the persistent schedule deals the
    last (up to three) heads of each launch rank by rank.  Only which
    workgroup runs an item changes, so the output equals the static grid's bit
    for bit (2, 3 and 5 heads; 20 heads in two launches of 16 and 4) and the
    oracle on every row."""
    from block_sparse_spatio_svattn_amd.layer import SparseVideoAttention
    heads = tuple([synth.Head("temporal", radius=2, order="tms")] * n_heads)
    wl = synth.Workload(name="onemap", seed=41, frames=5, height=6, width=9, head_dim=d, heads=heads,
                        tiles=((bq, bk),))
    inp = synth.make_inputs(wl)
    g = sv.Geom(wl.frames, wl.height, wl.width)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    masks = [sv_mask(h) for h in heads]
    o_p = SparseVideoAttention(g, masks, d, bq, bk, persistent=True)(q, k, v, scales)
    o_s = SparseVideoAttention(g, masks, d, bq, bk, persistent=False)(q, k, v, scales)
    torch.cuda.synchronize()
    assert (bits_of(o_p) == bits_of(o_s)).all()
    ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * wl.n_heads)
    for h in range(wl.n_heads):
        assert_close(f64_of(o_p[h]), ref[h][0], f"one map h{h} of {n_heads}")


@pytest.mark.parametrize("geom,r,order,bq,bk", [
    ((17, 3, 5), 1, "tm", 64, 64),    # F-1 = 16: patch runs of 16 keys, ragged tail (N = 255)
    ((21, 4, 6), 1, "tm", 256, 64),   # F-1 = 20, as the headline; N = 504
    ((21, 4, 6), 2, "tm", 64, 32),
    ((17, 3, 16), 1, "fm", 128, 64),  # W = 16: patch-row runs, frame-major
    ((5, 6, 40), 3, "fm", 64, 32),
    ((3, 2, 70), 9, "fm", 256, 64),   # rows longer than a tile
    ((21, 4, 6), 1, "tmb", 256, 64),  # blocked patch order: 4x4 and 4x2 blocks
    ((17, 9, 13), 2, "tmb", 128, 64), # ragged blocks in both directions, F-1 = 16
    ((21, 5, 7), 1, "tmb", 64, 32),
    ((21, 4, 6), 1, "tms", 256, 64),  # snake strips: three strips of 2 columns
    ((17, 9, 13), 2, "tms", 128, 64), # odd width: a last strip one patch wide, F-1 = 16
    ((21, 5, 7), 1, "tms", 64, 32),
])
def test_long_run_masks_all_rows(sv, geom, r, order, bq, bk):
    """Geometries whose key runs (F-1 frames of a patch in temporal-major order,
    W patches of a row in frame-major order) are at least 16 keys long, so
    boundary tiles take the run-mask path; every output row against the
    oracle, with spatial and dense heads beside them."""
    F, H, W = geom
    heads = (synth.Head("temporal", radius=r, order=order), synth.Head("spatial", window=1),
             synth.Head("temporal", radius=0, order=order), synth.Head("dense"))
    wl = synth.Workload(name="runs", seed=23, frames=F, height=H, width=W, head_dim=128,
                        heads=heads, tiles=((bq, bk),))
    inp = synth.make_inputs(wl)
    o = _run_layer(sv, wl, inp, bq, bk)
    ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * wl.n_heads)
    for h in range(wl.n_heads):
        assert_close(f64_of(o[h]), ref[h][0], f"runs {geom} r{r} {order} h{h} {bq}x{bk}")


@pytest.mark.parametrize("wl_name,bq,bk", [("tiny", 32, 32), ("tiny", 256, 64), ("small", 128, 64), ("small", 64, 32)])
def test_tile_aligned_traversal_all_rows(sv, wl_name, bq, bk):
    """Maps built with MAP_TILE_ALIGNED mark every non-empty tile full, so the
    forward attends to every pair of those tiles; every output row against the
    oracle's tile-snapped mask in each head's own token order."""
    wl = synth.WORKLOADS[wl_name]
    inp = synth.make_inputs(wl)
    o = _run_layer(sv, wl, inp, bq, bk, flags=sv.MAP_TILE_ALIGNED)
    g = oracle.Geometry(wl.frames, wl.height, wl.width)
    for h, head in enumerate(wl.heads):
        ref, _ = oracle.attend_head(inp.q[h], inp.k[h], inp.v[h], float(inp.scales[h]), g, head.kind, head.window,
                                    head.radius, tile_aligned=(head.order, bq, bk))
        assert_close(f64_of(o[h]), ref, f"tile-aligned {wl_name} h{h} {bq}x{bk}")


def test_tile_aligned_long_runs(sv):
    """Tile snapping with key runs of 20 frames (the headline's F - 1) and a
    ragged tail, temporal-major and frame-major temporal heads."""
    heads = (synth.Head("temporal", radius=1, order="tm"), synth.Head("temporal", radius=2, order="fm"),
             synth.Head("spatial", window=1), synth.Head("temporal", radius=1, order="tmb"),
             synth.Head("temporal", radius=1, order="tms"))
    wl = synth.Workload(name="ta", seed=29, frames=21, height=4, width=6, head_dim=128, heads=heads,
                        tiles=((128, 64),))
    inp = synth.make_inputs(wl)
    o = _run_layer(sv, wl, inp, 128, 64, flags=sv.MAP_TILE_ALIGNED)
    g = oracle.Geometry(wl.frames, wl.height, wl.width)
    for h, head in enumerate(heads):
        ref, _ = oracle.attend_head(inp.q[h], inp.k[h], inp.v[h], float(inp.scales[h]), g, head.kind, head.window,
                                    head.radius, tile_aligned=(head.order, 128, 64))
        assert_close(f64_of(o[h]), ref, f"tile-aligned long runs h{h}")


@pytest.mark.parametrize("wl_name,bq,bk,persistent", [("tiny", 256, 64, True), ("tiny", 32, 32, False),
                                                      ("small", 256, 64, True), ("small", 128, 32, False)])
def test_fused_permutation_bit_identical(sv, wl_name, bq, bk, persistent):
    """Temporal-major heads computed straight from the frame-major tensors
    (the row of each position worked out in the kernel, O scattered back)
    give the same bits as permute -> forward -> unpermute."""
    from block_sparse_spatio_svattn_amd.layer import SparseVideoAttention
    wl = synth.WORKLOADS[wl_name]
    inp = synth.make_inputs(wl)
    g = sv.Geom(wl.frames, wl.height, wl.width)
    masks = [sv_mask(h) for h in wl.heads]
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    o_sep = SparseVideoAttention(g, masks, wl.head_dim, bq, bk, persistent=persistent)(q, k, v, scales)
    o_fused = SparseVideoAttention(g, masks, wl.head_dim, bq, bk, persistent=persistent, fused=True)(q, k, v, scales)
    torch.cuda.synchronize()
    assert (bits_of(o_sep) == bits_of(o_fused)).all()


@pytest.mark.parametrize("geom,bq,bk,first,second", [
    ((4, 8, 8), 256, 64, "tmb", "tmb"), ((5, 24, 40), 128, 64, "tmb", "tmb"), ((17, 9, 13), 64, 32, "tmb", "tmb"),
    ((5, 24, 40), 256, 64, "tmb", "tm"), ((21, 9, 14), 256, 64, "tmb", "tm"),
    ((4, 8, 8), 256, 64, "tms", "tms"), ((17, 9, 13), 64, 32, "tms", "tms"), ((21, 9, 13), 256, 64, "tms", "tmb"),
    ((5, 24, 40), 128, 64, "tms", "tm")])
def test_fused_permutation_blocked_order_bit_identical(sv, geom, bq, bk, first, second):
    """Fused and separate paths agree bit for bit with temporal heads in the
    blocked or strip order (and a second temporal head of another
    temporal-major order in the same call); both within the bar of the oracle."""
    from block_sparse_spatio_svattn_amd.layer import SparseVideoAttention
    heads = (synth.Head("spatial", window=1), synth.Head("temporal", radius=2, order=first),
             synth.Head("temporal", radius=1, order=second))
    F, H, W = geom
    wl = synth.Workload(name="fb", seed=37, frames=F, height=H, width=W, head_dim=128, heads=heads,
                        tiles=((bq, bk),))
    inp = synth.make_inputs(wl)
    g = sv.Geom(F, H, W)
    masks = [sv_mask(h) for h in heads]
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    o_sep = SparseVideoAttention(g, masks, 128, bq, bk)(q, k, v, scales)
    o_fused = SparseVideoAttention(g, masks, 128, bq, bk, fused=True)(q, k, v, scales)
    torch.cuda.synchronize()
    assert (bits_of(o_sep) == bits_of(o_fused)).all()
    ref = _oracle_rows(wl, inp, [np.arange(wl.n_tokens)] * len(heads))
    for h in range(len(heads)):
        assert_close(f64_of(o_fused[h]), ref[h][0], f"fused {first}/{second} {geom} h{h}")


def test_fused_permutation_lse_and_ragged_long_runs(sv):
    """lse through the fused entry equals the separate path's lse moved back
    to frame-major rows; a geometry with 20-frame runs and a ragged tail."""
    heads = (synth.Head("temporal", radius=1, order="tm"), synth.Head("spatial", window=1),
             synth.Head("temporal", radius=2, order="tm"), synth.Head("dense", order="tm"))
    wl = synth.Workload(name="fused", seed=31, frames=21, height=4, width=6, head_dim=128, heads=heads,
                        tiles=((256, 64),))
    inp = synth.make_inputs(wl)
    g = sv.Geom(wl.frames, wl.height, wl.width)
    masks = [sv_mask(h) for h in heads]
    maps = [sv.build_tile_map(g, m, 256, 64) for m in masks]
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    perm, _ = sv.permutation_index(g)
    ws = sv.new_workspace()
    n = wl.n_tokens
    lse_f = torch.empty(len(heads), n, dtype=torch.float32, device="cuda")
    o_f = sv.forward_fused(g, q, k, v, masks, maps, scales, lse=lse_f, workspace=ws)
    # separate path: permuted copies of every temporal-major head
    tm = [h for h, m in enumerate(masks) if m.order == sv.TEMPORAL_MAJOR]
    qs, ks, vs = q.clone(), k.clone(), v.clone()
    for h in tm:
        for src, dst in ((q, qs), (k, ks), (v, vs)):
            dst[h:h + 1] = sv.permute_tokens(g, src[h:h + 1])
    lse_s = torch.empty_like(lse_f)
    o_s = sv.forward(g, qs, ks, vs, masks, maps, scales, lse=lse_s, workspace=ws)
    torch.cuda.synchronize()
    p = perm.long().cpu()
    o_s, lse_s = o_s.clone(), lse_s.clone()
    for h in tm:
        o_s[h] = sv.unpermute(g, o_s[h:h + 1])[0]
        row = torch.empty_like(lse_s[h].cpu())
        row[p] = lse_s[h].cpu()
        lse_s[h] = row.cuda()
    torch.cuda.synchronize()
    assert (bits_of(o_f) == bits_of(o_s)).all()
    assert torch.equal(lse_f, lse_s)
    ref = _oracle_rows(wl, inp, [np.arange(n)] * len(heads))
    for h in range(len(heads)):
        assert_close(f64_of(o_f[h]), ref[h][0], f"fused h{h}")


def _route_setup(sv, wl, window, radius, bq=64, bk=64):
    g = sv.Geom(wl.frames, wl.height, wl.width)
    sp = sv.Mask(sv.SPATIAL, sv.FRAME_MAJOR, window, 0)
    tp = sv.Mask(sv.TEMPORAL, sv.FRAME_MAJOR, 0, radius)
    dm = sv.build_tile_map(g, sv.Mask(sv.DENSE, sv.FRAME_MAJOR, 0, 0), bq, bk)
    sm = sv.build_tile_map(g, sp, bq, bk)
    tm = sv.build_tile_map(g, tp, bq, bk)
    return g, sp, tp, dm, sm, tm


def test_route_heads_closed_forms(sv):
    """A window covering every frame makes the spatial candidate the dense
    attention (deviation exactly 0, spatial chosen); a radius covering the
    grid does the same for the temporal one."""
    wl = synth.WORKLOADS["small"]
    inp = synth.make_inputs(wl)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    g, sp, tp, dm, sm, tm = _route_setup(sv, wl, wl.frames, 1)
    err, ch = sv.route_heads(g, q, k, v, sp, tp, dm, sm, tm, scales, [3, 40])
    torch.cuda.synchronize()
    assert (err[:, 0] == 0).all() and (err[:, 1] > 0).all() and (ch == sv.SPATIAL).all()
    g, sp, tp, dm, sm, tm = _route_setup(sv, wl, 0, max(wl.height, wl.width))
    err, ch = sv.route_heads(g, q, k, v, sp, tp, dm, sm, tm, scales, [0, 7, 74])
    torch.cuda.synchronize()
    assert (err[:, 1] == 0).all() and (err[:, 0] > 0).all() and (ch == sv.TEMPORAL).all()


def test_route_heads_128_key_maps(sv):
    """Routing over 128-key tile maps (two 64-key halves per entry) gives
    bit-identical deviations and choices to routing over 64-key maps."""
    wl = synth.WORKLOADS["small"]
    inp = synth.make_inputs(wl)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    out = []
    for bk in (64, 128):
        g, sp, tp, dm, sm, tm = _route_setup(sv, wl, 1, 2, bq=128, bk=bk)
        err, ch = sv.route_heads(g, q, k, v, sp, tp, dm, sm, tm, scales, [2, 17, 36])
        torch.cuda.synchronize()
        out.append((err.cpu().numpy(), ch.cpu().numpy()))
    assert np.array_equal(out[0][0].view(np.uint32), out[1][0].view(np.uint32))
    assert np.array_equal(out[0][1], out[1][1])


@pytest.mark.parametrize("window,radius,bq", [(1, 2, 64), (0, 6, 128), (1, 12, 256)])
def test_route_heads_against_oracle(sv, window, radius, bq):
    """Deviations within 5% of the oracle's (fp64 outputs of the same rows);
    the choice agrees wherever the oracle's two deviations differ by more
    than 10%."""
    wl = synth.WORKLOADS["small"]
    inp = synth.make_inputs(wl)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    g, sp, tp, dm, sm, tm = _route_setup(sv, wl, window, radius, bq=bq)
    n_qt = wl.n_tokens // bq
    qtiles = [1, n_qt // 2, n_qt - 2]
    err, ch = sv.route_heads(g, q, k, v, sp, tp, dm, sm, tm, scales, qtiles)
    torch.cuda.synchronize()
    err, ch = err.cpu().numpy(), ch.cpu().numpy()
    og = oracle.Geometry(wl.frames, wl.height, wl.width)
    rows = np.concatenate([np.arange(t * bq, (t + 1) * bq) for t in qtiles])
    for h in range(wl.n_heads):
        es, et, choice = oracle.route_head(inp.q[h], inp.k[h], inp.v[h], float(inp.scales[h]), og, window,
                                           radius, rows)
        assert abs(err[h, 0] - es) <= 0.05 * es + 1e-7, (h, err[h], es, et)
        assert abs(err[h, 1] - et) <= 0.05 * et + 1e-7, (h, err[h], es, et)
        if abs(es - et) > 0.1 * max(es, et):
            assert ch[h] == (sv.TEMPORAL if choice == "temporal" else sv.SPATIAL), (h, es, et)


@pytest.mark.parametrize("wl_name,bq,bk,qtiles", [("small", 64, 64, [0, 37, 74]), ("small", 256, 128, [3, 17]),
                                                  ("small", 128, 32, list(range(0, 36, 2))),
                                                  ("tiny", 32, 32, [0, 3, 7]), ("tiny", 64, 64, [1])])
def test_route_heads_equals_plain_forward(sv, wl_name, bq, bk, qtiles):
    """Routing runs its forward with the key list cut into splits merged by
    their lse; its deviations equal those of the plain forward's bf16 outputs
    over the same rows to 1% (a merged element may round to the neighbouring
    bf16 value), and its choice agrees wherever those differ by more than 2%.
    Covers head_dim 64 and 128, 32- to 128-key maps, 1 to 18 q-tiles (up to
    32 splits, many of them without a kept key on the small grids)."""
    wl = synth.WORKLOADS[wl_name]
    inp = synth.make_inputs(wl)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    g, sp, tp, dm, sm, tm = _route_setup(sv, wl, 1, 2, bq=bq, bk=bk)
    err, ch = sv.route_heads(g, q, k, v, sp, tp, dm, sm, tm, scales, qtiles)
    H = wl.n_heads
    outs = [sv.forward(g, q, k, v, [m] * H, [mp] * H, scales)
            for m, mp in ((sv.Mask(sv.DENSE, sv.FRAME_MAJOR, 0, 0), dm), (sp, sm), (tp, tm))]
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(t * bq, (t + 1) * bq) for t in qtiles])
    od, osp, ot = (f64_of(o)[:, rows] for o in outs)
    es = ((osp - od) ** 2).mean(axis=(1, 2))
    et = ((ot - od) ** 2).mean(axis=(1, 2))
    err, ch = err.cpu().numpy().astype(np.float64), ch.cpu().numpy()
    for h in range(H):
        assert abs(err[h, 0] - es[h]) <= 0.01 * es[h] + 1e-9, (h, err[h], es[h])
        assert abs(err[h, 1] - et[h]) <= 0.01 * et[h] + 1e-9, (h, err[h], et[h])
        if abs(es[h] - et[h]) > 0.02 * max(es[h], et[h]):
            assert ch[h] == (sv.TEMPORAL if et[h] < es[h] else sv.SPATIAL), (h, es[h], et[h])


def test_route_heads_repeat_is_deterministic(sv):
    """The split forward takes its work from a shared counter, but each split
    writes its own rows and the merge sums in a fixed order: two calls give
    bit-identical deviations."""
    wl = synth.WORKLOADS["small"]
    inp = synth.make_inputs(wl)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    g, sp, tp, dm, sm, tm = _route_setup(sv, wl, 1, 2, bq=64, bk=64)
    a, _ = sv.route_heads(g, q, k, v, sp, tp, dm, sm, tm, scales, [5, 50])
    b, _ = sv.route_heads(g, q, k, v, sp, tp, dm, sm, tm, scales, [5, 50])
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


def test_route_heads_sixteen_heads_two_group_schedule(sv):
    """16 heads: the routing forward's first launch then holds only dense
    slots, which at 256 x 32 tiles run the two-group schedule (static grid),
    with key splits and partial outputs; deviations equal the plain forward's
    to 1%."""
    heads = tuple([synth.Head("spatial", window=1)] * 16)
    wl = synth.Workload(name="route16", seed=41, frames=4, height=8, width=16, head_dim=128, heads=heads,
                        tiles=((256, 32),))
    inp = synth.make_inputs(wl)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    scales = [float(s) for s in inp.scales]
    g, sp, tp, dm, sm, tm = _route_setup(sv, wl, 1, 2, bq=256, bk=32)
    qtiles = [0, 1]
    err, ch = sv.route_heads(g, q, k, v, sp, tp, dm, sm, tm, scales, qtiles)
    H = wl.n_heads
    outs = [sv.forward(g, q, k, v, [m] * H, [mp] * H, scales)
            for m, mp in ((sv.Mask(sv.DENSE, sv.FRAME_MAJOR, 0, 0), dm), (sp, sm), (tp, tm))]
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(t * 256, (t + 1) * 256) for t in qtiles])
    od, osp, ot = (f64_of(o)[:, rows] for o in outs)
    es = ((osp - od) ** 2).mean(axis=(1, 2))
    et = ((ot - od) ** 2).mean(axis=(1, 2))
    err = err.cpu().numpy().astype(np.float64)
    for h in range(H):
        assert abs(err[h, 0] - es[h]) <= 0.01 * es[h] + 1e-9, (h, err[h], es[h])
        assert abs(err[h, 1] - et[h]) <= 0.01 * et[h] + 1e-9, (h, err[h], et[h])
