"""GPU parity: permutation index, token permutation and tile maps must match the
oracle bit-exactly (integer and byte work)."""
import numpy as np
import pytest
import torch

import oracle
import svattn_synth as synth
from _util import bits_of, sv_mask, to_dev

pytestmark = pytest.mark.gpu

GEOMS = [(4, 8, 8), (5, 24, 40), (21, 45, 80), (21, 90, 160), (3, 5, 7), (1, 4, 4), (2, 3, 5), (7, 1, 9)]


@pytest.fixture(scope="module")
def sv():
    import block_sparse_spatio_svattn_amd as m
    return m


ORDER_CODE = {"tm": 1, "tmb": 2, "tms": 3}  # SVATTN_TEMPORAL_MAJOR / _BLOCKED / _STRIPS


@pytest.mark.parametrize("order", ["tm", "tmb", "tms"])
@pytest.mark.parametrize("F,H,W", GEOMS + [(3, 9, 13), (4, 13, 17)])
def test_permutation_index_bit_exact(sv, F, H, W, order):
    g = sv.Geom(F, H, W)
    perm, inv = sv.permutation_index(g, order=ORDER_CODE[order])
    ref = oracle.layout_tokens(oracle.Geometry(F, H, W), order)
    p = perm.cpu().numpy()
    assert (p == ref).all()
    iv = inv.cpu().numpy()
    assert (iv[ref] == np.arange(g.n)).all()


@pytest.mark.parametrize("order", ["tm", "tmb", "tms"])
@pytest.mark.parametrize("F,H,W,d,heads", [(4, 8, 8, 64, 2), (5, 24, 40, 128, 3), (3, 5, 7, 128, 2),
                                           (21, 45, 80, 128, 5), (1, 4, 4, 64, 1), (3, 9, 13, 64, 2)])
def test_permute_unpermute_bit_exact(sv, F, H, W, d, heads, order):
    g = sv.Geom(F, H, W)
    x = synth.random_bf16((heads, g.n, d), seed=F * 1000 + W)
    xd = to_dev(x)
    perm = oracle.layout_tokens(oracle.Geometry(F, H, W), order)
    o = ORDER_CODE[order]
    y = sv.permute_tokens(g, xd, order=o)
    torch.cuda.synchronize()
    assert (bits_of(y) == x[:, perm]).all()
    back = sv.unpermute(g, y, order=o)
    torch.cuda.synchronize()
    assert (bits_of(back) == x).all()


def _compare_map(m, ref, qtiles=None):
    cls_ref, rp_ref, col_ref, cc_ref = ref
    cls = m.cls.cpu().numpy().reshape(m.n_qt, m.n_kt)
    rp = m.row_ptr.cpu().numpy()
    col = m.col.cpu().numpy()
    cc = m.col_cls.cpu().numpy()
    rows = range(m.n_qt) if qtiles is None else qtiles
    for i, qt in enumerate(rows):
        assert (cls[qt] == cls_ref[i]).all(), f"cls row {qt}"
        a, b = rp[qt], rp[qt + 1]
        ra, rb = rp_ref[i], rp_ref[i + 1]
        assert b - a == rb - ra, f"row {qt} nnz"
        assert (col[a:b] == col_ref[ra:rb]).all(), f"col row {qt}"
        assert (cc[a:b] == cc_ref[ra:rb]).all(), f"col_cls row {qt}"
    # whole-map invariants
    assert rp[0] == 0 and (np.diff(rp) >= 0).all()
    assert rp[-1] == int((cls != 0).sum())
    nz_cols = col[:rp[-1]]
    for qt in range(m.n_qt):
        seg = nz_cols[rp[qt]:rp[qt + 1]]
        assert (np.diff(seg) > 0).all()
    assert (cc[:rp[-1]] == cls[np.repeat(np.arange(m.n_qt), np.diff(rp)), nz_cols]).all()
    # q-tile visiting order: exact against the oracle on whole maps; on sampled
    # maps a permutation that is longest-row-first with ties by index
    order = m.qt_order.cpu().numpy()
    if qtiles is None:
        assert (order == oracle.qtile_order(rp_ref)).all()
    assert (np.sort(order) == np.arange(m.n_qt)).all()
    lens = np.diff(rp.astype(np.int64))[order]
    assert (np.diff(lens) <= 0).all()
    ties = np.diff(lens) == 0
    assert (np.diff(order)[ties] > 0).all()


SMALL_CASES = (
    [((4, 8, 8), k, w, r, o, bq, bk) for (k, w, r, o) in
     [("spatial", 1, 0, "fm"), ("temporal", 0, 1, "fm"), ("temporal", 0, 1, "tm"), ("dense", 0, 0, "fm"),
      ("temporal", 0, 0, "tm"), ("spatial", 0, 0, "fm")]
     for bq in (32, 64, 256) for bk in (32, 64, 128)]
    + [((5, 24, 40), k, w, r, o, bq, bk) for (k, w, r, o) in
       [("spatial", 1, 0, "fm"), ("temporal", 0, 2, "fm"), ("temporal", 0, 2, "tm")]
       for bq in (64, 128, 256) for bk in (32, 64, 128)]
    + [((3, 5, 7), "temporal", 0, 1, "tm", 32, 32), ((3, 5, 7), "spatial", 1, 0, "fm", 64, 32),
       ((1, 4, 4), "temporal", 0, 1, "tm", 32, 32), ((7, 1, 9), "temporal", 0, 2, "tm", 32, 64),
       ((2, 3, 5), "spatial", 0, 0, "fm", 32, 128)]
    # temporal-major over 4x4 patch blocks, with ragged edge blocks and tiles
    + [(geom, "temporal", 0, r, "tmb", bq, bk)
       for geom, r in [((4, 8, 8), 1), ((5, 24, 40), 2), ((3, 9, 13), 2), ((3, 5, 7), 1), ((7, 1, 9), 2),
                       ((1, 4, 4), 1), ((4, 13, 17), 5)]
       for bq, bk in [(32, 32), (128, 64), (256, 64)]]
    + [((4, 8, 8), "dense", 0, 0, "tmb", 64, 64)]
    # temporal-major over snake strips, odd widths (a last strip one patch wide) included
    + [(geom, "temporal", 0, r, "tms", bq, bk)
       for geom, r in [((4, 8, 8), 1), ((5, 24, 40), 2), ((3, 9, 13), 2), ((3, 5, 7), 1), ((7, 1, 9), 2),
                       ((1, 4, 4), 1), ((4, 13, 17), 5)]
       for bq, bk in [(32, 32), (128, 64), (256, 64)]]
    + [((4, 8, 8), "dense", 0, 0, "tms", 64, 64)]
)


@pytest.mark.parametrize("geom,kind,w,r,order,bq,bk", SMALL_CASES)
def test_tile_map_bit_exact(sv, geom, kind, w, r, order, bq, bk):
    g = sv.Geom(*geom)
    head = synth.Head(kind, window=w, radius=r, order=order)
    m = sv.build_tile_map(g, sv_mask(head), bq, bk)
    torch.cuda.synchronize()
    ref = oracle.tile_map(oracle.Geometry(*geom), kind, w, r, order, bq, bk)
    _compare_map(m, ref)


@pytest.mark.parametrize("wl_name,hi,order", [("headline", 0, "fm"), ("headline", 5, "tm"),
                                              ("headline", 5, "fm"), ("perm_study", 0, "tm"),
                                              ("p1440", 0, "fm"), ("p1440", 5, "tm"), ("headline", 5, "tmb"),
                                              ("perm_study", 0, "tmb"), ("p1440", 5, "tmb"),
                                              ("headline", 5, "tms"), ("perm_study", 0, "tms"),
                                              ("p1440", 5, "tms")])
@pytest.mark.parametrize("bq,bk", [(256, 64), (128, 32)])
def test_tile_map_large_sampled_rows(sv, wl_name, hi, order, bq, bk):
    wl = synth.WORKLOADS[wl_name]
    h = wl.heads[hi]
    g = sv.Geom(wl.frames, wl.height, wl.width)
    m = sv.build_tile_map(g, sv_mask(h, order), bq, bk)
    torch.cuda.synchronize()
    rng = np.random.default_rng(hi + bq)
    qtiles = sorted(set([0, m.n_qt - 1] + list(rng.choice(m.n_qt, 4, replace=False))))
    ref = oracle.tile_map(oracle.Geometry(wl.frames, wl.height, wl.width), h.kind, h.window, h.radius,
                          order, bq, bk, qtiles=qtiles)
    _compare_map(m, ref, qtiles)


def _oracle_map_threaded(geom, kind, w, r, order, bq, bk):
    """oracle.tile_map over every q-tile row, one row per task on a thread pool
    (numpy releases the GIL in its array loops); rows assembled in order, so the
    result is the same as oracle.tile_map over all rows."""
    from concurrent.futures import ThreadPoolExecutor
    g = oracle.Geometry(*geom)
    n_qt = -(-g.n // bq)

    def one(qt):
        return oracle.tile_map(g, kind, w, r, order, bq, bk, qtiles=[qt])
    with ThreadPoolExecutor(16) as ex:
        rows = list(ex.map(one, range(n_qt)))
    cls = np.concatenate([x[0] for x in rows])
    lens = np.array([x[1][1] for x in rows], dtype=np.int64)
    row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    col = np.concatenate([x[2] for x in rows]).astype(np.int32)
    col_cls = np.concatenate([x[3] for x in rows]).astype(np.uint8)
    return cls, row_ptr, col, col_cls


@pytest.mark.parametrize("wl_name,hi,order", [("headline", 0, "fm"), ("headline", 5, "tm"),
                                              ("headline", 5, "tmb"), ("perm_study", 0, "tmb"),
                                              ("headline", 5, "tms"), ("perm_study", 0, "tms")])
def test_tile_map_full_size_every_row(sv, wl_name, hi, order):
    """The benchmark's 256 x 64 maps at 75,600 tokens, whole: every q-tile row's
    classes, CSR list and the longest-first q-tile order, bit for bit."""
    wl = synth.WORKLOADS[wl_name]
    h = wl.heads[hi]
    g = sv.Geom(wl.frames, wl.height, wl.width)
    print(f"full map {wl_name} head {hi} ({h.kind}) order {order}", flush=True)
    m = sv.build_tile_map(g, sv_mask(h, order), 256, 64)
    torch.cuda.synchronize()
    ref = _oracle_map_threaded((wl.frames, wl.height, wl.width), h.kind, h.window, h.radius, order, 256, 64)
    _compare_map(m, ref)


def test_all_boundary_flag(sv):
    g = sv.Geom(5, 24, 40)
    mk = sv_mask(synth.Head("temporal", radius=2, order="tm"))
    a = sv.build_tile_map(g, mk, 128, 64)
    b = sv.build_tile_map(g, mk, 128, 64, flags=sv.MAP_ALL_BOUNDARY)
    torch.cuda.synchronize()
    ca, cb = a.cls.cpu().numpy(), b.cls.cpu().numpy()
    assert ((ca != 0) == (cb != 0)).all() and set(np.unique(cb)) <= {0, 1}
    assert (a.row_ptr.cpu().numpy() == b.row_ptr.cpu().numpy()).all()


def test_tile_aligned_flag_map(sv):
    """MAP_TILE_ALIGNED lists the same non-empty tiles as the exact map, every
    one FULL."""
    g = sv.Geom(5, 24, 40)
    for head in (synth.Head("temporal", radius=2, order="tm"), synth.Head("spatial", window=1)):
        a = sv.build_tile_map(g, sv_mask(head), 128, 64)
        b = sv.build_tile_map(g, sv_mask(head), 128, 64, flags=sv.MAP_TILE_ALIGNED)
        torch.cuda.synchronize()
        ca, cb = a.cls.cpu().numpy(), b.cls.cpu().numpy()
        assert ((ca != 0) == (cb != 0)).all()
        assert set(np.unique(cb).tolist()) <= {0, 2}
        nnz = a.nnz()
        assert nnz == b.nnz()
        assert (a.col[:nnz].cpu().numpy() == b.col[:nnz].cpu().numpy()).all()
        assert (b.col_cls[:nnz].cpu().numpy() == 2).all()
