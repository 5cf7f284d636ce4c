"""The library's token-order maps and tile classifier, built for the host and
compared with the oracle on the CPU.

The permutation-index and classification code of the HIP library is written
as host-and-device functions; `tests/host/index_check.cpp` compiles them for
the host (hipcc, host code only runs) and prints permutations and tile
classes, which must equal the oracle's bit for bit.  This covers many more
geometries than the GPU tests (ragged patch blocks, one-row and one-column
grids, a single frame) at no GPU cost.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "index_check.cpp")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ORDERS = {"fm": 0, "tm": 1, "tmb": 2, "tms": 3}
KINDS = {"spatial": 0, "temporal": 1, "dense": 2}


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not available")
    out = str(tmp_path_factory.mktemp("host") / "index_check")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "block_sparse_spatio_svattn_amd", "csrc"), SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


def _run(exe, *args):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    return r.stdout.split("\n")


GEOMS = [(3, 5, 6), (4, 8, 8), (5, 24, 40), (21, 45, 80), (2, 3, 5), (1, 4, 4), (3, 9, 13), (2, 1, 7),
         (3, 7, 1), (4, 13, 17), (2, 90, 160)]


@pytest.mark.parametrize("order", ["tm", "tmb", "tms"])
@pytest.mark.parametrize("F,H,W", GEOMS)
def test_permutation_maps_match_oracle(exe, F, H, W, order):
    g = oracle.Geometry(F, H, W)
    out = _run(exe, F, H, W, ORDERS[order])
    perm = np.array(out[0].split(), dtype=np.int64)
    inv = np.array(out[1].split(), dtype=np.int64)
    ref = oracle.layout_tokens(g, order)
    assert (perm == ref).all()
    assert (inv[ref] == np.arange(g.n)).all()


CLASS_CASES = (
    [((F, H, W), "temporal", 0, r, order, bq, bk)
     for order in ("tmb", "tms")
     for (F, H, W) in [(3, 5, 6), (4, 8, 8), (3, 9, 13), (2, 3, 5), (4, 13, 17), (3, 7, 1), (2, 1, 7)]
     for r in (0, 1, 2, 5)
     for bq, bk in [(32, 32), (64, 32), (32, 64), (128, 64), (256, 64)]]
    + [((5, 24, 40), "temporal", 0, r, order, bq, bk) for order in ("tmb", "tms") for r in (1, 3)
       for bq, bk in [(128, 64), (256, 64)]]
    + [((F, H, W), kind, w, r, order, bq, bk)
       for (F, H, W) in [(3, 5, 6), (4, 8, 8), (3, 9, 13)]
       for kind, w, r, order in [("temporal", 0, 1, "tm"), ("temporal", 0, 2, "fm"), ("spatial", 1, 0, "fm"),
                                 ("dense", 0, 0, "tmb"), ("dense", 0, 0, "tms")]
       for bq, bk in [(32, 32), (128, 64)]]
)


@pytest.mark.parametrize("geom,kind,w,r,order,bq,bk", CLASS_CASES)
def test_tile_classes_match_oracle(exe, geom, kind, w, r, order, bq, bk):
    F, H, W = geom
    out = [row for row in _run(exe, F, H, W, ORDERS[order], KINDS[kind], w, r, bq, bk) if row]
    got = np.array([[int(c) for c in row] for row in out], dtype=np.uint8)
    ref, *_ = oracle.tile_map(oracle.Geometry(F, H, W), kind, w, r, order, bq, bk)
    assert got.shape == ref.shape
    assert (got == ref).all()


# ---- full-size maps: every q-tile row of the 75,600-token maps, a stratified
# set of rows of the 302,400-token maps (256 x 64 tiles, the benchmark's) ----

def _oracle_rows_threaded(g, kind, w, r, order, bq, bk, rows):
    """oracle.tile_map row by row on a thread pool (numpy releases the GIL in
    its array loops, so the brute force runs on every core)."""
    from concurrent.futures import ThreadPoolExecutor

    def one(qt):
        return oracle.tile_map(g, kind, w, r, order, bq, bk, qtiles=[qt])[0][0]
    with ThreadPoolExecutor(min(16, os.cpu_count() or 4)) as ex:
        return np.stack(list(ex.map(one, rows)))


FULL_SIZE_MAPS = [
    ((21, 45, 80), "spatial", 1, 0, "fm", None),
    ((21, 45, 80), "temporal", 0, 31, "tm", None),
    ((21, 45, 80), "temporal", 0, 31, "tmb", None),
    ((21, 45, 80), "temporal", 0, 22, "tmb", None),
    ((21, 45, 80), "temporal", 0, 31, "tms", None),
    ((21, 45, 80), "temporal", 0, 22, "tms", None),
    ((21, 45, 80), "temporal", 0, 11, "tms", None),
    ((21, 45, 80), "spatial", 7, 0, "fm", 8),
    ((21, 90, 160), "spatial", 1, 0, "fm", 16),
    ((21, 90, 160), "temporal", 0, 62, "tmb", 16),
    ((21, 90, 160), "temporal", 0, 62, "tms", 16),
]


@pytest.mark.parametrize("geom,kind,w,r,order,stride", FULL_SIZE_MAPS)
def test_full_size_tile_classes_match_oracle(exe, geom, kind, w, r, order, stride):
    """Host build of the classifier vs the brute-force oracle on full-size
    maps.  stride None: every q-tile row; else rows 0, 1, the last two (the
    last one ragged when block_q does not divide N) and every stride-th row."""
    F, H, W = geom
    bq, bk = 256, 64
    g = oracle.Geometry(F, H, W)
    n_qt = -(-g.n // bq)
    out = [row for row in _run(exe, F, H, W, ORDERS[order], KINDS[kind], w, r, bq, bk) if row]
    assert len(out) == n_qt
    rows = list(range(n_qt)) if stride is None else sorted({0, 1, n_qt - 2, n_qt - 1, *range(0, n_qt, stride)})
    got = np.array([[int(c) for c in out[qt]] for qt in rows], dtype=np.uint8)
    ref = _oracle_rows_threaded(g, kind, w, r, order, bq, bk, rows)
    assert got.shape == ref.shape
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} blocks differ, first at q-tile row {rows[bad[0][0]]}, k-tile {bad[0][1]}"
