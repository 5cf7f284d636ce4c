"""CPU tests of the C ABI: the library loads, exports every entry point the
header declares, and rejects invalid arguments with the documented status
before any HIP call.  No call here reaches a kernel launch: every call carries
at least one invalid argument, except the no-device check, which only runs
when the process sees no GPU."""
import ctypes
import os
import re

import pytest
import torch

import block_sparse_spatio_svattn_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svattn.h")

OK, INVALID, UNSUPPORTED, HIP = 0, 1, 2, 3
FAKE = 0x100000  # 16-byte-aligned stand-in address; never dereferenced here


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SVATTN_API\s+[\w\s\*]*?\b(svattn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = sv.lib()
    names = _declared()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(L, n), n
    # and nothing else named svattn_ beyond the header
    syms = os.popen(f"nm -D --defined-only {sv.LIB_PATH}").read()
    exported = set(re.findall(r" T (svattn_\w+)", syms))
    assert exported == set(names), exported ^ set(names)


def test_version_and_status_strings():
    assert sv.version() == 10400
    L = sv.lib()
    for code, name in [(0, b"SVATTN_OK"), (1, b"SVATTN_ERR_INVALID_ARG"), (2, b"SVATTN_ERR_UNSUPPORTED"),
                       (3, b"SVATTN_ERR_HIP"), (99, b"SVATTN_ERR_UNKNOWN")]:
        assert L.svattn_status_string(code) == name


def _status(fn, *args):
    return fn(*args)


def _err():
    return sv.lib().svattn_last_error().decode()


def test_tile_map_dims_validation():
    L = sv.lib()
    a, b = ctypes.c_int32(), ctypes.c_int32()
    g = sv.Geom(21, 45, 80)
    assert L.svattn_tile_map_dims(ctypes.byref(g), 256, 64, ctypes.byref(a), ctypes.byref(b)) == OK
    assert (a.value, b.value) == (296, 1182)
    assert L.svattn_tile_map_dims(None, 256, 64, ctypes.byref(a), ctypes.byref(b)) == INVALID
    assert "geom" in _err()
    assert L.svattn_tile_map_dims(ctypes.byref(sv.Geom(0, 4, 4)), 32, 32, ctypes.byref(a), ctypes.byref(b)) == INVALID
    assert L.svattn_tile_map_dims(ctypes.byref(g), 48, 64, ctypes.byref(a), ctypes.byref(b)) == UNSUPPORTED
    assert L.svattn_tile_map_dims(ctypes.byref(g), 256, 256, ctypes.byref(a), ctypes.byref(b)) == UNSUPPORTED
    assert L.svattn_tile_map_dims(ctypes.byref(sv.Geom(1024, 128, 256)), 256, 64, ctypes.byref(a),
                                  ctypes.byref(b)) == UNSUPPORTED


def _map(g, bq, bk, **kw):
    n_qt, n_kt = -(-g.n // bq), -(-g.n // bk)
    c = sv._TileMapC(bq, bk, n_qt, n_kt, FAKE, FAKE, FAKE, FAKE)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_token_limit_is_the_headers():
    """N < 2^23 (the header's limit): N = 2^23 - 1 is accepted, 2^23 is not,
    by every entry point that takes a geometry or a token count."""
    L = sv.lib()
    a, b = ctypes.c_int32(), ctypes.c_int32()
    ok = sv.Geom(1, 1, (1 << 23) - 1)
    too_big = sv.Geom(2, 1 << 11, 1 << 11)        # exactly 2^23
    assert L.svattn_tile_map_dims(ctypes.byref(ok), 256, 64, ctypes.byref(a), ctypes.byref(b)) == OK
    assert (a.value, b.value) == (-(-((1 << 23) - 1) // 256), -(-((1 << 23) - 1) // 64))
    assert L.svattn_tile_map_dims(ctypes.byref(too_big), 256, 64, ctypes.byref(a), ctypes.byref(b)) == UNSUPPORTED
    assert "2^23" in _err()
    assert L.svattn_permute_tokens(ctypes.byref(too_big), 1, 128, FAKE, FAKE * 4, None) == UNSUPPORTED
    assert _fwd(L, too_big) == UNSUPPORTED
    sarr = (ctypes.c_float * 1)(0.1)
    assert L.svattn_forward_dense_mask(1, 1 << 23, 128, FAKE, 0, sarr, FAKE, FAKE, FAKE, FAKE * 4, None, 256, 64,
                                       None) == INVALID


def test_forward_rejects_oversize_maps():
    """A map of n_qt * n_kt >= 2^31 blocks (possible near the token limit with
    32 x 32 tiles) is rejected by the forward itself, before any HIP call; the
    kernel indexes map entries in 32-bit arithmetic."""
    L = sv.lib()
    g = sv.Geom(4, 1024, 2000)                     # N = 8,192,000 < 2^23
    big = _map(g, 32, 32)
    assert big.n_qt * big.n_kt >= 1 << 31
    masks = [sv.Mask(sv.SPATIAL, sv.FRAME_MAJOR, 1, 0)]
    assert _fwd(L, g, heads=1, masks=masks, maps=[big], q=FAKE, k=FAKE << 8, v=FAKE << 9, o=FAKE << 10) == UNSUPPORTED
    assert "too large" in _err()
    mask = sv.Mask(sv.SPATIAL, sv.FRAME_MAJOR, 1, 0)
    assert L.svattn_build_tile_map_ex(ctypes.byref(g), ctypes.byref(mask), ctypes.byref(big), 0, None) == UNSUPPORTED


def test_build_tile_map_validation():
    L = sv.lib()
    g = sv.Geom(5, 24, 40)
    good_mask = sv.Mask(sv.TEMPORAL, sv.TEMPORAL_MAJOR, 0, 2)
    cases = [
        (sv.Mask(7, 0, 0, 0), _map(g, 64, 64), 0, INVALID),                     # bad kind
        (sv.Mask(0, 4, 0, 0), _map(g, 64, 64), 0, INVALID),                     # bad order
        (sv.Mask(0, 0, -1, 0), _map(g, 64, 64), 0, INVALID),                    # negative window
        (sv.Mask(sv.SPATIAL, sv.TEMPORAL_MAJOR, 1, 0), _map(g, 64, 64), 0, UNSUPPORTED),
        (sv.Mask(sv.SPATIAL, sv.TEMPORAL_MAJOR_BLOCKED, 1, 0), _map(g, 64, 64), 0, UNSUPPORTED),
        (sv.Mask(sv.SPATIAL, sv.TEMPORAL_MAJOR_STRIPS, 1, 0), _map(g, 64, 64), 0, UNSUPPORTED),
        (good_mask, _map(g, 96, 64), 0, UNSUPPORTED),                           # bad block_q
        (good_mask, _map(g, 64, 64, n_qt=3), 0, INVALID),                       # wrong dims
        (good_mask, _map(g, 64, 64, col=None), 0, INVALID),                     # NULL buffer
        (good_mask, _map(g, 64, 64, row_ptr=FAKE + 2), 0, INVALID),             # misaligned
        (good_mask, _map(g, 64, 64, qt_order=FAKE + 2), 0, INVALID),            # misaligned order
        (good_mask, _map(g, 64, 64), 4, INVALID),                               # unknown flag
        (good_mask, _map(g, 64, 64), 3, INVALID),                               # both traversal flags
    ]
    for m, mp, flags, want in cases:
        got = L.svattn_build_tile_map_ex(ctypes.byref(g), ctypes.byref(m), ctypes.byref(mp), flags, None)
        assert got == want, (m, got, _err())


def test_permute_validation():
    L = sv.lib()
    g = sv.Geom(4, 8, 8)
    assert L.svattn_permute_tokens(ctypes.byref(g), 2, 96, FAKE, FAKE * 4, None) == UNSUPPORTED
    assert L.svattn_permute_tokens(ctypes.byref(g), 0, 64, FAKE, FAKE * 4, None) == INVALID
    assert L.svattn_permute_tokens(ctypes.byref(g), 2, 64, None, FAKE * 4, None) == INVALID
    assert L.svattn_permute_tokens(ctypes.byref(g), 2, 64, FAKE + 8, FAKE * 4, None) == INVALID
    assert L.svattn_unpermute(ctypes.byref(g), 2, 64, FAKE, FAKE + 64, None) == INVALID   # overlap
    assert "overlap" in _err()
    assert L.svattn_permutation_index(ctypes.byref(g), None, None, None) == INVALID
    assert L.svattn_permutation_index(ctypes.byref(g), FAKE, FAKE + 4, None) == INVALID  # perm/inv overlap
    # order-aware entries: frame-major cannot be permuted to, unknown orders are rejected
    for o in (sv.FRAME_MAJOR, 4, -1):
        assert L.svattn_permute_tokens_order(ctypes.byref(g), o, 2, 64, FAKE, FAKE * 4, None) == INVALID
        assert "order" in _err()
        assert L.svattn_unpermute_order(ctypes.byref(g), o, 2, 64, FAKE, FAKE * 4, None) == INVALID
    assert L.svattn_permutation_index_order(ctypes.byref(g), 4, FAKE, None, None) == INVALID
    assert L.svattn_permute_tokens_order(ctypes.byref(g), sv.TEMPORAL_MAJOR_BLOCKED, 2, 96, FAKE, FAKE * 4,
                                         None) == UNSUPPORTED
    assert L.svattn_unpermute_order(ctypes.byref(g), sv.TEMPORAL_MAJOR_BLOCKED, 2, 64, FAKE, FAKE + 64,
                                    None) == INVALID   # overlap
    # the strip order passes the order check and reaches the later ones
    assert L.svattn_permute_tokens_order(ctypes.byref(g), sv.TEMPORAL_MAJOR_STRIPS, 2, 96, FAKE, FAKE * 4,
                                         None) == UNSUPPORTED
    assert L.svattn_unpermute_order(ctypes.byref(g), sv.TEMPORAL_MAJOR_STRIPS, 2, 64, FAKE, FAKE + 64,
                                    None) == INVALID   # overlap
    assert "overlap" in _err()


def _fwd(L, g, heads=2, d=128, masks=None, maps=None, scales=None, q=FAKE, k=FAKE * 16, v=FAKE * 32,
         o=FAKE * 64, lse=None, workspace=None):
    masks = masks or [sv.Mask(sv.SPATIAL, 0, 1, 0)] * heads
    maps = maps or [_map(g, 256, 64)] * heads
    scales = scales or [0.1] * heads
    marr = (sv.Mask * heads)(*masks)
    P = ctypes.POINTER(sv._TileMapC)
    parr = (P * heads)(*[ctypes.pointer(m) for m in maps])
    sarr = (ctypes.c_float * heads)(*scales)
    return L.svattn_forward(ctypes.byref(g), heads, d, marr, parr, sarr, q, k, v, o, lse, workspace, None)


def test_forward_validation():
    L = sv.lib()
    g = sv.Geom(4, 8, 8)   # N = 256
    n_bytes = 2 * 256 * 128 * 2
    assert _fwd(L, g, d=96) == UNSUPPORTED
    assert _fwd(L, g, scales=[0.1, 0.0]) == INVALID
    assert _fwd(L, g, scales=[0.1, float("nan")]) == INVALID
    assert _fwd(L, g, q=None) == INVALID
    assert _fwd(L, g, k=FAKE * 16 + 4) == INVALID                            # misaligned
    assert _fwd(L, g, o=FAKE + n_bytes // 2) == INVALID                      # o overlaps q
    assert "overlap" in _err()
    assert _fwd(L, g, lse=FAKE * 64 + 16) == INVALID                         # lse overlaps o
    assert _fwd(L, g, maps=[_map(g, 256, 64), _map(g, 128, 64)]) == INVALID  # mixed tiles
    assert _fwd(L, g, maps=[_map(g, 256, 256)] * 2) == UNSUPPORTED           # block_k 256
    assert _fwd(L, g, maps=[_map(g, 256, 64, n_kt=5)] * 2) == INVALID
    assert _fwd(L, g, maps=[_map(g, 256, 64, col_cls=None)] * 2) == INVALID
    assert _fwd(L, g, masks=[sv.Mask(sv.SPATIAL, sv.TEMPORAL_MAJOR, 1, 0)] * 2) == UNSUPPORTED
    assert L.svattn_forward(ctypes.byref(g), 2, 128, None, None, None, FAKE, FAKE, FAKE, FAKE, None, None,
                            None) == INVALID
    assert _fwd(L, g, maps=[_map(g, 256, 64, qt_order=FAKE + 2)] * 2) == INVALID  # misaligned order
    assert _fwd(L, g, workspace=FAKE * 128 + 2) == INVALID                    # misaligned workspace
    assert _fwd(L, g, workspace=FAKE * 64 + 512) == INVALID                   # workspace inside o
    assert "workspace" in _err()


def test_forward_ptrs_and_dense_mask_validation():
    L = sv.lib()
    g = sv.Geom(4, 8, 8)
    heads, d = 2, 64
    hb = 256 * d * 2
    marr = (sv.Mask * heads)(*[sv.Mask(sv.TEMPORAL, sv.TEMPORAL_MAJOR, 0, 1)] * heads)
    m = _map(g, 64, 32)
    P = ctypes.POINTER(sv._TileMapC)
    parr = (P * heads)(ctypes.pointer(m), ctypes.pointer(m))
    sarr = (ctypes.c_float * heads)(0.1, 0.1)
    VP = ctypes.c_void_p * heads
    q, k, v = VP(FAKE, FAKE + hb), VP(FAKE * 16, FAKE * 16 + hb), VP(FAKE * 32, FAKE * 32 + hb)
    o_overlap = VP(FAKE * 64, FAKE * 64 + 16)                # two heads' outputs overlap
    assert L.svattn_forward_ptrs(ctypes.byref(g), heads, d, marr, parr, sarr, q, k, v, o_overlap, None,
                                 None, None) == INVALID
    o_in = VP(FAKE * 64, FAKE + hb)                           # head 1 writes over q of head 1
    assert L.svattn_forward_ptrs(ctypes.byref(g), heads, d, marr, parr, sarr, q, k, v, o_in, None,
                                 None, None) == INVALID
    assert L.svattn_forward_ptrs(ctypes.byref(g), heads, d, marr, parr, sarr, q, k, v, None, None,
                                 None, None) == INVALID
    # dense-mask entry
    assert L.svattn_forward_dense_mask(2, 0, 64, FAKE, 1, sarr, FAKE, FAKE * 16, FAKE * 32, FAKE * 64, None,
                                       64, 32, None) == INVALID
    assert L.svattn_forward_dense_mask(2, 256, 64, None, 1, sarr, FAKE, FAKE * 16, FAKE * 32, FAKE * 64, None,
                                       64, 32, None) == INVALID
    assert L.svattn_forward_dense_mask(2, 256, 64, FAKE * 128, 1, sarr, FAKE, FAKE * 16, FAKE * 32, FAKE * 64,
                                       None, 64, 128, None) == UNSUPPORTED


def test_binding_rejects_host_tensors():
    g = sv.Geom(4, 8, 8)
    x = torch.zeros(1, 256, 64, dtype=torch.bfloat16)
    with pytest.raises(sv.SvattnError):
        sv.permute_tokens(g, x, out=torch.zeros_like(x))
    # the forward bindings marshal their arguments, then refuse host tensors
    # before calling the library
    from types import SimpleNamespace
    mp = SimpleNamespace(c=_map(g, 256, 64))
    masks = [sv.Mask(sv.SPATIAL, sv.FRAME_MAJOR, 1, 0)]
    for fn in (sv.forward, sv.forward_noalloc):
        with pytest.raises(sv.SvattnError, match="CUDA \\(HIP\\) tensor"):
            fn(g, x, x, x, masks, [mp], [0.125])
        with pytest.raises(sv.SvattnError, match="one mask and one map per head"):
            fn(g, x, x, x, masks * 2, [mp], [0.125])


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-device error path")
def test_valid_call_without_device_reports_hip_error():
    L = sv.lib()
    g = sv.Geom(4, 8, 8)
    st = L.svattn_permutation_index(ctypes.byref(g), FAKE, None, None)
    assert st == HIP
    assert len(_err()) > 0


def test_workspace_size_matches_header():
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "svattn.h")).read()
    m = re.search(r"#define SVATTN_FORWARD_WORKSPACE_BYTES (\d+)", hdr)
    assert m and int(m.group(1)) == sv.FORWARD_WORKSPACE_BYTES


def test_traffic_summary_parses():
    """The committed counter summary carries a machine-readable record that
    bench.py can read (its traffic is reported only for matching sources)."""
    import json
    import sys
    root = os.path.join(os.path.dirname(__file__), "..")
    text = open(os.path.join(root, "profiles", "fwd2_kernel_headline_traffic.md")).read()
    rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    assert rec["traffic_bytes_per_launch"] > rec["algorithmic_bytes_per_launch"] > 0
    assert len(rec["sources_sha256"]) == 64
    sys.path.insert(0, root)
    import bench
    t = bench.measured_traffic("headline", rec["temporal_order"])
    assert t is None or t == rec["traffic_bytes_per_launch"]
    assert bench.measured_traffic("small", rec["temporal_order"]) is None
    other = "tmb" if rec["temporal_order"] != "tmb" else "tms"
    assert bench.measured_traffic("headline", other) is None          # counters of another token order


def test_forward_fused_validation():
    """The fused entry takes svattn_forward's arguments and checks them the
    same way; heads may mix the two temporal-major orders (each head's rows
    follow from its own order)."""
    L = sv.lib()
    g = sv.Geom(4, 8, 8)   # N = 256
    heads, d = 2, 64
    marr = (sv.Mask * heads)(sv.Mask(sv.TEMPORAL, sv.TEMPORAL_MAJOR, 0, 1), sv.Mask(sv.SPATIAL, 0, 1, 0))
    m = _map(g, 64, 32)
    P = ctypes.POINTER(sv._TileMapC)
    parr = (P * heads)(ctypes.pointer(m), ctypes.pointer(m))
    sarr = (ctypes.c_float * heads)(0.1, 0.1)
    q, k, v, o = FAKE, FAKE * 16, FAKE * 32, FAKE * 64
    f = lambda masks=marr, **kw: L.svattn_forward_fused(ctypes.byref(g), heads, d, masks, parr, sarr,
                                                        kw.get("q", q), k, v, kw.get("o", o), None, kw.get("ws"),
                                                        None)
    assert f(o=FAKE * 16 + 1024) == INVALID        # o inside k
    assert f(q=FAKE + 8) == INVALID                # misaligned q
    assert f(ws=FAKE * 64 + 256) == INVALID        # workspace inside o
    bad = (sv.Mask * heads)(sv.Mask(sv.TEMPORAL, sv.TEMPORAL_MAJOR, 0, 1), sv.Mask(7, 0, 1, 0))
    assert f(masks=bad) == INVALID                 # unknown mask kind
    # both temporal-major orders in one call pass validation (fails later only for lack of a device)
    mixed = (sv.Mask * heads)(sv.Mask(sv.TEMPORAL, sv.TEMPORAL_MAJOR, 0, 1),
                              sv.Mask(sv.TEMPORAL, sv.TEMPORAL_MAJOR_BLOCKED, 0, 1))
    assert f(masks=mixed) != INVALID


def test_route_validation():
    L = sv.lib()
    g = sv.Geom(4, 8, 8)   # N = 256, 4 q-tiles of 64
    heads, d = 2, 64
    b = ctypes.c_size_t()
    assert L.svattn_route_scratch_bytes(heads, d, 64, 2, ctypes.byref(b)) == 0
    # work counter, then per mask 32 key splits (1024 work items over 3 masks x 2 heads x 2 q-tiles, at
    # most 32) of fp32 rows and their lse, then one pair of sums per 16-row merge workgroup
    rows = heads * 2 * 32 * 64
    assert b.value == 256 + 3 * (rows * d * 4 + rows * 4) + heads * 2 * (64 // 16) * 8
    # the split count follows the work-item target: ceil(1024 / (3 heads n_qtiles)), clamped to [1, 32]
    for hh, dd, bq, nq, splits in [(10, 128, 256, 2, 18), (400, 128, 256, 1, 1), (1, 128, 256, 32, 11),
                                   (3, 64, 32, 5, 23), (342, 64, 128, 1, 1), (341, 64, 128, 1, 2)]:
        assert L.svattn_route_scratch_bytes(hh, dd, bq, nq, ctypes.byref(b)) == 0
        r = hh * nq * splits * bq
        assert b.value == 256 + 3 * (r * dd * 4 + r * 4) + hh * nq * (bq // (1024 // dd)) * 8, (hh, dd, bq, nq)
    assert L.svattn_route_scratch_bytes(heads, d, 64, 33, ctypes.byref(b)) == INVALID
    assert L.svattn_route_scratch_bytes(heads, 96, 64, 2, ctypes.byref(b)) == UNSUPPORTED
    sp, tp = sv.Mask(sv.SPATIAL, 0, 1, 0), sv.Mask(sv.TEMPORAL, 0, 0, 1)
    m = _map(g, 64, 32)
    sarr = (ctypes.c_float * heads)(0.1, 0.1)
    q, k, v, scr, err, ch = FAKE, FAKE * 16, FAKE * 32, FAKE * 64, FAKE * 128, FAKE * 128 + 256
    def call(qt, spatial=sp, temporal=tp, scratch_bytes=None, **kw):
        arr = (ctypes.c_int32 * len(qt))(*qt)
        return L.svattn_route_heads(ctypes.byref(g), heads, d, ctypes.byref(spatial), ctypes.byref(temporal),
                                    ctypes.byref(m), ctypes.byref(m), ctypes.byref(m), sarr, arr, len(qt), q, k, v,
                                    kw.get("scr", scr), scratch_bytes if scratch_bytes is not None else b.value,
                                    kw.get("err", err), ch, None)
    assert call([0, 4]) == INVALID                  # q-tile 4 is past N
    assert call([1, 1]) == INVALID                  # repeated
    assert call([0, 1], spatial=tp) == INVALID      # candidates swapped
    assert call([0, 1], temporal=sv.Mask(sv.TEMPORAL, sv.TEMPORAL_MAJOR, 0, 1)) == INVALID
    assert call([0, 1], scratch_bytes=16) == INVALID
    assert call([0, 1], scr=FAKE * 16 + 64) == INVALID   # scratch inside k
    assert call([0, 1], err=FAKE * 64 + 32) == INVALID   # err inside scratch
    assert "overlap" in _err()
