#!/usr/bin/env python3
"""Benchmark of the block-sparse spatio-temporal attention hot path on one MI355X.

One step = one pass of the hot path over the workload's synthetic inputs,
already resident in HBM: permute the temporal heads' Q/K/V to temporal-major
order -> block-sparse attention forward over all heads -> unpermute the
temporal heads' output.  Tile maps are built once per (geometry, mask, tile)
and reused across steps (they do not depend on the activations); the
classifier is timed separately, as are a dense-attention run of the same
kernel (every tile full, no masking) and the naive traversal that masks every
visited tile.

Prints one JSON line.  `value` is effective TFLOP/s of the whole step
(4 * head_dim * kept pairs, summed over heads, divided by ms_per_step);
`roofline` is for the dominant kernel (the attention forward), timed with
HIP events on the stream it is launched on.

    python bench.py [--steps K] [--warmup W] [--workload headline] [--temporal-order tms|tmb|tm|fm]

Temporal heads run by default in the temporal-major order over snake strips
of two patch columns (the library's layout); the pages' temporal-major order,
which lists patches row by row, and the one over 4x4 patch blocks are timed
beside it as `other_temporal_orders`.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse attn fwd ms + effective TFLOP/s (% bf16 MFMA peak), 75.6K tok×10h×d128"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "fwd2_kernel_headline_traffic.md")


def kernel_sources_sha256() -> str:
    """Hash of the kernel sources (csrc/*.hip, csrc/*.hpp, include/svattn.h)."""
    import glob
    import hashlib
    pkg = os.path.join(ROOT, "block_sparse_spatio_svattn_amd", "csrc")
    paths = sorted(glob.glob(os.path.join(pkg, "*.hip")) + glob.glob(os.path.join(pkg, "*.hpp")) +
                   [os.path.join(ROOT, "include", "svattn.h")])
    h = hashlib.sha256()
    for p in paths:
        h.update(os.path.relpath(p, ROOT).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, temporal_order: str):
    """HBM bytes per forward launch from the committed counter summary, or None
    when there is none for this workload and token order or the kernel sources
    changed since."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("temporal_order") != temporal_order or \
            rec.get("sources_sha256") != kernel_sources_sha256():
        return None
    return rec.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)   # >= 50 timed runs, 10 warm-up runs
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--block-q", type=int, default=256)
    ap.add_argument("--block-k", type=int, default=64)
    ap.add_argument("--temporal-order", choices=["tm", "tmb", "tms", "fm"], default="tms",
                    help="token order of the temporal heads: temporal-major (patches in raster order), "
                         "temporal-major over 4x4 patch blocks or over snake strips, or frame-major")
    ap.add_argument("--dense-steps", type=int, default=5)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-naive", action="store_true")
    ap.add_argument("--no-aligned", action="store_true", help="skip the tile-aligned traversal")
    ap.add_argument("--no-fused", action="store_true", help="skip the fused-permutation step")
    ap.add_argument("--no-routing", action="store_true", help="skip the head-routing timing")
    ap.add_argument("--no-alt-order", action="store_true",
                    help="skip the forwards with the temporal heads in the other temporal-major orders")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="skip the GPU clock sample taken under load")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="forward launches timed after a 512 MB write that evicts L2 and MALL (0: skip)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library runs the kernel on one MI355X and has no "
              f"multi-GPU path (--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_spatio_svattn_amd as sv
    from block_sparse_spatio_svattn_amd import metrics
    from block_sparse_spatio_svattn_amd.layer import SparseVideoAttention
    import svattn_synth as synth

    ORDER_CODES = {"tm": sv.TEMPORAL_MAJOR, "tmb": sv.TEMPORAL_MAJOR_BLOCKED, "tms": sv.TEMPORAL_MAJOR_STRIPS,
                   "fm": sv.FRAME_MAJOR}
    wl = synth.WORKLOADS[args.workload]
    g = sv.Geom(wl.frames, wl.height, wl.width)
    kinds = {synth.SPATIAL: sv.SPATIAL, synth.TEMPORAL: sv.TEMPORAL, synth.DENSE: sv.DENSE}
    masks = []
    for h in wl.heads:
        order = sv.FRAME_MAJOR
        if h.kind == synth.TEMPORAL:
            order = ORDER_CODES[args.temporal_order]
        masks.append(sv.Mask(kinds[h.kind], order, h.window, h.radius))
    H, N, D = wl.n_heads, wl.n_tokens, wl.head_dim

    log(f"workload {wl.name}: N={N} heads={H} d={D} tiles {args.block_q}x{args.block_k}")
    t0 = time.time()
    inp = synth.make_inputs(wl)
    log(f"inputs drawn on the host ({time.time() - t0:.1f} s)")

    # ---- CPU oracle baseline (bounded sample), before this process touches the GPU ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, inp, args.cpu_seconds)
        log(f"cpu oracle baseline {cpu}")

    t0 = time.time()
    dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    scales = [float(s) for s in inp.scales]
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    log(f"inputs resident in HBM ({3 * q.numel() * 2 / 1e9:.2f} GB, {time.time() - t0:.1f} s)")

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # ---- tile classifier (one-off per geometry/mask/tile), timed separately ----
    layer = SparseVideoAttention(g, masks, D, args.block_q, args.block_k)
    distinct = {}
    for m, mp in zip(layer.masks, layer.maps):
        distinct[(m.kind, m.order, m.window, m.radius)] = (m, mp)
    torch.cuda.synchronize()
    cls_ms = []
    for _ in range(3):
        a, b = ev(), ev()
        a.record(stream)
        for m, mp in distinct.values():
            mp.rebuild(m)
        b.record(stream)
        torch.cuda.synchronize()
        cls_ms.append(a.elapsed_time(b))
    nnz = {str(key): mp.nnz() for key, (m, mp) in distinct.items()}
    log(f"classifier {min(cls_ms):.3f} ms for {len(distinct)} maps; nnz {nnz}")

    # ---- warmup ----
    for _ in range(args.warmup):
        layer(q, k, v, scales, out=out)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # ---- timed steps ----
    K = args.steps
    marks = [[ev() for _ in range(4)] for _ in range(K)]
    start, end = ev(), ev()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        marks[i][0].record(stream)
        layer.permute_inputs(q, k, v)
        marks[i][1].record(stream)
        layer.attend(q, k, v, out, scales)
        marks[i][2].record(stream)
        layer.unpermute_output(out)
        marks[i][3].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / K
    perm_ms = float(np.mean([m[0].elapsed_time(m[1]) for m in marks]))
    fwd_all = np.array([m[1].elapsed_time(m[2]) for m in marks])
    fwd_ms = float(np.mean(fwd_all))
    unperm_ms = float(np.mean([m[2].elapsed_time(m[3]) for m in marks]))
    log(f"step {ms_step:.3f} ms: permute {perm_ms:.3f} + forward {fwd_ms:.3f} (min {fwd_all.min():.3f}) "
        f"+ unpermute {unperm_ms:.3f}")

    flops = metrics.effective_flops(g, masks, D)
    kept = sum(metrics.kept_pairs(g, m) for m in masks)
    kept_frac = kept / (H * N * N)
    fwd_tflops = flops / (fwd_ms * 1e-3) / 1e12
    peak = metrics.BF16_PEAK_TFLOPS

    extra = {}
    # ---- the other temporal-major orders (patches row by row, 4x4 blocks, snake strips) ----
    alts = [] if args.no_alt_order or args.temporal_order == "fm" else \
        [o for o in ("tm", "tmb", "tms") if o != args.temporal_order]
    for alt in alts:
        alt_order = ORDER_CODES[alt]
        amasks = [sv.Mask(m.kind, alt_order if m.order != sv.FRAME_MAJOR else m.order, m.window, m.radius)
                  for m in masks]
        alayer = SparseVideoAttention(g, amasks, D, args.block_q, args.block_k)
        aout = torch.empty_like(out)
        alayer.permute_inputs(q, k, v)
        alayer.attend(q, k, v, aout, scales)
        torch.cuda.synchronize()
        am = []
        for _ in range(args.dense_steps):
            a, b = ev(), ev()
            a.record(stream)
            alayer.attend(q, k, v, aout, scales)
            b.record(stream)
            am.append((a, b))
        torch.cuda.synchronize()
        alt_ms = float(np.mean([a.elapsed_time(b) for a, b in am]))
        anz = {str((m.kind, m.order, m.window, m.radius)): mp.nnz() for m, mp in zip(alayer.masks, alayer.maps)}
        log(f"forward with temporal heads in order {alt}: {alt_ms:.3f} ms; nnz {anz}")
        extra.setdefault("other_temporal_orders", []).append(
            {"order": alt, "ms": round(alt_ms, 4), "forward_ms_ratio": round(alt_ms / fwd_ms, 3)})
        del alayer, aout
    # ---- dense comparator: the same kernel, every tile full ----
    if not args.no_dense:
        dmask = [sv.Mask(sv.DENSE, sv.FRAME_MAJOR, 0, 0)] * H
        dense = SparseVideoAttention(g, dmask, D, args.block_q, args.block_k)
        dense.attend(q, k, v, out, scales)
        torch.cuda.synchronize()
        dm = []
        for _ in range(args.dense_steps):
            a, b = ev(), ev()
            a.record(stream)
            dense.attend(q, k, v, out, scales)
            b.record(stream)
            dm.append((a, b))
        torch.cuda.synchronize()
        dense_ms = float(np.mean([a.elapsed_time(b) for a, b in dm]))
        dense_flops = metrics.effective_flops(g, dmask, D)
        extra["dense"] = {"ms": round(dense_ms, 4),
                          "tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 2),
                          "pct_peak": round(100 * dense_flops / (dense_ms * 1e-3) / 1e12 / peak, 2),
                          "sparse_speedup": round(dense_ms / fwd_ms, 3)}
        log(f"dense comparator {dense_ms:.3f} ms -> sparse speedup {dense_ms / fwd_ms:.2f}x")
        del dense
    # ---- naive traversal: every visited tile masked ----
    if not args.no_naive:
        naive = SparseVideoAttention(g, masks, D, args.block_q, args.block_k, map_flags=sv.MAP_ALL_BOUNDARY)
        naive.permute_inputs(q, k, v)
        naive.attend(q, k, v, out, scales)
        torch.cuda.synchronize()
        nm = []
        for _ in range(max(3, args.dense_steps)):
            a, b = ev(), ev()
            a.record(stream)
            naive.attend(q, k, v, out, scales)
            b.record(stream)
            nm.append((a, b))
        torch.cuda.synchronize()
        naive_ms = float(np.mean([a.elapsed_time(b) for a, b in nm]))
        extra["naive_all_boundary"] = {"ms": round(naive_ms, 4), "slowdown_vs_full_boundary": round(naive_ms / fwd_ms, 3)}
        log(f"naive (every tile masked) {naive_ms:.3f} ms")
        del naive

    # ---- the step with the permutation fused into the forward (no separate passes) ----
    if not args.no_fused:
        fused = SparseVideoAttention(g, masks, D, args.block_q, args.block_k, fused=True)
        fused(q, k, v, scales, out=out)
        torch.cuda.synchronize()
        fm = []
        for _ in range(max(3, args.dense_steps)):
            a, b = ev(), ev()
            a.record(stream)
            fused(q, k, v, scales, out=out)
            b.record(stream)
            fm.append((a, b))
        torch.cuda.synchronize()
        fused_ms = float(np.mean([a.elapsed_time(b) for a, b in fm]))
        extra["fused_step"] = {"ms": round(fused_ms, 4), "tflops": round(flops / (fused_ms * 1e-3) / 1e12, 2),
                               "vs_separate_step": round(ms_step / fused_ms, 3)}
        log(f"step with the permutation fused into the forward {fused_ms:.3f} ms")
        del fused

    # ---- SVG head routing on two sampled q-tiles (excluded from the step, as on the pages) ----
    if not args.no_routing:
        sp = next((m for m in masks if m.kind == sv.SPATIAL), sv.Mask(sv.SPATIAL, sv.FRAME_MAJOR, 1, 0))
        tp = next((m for m in masks if m.kind == sv.TEMPORAL), sv.Mask(sv.TEMPORAL, sv.FRAME_MAJOR, 0, 1))
        sp = sv.Mask(sv.SPATIAL, sv.FRAME_MAJOR, sp.window, 0)
        tp = sv.Mask(sv.TEMPORAL, sv.FRAME_MAJOR, 0, tp.radius)
        rmaps = [sv.build_tile_map(g, m, args.block_q, args.block_k)
                 for m in (sv.Mask(sv.DENSE, sv.FRAME_MAJOR, 0, 0), sp, tp)]
        n_full = N // args.block_q
        qts = [n_full // 3, (2 * n_full) // 3]
        scratch = torch.empty(sv.route_scratch_bytes(H, D, args.block_q, len(qts)), dtype=torch.uint8, device=q.device)
        sv.route_heads(g, q, k, v, sp, tp, *rmaps, scales, qts, scratch=scratch)
        torch.cuda.synchronize()
        rm = []
        for _ in range(3):
            a, b = ev(), ev()
            a.record(stream)
            err_r, choice_r = sv.route_heads(g, q, k, v, sp, tp, *rmaps, scales, qts, scratch=scratch)
            b.record(stream)
            rm.append((a, b))
        torch.cuda.synchronize()
        route_ms = float(np.mean([a.elapsed_time(b) for a, b in rm]))
        extra["routing"] = {"ms": round(route_ms, 4), "sampled_qtiles": len(qts),
                            "temporal_heads_chosen": int((choice_r == sv.TEMPORAL).sum().item())}
        log(f"head routing on {len(qts)} q-tiles per head {route_ms:.3f} ms")
        del scratch, rmaps

    # ---- tile-aligned traversal: every non-empty tile full (a different mask) ----
    if not args.no_aligned:
        aligned = SparseVideoAttention(g, masks, D, args.block_q, args.block_k, map_flags=sv.MAP_TILE_ALIGNED)
        aligned.permute_inputs(q, k, v)
        aligned.attend(q, k, v, out, scales)
        torch.cuda.synchronize()
        am = []
        for _ in range(max(3, args.dense_steps)):
            a, b = ev(), ev()
            a.record(stream)
            aligned.attend(q, k, v, out, scales)
            b.record(stream)
            am.append((a, b))
        torch.cuda.synchronize()
        aligned_ms = float(np.mean([a.elapsed_time(b) for a, b in am]))
        # kept pairs of the snapped mask: the in-range area of every listed tile
        pairs = 0
        for mp in aligned.maps:
            nnz = mp.nnz()
            rp = mp.row_ptr.cpu().numpy().astype(np.int64)
            col = mp.col[:nnz].cpu().numpy().astype(np.int64)
            rows = np.minimum(args.block_q, N - np.arange(mp.n_qt) * args.block_q)
            cols = np.minimum(args.block_k, N - col * args.block_k)
            cs = np.concatenate([[0], np.cumsum(cols)])
            pairs += int((cs[rp[1:]] - cs[rp[:-1]]) @ rows)
        extra["tile_aligned"] = {"ms": round(aligned_ms, 4), "kept_pairs": pairs,
                                 "tflops_on_kept": round(4 * D * pairs / (aligned_ms * 1e-3) / 1e12, 2)}
        if "dense" in extra:
            extra["tile_aligned"]["speedup_vs_dense"] = round(extra["dense"]["ms"] / aligned_ms, 3)
        log(f"tile-aligned traversal {aligned_ms:.3f} ms ({pairs} kept pairs)")
        del aligned

    # ---- forward after evicting the caches: a 512 MB write between launches ----
    cold_ms = None
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=q.device)
        cm = []
        for i in range(args.cold_steps):
            flush.fill_(i & 0xff)
            a, b = ev(), ev()
            a.record(stream)
            layer.attend(q, k, v, out, scales)
            b.record(stream)
            cm.append((a, b))
        torch.cuda.synchronize()
        cold_ms = round(float(np.mean([a.elapsed_time(b) for a, b in cm])), 4)
        log(f"forward after a 512 MB cache-evicting write: {cold_ms:.3f} ms")
        del flush

    # ---- graphics clock under load (amd-smi, read while the forward runs back to back) ----
    sclk = None
    if not args.no_clock:
        sclk = clock_under_load(lambda: layer.attend(q, k, v, out, scales))
        log(f"graphics clock under load: {sclk}")

    traffic = measured_traffic(wl.name, args.temporal_order) if args.block_q == 256 and args.block_k == 64 else None
    log(f"traffic per forward launch (committed counters): {traffic}")

    result = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": N, "frames": wl.frames, "grid": [wl.height, wl.width],
                   "heads": H, "head_dim": D, "block_q": args.block_q, "block_k": args.block_k,
                   "spatial_heads": sum(1 for h in wl.heads if h.kind == synth.SPATIAL),
                   "temporal_heads": sum(1 for h in wl.heads if h.kind == synth.TEMPORAL),
                   "temporal_order": args.temporal_order, "kept_fraction": round(kept_frac, 6),
                   "parallelism": "single-gpu"},
        "fwd_kernel": {"ms": round(fwd_ms, 4), "ms_min": round(float(fwd_all.min()), 4),
                       "ms_median": round(float(np.median(fwd_all)), 4),
                       "ms_p90": round(float(np.percentile(fwd_all, 90)), 4),
                       "tflops": round(fwd_tflops, 2), "pct_bf16_peak": round(100 * fwd_tflops / peak, 2),
                       **({"ms_cold_cache": cold_ms} if cold_ms is not None else {})},
        "permute_ms": round(perm_ms, 4),
        "unpermute_ms": round(unperm_ms, 4),
        "classifier_ms": round(min(cls_ms), 4),
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(fwd_tflops / peak, 4),
                     # HBM bytes per forward launch (FETCH_SIZE + WRITE_SIZE, calibrated), or null
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "env": {"rocm": rocm_version(), "device": torch.cuda.get_device_name(0), "sclk_under_load": sclk},
        **extra,
    }
    print(json.dumps(result), flush=True)


def rocm_version():
    try:
        with open("/opt/rocm/.info/version") as f:
            return f.read().strip()
    except OSError:
        return None


AMD_SMI = "/opt/rocm/libexec/amdsmi_cli/amdsmi_cli.py"


def clock_under_load(run, seconds=1.5):
    """Graphics clock (MHz, per XCD) reported by amd-smi while `run` keeps the
    GPU busy.  amd-smi (a Python script) runs in a child interpreter started
    directly, so no launcher re-executes anything, and it only reads the
    driver's clock report.  Skipped under rocprofv3 (its tool library, which
    the child would inherit, sets up the GPU in every process it is loaded
    into) or when amd-smi is not installed."""
    import subprocess
    import threading
    import torch
    if any(k.startswith("ROCPROF") for k in os.environ) or not os.path.exists(AMD_SMI):
        return {"error": "skipped (running under rocprofv3, or amd-smi missing)"}
    found = {}

    def sample():
        time.sleep(0.5)
        try:
            r = subprocess.run([sys.executable, AMD_SMI, "metric", "-c", "--json"], capture_output=True, text=True,
                               timeout=30)
            data = json.loads(r.stdout)
            gpus = data["gpu_data"] if isinstance(data, dict) else data
            found["mhz"] = [[v["clk"]["value"] for k, v in sorted(g["clock"].items()) if k.startswith("gfx_")]
                            for g in gpus]
        except Exception as e:  # amd-smi missing or its output format differs
            found["error"] = f"{type(e).__name__}: {str(e)[:80]}"

    th = threading.Thread(target=sample)
    t_end = time.time() + seconds
    th.start()
    while th.is_alive() or time.time() < t_end:
        run()
        torch.cuda.synchronize()
    th.join()
    if "mhz" not in found:
        return {"error": found.get("error")}
    mhz = found["mhz"][0] if len(found["mhz"]) == 1 else found["mhz"]
    return {"mhz_per_xcd": mhz, "source": "amd-smi metric -c"}


# Inputs of the CPU baseline's worker processes (set before the fork).
_CPU_JOB = {}


def _cpu_worker_init():
    """One BLAS thread per worker process: the sample is spread over processes."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _cpu_task(task):
    """The oracle on one block of query rows of one head; returns (head, rows, seconds)."""
    import oracle
    wl, inp = _CPU_JOB["wl"], _CPU_JOB["inp"]
    h, rows = task
    head = wl.heads[h]
    g = oracle.Geometry(wl.frames, wl.height, wl.width)
    t = time.perf_counter()
    oracle.attend_head(inp.q[h], inp.k[h], inp.v[h], float(inp.scales[h]), g, head.kind, head.window,
                       head.radius, rows=rows)
    return h, rows, time.perf_counter() - t


def _cpu_kept(task):
    """Kept pairs of the query rows of one block (for the FLOP count, untimed)."""
    import oracle
    wl = _CPU_JOB["wl"]
    h, rows = task
    head = wl.heads[h]
    g = oracle.Geometry(wl.frames, wl.height, wl.width)
    return float(oracle.kept_counts_per_row(g, head.kind, head.window, head.radius, rows).sum())


def _cpu_facts():
    """Host CPU model, core counts and the BLAS numpy uses."""
    import numpy as np
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        np.dot(np.ones((64, 64)), np.ones((64, 64)))          # loads the BLAS library
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "blas": blas}


def cpu_baseline(wl, inp, seconds, max_procs=16):
    """The fp64 oracle, as it stands, timed row-parallel on the host cores.

    Worker processes (one per usable core, at most max_procs, one BLAS thread
    each) run the oracle on blocks of seeded query rows, heads in turn, until
    about `seconds` of wall time have passed; the value is the effective
    FLOP of the completed rows (4 d per kept pair) over that wall time.  The
    pool is forked before this process touches the GPU."""
    import multiprocessing as mp
    import svattn_synth as synth
    facts = _cpu_facts()
    procs = max(1, min(max_procs, facts["affinity_cores"]))
    _CPU_JOB.update(wl=wl, inp=inp)
    rows_all = synth.sample_rows(wl, min(wl.n_tokens, 32768))  # seeded, sorted per head; time-bounded below
    block = 64
    tasks = [(h, rows_all[h][i:i + block]) for i in range(0, rows_all.shape[1], block) for h in range(wl.n_heads)]
    done = []
    ctx = mp.get_context("fork")
    with ctx.Pool(procs, initializer=_cpu_worker_init) as pool:
        pool.map(_cpu_task, [(0, rows_all[0][:4])] * procs)   # start-up outside the timed region
        t0 = time.perf_counter()
        it = iter(tasks)
        pending = [pool.apply_async(_cpu_task, (next(it),)) for _ in range(2 * procs)]
        while pending:
            r = pending.pop(0).get()
            done.append(r)
            if time.perf_counter() - t0 < seconds:
                nxt = next(it, None)
                if nxt is not None:
                    pending.append(pool.apply_async(_cpu_task, (nxt,)))
        wall = time.perf_counter() - t0
        kept = pool.map(_cpu_kept, [(h, rows) for h, rows, _ in done])
    flops = 4 * wl.head_dim * float(sum(kept))
    n_rows = sum(len(rows) for _, rows, _ in done)
    full_rows = wl.n_heads * wl.n_tokens
    return {"value": round(flops / wall / 1e12, 6), "unit": "TFLOP/s", "cores": procs, "kind": "oracle",
            "sample": f"{n_rows} seeded query rows ({block}-row blocks, heads in turn) of the {wl.n_tokens}-token "
                      f"x {wl.n_heads}-head workload, fp64 numpy oracle, {procs} processes x 1 BLAS thread, "
                      f"{wall:.1f} s wall",
            "seconds": round(wall, 2), "processes": procs, "blas_threads_per_process": 1, **facts,
            "full_workload_seconds_extrapolated": round(wall * full_rows / max(n_rows, 1), 1)}


if __name__ == "__main__":
    main()
