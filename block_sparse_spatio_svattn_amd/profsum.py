"""Summarise a rocprofv3 kernel trace (``--kernel-trace --output-format csv``).

    python -m block_sparse_spatio_svattn_amd.profsum TRACE.csv [--kernel fwd2_kernel]
        [--skip W] [--flop F] [--bench-line BENCH.json]
    python -m block_sparse_spatio_svattn_amd.profsum --counters COUNTERS.csv [...] [--kernel NAME]

Prints a markdown table of every kernel (calls, mean / median / min / max
duration) and, for the kernel whose name contains ``--kernel``, the same
figures over its dispatches after the first ``--skip`` (the bench's warm-up
calls), so the trace can be checked against the bench line of the same run:
with ``--flop`` (algorithmic FLOP per dispatch) it adds the effective TFLOP/s
and the fraction of the bf16 dense MFMA peak, and with ``--bench-line`` it
prints that line's forward time and roofline fraction beside them.  With
``--counters`` it reads rocprofv3 --pmc counter_collection.csv files instead
and prints each counter's mean per dispatch of the named kernel.
"""
from __future__ import annotations

import argparse
import csv
import json
import statistics
from collections import OrderedDict

BF16_PEAK_TFLOPS = 2500.0  # published dense bf16 MFMA peak of MI355X


def load(path):
    """(kernel name, start ns, end ns) of every dispatch, in dispatch order."""
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    return [(name, s, e) for _, name, s, e in rows]


def stats_us(durs_ns):
    d = [x / 1e3 for x in durs_ns]
    return {"calls": len(d), "mean_us": statistics.fmean(d), "median_us": statistics.median(d),
            "min_us": min(d), "max_us": max(d), "total_us": sum(d)}


def load_counters(path, kernel):
    """{counter: [value per dispatch]} for the dispatches of kernels whose name
    contains `kernel`, from a rocprofv3 --pmc counter_collection.csv."""
    per = OrderedDict()
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"]:
                per.setdefault(r["Counter_Name"], OrderedDict()).setdefault(int(r["Dispatch_Id"]), 0.0)
                per[r["Counter_Name"]][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def counters_main(argv):
    """--counters CSV [CSV ...] --kernel NAME: per-dispatch mean of every
    counter of the named kernel (one JSON object)."""
    ap = argparse.ArgumentParser()
    ap.add_argument("--counters", nargs="+", required=True)
    ap.add_argument("--kernel", default="fwd2_kernel")
    a = ap.parse_args(argv)
    out = {}
    for path in a.counters:
        for name, vals in load_counters(path, a.kernel).items():
            out[name] = {"dispatches": len(vals), "mean": statistics.fmean(vals)}
    print(json.dumps(out, indent=1))


def main(argv=None):
    import sys
    argv = sys.argv[1:] if argv is None else argv
    if argv and argv[0] == "--counters":
        return counters_main(argv)
    ap = argparse.ArgumentParser()
    ap.add_argument("trace")
    ap.add_argument("--kernel", default="fwd2_kernel")
    ap.add_argument("--skip", type=int, default=0, help="leading dispatches of --kernel to leave out (warm-up)")
    ap.add_argument("--flop", type=float, default=None, help="algorithmic FLOP per dispatch of --kernel")
    ap.add_argument("--bench-line", default=None, help="file holding the bench JSON line of the same run")
    a = ap.parse_args(argv)

    disp = load(a.trace)
    per = OrderedDict()
    for name, s, e in disp:
        per.setdefault(name, []).append(e - s)
    total = sum(sum(v) for v in per.values())
    print("| Kernel | Calls | Mean (us) | Median (us) | Min (us) | Max (us) | Share |")
    print("|---|---|---|---|---|---|---|")
    for name, durs in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        st = stats_us(durs)
        print(f"| `{name[:110]}` | {st['calls']} | {st['mean_us']:.1f} | {st['median_us']:.1f} | {st['min_us']:.1f} | "
              f"{st['max_us']:.1f} | {100 * sum(durs) / total:.2f}% |")
    sel = [e - s for name, s, e in disp if a.kernel in name]
    if not sel:
        raise SystemExit(f"no dispatch of a kernel named *{a.kernel}*")
    timed = sel[a.skip:]
    st = stats_us(timed)
    out = {"kernel": a.kernel, "dispatches": len(sel), "skipped": a.skip, **{k: round(v, 2) for k, v in st.items()}}
    if a.flop:
        tf = a.flop / (st["mean_us"] * 1e-6) / 1e12
        out.update(tflops=round(tf, 2), frac=round(tf / BF16_PEAK_TFLOPS, 4))
    if a.bench_line:
        with open(a.bench_line) as f:
            line = next(json.loads(l) for l in f if l.lstrip().startswith("{"))
        out["bench"] = {"fwd_ms": line["fwd_kernel"]["ms"], "ms_per_step": line["ms_per_step"],
                        "roofline_frac": line["roofline"]["frac"]}
        if a.flop:
            out["frac_rel_diff"] = round(out["frac"] / line["roofline"]["frac"] - 1, 4)
    print()
    print("```json")
    print(json.dumps(out, indent=1))
    print("```")


if __name__ == "__main__":
    main()
