"""Condense rocprofv3 CSV output into the short text summaries kept with the
benchmarks.

Two inputs are understood:

* ``--stats DIR``: the ``*_kernel_stats.csv`` of a ``rocprofv3 --kernel-trace
  --stats --output-format csv`` run; prints per-kernel calls and durations.
* ``--trace DIR --kernel SUBSTR --skip A --count B``: from the
  ``*_kernel_trace.csv`` of the same run, the durations of dispatches A .. A+B-1
  (in dispatch order) of the kernels whose name contains SUBSTR: the timed
  launches of one workload when several workloads share a kernel instance.
* ``--pmc DIR``: the ``*counter_collection.csv`` of a ``rocprofv3 --pmc
  FETCH_SIZE`` (or ``WRITE_SIZE``) run of ``bench.py --calib-probe MIB``;
  prints the counter per dispatch of the attention kernel and of the probe
  that calibrates it (a read-only sum for FETCH_SIZE, a write-only fill for
  WRITE_SIZE), the probe's scale factor (counter / known bytes) and the
  attention kernel's scaled bytes per launch.

``kernel_source_hash()`` is the SHA-256 of the sources that decide what the
forward kernel reads and writes; a traffic figure is only reported for the
hash it was measured with.
"""

import argparse
import collections
import csv
import glob
import hashlib
import os
import re
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("csrc/fwd_kernel.h", "csrc/plan.h", "csrc/plan.cpp", "csrc/device_index.h")
FWD_KERNEL = "rpe_fwd_kernel"


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()[:16]


_FWD = re.compile(r"_ZN3rpe14rpe_fwd_kernelI(DF16b|f)Li(\d+)ELi(\d)ELj(\d)ELb(\d)ELb(\d)ELi(\d)EEEvNS_6ParamsE")
_MODES = {"0": "none", "1": "bias", "2": "contextual"}
_MAPS = {"0": "", "1": ", Cross", "2": ", undirected"}


def fwd_name(name):
    """Readable name of a forward-kernel instance, or None."""
    m = _FWD.search(name)
    if not m:
        return None
    dt, d, mode, terms, wide, multi, mk = m.groups()
    t = "".join(c for bit, c in ((1, "K"), (2, "Q"), (4, "V")) if int(terms) & bit)
    # the fifth flag: several units per workgroup, or (with wide rows) rows of
    # more than 64 key slots
    rows = {("1", "0"): ", 64-slot rows", ("1", "1"): ", rows over 64 slots"}.get((wide, multi), "")
    return (f"rpe_fwd_kernel<{'bf16' if dt == 'DF16b' else 'fp32'}, d{d}, {_MODES[mode]}"
            f"{' ' + t if t else ''}{rows}"
            f"{', several units per workgroup' if multi == '1' and wide == '0' else ''}{_MAPS[mk]}>")


def demangle(names):
    own = [fwd_name(n) for n in names]
    if all(own):
        return own
    try:
        r = subprocess.run(["c++filt"], input="\n".join(names), stdout=subprocess.PIPE, text=True, timeout=10)
        out = r.stdout.splitlines()
        if len(out) == len(names):
            return [o if f is None else f for o, f in zip(out, own)]
    except Exception:
        pass
    return [n if f is None else f for n, f in zip(names, own)]


def _one(pattern, d):
    files = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not files:
        raise SystemExit(f"no {pattern} under {d}")
    return files[0]


def stats_summary(d):
    rows = list(csv.DictReader(open(_one("*kernel_stats.csv", d))))
    names = demangle([r["Name"] for r in rows])
    lines = [f"{'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_%':>8}  kernel"]
    for r, n in zip(rows, names):
        if len(n) > 110:
            n = n[:107] + "..."
        lines.append(f"{int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):8.2f}  {n}")
    return "\n".join(lines)


def trace_summary(d, substr, skip, count):
    rows = [r for r in csv.DictReader(open(_one("*kernel_trace.csv", d))) if substr in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    sel = rows[skip:skip + count]
    if len(sel) < count:
        raise SystemExit(f"only {len(rows)} dispatches of {substr}")
    us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel]
    name = demangle([sel[0]["Kernel_Name"]])[0]
    return (f"{name}: dispatches {skip}..{skip + count - 1} of {len(rows)} (dispatch order): "
            f"avg {sum(us) / len(us):.2f} us, min {min(us):.2f}, max {max(us):.2f}")


def pmc_summary(d, probe_mib):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE of the forward kernel, scaled by what the
    same counter reads for the calibration probes that ran after it (``bench.py
    --calib-probe MIB``): a sum that reads MIB MiB (FETCH_SIZE) and a fill that
    writes MIB MiB (WRITE_SIZE)."""
    rows = list(csv.DictReader(open(_one("*counter_collection.csv", d))))
    by = collections.defaultdict(lambda: collections.defaultdict(list))
    last_fwd = max((int(r["Dispatch_Id"]) for r in rows if FWD_KERNEL in r["Kernel_Name"]), default=-1)
    counters = sorted({r["Counter_Name"] for r in rows})
    for r in rows:
        name = r["Kernel_Name"]
        after = int(r["Dispatch_Id"]) > last_fwd
        if FWD_KERNEL in name:
            key = demangle([name])[0]
        elif after and "reduce_kernel" in name:
            key = "read probe"
        elif after and "FillFunctor" in name:
            key = "write probe"
        else:
            continue
        by[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = []
    probe_bytes = probe_mib * (1 << 20)
    probe_of = {"FETCH_SIZE": "read probe", "WRITE_SIZE": "write probe"}
    for c in counters:
        probe = probe_of.get(c)
        vals = by.get(probe, {}).get(c, []) if probe else []
        factor = None
        if len(vals) >= 3:
            # the three passes are the three largest dispatches of the probe kernel
            # (other sums and fills after the last forward launch, such as the
            # finite check's reductions or the probe buffer's allocation, are
            # smaller or not counted by this counter)
            top = sorted(vals)[-3:]
            per_pass = sum(top) / 3.0
            factor = per_pass * 1024.0 / probe_bytes
            out.append(f"{probe} ({probe_mib} MiB {'read' if probe == 'read probe' else 'written'} per pass, "
                       f"3 passes = the 3 largest of {len(vals)} dispatches, {min(top):.1f} .. {max(top):.1f} KiB): "
                       f"{c} {per_pass:.1f} KiB per pass; factor = {factor:.4f} (counter / known bytes)")
        for k, cs in by.items():
            if k in ("read probe", "write probe") or c not in cs:
                continue
            v = cs[c]
            mean_kib = sum(v) / len(v)
            scaled = mean_kib * 1024.0 / factor if factor else float("nan")
            out.append(f"{k}: {c} mean {mean_kib:.1f} KiB over {len(v)} dispatches "
                       f"(min {min(v):.1f}, max {max(v):.1f}); scaled bytes per launch {scaled:.0f}")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stats")
    ap.add_argument("--pmc")
    ap.add_argument("--trace")
    ap.add_argument("--kernel", default=FWD_KERNEL)
    ap.add_argument("--skip", type=int, default=0)
    ap.add_argument("--count", type=int, default=1)
    ap.add_argument("--probe-mib", type=int, default=256)
    ap.add_argument("--hash", action="store_true", help="print the forward kernel's source hash")
    a = ap.parse_args()
    if a.hash:
        print(kernel_source_hash())
    if a.stats:
        print(stats_summary(a.stats))
    if a.trace:
        print(trace_summary(a.trace, a.kernel, a.skip, a.count))
    if a.pmc:
        print(pmc_summary(a.pmc, a.probe_mib))


if __name__ == "__main__":
    main()
