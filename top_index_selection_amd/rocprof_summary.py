"""Short text summaries of rocprofv3 CSV output, for the files under profiles/.

Two inputs are understood:
  * kernel statistics: ``rocprofv3 --kernel-trace --stats -f csv`` writes
    ``<dir>/<name>_kernel_stats.csv`` (Name, Calls, TotalDurationNs, AverageNs, ...);
  * counter collections: ``rocprofv3 --pmc FETCH_SIZE -f csv`` (and a second run
    with ``WRITE_SIZE``) write ``<dir>/<name>_counter_collection.csv`` with one row
    per (dispatch, counter).

``mfma`` turns one counter run with ``SQ_VALU_MFMA_BUSY_CYCLES``,
``SQ_INSTS_VALU_MFMA_MOPS_BF16`` and ``GRBM_GUI_ACTIVE`` into the fraction of SIMD
cycles the matrix cores were busy during one kernel (the ``MfmaUtil`` formula:
busy cycles summed over the SIMDs / (active cycles of one XCD x SIMD count); the
CSV sums GRBM_GUI_ACTIVE over the XCDs) and the bf16 MFMA work it executed
(512 flop per MOPS unit).

``traffic`` turns the two counter runs into HBM bytes per launch of one kernel.
Each counter is scaled by what it reads for a plain copy kernel of known size
that ran in the same process (``bench.py --copy-probe-mib N`` runs ``torch.neg``
over N MiB of fp32, reading N MiB and writing N MiB): factor = known bytes /
counted bytes, so the counters' units and any systematic over- or under-count
cancel. The record is keyed by the SHA-256 of the kernel's sources, so that
``bench.py`` reports it only while the kernel is unchanged.

Usage:
  python -m top_index_selection_amd.rocprof_summary stats STATS_CSV --title T --command C
  python -m top_index_selection_amd.rocprof_summary traffic --fetch CSV --write CSV \\
      --kernel NAME --workload W --copy-mib N --algorithmic-bytes B --sources F [F ...] \\
      --command C [--json profiles/traffic.json]
  python -m top_index_selection_amd.rocprof_summary mfma COUNTER_CSV --kernel NAME \
      --workload W --sources F [F ...] --command C [--xcds 8] [--simds 1024] \
      [--json profiles/mfma.json]
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")


def sources_sha(names) -> str:
    """SHA-256 (first 16 hex digits) of the named csrc files, in order."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stats_markdown(path: str, title: str, command: str, match: str = "tis::") -> str:
    rows = list(csv.DictReader(open(path)))
    lines = [f"# {title}", "", "Command:", "", "```", command, "```", "",
             "Kernel durations from rocprofv3 kernel statistics (microseconds).", "",
             "| kernel | calls | total us | average us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|---|"]
    other = 0.0
    for r in rows:
        name = r["Name"].strip('"')
        if match not in name:
            other += float(r["TotalDurationNs"]) / 1e3
            continue
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    lines.append(f"| (other kernels: input generation, copies) | | {other:.1f} | | | | |")
    return "\n".join(lines) + "\n"


def per_dispatch(path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter."""
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def _pick(vals, needle):
    hits = {k: v for k, v in vals.items() if needle in k}
    if not hits:
        raise SystemExit(f"no dispatch of a kernel matching {needle!r}")
    if len(hits) > 1:  # the largest instantiation (most work per dispatch)
        k = max(hits, key=lambda k: max(hits[k]))
        return k, hits[k]
    k = next(iter(hits))
    return k, hits[k]


def traffic(fetch_csv, write_csv, kernel, copy_mib, algorithmic_bytes):
    fetch = per_dispatch(fetch_csv, "FETCH_SIZE")
    write = per_dispatch(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib * (1 << 20)
    _, cf = _pick(fetch, "neg")
    _, cw = _pick(write, "neg")
    # the three largest copy dispatches are the probe
    cf = sorted(cf)[-3:]
    cw = sorted(cw)[-3:]
    f_copy = sum(cf) / len(cf) * 1024.0
    w_copy = sum(cw) / len(cw) * 1024.0
    kf_name, kf = _pick(fetch, kernel)
    _, kw = _pick(write, kernel)
    factor_f = copy_bytes / f_copy
    factor_w = copy_bytes / w_copy
    kfetch = sum(kf) / len(kf) * 1024.0 * factor_f
    kwrite = sum(kw) / len(kw) * 1024.0 * factor_w
    return {
        "kernel": kf_name, "dispatches": len(kf),
        "fetch_bytes_per_launch": kfetch, "write_bytes_per_launch": kwrite,
        "hbm_bytes_per_launch": kfetch + kwrite,
        "copy_probe_bytes": copy_bytes,
        "copy_fetch_counted_bytes": f_copy, "copy_write_counted_bytes": w_copy,
        "factor_fetch": factor_f, "factor_write": factor_w,
        "algorithmic_bytes_per_launch": algorithmic_bytes,
        "traffic_over_algorithmic": (kfetch + kwrite) / algorithmic_bytes if algorithmic_bytes else None,
    }


def mfma(path, kernel, xcds, simds):
    """MFMA busy fraction and executed bf16 MFMA work per launch of the kernel
    whose name contains `kernel` (the instantiation with the most MFMA work if
    several match), from one counter run."""
    per = defaultdict(dict)  # (name, dispatch) -> {counter: value, "ns": duration}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        if kernel not in name:
            continue
        d = per[(name, r["Dispatch_Id"])]
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    if not per:
        raise SystemExit(f"no dispatch of a kernel matching {kernel!r}")
    names = defaultdict(list)
    for (name, _), d in per.items():
        names[name].append(d)
    name = max(names, key=lambda n: sum(d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for d in names[n]))
    ds = names[name]
    mean = lambda k: sum(d[k] for d in ds) / len(ds)
    busy, gui = mean("SQ_VALU_MFMA_BUSY_CYCLES"), mean("GRBM_GUI_ACTIVE") / xcds
    flop = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512.0
    ns = mean("ns")
    return {"kernel": name, "dispatches": len(ds), "mfma_busy_cycles": busy,
            "gui_active_cycles_per_xcd": gui, "simds": simds, "xcds": xcds,
            "mfma_busy_frac": busy / (gui * simds) if gui else None,
            "mfma_bf16_flop_per_launch": flop, "avg_duration_us_profiled": ns / 1e3,
            "executed_tflops_profiled": flop / ns / 1e3 if ns else None}


def _store(path, workload, key, rec):
    data = {}
    if os.path.exists(path):
        data = json.load(open(path))
    data.setdefault(workload, {})[key] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--algorithmic-bytes", type=float, required=True)
    t.add_argument("--sources", nargs="+", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--json")
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    m.add_argument("--kernel", required=True)
    m.add_argument("--workload", required=True)
    m.add_argument("--sources", nargs="+", required=True)
    m.add_argument("--command", required=True)
    m.add_argument("--xcds", type=int, default=8)
    m.add_argument("--simds", type=int, default=1024)
    m.add_argument("--json")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        sys.stdout.write(stats_markdown(a.csv, a.title, a.command))
        return
    if a.cmd == "mfma":
        rec = mfma(a.csv, a.kernel, a.xcds, a.simds)
        rec.update({"sources": a.sources, "source_sha": sources_sha(a.sources), "command": a.command})
        print(json.dumps(rec, indent=1))
        if a.json:
            _store(a.json, a.workload, a.kernel, rec)
        return
    rec = traffic(a.fetch, a.write, a.kernel, a.copy_mib, a.algorithmic_bytes)
    rec.update({"sources": a.sources, "source_sha": sources_sha(a.sources), "command": a.command})
    print(json.dumps(rec, indent=1))
    if a.json:
        _store(a.json, a.workload, a.kernel, rec)


if __name__ == "__main__":
    main()
