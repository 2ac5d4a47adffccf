"""Summaries of rocprofv3 CSV output (kernel statistics and FETCH_SIZE / WRITE_SIZE counters)
for the profiles/ folder.

HBM bytes of a kernel are taken from the TCC counters FETCH_SIZE and WRITE_SIZE (KiB per
dispatch), each scaled by the ratio between the known byte count of a plain device copy and
what the same counter reads for that copy in the same run.

usage:
  python -m molecular_dynamics_hilbert_amd.profiling stats <run_kernel_stats.csv>
  python -m molecular_dynamics_hilbert_amd.profiling traffic <fetch.csv> <write.csv> <kernel>
         <copy_MiB> <out.json>
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def short_name(name: str) -> str:
    n = re.sub(r"\(anonymous namespace\)::", "", name)
    n = re.sub(r"^void ", "", n)
    n = n.split("(")[0]
    return n.replace("tess::", "")


def kernel_stats_md(path: str, top: int = 20) -> str:
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["| kernel | calls | avg us | min us | max us | share % |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows[:top]:
        out.append("| %s | %s | %.1f | %.1f | %.1f | %.2f |" % (
            short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(out)


def _counter_rows(path: str, counter: str):
    return [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]


def _per_dispatch(rows):
    """Counter values summed per dispatch (a counter may be reported per XCD/instance)."""
    acc = {}
    for r in rows:
        k = (r["Dispatch_Id"], r["Kernel_Name"])
        acc[k] = acc.get(k, 0.0) + float(r["Counter_Value"])
    return acc


def traffic(fetch_csv: str, write_csv: str, kernel: str, copy_mib: int) -> dict:
    """Bytes per launch of `kernel` (regular expression searched in the demangled name),
    scaled by the copy."""
    res = {}
    for label, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        d = _per_dispatch(_counter_rows(path, counter))
        copies = [v for (i, n), v in d.items() if "copyBuffer" in n or "copy" in n.lower()]
        copy_kib = max(copies) if copies else None
        scale = (copy_mib * 1024.0) / copy_kib if copy_kib else 1.0
        vals = [v for (i, n), v in d.items() if re.search(kernel, n)]
        res[label] = {"kib_per_launch_raw": sum(vals) / max(len(vals), 1), "launches": len(vals),
                      "copy_kib_raw": copy_kib, "copy_scale": scale,
                      "bytes_per_launch": 1024.0 * scale * sum(vals) / max(len(vals), 1)}
    res["kernel"] = kernel
    res["bytes_per_launch"] = res["fetch"]["bytes_per_launch"] + res["write"]["bytes_per_launch"]
    return res


# Sources of the energy/forces kernels (the edge kernels and GEMMs whose counters the traffic
# summaries hold): a change to the rebuild or API sources leaves those counters valid.
EF_SOURCES = ("model.hip", "tess_common.h")
NBR_SOURCES = ("nbr.hip", "tess_common.h")  # the rebuild kernels


def source_digest(files=None) -> str:
    """sha256 over csrc/ (or over the named files of csrc/, in sorted order)."""
    h = hashlib.sha256()
    names = sorted(files) if files else sorted(os.listdir(os.path.join(HERE, "csrc")))
    for f in names:
        with open(os.path.join(HERE, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def write_summaries(stats_csv: str, fetch_csv: str, write_csv: str, kernel_key: str,
                    kernel_name: str, workload: str, copy_mib: int, commands: list,
                    out_dir: str) -> None:
    """profiles/<kernel>_<workload>.md (kernel statistics + counter traffic) and
    profiles/traffic_<kernel>_<workload>.json (bytes per launch, source digest)."""
    t = traffic(fetch_csv, write_csv, kernel_name, copy_mib)
    t["source_files"] = list(EF_SOURCES)
    t["source_digest"] = source_digest(EF_SOURCES)
    t["workload"] = workload
    with open(os.path.join(out_dir, "traffic_%s_%s.json" % (kernel_key, workload)), "w") as f:
        json.dump(t, f, indent=1)
    md = ["# %s at %s: rocprofv3 summary" % (kernel_key, workload), "",
          "Commands (run from the repository root):", ""]
    md += ["    " + c for c in commands]
    md += ["", "## Kernel statistics (--kernel-trace --stats)", "", kernel_stats_md(stats_csv), "",
           "## HBM traffic of %s (FETCH_SIZE / WRITE_SIZE, copy-calibrated)" % kernel_key, "",
           "| counter | raw KiB/launch | copy raw KiB (%d MiB copy) | scale | bytes/launch |" % copy_mib,
           "|---|---:|---:|---:|---:|"]
    for lab, cnt in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        r = t[lab]
        md.append("| %s | %.1f | %.1f | %.4f | %.4g |" % (cnt, r["kib_per_launch_raw"],
                                                        r["copy_kib_raw"] or 0, r["copy_scale"],
                                                        r["bytes_per_launch"]))
    rows = [r for r in csv.DictReader(open(stats_csv)) if re.search(kernel_name, r["Name"])]
    calls = sum(int(r["Calls"]) for r in rows)
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    md += ["", "All launches matching `%s` (every layer): %d calls, average %.1f us." % (
        kernel_name, calls, tot / max(calls, 1) / 1e3)]
    md += ["", "Launches counted: %d. Source digest (%s): %s." % (
        t["fetch"]["launches"], ", ".join(t["source_files"]), t["source_digest"])]
    with open(os.path.join(out_dir, "%s_%s.md" % (kernel_key, workload)), "w") as f:
        f.write("\n".join(md) + "\n")


REBUILD_KERNELS = ("k_wrap_key", "k_radix_hist", "k_radix_scatter", "k_scan_one", "k_scan_partial",
                   "k_scan_sums", "k_scan_final", "k_permute", "k_cell_fill", "k_cell_pairs",
                   "k_rev", "k_rev_grouped")


def rebuild_md(stats_csv: str, workload: str, command: str, calls_per_rebuild: dict = None) -> str:
    """Kernel statistics of the neighbour-rebuild kernels alone."""
    rows = [r for r in csv.DictReader(open(stats_csv))
            if short_name(r["Name"]).split("<")[0] in REBUILD_KERNELS]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["# Neighbour rebuild at %s: rocprofv3 kernel statistics" % workload, "",
           "Command (run from the repository root):", "", "    " + command, "",
           "| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        out.append("| %s | %s | %.1f | %.1f | %.1f |" % (
            short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    out += ["", "Source digest (%s): %s." % (", ".join(NBR_SOURCES), source_digest(NBR_SOURCES))]
    return "\n".join(out) + "\n"


def main(argv):
    if argv[0] == "rebuild":
        # rebuild <stats_csv> <workload> <out_md> <command...>
        md = rebuild_md(argv[1], argv[2], " ".join(argv[4:]))
        with open(argv[3], "w") as f:
            f.write(md)
        print(md)
    elif argv[0] == "stats":
        print(kernel_stats_md(argv[1]))
    elif argv[0] == "summarize":
        # summarize <prof_dir> <pmc_fetch_dir> <pmc_write_dir> <kernel_key> <kernel_name> <workload> <copy_mib>
        d, f, w, key, name, wl, mib = argv[1:8]
        cmds = ["rocprofv3 --kernel-trace --stats -f csv -d %s -o run -- python bench.py --steps 20 "
                "--warmup 20 --no-cpu-baseline --no-large" % d,
                "rocprofv3 --pmc FETCH_SIZE -f csv -d %s -o run -- python bench.py --steps 1 "
                "--warmup 1 --no-cpu-baseline --no-large --copy-calibration-mib %s" % (f, mib),
                "rocprofv3 --pmc WRITE_SIZE -f csv -d %s -o run -- python bench.py --steps 1 "
                "--warmup 1 --no-cpu-baseline --no-large --copy-calibration-mib %s" % (w, mib)]
        write_summaries(os.path.join(d, "run_kernel_stats.csv"),
                        os.path.join(f, "run_counter_collection.csv"),
                        os.path.join(w, "run_counter_collection.csv"), key, name, wl, int(mib),
                        cmds, os.path.join(os.path.dirname(HERE), "profiles"))
    elif argv[0] == "traffic":
        t = traffic(argv[1], argv[2], argv[3], int(argv[4]))
        t["source_files"] = list(EF_SOURCES)
        t["source_digest"] = source_digest(EF_SOURCES)
        with open(argv[5], "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t, indent=1))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
