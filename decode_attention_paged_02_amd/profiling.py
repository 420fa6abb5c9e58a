"""Summaries of rocprofv3 output for the profiles/ directory.

    python -m decode_attention_paged_02_amd.profiling stats  DIR [--match SUBSTR]
    python -m decode_attention_paged_02_amd.profiling counters DIR [--match SUBSTR]
    python -m decode_attention_paged_02_amd.profiling summary trace|counters DIR \
        --workload NAME --command "ROCPROF COMMAND" --out FILE
    python -m decode_attention_paged_02_amd.profiling traffic --workload NAME \\
        --fetch DIR --write DIR --kernel SUBSTR --bytes-per-launch N --copy-kernel SUBSTR

`stats` prints the kernel-time table of a `rocprofv3 --kernel-trace --stats`
run, `counters` the mean per-dispatch value of each counter of a `--pmc` run;
`summary` writes either table with a header that records the commands and the
digest of the kernel sources (the files kept under profiles/).  `traffic` reads two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE`
runs (KiB per dispatch) and calibrates each counter against the plain device
copy that bench.py's bandwidth probe performs in the same process: a copy of
known size must read and write exactly its buffer, so factor = known bytes /
counted bytes.  The result (bytes per launch of the kernel, calibrated) is
written to profiles/traffic_<workload>.json together with a digest of the
kernel sources, so bench.py reports it only while the kernels are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_paged_02_amd", "csrc")


# The sources a kernel is built and launched from: its own file, the shared
# device and argument headers, and the host code that plans and launches it.
_COMMON = ["pda_device.h", "pda_internal.h", "pda_host.cpp"]
KERNEL_SOURCES = {"gqa_mfma_kernel": ["pda_gqa_mfma.hip"] + _COMMON,
                  "gqa_split_kernel": ["pda_gqa.hip"] + _COMMON,
                  "mla_mfma_kernel": ["pda_mla.hip"] + _COMMON}


def source_digest(kernel: str = None) -> str:
    """Digest of the HIP/C++ sources the counters were taken on: those of
    `kernel` (KERNEL_SOURCES), or every source when it is None."""
    h = hashlib.sha256()
    files = KERNEL_SOURCES[kernel] if kernel else sorted(
        f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".h")))
    for f in files:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def _find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, d))
    return hits[0]


def kernel_stats(d):
    """Rows of the kernel_stats.csv of a --kernel-trace --stats run."""
    with open(_find(d, "kernel_stats.csv")) as f:
        return list(csv.DictReader(f))


def short_name(name: str) -> str:
    name = name.replace("pda::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    return name if len(name) < 110 else name[:107] + "..."


def stats_text(d, match=""):
    rows = [r for r in kernel_stats(d) if match in r["Name"]]
    out = ["%-8s %12s %12s %12s  %s" % ("calls", "avg_us", "min_us", "max_us", "kernel")]
    for r in rows:
        out.append("%-8s %12.3f %12.3f %12.3f  %s" % (
            r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, short_name(r["Name"])))
    return "\n".join(out)


def counter_values(d):
    """{kernel name: {counter: [value per dispatch]}} of a --pmc run."""
    res = defaultdict(lambda: defaultdict(list))
    with open(_find(d, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            res[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return res


def _pick(vals, substr):
    names = [k for k in vals if substr in k]
    if not names:
        raise KeyError("no kernel matching %r" % substr)
    return names[0]


def traffic(fetch_dir, write_dir, kernel, copy_kernel, copy_bytes):
    """Calibrated HBM bytes per dispatch of `kernel`.

    The copy kernel's dispatches of exactly `copy_bytes` each (the largest
    dispatches recorded for it) give the calibration of each counter."""
    fv, wv = counter_values(fetch_dir), counter_values(write_dir)
    k = _pick(fv, kernel)
    c = _pick(fv, copy_kernel)
    f_kib = statistics.mean(fv[k]["FETCH_SIZE"])
    w_kib = statistics.mean(wv[_pick(wv, kernel)]["WRITE_SIZE"])
    cf = max(fv[c]["FETCH_SIZE"])
    cw = max(wv[_pick(wv, copy_kernel)]["WRITE_SIZE"])
    f_fac = copy_bytes / (cf * 1024.0)
    w_fac = copy_bytes / (cw * 1024.0)
    return {
        "kernel": short_name(k),
        "dispatches": len(fv[k]["FETCH_SIZE"]),
        "fetch_kib_raw": f_kib, "write_kib_raw": w_kib,
        "copy_fetch_kib_raw": cf, "copy_write_kib_raw": cw, "copy_bytes": copy_bytes,
        "fetch_factor": f_fac, "write_factor": w_fac,
        "fetch_bytes": f_kib * 1024.0 * f_fac, "write_bytes": w_kib * 1024.0 * w_fac,
    }


def counters_text(d, match):
    """Mean value per dispatch of every counter of the kernels matching `match`."""
    vals = counter_values(d)
    out = []
    for k in vals:
        if match not in k:
            continue
        out.append("kernel: %s  (%d dispatches)" % (short_name(k),
                                                    len(next(iter(vals[k].values())))))
        for c in sorted(vals[k]):
            out.append("  %-28s %18.1f" % (c, statistics.mean(vals[k][c])))
    return "\n".join(out)


def summary_text(kind, d, workload, command, match="pda"):
    """A profiles/ summary: header (commands, source digest) + the table."""
    if kind == "trace":
        title = "rocprofv3 kernel trace, workload %s (bench.py; rotating KV pools)" % workload
        table = stats_text(d, match)
        tool = "stats"
    else:
        title = "rocprofv3 counters, workload %s" % workload
        table = counters_text(d, match)
        tool = "counters"
    head = ["# " + title,
            "# commands (GPU host, repository root as R; run from /tmp):",
            "#   " + command,
            "#   python -m decode_attention_paged_02_amd.profiling %s OUT" % tool,
            "# source digest " + source_digest()]
    if kind != "trace":
        head.append("# counters are summed over the GPU's XCDs/SEs as rocprofv3 reports them")
    return "\n".join(head) + "\n" + table + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--match", default="")
    cn = sub.add_parser("counters")
    cn.add_argument("dir")
    cn.add_argument("--match", default="")
    sm = sub.add_parser("summary")
    sm.add_argument("kind", choices=["trace", "counters"])
    sm.add_argument("dir")
    sm.add_argument("--workload", required=True)
    sm.add_argument("--command", required=True)
    sm.add_argument("--match", default="pda")
    sm.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--workload", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-kernel", default="copyBuffer")
    t.add_argument("--copy-bytes", type=int, default=2 << 30)
    t.add_argument("--bytes-per-launch", type=int, required=True,
                   help="algorithmic bytes one launch must read")
    t.add_argument("--command", default="", help="the rocprofv3 command lines, for the record")
    t.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats_text(a.dir, a.match))
        return
    if a.cmd == "counters":
        print(counters_text(a.dir, a.match))
        return
    if a.cmd == "summary":
        txt = summary_text(a.kind, a.dir, a.workload, a.command, a.match)
        with open(a.out, "w") as f:
            f.write(txt)
        print(txt)
        return
    r = traffic(a.fetch, a.write, a.kernel, a.copy_kernel, a.copy_bytes)
    r.update({"workload": a.workload, "source_digest": source_digest(a.kernel),
              "source_files": KERNEL_SOURCES[a.kernel],
              "algorithmic_bytes_per_launch": a.bytes_per_launch,
              "fetch_over_algorithmic": r["fetch_bytes"] / a.bytes_per_launch,
              "bytes_per_launch": round(r["fetch_bytes"] + r["write_bytes"]),
              "command": a.command})
    out = a.out or os.path.join(ROOT, "profiles", "traffic_%s.json" % a.workload)
    with open(out, "w") as f:
        json.dump(r, f, indent=1)
    print(json.dumps(r, indent=1))


if __name__ == "__main__":
    main(sys.argv[1:])
