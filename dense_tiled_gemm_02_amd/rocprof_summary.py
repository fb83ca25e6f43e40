"""Summarise rocprofv3 CSV output per kernel.

    python -m dense_tiled_gemm_02_amd.rocprof_summary DIR [--match SUBSTR]

DIR holds the CSV files of one or more rocprofv3 runs (kernel_stats,
kernel_trace, counter_collection).  Prints, per kernel name: dispatch count
and average duration from the kernel trace, and the average per dispatch of
every collected counter.  If a copy kernel is present (a torch elementwise
copy), its FETCH_SIZE / WRITE_SIZE per byte copied is printed as the
calibration factor of those counters.
"""
import csv
import glob
import os
import sys
from collections import defaultdict


def _short(name, n=110):
    return name if len(name) <= n else name[:n - 3] + "..."


def summarise(d, match=None):
    out = []
    traces = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    dur = defaultdict(list)
    for t in traces:
        for r in csv.DictReader(open(t)):
            dur[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if dur:
        out.append("kernel trace (%s):" % ", ".join(os.path.relpath(t, d) for t in traces))
        for k, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
            if match and match not in k:
                continue
            v2 = sorted(v)
            out.append("  %-110s n=%4d avg=%9.2f us  min=%9.2f  median=%9.2f  max=%9.2f" % (
                _short(k), len(v), sum(v) / len(v) / 1e3, v2[0] / 1e3, v2[len(v2) // 2] / 1e3, v2[-1] / 1e3))
    ctr = defaultdict(lambda: defaultdict(list))
    for c in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        per = defaultdict(lambda: defaultdict(float))
        for r in csv.DictReader(open(c)):
            key = (r.get("Dispatch_Id"), r["Kernel_Name"])
            per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        for (_, k), cs in per.items():
            for cn, v in cs.items():
                ctr[k][cn].append(v)
    if ctr:
        out.append("counters (average per dispatch):")
        for k, cs in ctr.items():
            if match and match not in k and "copy" not in k.lower():
                continue
            out.append("  " + _short(k))
            for cn, v in sorted(cs.items()):
                out.append("    %-32s %16.1f   (n=%d)" % (cn, sum(v) / len(v), len(v)))
    return "\n".join(out)


if __name__ == "__main__":
    args = sys.argv[1:]
    m = None
    if "--match" in args:
        i = args.index("--match")
        m = args[i + 1]
        del args[i:i + 2]
    print(summarise(args[0], m))
