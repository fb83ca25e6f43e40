"""Summarise rocprofv3 CSV output per kernel.

    python -m dense_tiled_gemm_02_amd.rocprof_summary DIR [--match SUBSTR]
    python -m dense_tiled_gemm_02_amd.rocprof_summary --traffic FETCH_DIR WRITE_DIR COPY_BYTES OUT.json
    python -m dense_tiled_gemm_02_amd.rocprof_summary --report OUT MATCH "WORKLOAD" "WORK" COPY_BYTES
    python -m dense_tiled_gemm_02_amd.rocprof_summary --report-mx OUT MATCH "WORKLOAD" "WORK" COPY_BYTES
    python -m dense_tiled_gemm_02_amd.rocprof_summary --report-cmd OUT PREFIX "BENCH" MATCH "WORKLOAD" "WORK" COPY_BYTES TRAFFIC

--report composes the per-kernel summary kept under profiles/ from the five
passes OUT/prof_{trace,fetch,write,mfma,lds} that profile_commands() lists,
for the kernels whose name contains MATCH; --report-mx does the same from the
OUT/mxprof_* passes of bench.py --mx.

DIR holds the CSV files of one or more rocprofv3 runs (kernel_stats,
kernel_trace, counter_collection).  Prints, per kernel name: dispatch count
and average duration from the kernel trace, and the average per dispatch of
every collected counter.  If a copy kernel is present (a torch elementwise
copy), its FETCH_SIZE / WRITE_SIZE per byte copied is printed as the
calibration factor of those counters.
"""
import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def source_hash():
    """sha256 over the device-code sources (kernels and the headers they
    include; not the host-side planner); measured counters are valid only for it."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if f.endswith((".hip", ".h")):
            h.update(os.path.basename(f).encode())
            h.update(open(f, "rb").read())
    return h.hexdigest()


def counter_dispatches(d, name):
    """{kernel name: {dispatch id: counter `name`}} from a --pmc run."""
    per = defaultdict(lambda: defaultdict(float))
    for c in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(c)):
            if r["Counter_Name"] == name:
                per[r["Kernel_Name"]][r.get("Dispatch_Id")] += float(r["Counter_Value"])
    return per


def counter_means(d, name):
    """{kernel name: mean per dispatch of counter `name`} from a --pmc run."""
    return {k: sum(v.values()) / len(v) for k, v in counter_dispatches(d, name).items()}


def _largest_copy(d, name):
    """The counter of the largest copy dispatch (the calibration copy; the runs
    also hold small host-to-device copies of the inputs)."""
    vals = [x for k, v in counter_dispatches(d, name).items() if "copy" in k.lower() for x in v.values()]
    return max(vals) if vals else None


def traffic(fetch_dir, write_dir, copy_bytes):
    """Bytes per launch between the L2s and the memory fabric (MALL hits
    included) of every kernel: FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled so that the copy kernel of copy_bytes reads and writes exactly
    copy_bytes."""
    fetch = counter_means(fetch_dir, "FETCH_SIZE")
    write = counter_means(write_dir, "WRITE_SIZE")
    copy_f = _largest_copy(fetch_dir, "FETCH_SIZE")
    copy_w = _largest_copy(write_dir, "WRITE_SIZE")
    if not copy_f or not copy_w:
        raise SystemExit("no copy kernel in the counter runs")
    ff = copy_bytes / (copy_f * 1024.0)
    fw = copy_bytes / (copy_w * 1024.0)
    out = {"source_sha256": source_hash(), "copy_bytes": copy_bytes,
           "fetch_scale": ff, "write_scale": fw, "kernels": {}}
    for k in fetch:
        if "copy" in k.lower() or k not in write:
            continue
        out["kernels"][k] = {"fetch_kib": fetch[k], "write_kib": write[k],
                             "bytes": fetch[k] * 1024.0 * ff + write[k] * 1024.0 * fw}
    return out


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


BENCH = "python3 bench.py --steps 100 --warmup 10 --no-cpu --copy-mb 512"
BENCH_MX = "python3 bench.py --mx --rounds 3 --copy-mb 512"
PASSES = [("trace", "--kernel-trace --stats", "gemm"),
          ("fetch", "--kernel-trace --pmc FETCH_SIZE", "p"),
          ("write", "--kernel-trace --pmc WRITE_SIZE", "p"),
          ("mfma", "--kernel-trace --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_MFMA GRBM_GUI_ACTIVE", "p"),
          ("lds", "--kernel-trace --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS", "p")]
TITLES = {"trace": "kernel trace (rocprofv3 --kernel-trace --stats)", "fetch": "FETCH_SIZE pass",
          "write": "WRITE_SIZE pass", "mfma": "MFMA / clock pass", "lds": "LDS pass"}


def profile_commands(out="OUT", bench=BENCH, prefix="prof_"):
    """The rocprofv3 runs behind a committed profile summary (one counter set per run)."""
    return ["rocprofv3 %s -f csv -d %s/%s%s -o %s -- %s" % (flags, out, prefix, name, o, bench)
            for name, flags, o in PASSES]


def report(out, match, workload, work, copy_bytes, mx=False, bench=None, prefix=None, traffic_file=None):
    """Text summary of one kernel over the five passes under `out` (the
    prof_* passes of the default benchmark, the mxprof_* passes of
    bench.py --mx with mx=True, or the passes `prefix`* of another bench.py
    command `bench`)."""
    custom = bench is not None
    prefix = prefix or ("mxprof_" if mx else "prof_")
    bench = bench or (BENCH_MX if mx else BENCH)
    lines = []
    names = set()
    for name, _, _ in PASSES:
        for t in glob.glob(os.path.join(out, prefix + name, "**", "*kernel_trace.csv"), recursive=True):
            for r in csv.DictReader(open(t)):
                if match in r["Kernel_Name"]:
                    names.add(r["Kernel_Name"])
    kname = sorted(names)[0] if names else match
    short = kname.split("namespace)::")[-1].split("(dtg::")[0]
    lines.append("Kernel:   " + short)
    lines.append("Workload: " + workload)
    lines.append("Algorithmic work per launch: " + work)
    lines.append("")
    lines.append("Commands (run from the repository root on one MI355X, after")
    if custom:
        lines.append('"python -m dense_tiled_gemm_02_amd.build"; the bench.py command runs the workload named')
        lines.append("above and ends with one 512 MiB device")
    elif mx:
        lines.append('"python -m dense_tiled_gemm_02_amd.build"; bench.py --mx runs the five block-scaled')
        lines.append("workloads (FP4 16x8192x8192; FP4, E4M3, FP6 E2M3 and E4M3 x FP4 at 4096^3) and ends with one")
        lines.append("512 MiB device")
    else:
        lines.append('"python -m dense_tiled_gemm_02_amd.build"; bench.py runs the bf16 4096^3 and the')
        lines.append("skinny bf16 16x8192x8192 workloads back to back and ends with one 512 MiB device")
    lines.append("copy used to calibrate the memory counters):")
    for c in profile_commands(bench=bench, prefix=prefix):
        lines.append("  " + c)
    lines.append("  python3 -m dense_tiled_gemm_02_amd.rocprof_summary --traffic OUT/%sfetch OUT/%swrite "
                 "%d profiles/%s" % (prefix, prefix, copy_bytes,
                                     traffic_file or ("traffic_mx.json" if mx else "traffic.json")))
    if custom:
        lines.append('  python3 -m dense_tiled_gemm_02_amd.rocprof_summary --report-cmd OUT %s "%s" "%s" ...   '
                     '(this file)' % (prefix, bench, match))
    else:
        lines.append('  python3 -m dense_tiled_gemm_02_amd.rocprof_summary --report%s OUT "%s" ...   (this file)' % (
            "-mx" if mx else "", match))
    for name, _, _ in PASSES:
        lines.append("")
        lines.append("--- %s ---" % TITLES[name])
        body = summarise(os.path.join(out, prefix + name), match)
        under = False
        for l in body.splitlines():
            if l.startswith("    "):
                if under:
                    lines.append("  " + l.strip())
            elif l.startswith("  "):
                under = match in l
                if under:
                    lines.append(l.strip())
        if name == "write":
            t = traffic(os.path.join(out, prefix + "fetch"), os.path.join(out, prefix + "write"), copy_bytes)
            for k, v in t["kernels"].items():
                if match in k:
                    lines.append("Calibration: the %d MiB copy kernel sets FETCH_SIZE x %.4f and WRITE_SIZE x %.4f,"
                                 % (copy_bytes >> 20, t["fetch_scale"], t["write_scale"]))
                    lines.append("so L2-to-fabric traffic per launch (MALL hits included) = %.1f KiB x %.4f + %.1f KiB x %.4f = %.1f MB" % (
                        v["fetch_kib"], t["fetch_scale"], v["write_kib"], t["write_scale"], v["bytes"] / 1e6))
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    args = sys.argv[1:]
    if args and args[0] == "--traffic":
        t = traffic(args[1], args[2], int(args[3]))
        with open(args[4], "w") as f:
            json.dump(t, f, indent=1)
        for k, v in t["kernels"].items():
            print("%-100s fetch %10.1f KiB  write %10.1f KiB  -> %.1f MB per launch" % (
                _short(k, 100), v["fetch_kib"], v["write_kib"], v["bytes"] / 1e6))
        print("scales: fetch %.4f  write %.4f  (copy of %d bytes)" % (t["fetch_scale"], t["write_scale"],
                                                                     t["copy_bytes"]))
        sys.exit(0)
    if args and args[0] == "--report-cmd":
        # --report-cmd OUT PREFIX "BENCH COMMAND" MATCH WORKLOAD WORK COPY_BYTES TRAFFIC_FILE
        sys.stdout.write(report(args[1], args[4], args[5], args[6], int(args[7]), bench=args[3], prefix=args[2],
                                traffic_file=args[8]))
        sys.exit(0)
    if args and args[0] in ("--report", "--report-mx"):
        sys.stdout.write(report(args[1], args[2], args[3], args[4], int(args[5]), mx=args[0] == "--report-mx"))
        sys.exit(0)
    m = None
    if "--match" in args:
        i = args.index("--match")
        m = args[i + 1]
        del args[i:i + 2]
    print(summarise(args[0], m))
