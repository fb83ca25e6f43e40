#!/usr/bin/env python3
"""Benchmark of the gfx950 tiled GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--sweep] [--no-cpu] [--config k=v,...]

A step is one launch of the whole hot path, D = A x B (+C), on the workload's
synthetic inputs, which are resident in HBM before timing starts.  First the
median and its spread: 12 (--batches, at least 10) batches of >= 1 ms, at
least 10 launches each, every batch timed between two HIP events on the
launch stream ("Tuning Triton kernels", section 2: report the median with its
spread).  Then, in the same warm regime, the timed region: W untimed launches,
then exactly K launches on one stream between two HIP events, preceded and
followed by a device synchronization; ms_per_step is elapsed / K.

One JSON line is printed (rank 0, N = 1):
  value     TFLOP/s of the headline workload (bf16 4096^3 by default) over
            the timed region; spread.median_ms and spread.tflops_at_median
            give the batches' median beside it
  roofline  the kernel's achieved flop rate against the dense bf16 MFMA peak
            (256 CUs x 2.4 GHz x 4096 flop/clk/CU = 2516.6 TFLOP/s), plus the
            HBM roofline figures of the skinny workload (bf16 16 x 8192 x 8192,
            B rotated over 4 copies so every launch reads it from HBM)
  cpu_baseline  the CPU oracle timed on this host on a bounded sample of rows
            of the same workload, scaled to TFLOP/s

--sweep times interleaved variants (GROUP_M, instruction shape, tile sizes):
every round visits the variants in a fresh seeded-random order and times a
batch of launches per visit; the median and spread = (max - min) / median
over the rounds are reported ("Tuning Triton kernels", section 2: compare a delta with
the spread, not with zero).
"""
import argparse
import json
import os
import random
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12        # 2516.6
PEAK_MX_TFLOPS = {"e4m3": 5000.0, "e5m2": 5000.0, "e2m3": 10100.0, "e3m2": 10100.0,
                  "e2m1": 10100.0}   # MI355X dense fp8 / fp6 / fp4


def mx_peak(fa, fb):
    """Dense peak of a block-scaled pair: the slower operand's rate (an 8-bit
    operand runs the instruction at the fp8 rate)."""
    return min(PEAK_MX_TFLOPS[fa], PEAK_MX_TFLOPS[fb])
PEAK_HBM_GBS = 8000.0
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
TRAFFIC_MX_JSON = os.path.join(ROOT, "profiles", "traffic_mx.json")
TRAFFIC_I8_JSON = os.path.join(ROOT, "profiles", "traffic_i8.json")
# What the counters behind "traffic" count: FETCH_SIZE and WRITE_SIZE are the
# L2's requests to the memory fabric, so re-reads that hit the last-level
# cache in front of HBM (the 256 MB MALL) count too.
TRAFFIC_KIND = "L2-to-fabric bytes per launch (FETCH_SIZE x 2 + WRITE_SIZE, copy-calibrated; MALL hits included)"


def plan_kernel_name(profiled):
    """A profiler's demangled kernel name in the form plans describe it:
    'void dtg::(anonymous namespace)::gemm_dma_kernel<256, 256, 64, 2, 4, 16,
    2, true, false, false>(dtg::KArgs)' -> 'gemm_dma_kernel<256,256,64,2,4,16,
    2,1,lay0>' (booleans as 0 / 1; the direct-to-LDS kernel's two layout flags
    as its layout code, bit 0 for A stored K x M, bit 1 for B stored N x K)."""
    n = profiled.replace(" ", "").split("(dtg::")[0].split("::")[-1]
    if "<" not in n:
        return n
    head, args = n[:-1].split("<", 1)
    a = ["1" if x == "true" else "0" if x == "false" else x for x in args.split(",")]
    if head == "gemm_dma_kernel" and len(a) == 10:
        a = a[:8] + ["lay%d" % (int(a[8]) + 2 * int(a[9]))]
    return "%s<%s>" % (head, ",".join(a))


def measured_traffic(kernel_name, path=TRAFFIC_JSON):
    """L2-to-fabric bytes per launch of this kernel (MALL hits included) from
    the committed counter runs, or None if there are none or the kernel
    sources changed since."""
    try:
        import json as _json
        from dense_tiled_gemm_02_amd import rocprof_summary
        t = _json.load(open(path))
        if t.get("source_sha256") != rocprof_summary.source_hash():
            return None
        for k, v in t["kernels"].items():
            if plan_kernel_name(k) == kernel_name:
                return v["bytes"]
    except (OSError, ValueError, KeyError):
        return None
    return None


def kernel_of(plan_desc):
    """'gemm_dma_kernel<256,256,...>' from a plan description."""
    return plan_desc.split("kernel=")[1].split(" ")[0]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="square_bf16_4096")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--layouts", action="store_true",
                    help="time bf16 4096^3 with A and / or B stored transposed")
    ap.add_argument("--decode", action="store_true",
                    help="time the decode regime: M in {1,2,4,8,16,32}, N = K in {4096, 8192}, bf16")
    ap.add_argument("--mx", action="store_true",
                    help="block-scaled (MX) workloads: FP8 / FP4 elements with E8M0 scales per 32 k")
    ap.add_argument("--configs", action="store_true",
                    help="every named workload against torch.matmul, batches of 10 launches captured in a HIP graph")
    ap.add_argument("--i8", action="store_true",
                    help="int8 workloads (int8 operands, int32 output) against the dense int8 peak")
    ap.add_argument("--mx-sweep", action="store_true",
                    help="block-scaled tile / slice variants of the decode and square workloads, interleaved")
    ap.add_argument("--rounds", type=int, default=30)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-skinny", action="store_true")
    ap.add_argument("--config", default="", help="forced config fields, e.g. bm=128,bn=128,mfma=32")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--out", default="")
    ap.add_argument("--save", default="", help="sweep modes: write the records and the command to this JSON file")
    ap.add_argument("--batches", type=int, default=12,
                    help="batches of >= 1 ms for the headline median and spread (at least 10)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="after timing, run one device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def _cfg(s):
    if not s:
        return None
    d = {}
    for kv in s.split(","):
        k, v = kv.split("=")
        d[k.strip()] = int(v)
    return d


class Case:
    """Device-resident inputs of one workload plus rotation copies of B."""

    def __init__(self, w, rotate=1):
        import torch
        import gemm_inputs
        self.w = w
        A, B, C = gemm_inputs.make(w)
        self.A = A.cuda()
        self.Bs = [B.cuda()]
        for r in range(1, rotate):
            self.Bs.append(gemm_inputs.draw((w.K, w.N), w.seeds[1] + 1000 * r, w.dtype, w.dist,
                                            w.scale).cuda())
        self.C = C.cuda() if C is not None else None
        self.D = torch.empty((w.M, w.N), dtype=self.A.dtype, device="cuda")
        self.host = (A, B, C)

    def launcher(self, config=None):
        import torch
        import dense_tiled_gemm_02_amd as g
        pl = g.plan_for(self.A, self.Bs[0], self.C, self.D, config)
        stream = torch.cuda.current_stream().cuda_stream
        lib = g.lib()
        h = pl.handle
        a = self.A.data_ptr()
        bs = [b.data_ptr() for b in self.Bs]
        c = self.C.data_ptr() if self.C is not None else None
        d = self.D.data_ptr()
        ws, ws_bytes = g.workspace_for(pl, torch.cuda.current_device(), stream)
        run = lib.gemm_run
        nb = len(bs)
        state = {"i": 0}

        def launch(n):
            i = state["i"]
            for _ in range(n):
                st = run(h, a, bs[i % nb], c, d, ws, ws_bytes, stream)
                if st != 0:
                    raise g.GemmError(st, g.gemm_last_error())
                i += 1
            state["i"] = i
        return launch, pl


def time_region(launch, steps, warmup):
    """(ms per launch) over `steps` launches between two events on the launch stream."""
    import torch
    launch(warmup)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    launch(steps)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def batch_times(launch, batch, rounds, back_to_back=False):
    """Per-launch ms of `rounds` batches of `batch` launches (for median/spread).
    back_to_back: the batches are enqueued one after another with an event
    between each two and the host waits once at the end, so the GPU never
    idles between them (the regime of a long timed region); otherwise the
    host waits after every batch (interleaved comparisons of variants)."""
    import torch
    if back_to_back:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(rounds + 1)]
        ev[0].record()
        for r in range(rounds):
            launch(batch)
            ev[r + 1].record()
        ev[-1].synchronize()
        return [ev[r].elapsed_time(ev[r + 1]) / batch for r in range(rounds)]
    out = []
    for _ in range(rounds):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        launch(batch)
        e.record()
        e.synchronize()
        out.append(s.elapsed_time(e) / batch)
    return out


def stats(ts):
    med = statistics.median(ts)
    q = statistics.quantiles(ts, n=4) if len(ts) >= 4 else [med, med, med]
    return {"median_ms": med, "spread": (max(ts) - min(ts)) / med, "p25_ms": q[0], "p75_ms": q[2],
            "min_ms": min(ts), "max_ms": max(ts), "n": len(ts)}


def batch_len(launch, target_ms=1.0, least=10):
    """Launches per timed batch: at least `least`, and enough for >= target_ms."""
    probe = time_region(launch, 5, 3)
    return max(least, int(-(-target_ms // max(probe, 1e-4))))


def headline_times(launch, steps, warmup, rounds):
    """The headline measurement of one kernel, in one warm regime:
    `rounds` batches of >= 1 ms (>= 10 launches) enqueued back to back with
    an event on the launch stream between each two, for the median and its
    spread; then the timed region proper, `warmup` untimed launches and
    exactly `steps` launches between two events (ms_per_step).  Before the
    batches, ~100 ms of untimed launches let the clock settle (timed from a
    cold start, the first batches ran ~10 % slower than the region).
    Returns (ms_per_step, stats of the batches with the batch length
    added)."""
    batch = batch_len(launch)
    # ~100 ms of untimed launches first: the clock settles before anything is timed
    launch(max(warmup, batch * 100))
    st = stats(batch_times(launch, batch, rounds, back_to_back=True))
    st["batch_launches"] = batch
    ms = time_region(launch, steps, warmup)
    return ms, st


def cpu_baseline(w, seconds):
    """Time the CPU oracle on the first rows of the workload (bounded sample)."""
    import oracle
    import gemm_inputs
    A, B, C = gemm_inputs.make(w)
    Ab, Bb = gemm_inputs.bits(A), gemm_inputs.bits(B)
    Cb = gemm_inputs.bits(C) if C is not None else None
    # calibrate: the oracle decodes all of B once per call, then costs per row
    def timed(r):
        t0 = time.perf_counter()
        oracle.gemm_f64(Ab[:r], Bb, Cb[:r] if Cb is not None else None, w.dtype)
        return time.perf_counter() - t0
    r1 = min(w.M, 8)
    r2 = min(w.M, 40)
    t1, t2 = timed(r1), timed(r2)
    per_row = max((t2 - t1) / max(r2 - r1, 1), 1e-6)
    rows = int(max(r2, min(w.M, (seconds - t1) / per_row)))
    t = timed(rows)
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "first %d of %d rows of %s (%dx%dx%d), full K and N; %.2f s" % (
                rows, w.M, w.name, rows, w.N, w.K, t)}


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def sweep(args):
    import gemm_inputs
    variants = {
        # GROUP_M {1, 4, 8} x instruction {16x16x32, 32x32x16} at the 256 x 256
        # tile with 8 waves (2 per SIMD) and with 4 (one per SIMD, AGPR
        # accumulators), deeper rings of 32-deep K steps, and the smaller tiles
        "square_bf16_4096": [dict(kernel=3, bm=256, bn=256, bk=64, stages=2, mfma=mf, waves_m=2, waves_n=wn,
                                  group_m=gm) for wn in (4, 2) for mf in (16, 32) for gm in (1, 4, 8)] +
                            [dict(kernel=3, bm=256, bn=256, bk=32, stages=4, mfma=16, waves_m=2, waves_n=4,
                                  group_m=8),
                             dict(kernel=3, bm=256, bn=128, bk=64, stages=3, mfma=16, group_m=8),
                             dict(kernel=3, bm=128, bn=128, bk=64, stages=4, mfma=16, group_m=8)],
        # the planner's plan, the three tiles of the tile-size sweep (32^3 and 64 x 64 x 32 register-staged,
        # 128 x 128 x 64 both ways), then other direct-to-LDS tiles and K slices
        "square_f16_1024": [dict(), dict(kernel=1, bm=32, bn=32, bk=32), dict(kernel=1, bm=64, bn=64, bk=32, stages=2),
                            dict(kernel=1, bm=128, bn=128, bk=64, stages=2),
                            dict(kernel=3, bm=128, bn=128, bk=64, stages=4, waves_m=2, waves_n=4),
                            dict(kernel=3, bm=128, bn=128, bk=32, stages=4, waves_m=2, waves_n=4),
                            dict(kernel=3, bm=128, bn=128, bk=32, stages=4, waves_m=2, waves_n=4, splitk=2),
                            dict(kernel=3, bm=128, bn=128, bk=64, stages=4, waves_m=2, waves_n=4, splitk=2),
                            dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=4, splitk=2),
                            dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=4, splitk=8),
                            dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=2, splitk=4),
                            dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=4, splitk=1),
                            dict(bm=64, bn=64, bk=64),
                            dict(kernel=3, bm=128, bn=128, bk=64, stages=2, mfma=16),
                            dict(kernel=3, bm=128, bn=128, bk=64, stages=2, mfma=32),
                            dict(kernel=3, bm=256, bn=128, bk=64, stages=2, mfma=16)],
        "square_f16_256": [dict(), dict(bm=64, bn=64, bk=64), dict(bm=16, bn=64, bk=64),
                           dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=4, splitk=1)],
        "decode_bf16_1x4096x4096": [dict()] + [dict(kernel=2, bm=16, bn=bn, waves_n=w, bk=bk, stages=st, splitk=sk)
                                             for (bn, w, bk, st) in ((128, 8, 32, 2), (64, 8, 64, 2), (32, 8, 64, 3),
                                                                     (16, 8, 64, 3), (128, 4, 32, 3))
                                             for sk in (1, 2, 4, 8)],
        "deepk_bf16_512x512x32768": [dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=4, splitk=s)
                                     for s in (1, 2, 4, 8, 12, 16)] +
                                    [dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=2, splitk=s)
                                     for s in (4, 16)] + [dict()],
        "skinny_bf16_16x8192": [dict(kernel=2, bn=32, waves_n=8, bk=64, stages=3, splitk=1)] +
                               [dict(kernel=2, bn=128, waves_n=8, bk=32, stages=2, splitk=s) for s in (4, 6)] +
                               [dict(kernel=2, bn=128, waves_n=4, bk=32, stages=st, splitk=s)
                                for st in (3, 4) for s in (4, 6, 8)] +
                               [dict(kernel=2, bn=128, waves_n=2, bk=32, stages=st, splitk=s)
                                for st in (6, 8) for s in (4, 8)],
        "tail_f16_4000x3000x1000_c": [dict(), dict(kernel=3, bm=256, bn=128, waves_m=4, waves_n=2),
                                      dict(kernel=3, bm=128, bn=256, waves_m=2, waves_n=4),
                                      dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=4),
                                      dict(kernel=3, bm=256, bn=128, bk=64, stages=2, mfma=16),
                                      dict(kernel=3, bm=256, bn=128, bk=64, stages=3, mfma=16),
                                      dict(kernel=3, bm=128, bn=128, bk=64, stages=2, mfma=16),
                                      dict(kernel=3, bm=128, bn=128, bk=64, stages=4, mfma=16),
                                      dict(kernel=3, bm=256, bn=256, bk=64, stages=2, mfma=16),
                                      dict(kernel=3, bm=128, bn=256, bk=64, stages=2, mfma=16),
                                      dict(bm=128, bn=128, bk=64)],
    }[args.workload]
    w = gemm_inputs.WORKLOADS[args.workload]
    # B rotated over enough copies (> 300 MB) that HBM-bound shapes read it from HBM
    rot = max(4, -(-300 * (1 << 20) // (2 * w.K * w.N))) if w.M <= 32 else 1
    case = Case(w, rotate=rot)
    ls = []
    for v in variants:
        launch, pl = case.launcher(v)
        launch(3)
        ls.append((v, launch, pl))
    import torch
    torch.cuda.synchronize()
    # batch so that one visit is >= ~1 ms
    probe = time_region(ls[0][1], 5, 2)
    batch = max(4, int(1.0 / max(probe, 1e-3)))
    times = {i: [] for i in range(len(ls))}
    rng = random.Random(1234)
    for _ in range(args.rounds):
        order = list(range(len(ls)))
        rng.shuffle(order)
        for i in order:
            times[i].extend(batch_times(ls[i][1], batch, 1))
    rows = []
    for i, (v, _, pl) in enumerate(ls):
        st = stats(times[i])
        ms = st["median_ms"]
        rec = {"workload": w.name, "variant": v, "plan": pl.describe(), **st, "batch_launches": batch,
               "tflops": w.flops() / ms / 1e9, "pct_mfma": 100 * w.flops() / ms / 1e9 / PEAK_BF16_TFLOPS,
               "gbs": w.bytes() / ms / 1e6, "pct_hbm": 100 * w.bytes() / ms / 1e6 / PEAK_HBM_GBS}
        rows.append(rec)
        print(json.dumps(rec), flush=True)
    if args.save:
        save_rows(args.save, rows, "interleaved sweep of %s: %d rounds in seeded-random order, one batch of %d "
                                   "launches per variant per round" % (w.name, args.rounds, batch))
    return rows


def save_rows(path, rows, what):
    """Sweep records with the command that made them and the device, as one JSON file."""
    import torch
    doc = {"what": what, "command": "python " + " ".join(sys.argv), "device": torch.cuda.get_device_name(0),
           "rows": rows}
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


def layouts(args):
    """bf16 4096^3 with each operand layout (A stored M x K or K x M, B stored
    K x N or N x K), the planner's plan against torch.matmul on the same views.
    One JSON line per layout."""
    import torch
    import gemm_inputs
    import dense_tiled_gemm_02_amd as g
    w = gemm_inputs.WORKLOADS["square_bf16_4096"]
    A, B, _ = gemm_inputs.make(w)
    D = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for ta in (False, True):
        for tb in (False, True):
            dA = A.t().contiguous().cuda().t() if ta else A.cuda()
            dB = B.t().contiguous().cuda().t() if tb else B.cuda()
            pl = g.plan_for(dA, dB, None, D)
            ws, wsb = g.workspace_for(pl, torch.cuda.current_device(), stream)
            run = g.lib().gemm_run

            def launch(c):
                for _ in range(c):
                    assert run(pl.handle, dA.data_ptr(), dB.data_ptr(), None, D.data_ptr(), ws, wsb, stream) == 0

            def launch_torch(c):
                for _ in range(c):
                    torch.matmul(dA, dB, out=D)
            ours = stats(batch_times(launch, 10, args.rounds))["median_ms"]
            ref = stats(batch_times(launch_torch, 10, args.rounds))["median_ms"]
            print(json.dumps({"workload": w.name, "A": "K x M" if ta else "M x K", "B": "N x K" if tb else "K x N",
                              "plan": pl.describe(), "us": ours * 1e3, "tflops": w.flops() / ours / 1e9,
                              "torch_matmul_us": ref * 1e3}), flush=True)
            del dA, dB


def decode(args):
    """The M-bucketed decode regime: for each M, the planner's plan against
    torch.matmul, B rotated over enough copies (> 256 MB) that every launch
    reads it from HBM.  One JSON line per (M, N)."""
    import torch
    import gemm_inputs
    import dense_tiled_gemm_02_amd as g
    for n in (4096, 8192):
        k = n
        copies = max(4, -(-300 * (1 << 20) // (2 * k * n)))
        Bs = [gemm_inputs.draw((k, n), 900 + r, "bf16", "normal", 1 / 64).cuda() for r in range(copies)]
        for m in (1, 2, 4, 8, 16, 32):
            A = gemm_inputs.draw((m, k), 800 + m, "bf16", "normal", 1 / 64).cuda()
            D = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
            pl = g.plan_for(A, Bs[0], None, D)
            stream = torch.cuda.current_stream().cuda_stream
            ws, wsb = g.workspace_for(pl, torch.cuda.current_device(), stream)
            run = g.lib().gemm_run
            st = {"i": 0}

            def launch(c, st=st):
                for _ in range(c):
                    b = Bs[st["i"] % copies]
                    assert run(pl.handle, A.data_ptr(), b.data_ptr(), None, D.data_ptr(), ws, wsb, stream) == 0
                    st["i"] += 1

            def launch_torch(c, st=st):
                for _ in range(c):
                    torch.matmul(A, Bs[st["i"] % copies], out=D)
                    st["i"] += 1
            ours = stats(batch_times(launch, 20, args.rounds))["median_ms"]
            ref = stats(batch_times(launch_torch, 20, args.rounds))["median_ms"]
            byt = 2.0 * (m * k + k * n + m * n)
            print(json.dumps({"workload": "decode_bf16_%dx%dx%d" % (m, n, k), "M": m, "N": n, "K": k,
                              "plan": pl.describe(), "us": ours * 1e3, "gbs": byt / ours / 1e6,
                              "pct_hbm": 100 * byt / ours / 1e6 / PEAK_HBM_GBS,
                              "torch_matmul_us": ref * 1e3}), flush=True)
        del Bs


def configs(args):
    """Every named workload (the planner's plan) against torch.matmul (torch.addmm
    with an addend): each timed batch is one HIP graph of 10 launches, so host
    launch cost is out of both; rounds in seeded-random order, medians.  The
    skinny and decode workloads rotate B over 4 copies (read from HBM).  One
    JSON line per workload."""
    import random
    import torch
    import gemm_inputs
    import dense_tiled_gemm_02_amd as g
    for name, w in gemm_inputs.WORKLOADS.items():
        A, B, C = gemm_inputs.make(name)
        dA = A.cuda()
        ncopy = 4 if w.M <= 16 else 1
        Bs = [B.cuda()] + [gemm_inputs.draw((w.K, w.N), 990 + r, w.dtype, w.dist, w.scale).cuda()
                           for r in range(1, ncopy)]
        dC = C.cuda() if C is not None else None
        D1 = torch.empty((w.M, w.N), dtype=dA.dtype, device="cuda")
        D2 = torch.empty_like(D1)

        def ours(i):
            g.matmul(dA, Bs[i % ncopy], dC, out=D1)

        def theirs(i):
            if dC is None:
                torch.matmul(dA, Bs[i % ncopy], out=D2)
            else:
                torch.addmm(dC, dA, Bs[i % ncopy], out=D2)
        graphs = {}
        side = torch.cuda.Stream()
        # a K-sliced plan's workspace for the capture stream, zero-filled before the capture
        g.workspace_for(g.plan_for(dA, Bs[0], dC, D1), torch.cuda.current_device(), side.cuda_stream)
        for key, f in (("ours", ours), ("torch", theirs)):
            for i in range(3):
                f(i)
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.graph(gr, stream=side):
                for i in range(10):
                    f(i)
            torch.cuda.synchronize()
            graphs[key] = gr
        t = {k: [] for k in graphs}
        rng = random.Random(1)
        for _ in range(args.rounds):
            order = list(graphs)
            rng.shuffle(order)
            for k in order:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                graphs[k].replay()
                e1.record()
                torch.cuda.synchronize()
                t[k].append(e0.elapsed_time(e1) / 10)
        us = {k: stats(v)["median_ms"] * 1e3 for k, v in t.items()}
        byt = 2.0 * (w.M * w.K + w.K * w.N + w.M * w.N * (2 if dC is not None else 1))
        print(json.dumps({"workload": name, "plan": g.plan_for(dA, Bs[0], dC, D1).describe().split(" bm=")[0],
                          "us": round(us["ours"], 2), "torch_us": round(us["torch"], 2),
                          "tflops": round(w.flops() / us["ours"] / 1e6, 1), "gbs": round(byt / us["ours"] / 1e3, 1)}),
              flush=True)


def mx(args):
    """Block-scaled (MX) workloads: the planner's plan, median and spread over
    interleaved rounds, against the dense MFMA peak of the element type (square)
    or HBM (M = 16, B rotated over > 256 MB of copies).  A per-tensor scaled
    fp8 GEMM of torch (torch._scaled_mm, hipBLASLt) on the same bytes is timed
    beside the fp8 case as a library reference (no block scales), and the same
    block-scaled product through torch._scaled_mm where the build has it.  One
    JSON line per workload."""
    import torch
    import gemm_inputs
    import dense_tiled_gemm_02_amd.mx as mxb
    for name in sorted(gemm_inputs.MX_WORKLOADS):
        w = gemm_inputs.MX_WORKLOADS[name]
        A, SA, B, SB, _ = gemm_inputs.make_mx(w)
        dA, dSA = torch.from_numpy(A).cuda(), torch.from_numpy(SA).cuda()
        copies = 1
        if w.M <= 32:
            copies = max(4, -(-300 * (1 << 20) // B.nbytes))
        Bs = [torch.from_numpy(B).cuda()]
        SBs = [torch.from_numpy(SB).cuda()]
        for r in range(1, copies):
            b2, s2 = gemm_inputs.draw_mx(w.N, w.K, w.fmt_b, w.seeds[1] + 1000 * r)
            Bs.append(torch.from_numpy(b2).cuda())
            SBs.append(torch.from_numpy(s2).cuda())
        D = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        p = mxb.mx_problem(w.M, w.N, w.K, w.fmt_a, w.fmt_b, mxb.GEMM_MX_OUT_BF16, lda=A.shape[1], ldb=B.shape[1],
                           ldsa=SA.shape[1], ldsb=SB.shape[1])
        pl = mxb.gemm_mx_plan_create(p, torch.cuda.current_device())
        stream = torch.cuda.current_stream().cuda_stream
        ws, wsb = mxb._workspace(pl, torch.cuda.current_device(), stream)
        run = mxb.mxlib().gemm_mx_run
        st = {"i": 0}

        def launch(c, st=st):
            for _ in range(c):
                i = st["i"] % copies
                assert run(pl.handle, dA.data_ptr(), dSA.data_ptr(), Bs[i].data_ptr(), SBs[i].data_ptr(), None,
                           D.data_ptr(), ws, wsb, stream) == 0
                st["i"] += 1
        launch(5)
        torch.cuda.synchronize()
        ts = stats(batch_times(launch, 20, args.rounds))
        ms = ts["median_ms"]
        rec = {"workload": name, **w.describe(), "plan": pl.describe(), "us": ms * 1e3, "spread": ts["spread"],
               "tflops": w.flops() / ms / 1e9}
        if w.M <= 32:
            gbs = w.bytes() / ms / 1e6
            rec["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": gbs / PEAK_HBM_GBS}
        else:
            peak = mx_peak(w.fmt_a, w.fmt_b)
            rec["roofline"] = {"bound": "mfma", "achieved": round(rec["tflops"], 1), "peak": peak,
                               "unit": "TFLOP/s", "frac": rec["tflops"] / peak}
        rec["roofline"]["traffic"] = measured_traffic(kernel_of(pl.describe()), TRAFFIC_MX_JSON)
        if w.fmt_a == "e4m3" and w.fmt_b == "e4m3":
            try:
                a8 = dA.view(torch.float8_e4m3fn)
                b8 = Bs[0].view(torch.float8_e4m3fn)
                one = torch.ones((), dtype=torch.float32, device="cuda")

                def launch_torch(c):
                    for _ in range(c):
                        torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
                launch_torch(3)
                torch.cuda.synchronize()
                rec["torch_scaled_mm_per_tensor_us"] = stats(batch_times(launch_torch, 20, args.rounds))[
                    "median_ms"] * 1e3
            except Exception as e:   # not every build has a scaled fp8 GEMM
                rec["torch_scaled_mm_per_tensor_us"] = None
                rec["torch_scaled_mm_error"] = str(e)[:200]
        # the same block-scaled product through torch._scaled_mm (E8M0 scales per
        # 32 k), where the build has it: time, and the largest difference from
        # this library's D relative to max |D|
        nb = w.K // 32
        if w.M > 32 and w.K % 32 == 0 and SA.shape[1] >= nb:
            try:
                el = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}.get(w.fmt_a)
                if w.fmt_a == "e2m1" and w.fmt_b == "e2m1":
                    el = torch.float4_e2m1fn_x2
                if el is None or w.fmt_b != w.fmt_a:
                    raise ValueError("no torch element type for %s x %s" % (w.fmt_a, w.fmt_b))
                ta, tb = dA.view(el), Bs[0].view(el)
                tsa = dSA[:, :nb].contiguous().view(torch.float8_e8m0fnu)
                tsb = SBs[0][:, :nb].contiguous().view(torch.float8_e8m0fnu)

                def launch_block(c):
                    for _ in range(c):
                        torch._scaled_mm(ta, tb.t(), scale_a=tsa, scale_b=tsb, out_dtype=torch.bfloat16)
                Dt = torch._scaled_mm(ta, tb.t(), scale_a=tsa, scale_b=tsb, out_dtype=torch.bfloat16)
                launch(1)
                torch.cuda.synchronize()
                rec["torch_scaled_mm_block_us"] = stats(batch_times(launch_block, 20, args.rounds))["median_ms"] * 1e3
                ours = D.float()
                rec["torch_block_max_rel_diff"] = ((Dt.float() - ours).abs().max() / ours.abs().max()).item()
            except Exception as e:
                rec["torch_scaled_mm_block_us"] = None
                rec["torch_scaled_mm_block_error"] = str(e)[:200]
        print(json.dumps(rec), flush=True)
        del Bs, SBs, dA, dSA
    if args.copy_mb:
        copy_calibration(args.copy_mb)


def mx_sweep(args):
    """The block-scaled workloads in their planned configuration beside other
    tiles / K-slice counts, interleaved in seeded-random order (median and
    spread over the rounds)."""
    import torch
    import gemm_inputs
    import dense_tiled_gemm_02_amd.mx as mxb
    cases = {
        "mx_e2m1_16x8192x8192": [dict()] + [dict(bm=32, bn=64, splitk=k) for k in (1, 3, 4, 8)],
        "mx_e4m3_4096": [dict()] + [dict(bm=bm, bn=bn) for (bm, bn) in ((256, 128), (128, 256), (128, 128))],
        "mx_e2m1_4096": [dict()] + [dict(bm=bm, bn=bn) for (bm, bn) in ((256, 128), (128, 256), (128, 128))],
        # FP6 and mixed widths: the planned tile kernel, its 128 x 128 tile and the register-direct kernel
        "mx_e2m3_4096": [dict(), dict(kernel=4, bm=128, bn=128), dict(kernel=5)],
        "mx_e4m3xe2m1_4096": [dict(), dict(kernel=4, bm=128, bn=128), dict(kernel=5)],
    }
    rows = []
    for name, variants in cases.items():
        w = gemm_inputs.MX_WORKLOADS[name]
        A, SA, B, SB, _ = gemm_inputs.make_mx(w)
        copies = max(4, -(-300 * (1 << 20) // B.nbytes)) if w.M <= 32 else 1
        dA, dSA = torch.from_numpy(A).cuda(), torch.from_numpy(SA).cuda()
        Bs = [torch.from_numpy(B).cuda()] + [torch.from_numpy(gemm_inputs.draw_mx(w.N, w.K, w.fmt_b, 5000 + r)[0]).cuda()
                                             for r in range(1, copies)]
        dSB = torch.from_numpy(SB).cuda()
        D = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        run = mxb.mxlib().gemm_mx_run
        ls = []
        for v in variants:
            p = mxb.mx_problem(w.M, w.N, w.K, w.fmt_a, w.fmt_b, mxb.GEMM_MX_OUT_BF16, lda=A.shape[1], ldb=B.shape[1],
                               ldsa=SA.shape[1], ldsb=SB.shape[1])
            pl = mxb.gemm_mx_plan_create(p, torch.cuda.current_device(), v or None)
            ws, wsb = mxb._workspace(pl, torch.cuda.current_device(), stream)
            st = {"i": 0}

            def launch(c, pl=pl, ws=ws, wsb=wsb, st=st):
                for _ in range(c):
                    b = Bs[st["i"] % copies]
                    assert run(pl.handle, dA.data_ptr(), dSA.data_ptr(), b.data_ptr(), dSB.data_ptr(), None,
                               D.data_ptr(), ws, wsb, stream) == 0
                    st["i"] += 1
            launch(3)
            ls.append((v, launch, pl))
        torch.cuda.synchronize()
        times = {i: [] for i in range(len(ls))}
        rng = random.Random(99)
        for _ in range(args.rounds):
            order = list(range(len(ls)))
            rng.shuffle(order)
            for i in order:
                times[i].extend(batch_times(ls[i][1], 20, 1))
        for i, (v, _, pl) in enumerate(ls):
            s = stats(times[i])
            ms = s["median_ms"]
            rec = {"workload": name, "variant": v, "plan": pl.describe(), "us": ms * 1e3, "spread": s["spread"],
                   "p25_us": s["p25_ms"] * 1e3, "p75_us": s["p75_ms"] * 1e3,
                   "tflops": w.flops() / ms / 1e9, "gbs": w.bytes() / ms / 1e6}
            rows.append(rec)
            print(json.dumps(rec), flush=True)
        del Bs
    if args.save:
        save_rows(args.save, rows, "block-scaled workloads: planned plan beside other tiles, K-slice counts and "
                                   "kernels, %d interleaved rounds of 20-launch batches" % args.rounds)


PEAK_I8_TOPS = 5000.0   # MI355X dense int8 matrix peak (2:1 sparsity excluded)


def i8(args):
    """int8 workloads (int8 A and B stored N x K, int32 D): the planner's plan
    and the 32 x 32 x 32 instruction at the same tile, timed in interleaved
    rounds of >= 1 ms batches (median, spread), against the dense int8 peak.
    One JSON line per workload and variant."""
    import torch
    import gemm_inputs
    import dense_tiled_gemm_02_amd as g
    rows = []
    names = [args.workload] if args.workload in gemm_inputs.I8_WORKLOADS else list(gemm_inputs.I8_WORKLOADS)
    for name in names:
        w = gemm_inputs.I8_WORKLOADS[name]
        A, Bt, C = gemm_inputs.make_i8(w)
        dA, dBt = torch.from_numpy(A).cuda(), torch.from_numpy(Bt).cuda()
        dC = torch.from_numpy(C).cuda() if C is not None else None
        D = torch.empty((w.M, w.N), dtype=torch.int32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        variants = [None]
        base = g.plan_for(dA, dBt.t(), dC, D).config
        if base.mfma == 16:
            variants.append(dict(kernel=3, bm=base.bm, bn=base.bn, bk=base.bk, waves_m=base.waves_m,
                                 waves_n=base.waves_n, stages=base.stages, mfma=32))
        ls = []
        for v in variants:
            try:
                pl = g.plan_for(dA, dBt.t(), dC, D, v)
            except g.GemmError:
                continue
            run = g.lib().gemm_run

            def launch(n, pl=pl):
                for _ in range(n):
                    st = run(pl.handle, dA.data_ptr(), dBt.data_ptr(), dC.data_ptr() if dC is not None else None,
                             D.data_ptr(), None, 0, stream)
                    if st != 0:
                        raise g.GemmError(st, g.gemm_last_error())
            launch(3)
            ls.append((v, launch, pl))
        torch.cuda.synchronize()
        batch = batch_len(ls[0][1])
        times = {i: [] for i in range(len(ls))}
        rng = random.Random(7)
        for _ in range(args.rounds):
            order = list(range(len(ls)))
            rng.shuffle(order)
            for i in order:
                times[i].extend(batch_times(ls[i][1], batch, 1))
        for i, (v, _, pl) in enumerate(ls):
            st = stats(times[i])
            tops = w.flops() / st["median_ms"] / 1e9
            rec = {"workload": name, **w.describe(), "variant": v, "plan": pl.describe(), "us": st["median_ms"] * 1e3,
                   "spread": st["spread"], "batch_launches": batch,
                   "roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": PEAK_I8_TOPS, "unit": "TOP/s",
                                "frac": tops / PEAK_I8_TOPS,
                                "traffic": measured_traffic(kernel_of(pl.describe()), TRAFFIC_I8_JSON)},
                   "gbs": w.bytes() / st["median_ms"] / 1e6}
            rows.append(rec)
            print(json.dumps(rec), flush=True)
        del dA, dBt, dC, D
    if args.save:
        save_rows(args.save, rows, "int8 workloads: planner plan and the other instruction shape, %d interleaved "
                                   "rounds" % args.rounds)
    if args.copy_mb:
        copy_calibration(args.copy_mb)


def copy_calibration(mb):
    """One device copy of `mb` MiB, the reference kernel of the memory counters."""
    import torch
    n = mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    return 4 * n


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the GEMM of this library is a single-GPU kernel "
              "(multi-GPU sharding is described, not built); got --gpus %d" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import gemm_inputs
    import dense_tiled_gemm_02_amd as g
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.sweep:
        sweep(args)
        return
    if args.decode:
        decode(args)
        return
    if args.configs:
        configs(args)
        return
    if args.layouts:
        layouts(args)
        return
    if args.mx:
        mx(args)
        return
    if args.mx_sweep:
        mx_sweep(args)
        return
    if args.i8:
        i8(args)
        return
    w = gemm_inputs.WORKLOADS[args.workload]
    case = Case(w, rotate=4 if w.name.startswith("skinny") else 1)
    launch, pl = case.launcher(_cfg(args.config))
    torch.cuda.synchronize()
    rounds = max(10, args.batches)
    ms, spread = headline_times(launch, args.steps, args.warmup, rounds)
    flops = w.flops()
    tflops = flops / ms / 1e9
    spread["tflops_at_median"] = flops / spread["median_ms"] / 1e9
    spread["region_within_spread"] = spread["min_ms"] <= ms <= spread["max_ms"]
    rec = {
        "metric": "GEMM TFLOPS + % of MFMA peak at 4096^3 bf16; % HBM BW on skinny",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f16",
        "data": "synthetic",
        "config": {**w.describe(), "plan": pl.describe(), "parallelism": "single-gpu"},
        "spread": spread,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(kernel_of(pl.describe())), "traffic_kind": TRAFFIC_KIND},
    }
    if not args.no_skinny and args.workload != "skinny_bf16_16x8192":
        sw = gemm_inputs.WORKLOADS["skinny_bf16_16x8192"]
        sc = Case(sw, rotate=4)
        sl, spl = sc.launcher()
        sms, sspread = headline_times(sl, max(40, args.steps), 8, rounds)
        gbs = sw.bytes() / sms / 1e6
        sspread["gbs_at_median"] = sw.bytes() / sspread["median_ms"] / 1e6
        sspread["region_within_spread"] = sspread["min_ms"] <= sms <= sspread["max_ms"]
        rec["skinny"] = {"workload": sw.name, "plan": spl.describe(), "ms_per_step": sms, "steps": max(40, args.steps),
                         "spread": sspread,
                         "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                      "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                      "traffic": measured_traffic(kernel_of(spl.describe())),
                                      "traffic_kind": TRAFFIC_KIND},
                         "tflops": sw.flops() / sms / 1e9}
        del sc
    if args.copy_mb:
        rec["copy_calibration_bytes"] = copy_calibration(args.copy_mb)
    if not args.no_cpu:
        cb = cpu_baseline(w, args.cpu_seconds)
        cb["host_cpu"] = host_cpu_model()
        rec["cpu_baseline"] = cb
    line = json.dumps(rec)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
