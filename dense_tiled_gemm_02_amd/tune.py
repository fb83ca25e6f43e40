"""Per-shape tile-configuration table: a pruned sweep, every candidate probed
in its own process, finalists raced interleaved, the winners frozen into the
planner.

    python -m dense_tiled_gemm_02_amd.tune [--shapes NAME,...] [--rounds R] [--out FILE.json]
    python -m dense_tiled_gemm_02_amd.tune --one NAME CONFIG_JSON     (one candidate; its own process)
    python -m dense_tiled_gemm_02_amd.tune --emit FILE.json ...        (merges sweeps; writes csrc/tuned_table.inc)

The method is the one "Tuning Triton kernels" describes: the table is keyed
on every tiled dimension and the storage type (section 3: a key that omits M
serves a 4096-row tile to a one-row problem); the candidate space is pruned
before anything runs (section 4); a candidate is probed in a process of its
own, judged by its exit code, because a configuration that fails can take
the process down with it (section 6: a failing kernel aborts, and abort()
cannot be caught); the finalists are raced in interleaved rounds and a
candidate replaces the planner's own choice only when it wins beyond the
noise (section 2: compare a win with the spread, not with zero).

Steps:
  1. candidates: the cross product of the tile axes (kernel family, tile,
     K step, depth, instruction, wave grid, K slices), each point planned on
     the host against a gfx950 description with every field forced; what
     plans is compiled and fits the LDS (deduplicated by the plan's own
     configuration), times GROUP_M 1 / 4 / 8 where the grid has two rounds
     of tiles or more; then `prune`: no tile dimension over twice the
     problem's, K slices of >= 16 K steps (>= 512 k on the skinny kernel)
     and at most one round of workgroups;
  2. probe: every candidate runs `--one` in a subprocess: plan, run, time
     10 batches of >= 1 ms, print the median; a non-zero exit code or a
     non-finite output rejects it;
  3. race: the heuristic's plan (the planner with GEMM_TUNED_TABLE=0) and
     the four fastest probed candidates other than it, interleaved in
     seeded-random order for R rounds, one batch each per round; the fastest
     median wins if its 75th percentile is below the heuristic's 25th
     (non-overlapping interquartile ranges), else the heuristic stays;
  4. emit: merges the sweep files into profiles/tuned_table.json and writes
     csrc/tuned_table.inc, one entry per shape where a candidate won; the
     planner consults it before its heuristic (exact key: M, N, K, dtype,
     addend, row-major operands).

The shapes are the named workloads (NAMED) unless --shapes names others as
MxNxK[dtype][+C]; inputs are random (their values do not change the time);
for M <= 32 B rotates over enough copies that every launch reads it from
HBM.
"""
import argparse
import itertools
import json
import os
import random
import statistics
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INC = os.path.join(PKG, "csrc", "tuned_table.inc")

# name -> (M, N, K, dtype, has_c)
NAMED = {
    "square_f16_256": (256, 256, 256, "f16", False),
    "square_f16_1024": (1024, 1024, 1024, "f16", False),
    "square_bf16_4096": (4096, 4096, 4096, "bf16", False),
    "skinny_bf16_16x8192": (16, 8192, 8192, "bf16", False),
    "tail_f16_4000x3000x1000_c": (4000, 3000, 1000, "f16", True),
    "decode_bf16_1x4096x4096": (1, 4096, 4096, "bf16", False),
    "deepk_bf16_512x512x32768": (512, 512, 32768, "bf16", False),
}

CUS = 256
# The axes of the space; `candidates` keeps the points the library compiled.
KERNELS = (1, 2, 3, 6)          # register-staged tile, skinny, direct-to-LDS tile, its stream-K form
BMS, BNS, BKS = (16, 32, 64, 128, 192, 256), (16, 32, 64, 128, 256), (32, 64, 128)
STAGES, MFMAS = (2, 3, 4, 8), (16, 32)
WAVES = ((1, 2), (1, 4), (1, 8), (2, 1), (2, 2), (2, 4), (4, 2), (4, 1))
SPLITS = (1, 2, 4, 8, 16)


def parse_shape(s):
    """(name, (M, N, K, dtype, has_c)) of a named workload or of MxNxK[f16|bf16][+C]."""
    if s in NAMED:
        return s, NAMED[s]
    has_c = s.endswith("+C")
    body = s[:-2] if has_c else s
    dt = "bf16" if body.endswith("bf16") else "f16"
    m, n, k = (int(x) for x in body.replace("bf16", "").replace("f16", "").split("x"))
    return s, (m, n, k, dt, has_c)


def _fake_gfx950():
    import dense_tiled_gemm_02_amd as g
    d = g.gemm_device_info()
    d.arch, d.cu_count, d.xcd_count, d.clock_khz = 950, CUS, 8, 2400000
    d.lds_per_cu = d.lds_per_wg = 160 * 1024
    d.wave_size = 64
    return d


def candidates(M, N, K, dt="bf16", has_c=False):
    """Every compiled configuration that can plan this problem: the cross
    product of the axes, each point planned on the host (no GPU) with every
    tile field forced, deduplicated by the configuration the plan took."""
    import dense_tiled_gemm_02_amd as g
    prob = g.problem(M, N, K, g.GEMM_BF16 if dt == "bf16" else g.GEMM_F16, has_c)
    dev = _fake_gfx950()
    seen, out = set(), []
    for kern, bm, bn, bk, st, mf, (wm, wn) in itertools.product(KERNELS, BMS, BNS, BKS, STAGES, MFMAS, WAVES):
        if kern == 2 and bm > 32:
            continue
        # stream-K: splitk is the workgroup count; 0 lets the plan take one per CU
        for sk in (SPLITS if kern in (2, 3) else (0,) if kern == 6 else (1,)):
            f = dict(kernel=kern, bm=bm, bn=bn, bk=bk, stages=st, mfma=mf, waves_m=wm, waves_n=wn, splitk=sk)
            try:
                pl = g.gemm_plan_create_for(prob, dev, f)
            except g.GemmError:
                continue
            c = pl.config.as_dict()
            if kern == 6:
                f["splitk"] = c["splitk"]
            key = tuple(c[k] for k in ("kernel", "bm", "bn", "bk", "stages", "mfma", "waves_m", "waves_n", "splitk"))
            if key in seen:
                continue
            seen.add(key)
            tiles = -(-M // c["bm"]) * -(-N // c["bn"])
            for gm in ((1, 4, 8) if kern in (1, 3) and sk == 1 and tiles >= 2 * CUS else (c["group_m"],)):
                out.append(dict(f, group_m=gm))
    return out


def prune(M, N, K, cands):
    """(kept, reasons): a tile may exceed a dimension by at most 2x (rounded
    to 16); K slices need >= 16 K steps each and at most one round of
    workgroups; the skinny kernels only for M <= 32 (their slab height);
    stream-K only with >= 16 K steps per workgroup range."""
    kept, why = [], {}
    cdiv = lambda a, b: -(-a // b)
    for c in cands:
        r = None
        if c["kernel"] != 2 and (c["bm"] > 2 * max(16, M) or c["bn"] > 2 * max(16, N)):
            r = "tile more than twice the problem"
        elif c["kernel"] == 6:
            total = cdiv(M, c["bm"]) * cdiv(N, c["bn"]) * cdiv(K, c["bk"])
            if total < 16 * c["splitk"]:
                r = "stream-K ranges of fewer than 16 K steps"
        elif c["splitk"] > 1:
            steps = cdiv(K, c["bk"])
            wgs = cdiv(M, c["bm"]) * cdiv(N, c["bn"]) * c["splitk"]
            if steps // c["splitk"] < 16 and c["kernel"] == 3:
                r = "K slices of fewer than 16 K steps"
            elif c["kernel"] == 2 and K // c["splitk"] < 512:
                r = "skinny K slices below 512 k"
            elif wgs > CUS:
                r = "K slices beyond one round of workgroups"
        if r:
            why[r] = why.get(r, 0) + 1
        else:
            kept.append(c)
    return kept, why


def _inputs(M, N, K, dt, has_c, copies):
    import torch
    g = torch.Generator().manual_seed(M * 7 + N * 3 + K)
    t = torch.bfloat16 if dt == "bf16" else torch.float16
    A = (torch.randn(M, K, generator=g) / 16).to(t).cuda()
    Bs = [(torch.randn(K, N, generator=g) / 16).to(t).cuda() for _ in range(copies)]
    C = (torch.randn(M, N, generator=g) / 16).to(t).cuda() if has_c else None
    D = torch.empty(M, N, dtype=t, device="cuda")
    return A, Bs, C, D


def _launcher(A, Bs, C, D, cfg):
    """(launch(n), plan) for one configuration (None: the planner's own)."""
    import torch
    import dense_tiled_gemm_02_amd as g
    pl = g.plan_for(A, Bs[0], C, D, cfg)
    stream = torch.cuda.current_stream().cuda_stream
    dev = torch.cuda.current_device()
    st = {"i": 0}

    def launch(n):
        # the shared workspace grows when a later plan needs more: fetch it per batch
        ws, wsb = g.workspace_for(pl, dev, stream)
        for _ in range(n):
            b = Bs[st["i"] % len(Bs)]
            g.gemm_run(pl, A.data_ptr(), b.data_ptr(), C.data_ptr() if C is not None else None, D.data_ptr(),
                       ws, wsb, stream)
            st["i"] += 1
    return launch, pl


def _batch_ms(launch, n):
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    launch(n)
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / n


def _copies(M, N, K):
    return max(4, -(-300 * (1 << 20) // (2 * K * N))) if M <= 32 else 1


def one(name, cfg):
    """Probe one candidate (run in its own process): plan, run, check the
    output is finite, time 10 batches of >= 1 ms; print the median in us."""
    import torch
    _, (M, N, K, dt, has_c) = parse_shape(name)
    A, Bs, C, D = _inputs(M, N, K, dt, has_c, _copies(M, N, K))
    launch, pl = _launcher(A, Bs, C, D, cfg)
    launch(3)
    torch.cuda.synchronize()
    if not torch.isfinite(D.float()).all():
        print(json.dumps({"error": "non-finite output"}))
        return 3
    n = max(10, int(1.0 / max(_batch_ms(launch, 3), 1e-4)) + 1)
    ts = sorted(_batch_ms(launch, n) for _ in range(10))
    print(json.dumps({"us": statistics.median(ts) * 1e3, "plan": pl.describe()}))
    return 0


def race(name, cfgs, rounds):
    """Interleaved rounds over cfgs (None: the planner's plan); per config the
    median, p25 / p75 and spread in us."""
    import torch
    _, (M, N, K, dt, has_c) = parse_shape(name)
    A, Bs, C, D = _inputs(M, N, K, dt, has_c, _copies(M, N, K))
    ls = []
    for c in cfgs:
        launch, pl = _launcher(A, Bs, C, D, c)
        launch(3)
        ls.append((c, launch, pl))
    torch.cuda.synchronize()
    n = max(10, int(1.0 / max(_batch_ms(ls[0][1], 3), 1e-4)) + 1)
    times = [[] for _ in ls]
    rng = random.Random(17)
    for _ in range(rounds):
        order = list(range(len(ls)))
        rng.shuffle(order)
        for i in order:
            times[i].append(_batch_ms(ls[i][1], n) * 1e3)
    out = []
    for (c, _, pl), ts in zip(ls, times):
        q = statistics.quantiles(ts, n=4)
        med = statistics.median(ts)
        out.append({"config": c, "plan": pl.describe(), "median_us": med, "p25_us": q[0], "p75_us": q[2],
                    "spread": (max(ts) - min(ts)) / med})
    return out


CFG_KEYS = ("kernel", "bm", "bn", "bk", "stages", "mfma", "waves_m", "waves_n", "splitk", "group_m")


def heuristic_config(M, N, K, dt, has_c):
    """The configuration the planner's heuristic takes for this problem."""
    import dense_tiled_gemm_02_amd as g
    prob = g.problem(M, N, K, g.GEMM_BF16 if dt == "bf16" else g.GEMM_F16, has_c)
    c = g.gemm_plan_create_for(prob, _fake_gfx950()).config.as_dict()
    return {k: c[k] for k in CFG_KEYS}


def sweep(shapes, rounds, out_path):
    os.environ["GEMM_TUNED_TABLE"] = "0"       # race against the heuristic (inherited by the probes)
    doc = {"command": "python -m dense_tiled_gemm_02_amd.tune " + " ".join(sys.argv[1:]), "shapes": {}}
    for s in shapes:
        name, (M, N, K, dt, has_c) = parse_shape(s)
        cands = candidates(M, N, K, dt, has_c)
        kept, why = prune(M, N, K, cands)
        heur = heuristic_config(M, N, K, dt, has_c)
        probed = []
        for i, c in enumerate(kept):
            r = subprocess.run([sys.executable, "-m", "dense_tiled_gemm_02_amd.tune", "--one", name, json.dumps(c)],
                               cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
            rec = {"config": c, "exit": r.returncode}
            if r.returncode == 0:
                rec.update(json.loads(r.stdout.strip().splitlines()[-1]))
            else:
                tail = (r.stdout + r.stderr).strip().splitlines()
                rec["error"] = tail[-1][:200] if tail else ""
            probed.append(rec)
            print("probe %s %d/%d exit %d %s" % (name, i + 1, len(kept), r.returncode,
                                                 "%.2f us" % rec["us"] if "us" in rec else rec.get("error", "")),
                  flush=True)
        ok = sorted((p for p in probed if p["exit"] == 0), key=lambda p: p["us"])
        others = [p["config"] for p in ok if {k: p["config"][k] for k in CFG_KEYS} != heur]
        raced = race(name, [None] + others[:4], rounds)
        base = raced[0]
        best = min(raced, key=lambda r: r["median_us"])
        won = best is not base and best["p75_us"] < base["p25_us"]
        doc["shapes"][name] = {"M": M, "N": N, "K": K, "dtype": dt, "has_c": has_c,
                               "candidates": len(cands), "pruned": why, "heuristic": heur, "probed": probed,
                               "raced": raced, "winner": best["config"] if won else None,
                               "planner_plan": base["plan"], "planner_us": base["median_us"],
                               "best_us": best["median_us"]}
        print(json.dumps({"shape": name, "candidates": len(cands), "kept": len(kept),
                          "failed": sum(1 for p in probed if p["exit"] != 0), "planner_us": round(base["median_us"], 2),
                          "best_us": round(best["median_us"], 2), "winner": best["config"] if won else None}),
              flush=True)
    with open(out_path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


def table_lines(doc):
    """The initializers of the winning shapes of a (merged) sweep document."""
    lines, keys = [], set()
    for name, s in sorted(doc["shapes"].items()):
        w = s["winner"]
        key = (s["M"], s["N"], s["K"], s["dtype"], bool(s["has_c"]))
        if not w or key in keys:       # one entry per key (a shape raced under two names)
            continue
        keys.add(key)
        dt = 1 if s["dtype"] == "bf16" else 0
        lines.append("{%d, %d, %d, %d, %d, {%d, %d, %d, %d, %d, %d, %d, %d, %d, 0, %d}, %d, 1},   // %s: %.1f us "
                     "(heuristic %.1f us)" % (s["M"], s["N"], s["K"], dt, int(s["has_c"]), w["bm"], w["bn"], w["bk"],
                                              w["stages"], w["mfma"], w["waves_m"], w["waves_n"], w["group_m"],
                                              w["splitk"], w["kernel"], w["group_m"], name, s["best_us"],
                                              s["planner_us"]))
    return lines


def emit(paths, inc=INC, merged=os.path.join(ROOT, "profiles", "tuned_table.json")):
    """Merge sweep files into `merged` and write the planner's include `inc`:
    one initializer {M, N, K, dtype, has_c, {gemm_config}, group_m, xcd} per
    shape where a candidate won."""
    doc = {"commands": [], "shapes": {}}
    for p in paths:
        d = json.load(open(p))
        doc["commands"].append(d.get("command", ""))
        doc["shapes"].update(d["shapes"])
    slim = {"commands": doc["commands"], "shapes": {}}
    for name, s in doc["shapes"].items():
        t = dict(s)
        if "probed" in t:   # one line per probe: the configuration's fields in CFG_KEYS order, us or the error
            t["probed"] = ["%s: %s" % ("/".join(str(p["config"][k]) for k in CFG_KEYS),
                                       "%.2f us" % p["us"] if p.get("exit") == 0 else "exit %d %s" %
                                       (p.get("exit", -1), p.get("error", ""))) for p in t["probed"]]
            t["probed_fields"] = "/".join(CFG_KEYS)
        slim["shapes"][name] = t
    with open(merged, "w") as f:
        json.dump(slim, f, indent=1)
        f.write("\n")
    head = ["// Generated by python -m dense_tiled_gemm_02_amd.tune --emit (from %s); do not edit." %
            os.path.relpath(merged, ROOT),
            "// {M, N, K, dtype, has_c, {bm, bn, bk, stages, mfma, waves_m, waves_n, group_m, splitk, xcd_remap,",
            "//  kernel}, group_m, xcd}: the winners of the interleaved races, median times in the comments."]
    with open(inc, "w") as f:
        f.write("\n".join(head + table_lines(doc)) + "\n")
    print(inc)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--one", nargs=2, metavar=("SHAPE", "CONFIG"))
    ap.add_argument("--emit", nargs="+", metavar="SWEEP_JSON")
    ap.add_argument("--shapes", default=",".join(NAMED))
    ap.add_argument("--rounds", type=int, default=20)
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "tune_sweep.json"))
    a = ap.parse_args()
    if a.one:
        sys.exit(one(a.one[0], json.loads(a.one[1])))
    if a.emit:
        emit(a.emit)
        return
    sweep(a.shapes.split(","), a.rounds, a.out)


if __name__ == "__main__":
    main()
