"""Host checks of the per-shape tuning tool and of the table it freezes into
the planner (no GPU): the candidate space plans, the pruning rules hold, the
emitted include has the planner's entry layout, and every committed entry is
the plan the planner takes for its shape (engagement), unless the table is
switched off with GEMM_TUNED_TABLE=0, when the heuristic plans it."""
import json
import os
import re
import subprocess
import sys

import pytest

import dense_tiled_gemm_02_amd as g
from dense_tiled_gemm_02_amd import tune

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENTRY = re.compile(r"^\{(\d+), (\d+), (\d+), (\d), (\d), \{([\d, ]+)\}, (\d+), (\d)\},")
FIELDS = ("bm", "bn", "bk", "stages", "mfma", "waves_m", "waves_n", "group_m", "splitk", "xcd_remap", "kernel")


def committed_entries():
    out = []
    for line in open(tune.INC):
        m = ENTRY.match(line)
        if m:
            M, N, K, dt, c = (int(x) for x in m.groups()[:5])
            cfg = dict(zip(FIELDS, (int(x) for x in m.group(6).split(","))))
            out.append((M, N, K, dt, c, cfg, int(m.group(7))))
    return out


@pytest.mark.parametrize("name", sorted(tune.NAMED))
def test_candidates_plan_and_include_the_heuristic(name):
    M, N, K, dt, c = tune.NAMED[name]
    cands = tune.candidates(M, N, K, dt, c)
    keys = [tuple(x[k] for k in tune.CFG_KEYS) for x in cands]
    assert len(keys) == len(set(keys)) and len(keys) >= 20
    prob = g.problem(M, N, K, g.GEMM_BF16 if dt == "bf16" else g.GEMM_F16, c)
    dev = tune._fake_gfx950()
    for x in cands:
        got = g.gemm_plan_create_for(prob, dev, x).config.as_dict()
        assert all(got[k] == x[k] for k in tune.CFG_KEYS if k != "group_m"), (x, got)
    # the heuristic's tile is in the space (its GROUP_M may differ)
    h = tune.heuristic_config(M, N, K, dt, c)
    tiles = {tuple(x[k] for k in tune.CFG_KEYS if k != "group_m") for x in cands}
    assert tuple(h[k] for k in tune.CFG_KEYS if k != "group_m") in tiles


def test_prune_rules():
    M, N, K = 16, 8192, 8192
    kept, why = tune.prune(M, N, K, tune.candidates(M, N, K))
    for x in kept:
        if x["kernel"] != 2:
            assert x["bm"] <= 32 and x["bn"] <= 2 * N
        grid = -(-M // x["bm"]) * -(-N // x["bn"]) * x["splitk"]
        assert x["splitk"] == 1 or grid <= tune.CUS
        if x["kernel"] == 2 and x["splitk"] > 1:
            assert K // x["splitk"] >= 512
    assert sum(why.values()) > 0
    kept, _ = tune.prune(256, 256, 256, tune.candidates(256, 256, 256))
    assert all(x["splitk"] == 1 for x in kept if x["kernel"] == 3)   # 4 K steps: no slices


def test_emit_writes_the_planner_layout(tmp_path):
    w = dict(kernel=3, bm=256, bn=256, bk=64, stages=2, mfma=16, waves_m=2, waves_n=4, splitk=1, group_m=4)
    doc = {"command": "test", "shapes": {
        "a": {"M": 4096, "N": 4096, "K": 4096, "dtype": "bf16", "has_c": False, "winner": w,
              "best_us": 90.0, "planner_us": 97.0},
        "b": {"M": 1, "N": 2, "K": 3, "dtype": "f16", "has_c": True, "winner": None,
              "best_us": 1.0, "planner_us": 1.0}}}
    src = tmp_path / "s.json"
    src.write_text(json.dumps(doc))
    inc, merged = tmp_path / "t.inc", tmp_path / "m.json"
    tune.emit([str(src)], inc=str(inc), merged=str(merged))
    lines = [l for l in inc.read_text().splitlines() if ENTRY.match(l)]
    assert len(lines) == 1
    m = ENTRY.match(lines[0])
    assert tuple(int(x) for x in m.groups()[:5]) == (4096, 4096, 4096, 1, 0)
    cfg = dict(zip(FIELDS, (int(x) for x in m.group(6).split(","))))
    assert all(cfg[k] == w[k] for k in w) and int(m.group(7)) == 4
    assert set(json.loads(merged.read_text())["shapes"]) == {"a", "b"}


def test_committed_entries_are_what_the_planner_takes():
    dev = tune._fake_gfx950()
    for (M, N, K, dt, c, cfg, gm) in committed_entries():
        got = g.gemm_plan_create_for(g.problem(M, N, K, dt, bool(c)), dev).config.as_dict()
        for k in ("kernel", "bm", "bn", "bk", "stages", "mfma", "waves_m", "waves_n", "splitk"):
            assert got[k] == cfg[k], (M, N, K, k, got, cfg)
        assert got["group_m"] == min(gm, -(-M // cfg["bm"]))


def test_table_switch_restores_the_heuristic():
    """A fresh process with GEMM_TUNED_TABLE=0 plans each entry's shape by the
    heuristic; the plan must then be the configuration the sweep raced as
    the heuristic's (checked through profiles/tuned_table.json)."""
    entries = committed_entries()
    if not entries:
        pytest.skip("no tuned entries committed")
    doc = json.load(open(os.path.join(ROOT, "profiles", "tuned_table.json")))
    code = ("import json,sys; from dense_tiled_gemm_02_amd import tune; "
            "print(json.dumps([tune.heuristic_config(*tune.parse_shape(n)[1]) for n in sys.argv[1:]]))")
    names = sorted(doc["shapes"])
    env = dict(os.environ, GEMM_TUNED_TABLE="0")
    out = subprocess.run([sys.executable, "-c", code] + names, cwd=ROOT, env=env, check=True,
                         stdout=subprocess.PIPE, text=True).stdout
    for n, h in zip(names, json.loads(out.strip().splitlines()[-1])):
        assert h == doc["shapes"][n]["heuristic"], n
