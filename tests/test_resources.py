"""Resource gate of the compiled kernel table (CPU).

The build writes the compiler's own resource report of every kernel in
libgemm.so (its kernel-resource-usage remarks: VGPRs, AGPRs, scratch bytes
per lane, spills, LDS, occupancy) to _build/kernel_resources.json.  A kernel
that needs scratch memory spills registers to memory inside its loop ("DCU
K100 节点初探", section 4.3: a non-zero scratch size in the compiler's report
means spills; FlagGems "Hygon optimization", section "Software pipelining":
check the resource report of a pipelined kernel).  Every compiled variant can
be reached through a forced configuration, so every one is gated.
"""
import json
import os
import subprocess

import pytest

from dense_tiled_gemm_02_amd import build

LDS_BYTES = 160 * 1024   # per workgroup on gfx950
FAMILIES = ("gemm_dma_kernel", "gemm_tile_kernel", "gemm_skinny_kernel", "gemm_mx_kernel", "gemm_i8_kernel",
            "gemm_mx_direct_kernel")


@pytest.fixture(scope="module")
def report():
    if not os.path.exists(build.RESOURCES):
        pytest.fail("no resource report at %s: run python -m dense_tiled_gemm_02_amd.build" % build.RESOURCES)
    r = json.load(open(build.RESOURCES))
    assert r["sources_sha256"] == build.source_digest(), (
        "the resource report is older than the sources: run python -m dense_tiled_gemm_02_amd.build")
    return r


def _demangle(names):
    out = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True).stdout
    return dict(zip(names, out.splitlines()))


def test_report_covers_every_kernel_family(report):
    names = _demangle(list(report["kernels"]))
    fam = {}
    for d in names.values():
        for f in FAMILIES:
            if f + "<" in d:
                fam[f] = fam.get(f, 0) + 1
    assert set(fam) == set(FAMILIES), fam
    assert fam["gemm_dma_kernel"] >= 40 and fam["gemm_mx_kernel"] >= 10, fam
    assert fam["gemm_i8_kernel"] >= 7 and fam["gemm_mx_direct_kernel"] >= 25, fam


def test_no_kernel_uses_scratch_or_spills_vector_registers(report):
    names = _demangle(list(report["kernels"]))
    bad = [(names[k], v) for k, v in report["kernels"].items()
           if v.get("ScratchSize", 0) != 0 or v.get("VGPRs Spill", 0) != 0 or v.get("Dynamic Stack") != "False"]
    assert not bad, "kernels with scratch / VGPR spills: %s" % bad


def test_register_and_lds_budgets(report):
    """Every kernel fits gfx950's 512 registers per lane (VGPRs + AGPRs, at one
    wave per SIMD) and 160 KiB of LDS per workgroup, and the one-wave-per-SIMD
    tiles hold their 256 accumulators in AGPRs."""
    names = _demangle(list(report["kernels"]))
    for k, v in report["kernels"].items():
        assert v["VGPRs"] + v.get("AGPRs", 0) <= 512, (names[k], v)
        assert v.get("LDS Size", 0) <= LDS_BYTES, (names[k], v)
        d = names[k]
        if "gemm_dma_kernel<256, 256, 64, 2, 2," in d:
            assert v["AGPRs"] == 256 and v["VGPRs"] <= 256 and v["Occupancy"] == 1, (d, v)
        if "gemm_dma_kernel<256, 256, 64, 2, 4, 16, 2," in d:   # the 4096^3 plan: two waves per SIMD
            assert v["VGPRs"] + v.get("AGPRs", 0) <= 256 and v["Occupancy"] >= 2, (d, v)


def _plan_name(demangled):
    """'void dtg::(anonymous namespace)::gemm_dma_kernel<256, 256, 64, 2, 4, 16,
    2, true, false, false>(dtg::KArgs)' -> 'gemm_dma_kernel<256,256,64,2,4,16,2,1,lay0>'
    (the form plans describe their kernel in)."""
    import bench
    return bench.plan_kernel_name(demangled)


def test_every_knob_reaches_the_compiled_kernel(report):
    """"Tuning Triton kernels", section 6: a knob the kernel accepts but never reads
    gives a fake win in a sweep.  Every tile knob here is a template argument:
    forcing a value selects a kernel whose name carries it, and that kernel is
    a distinct function in the compiler's report (its code is specialized on
    the value).  GROUP_M, the XCD order and the K slices are launch arguments,
    checked by the tile-order export and the GPU tests."""
    from test_abi import plan
    compiled = {_plan_name(d) for d in _demangle(list(report["kernels"])).values()}
    knobs = ("bm", "bn", "bk", "waves_m", "waves_n", "mfma", "stages")
    cases = [dict(kernel=3, bm=256, bn=256, bk=64, waves_m=2, waves_n=4, mfma=16, stages=2),
             dict(kernel=3, bm=256, bn=256, bk=64, waves_m=2, waves_n=4, mfma=32, stages=2),
             dict(kernel=3, bm=256, bn=256, bk=32, waves_m=2, waves_n=4, mfma=16, stages=4),
             dict(kernel=3, bm=256, bn=256, bk=64, waves_m=2, waves_n=2, mfma=16, stages=2),
             dict(kernel=3, bm=256, bn=128, bk=64, waves_m=4, waves_n=2, mfma=16, stages=3),
             dict(kernel=3, bm=256, bn=128, bk=64, waves_m=4, waves_n=2, mfma=16, stages=2),
             dict(kernel=3, bm=128, bn=128, bk=64, waves_m=2, waves_n=4, mfma=16, stages=4),
             dict(kernel=3, bm=128, bn=128, bk=32, waves_m=2, waves_n=4, mfma=16, stages=4),
             dict(kernel=3, bm=64, bn=64, bk=64, waves_m=2, waves_n=2, mfma=16, stages=4),
             dict(kernel=1, bm=64, bn=64, bk=32, waves_m=2, waves_n=2, mfma=16, stages=2),
             dict(kernel=1, bm=64, bn=64, bk=32, waves_m=2, waves_n=2, mfma=16, stages=1),
             dict(kernel=1, bm=128, bn=128, bk=64, waves_m=2, waves_n=2, mfma=32, stages=2)]
    seen = {}
    for cfg in cases:
        p = plan(2048, 2048, 2048, force=cfg)
        c = p.config
        for k in knobs:
            assert getattr(c, k) == cfg[k], (cfg, k, getattr(c, k))
        name = p.describe().split("kernel=")[1].split(" ")[0]
        assert name in compiled, name
        # both families: <BM, BN, BK, WM, WN, MF, ST, BF16, layout or vector flag>
        args = name.split("<")[1].rstrip(">").split(",")
        assert [int(a) for a in args[:7]] == [cfg[k] for k in ("bm", "bn", "bk", "waves_m", "waves_n",
                                                              "mfma", "stages")], (name, cfg)
        seen[tuple(cfg[k] for k in ("kernel",) + knobs)] = name
    # configurations that differ in any one knob run different compiled kernels
    assert len(set(seen.values())) == len(seen)
