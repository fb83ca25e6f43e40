"""Host-side tests of the C ABI and planner (CPU only: no kernel is launched).

The planner is a pure function of (problem, device facts), so it is tested
with a hand-made gfx950 device description: 256 CUs, 8 XCDs, 2.4 GHz,
160 KiB of LDS per CU.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import dense_tiled_gemm_02_amd as g
import dense_tiled_gemm_02_amd.mx as mx
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def fake_gfx950():
    d = g.gemm_device_info()
    d.arch, d.cu_count, d.xcd_count, d.clock_khz = 950, 256, 8, 2400000
    d.lds_per_cu = d.lds_per_wg = 160 * 1024
    d.wave_size = 64
    return d


def declared_functions(header="gemm.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(gemm\w*)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 14
    L = g.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(n for n, _, _ in g.SIGNATURES) == names
    mx_names = declared_functions("gemm_mx.h")
    assert len(mx_names) == 9
    L = mx.mxlib()
    for n in mx_names:
        assert hasattr(L, n), n
    assert sorted(n for n, _, _ in mx.MX_SIGNATURES) == mx_names
    # every header under include/ is covered
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["gemm.h", "gemm_mx.h"]


def test_status_strings():
    assert g.gemm_status_string(g.GEMM_OK) == "GEMM_OK"
    assert g.gemm_status_string(g.GEMM_ERR_UNSUPPORTED) == "GEMM_ERR_UNSUPPORTED"
    assert g.gemm_status_string(99) == "GEMM_ERR_UNKNOWN"


def test_lds_formula_worked_value():
    # FlagGems "Hygon optimization", section "Software pipelining": one A/B tile
    # pair of 64 x 64 x 32 fp16 is 8 KiB.
    assert g.gemm_lds_bytes(64, 64, 32, 1, g.GEMM_F16) == 8 * 1024
    assert g.gemm_lds_bytes(64, 64, 32, 2, g.GEMM_F16) == 16 * 1024
    assert g.gemm_lds_bytes(256, 256, 64, 2, g.GEMM_BF16) == 128 * 1024
    assert g.gemm_lds_bytes(0, 64, 32, 1, g.GEMM_F16) == -1


@pytest.mark.parametrize("npm,npn,gm", [(5, 3, 2), (16, 16, 8), (7, 11, 4), (1, 9, 8), (9, 1, 1),
                                        (32, 24, 8), (13, 13, 3)])
def test_tile_order_matches_enumerated_grouped_order(npm, npn, gm):
    want = oracle.grouped_order(npm, npn, gm)
    got = [g.gemm_tile_of_workgroup(w, npm, npn, gm, 1) for w in range(npm * npn)]
    assert got == want


@pytest.mark.parametrize("npm,npn,gm,x", [(16, 16, 8, 8), (32, 24, 8, 8), (5, 3, 2, 8), (7, 11, 4, 8),
                                          (3, 3, 1, 8), (10, 13, 4, 3)])
def test_xcd_permutation_is_a_bijection_with_contiguous_ranges(npm, npn, gm, x):
    grid = npm * npn
    order = oracle.grouped_order(npm, npn, gm)
    pos_of = {t: i for i, t in enumerate(order)}
    tiles = [g.gemm_tile_of_workgroup(w, npm, npn, gm, x) for w in range(grid)]
    assert sorted(tiles) == sorted(order)            # every tile exactly once
    # workgroups of one die (w % x) cover one contiguous run of the tile order
    for die in range(x):
        ps = sorted(pos_of[tiles[w]] for w in range(die, grid, x))
        assert ps == list(range(ps[0], ps[0] + len(ps))) if ps else True
        # and in dispatch order
        assert [pos_of[tiles[w]] for w in range(die, grid, x)] == ps


def test_tile_order_rejects_bad_arguments():
    with pytest.raises(g.GemmError) as e:
        g.gemm_tile_of_workgroup(9, 3, 3, 1, 1)
    assert e.value.status == g.GEMM_ERR_INVALID_ARG
    with pytest.raises(g.GemmError):
        g.gemm_tile_of_workgroup(0, 3, 3, 0, 1)


def plan(M, N, K, dt=g.GEMM_BF16, has_c=False, force=None, **ld):
    return g.gemm_plan_create_for(g.problem(M, N, K, dt, has_c, **ld), fake_gfx950(), force)



def test_plans_for_the_five_workloads_fit_the_device():
    cases = [(256, 256, 256, g.GEMM_F16, False), (1024, 1024, 1024, g.GEMM_F16, False),
             (4096, 4096, 4096, g.GEMM_BF16, False), (16, 8192, 8192, g.GEMM_BF16, False),
             (4000, 3000, 1000, g.GEMM_F16, True)]
    for M, N, K, dt, c in cases:
        p = plan(M, N, K, dt, c)
        cfg = p.config
        grid, threads, lds = g.gemm_plan_launch(p)
        assert lds <= 160 * 1024
        assert threads % 64 == 0 and threads <= 1024
        assert grid == -(-M // cfg.bm) * -(-N // cfg.bn) * cfg.splitk or cfg.kernel == 2
        assert lds == g.gemm_lds_bytes(cfg.bm, cfg.bn, cfg.bk, cfg.stages, dt) or cfg.kernel == 2
        assert "kernel=" in p.describe()
    assert plan(4096, 4096, 4096).config.kernel == 3          # direct-to-LDS family when aligned


def test_few_tiles_and_deep_k_take_k_slices():
    # 512 x 512 x 32768 at 128 x 128: 16 tiles, 512 K steps: 16 slices of 32 steps fill the CUs
    p = plan(512, 512, 32768)
    c = p.config
    assert c.kernel == 3 and (c.bm, c.bn) == (128, 128) and c.splitk == 16
    grid, _, _ = g.gemm_plan_launch(p)
    assert grid == 16 * 16
    need = g.gemm_workspace_size(p)
    assert need >= 16384 + 16 * 16 * 128 * 128 * 4               # counters + fp32 partial tiles
    # 1024^3: 16 K steps per tile, too shallow to pay for the fused reduce
    assert plan(1024, 1024, 1024, g.GEMM_F16).config.splitk == 1
    # one tile, K = 65536: capped at 16 slices
    c = plan(128, 128, 65536).config
    assert c.splitk == 16
    # the one-shot path has no workspace: no slices
    p = g.gemm_plan_create_for(g.problem(1024, 1024, 1024, g.GEMM_F16), fake_gfx950(), {"kernel": 3, "bm": 128,
                                                                                     "bn": 128, "splitk": 4})
    assert p.config.splitk == 4
    # the 256 x 256 tile keeps too many accumulators per lane for K slices
    with pytest.raises(g.GemmError) as e:
        plan(1024, 1024, 1024, force={"kernel": 3, "bm": 256, "bn": 256, "splitk": 2})
    assert e.value.status == g.GEMM_ERR_UNSUPPORTED


def test_key_includes_m():
    # "Tuning Triton kernels", section 3: M=1 and M=4096 with equal N, K must not share a tile.
    big = plan(4096, 4096, 4096).config
    small = plan(1, 4096, 4096).config
    assert (big.bm, big.bn, big.kernel) != (small.bm, small.bn, small.kernel)
    assert small.bm <= 16


def test_forced_config_is_honoured_or_rejected():
    p = plan(1024, 1024, 1024, g.GEMM_F16, force={"bm": 128, "bn": 128, "bk": 64, "mfma": 32})
    c = p.config
    assert (c.bm, c.bn, c.bk, c.mfma) == (128, 128, 64, 32)
    p = plan(1024, 1024, 1024, force={"group_m": 4, "xcd_remap": g.GEMM_XCD_OFF})
    assert p.config.group_m == 4 and p.config.xcd_remap == g.GEMM_XCD_OFF
    with pytest.raises(g.GemmError) as e:
        plan(1024, 1024, 1024, force={"bm": 48})
    assert e.value.status == g.GEMM_ERR_UNSUPPORTED
    small = fake_gfx950()
    small.lds_per_wg = 48 * 1024
    with pytest.raises(g.GemmError) as e:
        g.gemm_plan_create_for(g.problem(4096, 4096, 4096, g.GEMM_BF16), small, {"bm": 256, "bn": 256})
    assert e.value.status == g.GEMM_ERR_UNSUPPORTED


def test_unaligned_shapes_take_the_element_path():
    p = plan(100, 30, 17, g.GEMM_F16)
    assert "VEC" not in p.describe()
    assert "vec=0 " in p.describe()
    p = plan(128, 64, 64, g.GEMM_F16)
    assert "vec=1 " in p.describe()


def test_validation_errors():
    info = fake_gfx950()

    def status(prob, force=None):
        h = ctypes.c_void_p()
        s = g.lib().gemm_plan_create_for(ctypes.byref(prob), ctypes.byref(info), None, ctypes.byref(h))
        if h.value:
            g.lib().gemm_plan_destroy(h)
        return s

    assert status(g.problem(-1, 4, 4, g.GEMM_F16)) == g.GEMM_ERR_INVALID_ARG
    p = g.problem(4, 4, 4, g.GEMM_F16)
    p.dtype = 7
    assert status(p) == g.GEMM_ERR_INVALID_ARG
    p = g.problem(4, 4, 4, g.GEMM_F16)
    p.has_c = 2
    assert status(p) == g.GEMM_ERR_INVALID_ARG
    p = g.problem(4, 4, 4, g.GEMM_F16, True)
    p.sc_n = 2                                   # C and D must stay row-major
    assert status(p) == g.GEMM_ERR_UNSUPPORTED
    assert "column stride" in g.gemm_last_error()
    p = g.problem(4, 4, 4, g.GEMM_F16)
    p.sa_k = 2                                   # any A and B strides: element-wise path
    assert status(p) == g.GEMM_OK
    p = g.problem(4, 8, 4, g.GEMM_F16, ldd=4)    # output rows would overlap
    assert status(p) == g.GEMM_ERR_INVALID_ARG
    p = g.problem(1 << 31, 4, 4, g.GEMM_F16)
    assert status(p) == g.GEMM_ERR_UNSUPPORTED
    assert status(g.problem(0, 4, 4, g.GEMM_F16)) == g.GEMM_OK
    assert status(g.problem(4, 4, 0, g.GEMM_BF16, True)) == g.GEMM_OK
    assert g.lib().gemm_plan_create_for(None, ctypes.byref(info), None,
                                        ctypes.byref(ctypes.c_void_p())) == g.GEMM_ERR_INVALID_ARG


def test_run_rejects_bad_pointers_without_launching():
    p = plan(64, 64, 64, g.GEMM_F16, True)
    with pytest.raises(g.GemmError) as e:
        g.gemm_run(p, 4096, 8192, None, 1 << 20)         # C missing
    assert e.value.status == g.GEMM_ERR_INVALID_ARG
    p = plan(64, 64, 64, g.GEMM_F16)
    with pytest.raises(g.GemmError):
        g.gemm_run(p, 4096, 8192, 1 << 24, 1 << 20)      # C given, problem has none
    with pytest.raises(g.GemmError) as e:
        g.gemm_run(p, 1 << 20, 1 << 24, None, (1 << 20) + 64)   # D overlaps A
    assert "overlaps A" in e.value.detail
    with pytest.raises(g.GemmError):
        g.gemm_run(p, 1 << 20, 1 << 24, None, None)      # D missing
    # M = 0: nothing to do, nothing launched, even with no pointers
    g.gemm_run(plan(0, 64, 64, g.GEMM_F16), None, None, None, None)


def test_in_place_addend_allowed_only_with_equal_strides():
    p = plan(64, 64, 64, g.GEMM_F16, True)
    with pytest.raises(g.GemmError) as e:
        g.gemm_run(p, 1 << 20, 1 << 24, (1 << 28) + 2, 1 << 28)   # shifted alias
    assert "overlaps C" in e.value.detail


def test_decode_slab_rule():
    """M <= 32: the widest slab (128, 64 or 32 columns) whose slabs fill the
    CUs with 4 K slices; 128-column slabs instead when they fill the CUs with
    up to 8 slices of at least 512 k (1024 k for the 32-row slabs of M > 16;
    shapes outside the tuned table)."""
    def slab(M, N, K):
        c = plan(M, N, K).config
        return (c.kernel, c.bm, c.bn, c.splitk)
    assert slab(1, 2048, 2048) == (2, 16, 32, 4)
    assert slab(8, 4096, 4096) == (2, 16, 128, 8)
    assert slab(8, 4096, 2048) == (2, 16, 64, 4)       # 8 slices would be 256 k each
    assert slab(4, 8192, 8192) == (2, 16, 128, 4)
    assert slab(8, 6144, 4096) == (2, 16, 64, 2)
    assert slab(4, 4096, 6144) == (2, 16, 128, 8)
    assert slab(4, 4096, 11008) == (2, 16, 128, 8)
    assert slab(1, 4096, 14336) == (2, 16, 128, 8)
    assert slab(24, 4096, 14336) == (2, 32, 128, 8)
    assert slab(24, 4096, 4096) == (2, 32, 64, 4)       # 32-row slabs: slices of >= 1024 k


def test_one_row_of_tiles_streams_b():
    """A grid of one row of direct-to-LDS tiles reads each byte of B once per
    K slice: the planner swaps in the streamed-B twin of the tile (non-temporal
    B loads) where one is compiled (the 64 x 64 tile, row-major operands)."""
    for shape in ((32, 8192, 8192), (64, 8192, 8192), (64, 4096, 4096)):
        d = plan(*shape).describe()
        assert "gemm_dma_sb_kernel<64,64,64,2,2,16,4,1>" in d, (shape, d)
    d = plan(48, 2048, 8192).describe()                   # one row of K-sliced 128 x 128 tiles: no twin
    assert "gemm_dma_kernel<128,128,64,2,4,16,4,1" in d and "splitk=8" in d, d
    for shape, kw in (((128, 4096, 4096), {}), ((1024, 1024, 1024), {}), ((64, 4096, 4096), {"tb": True})):
        d = plan(*shape, **kw).describe()
        assert "gemm_dma_sb_kernel" not in d, (shape, d)
    # a forced 64 x 64 configuration on one row of tiles takes the twin too
    d = plan(64, 1024, 2048, force={"kernel": 3, "bm": 64, "bn": 64, "bk": 64, "stages": 4, "waves_m": 2,
                                    "waves_n": 2, "splitk": 2}).describe()
    assert "gemm_dma_sb_kernel" in d and "splitk=2" in d


def test_split_k_plans_need_and_check_a_workspace():
    p = plan(16, 8192, 8192)
    c = p.config
    assert c.kernel == 2 and c.bn >= 64 and c.splitk > 1          # 128-byte bands, K slices
    grid, _, _ = g.gemm_plan_launch(p)
    assert grid == -(-8192 // c.bn) * c.splitk
    need = g.gemm_workspace_size(p)
    assert need >= c.splitk * 8192 * 16 * 4
    with pytest.raises(g.GemmError) as e:
        g.gemm_run(p, 1 << 20, 1 << 30, None, 1 << 24)              # no workspace
    assert e.value.status == g.GEMM_ERR_WORKSPACE
    with pytest.raises(g.GemmError) as e:
        g.gemm_run(p, 1 << 20, 1 << 30, None, 1 << 24, 1 << 34, need - 4)
    assert e.value.status == g.GEMM_ERR_WORKSPACE
    with pytest.raises(g.GemmError) as e:
        g.gemm_workspace_init(p, None, 0)
    assert e.value.status == g.GEMM_ERR_WORKSPACE
    p1 = plan(16, 8192, 8192, force={"kernel": 2, "bn": 32, "splitk": 1})
    assert g.gemm_workspace_size(p1) == 0


def test_layouts_pick_matching_kernels():
    # A stored K x M and/or B stored N x K: direct-to-LDS variants of that layout
    for ta, tb in ((False, True), (True, False), (True, True)):
        p = plan(4096, 4096, 4096, ta=ta, tb=tb)
        lay = (1 if ta else 0) | (2 if tb else 0)
        assert p.config.kernel == 3 and p.describe().endswith("vec=1 layout=%d" % lay)
        assert ",lay%d>" % lay in p.describe()
    # row-major: the plain variants
    assert plan(4096, 4096, 4096).describe().endswith("vec=1 layout=0")
    # a transposed operand whose contiguous extent is not a multiple of 8: element path
    p = plan(4000, 1000, 1004, ta=True)             # M = 4000 is fine, but
    assert p.describe().endswith("vec=1 layout=1")
    p = plan(4004 - 2, 1000, 1000, ta=True)         # M % 8 != 0 for a K x M A
    assert p.describe().endswith("vec=0 layout=1")
    # strides that are neither (element-wise path, layout -1)
    pr = g.problem(64, 64, 64, g.GEMM_F16)
    pr.sa_m, pr.sa_k = 130, 2
    p = g.gemm_plan_create_for(pr, fake_gfx950())
    assert p.describe().endswith("vec=0 layout=-1")
    # the decode regime needs row-major operands; a transposed B goes to the tile ladder
    assert plan(16, 8192, 8192).config.kernel == 2
    assert plan(16, 8192, 8192, tb=True).config.kernel != 2


# ---------------------------------------------------------------- block-scaled (MX) path


def mx_plan(M, N, K, fmt="e4m3", **kw):
    return mx.gemm_mx_plan_create_for(mx.mx_problem(M, N, K, fmt, **kw), fake_gfx950())


def test_mx_plans_fit_the_device_and_pick_by_tile_count():
    for fmt in ("e4m3", "e5m2", "e2m1"):
        for (M, N, K) in [(4096, 4096, 4096), (512, 512, 1024), (16, 8192, 8192), (1000, 3000, 992)]:
            p = mx_plan(M, N, K, fmt)
            c = p.config
            grid, threads, lds = mx.gemm_mx_plan_launch(p)
            assert c.kernel == mx.KERNEL_MX and c.mfma == 32 and c.splitk >= 1
            assert c.bk == (256 if fmt == "e2m1" else 128)
            assert lds <= 160 * 1024 and threads in (128, 256, 512)
            assert grid == -(-M // c.bm) * -(-N // c.bn) * c.splitk
            assert (mx.gemm_mx_workspace_size(p) > 0) == (c.splitk > 1)
            assert ("fmt=%d/%d" % (mx.FORMATS[fmt], mx.FORMATS[fmt])) in p.describe()
    assert (mx_plan(4096, 4096, 4096).config.bm, mx_plan(4096, 4096, 4096).config.bn) == (256, 256)
    assert (mx_plan(512, 512, 1024).config.bm, mx_plan(512, 512, 1024).config.bn) == (64, 64)
    # decode regime: 32-row slabs with K slices and a workspace
    d = mx_plan(16, 8192, 8192, "e2m1")
    c = d.config
    assert (c.bm, c.bn, c.splitk) == (32, 64, 2)
    assert mx.gemm_mx_workspace_size(d) == 16384 + 128 * 2 * 32 * 64 * 4
    assert mx.gemm_mx_workspace_size(mx_plan(4096, 4096, 4096)) == 0
    # few square tiles over a deep K: slices of at least 8 K steps
    c = mx_plan(512, 512, 32768).config
    assert (c.bm, c.bn, c.splitk) == (128, 128, 16)
    p = mx_plan(4096, 4096, 4096, fmt_b="e5m2")
    assert "fmt=0/1" in p.describe()


def test_mx_forced_config_is_honoured_or_rejected():
    p = mx.gemm_mx_plan_create_for(mx.mx_problem(4096, 4096, 4096), fake_gfx950(), {"bm": 128, "bn": 256})
    assert (p.config.bm, p.config.bn) == (128, 256)
    for bad in ({"bm": 96}, {"bm": 256, "bn": 256, "splitk": 2}, {"mfma": 16}, {"kernel": 3}, {"splitk": 65}):
        with pytest.raises(g.GemmError) as e:
            mx.gemm_mx_plan_create_for(mx.mx_problem(4096, 4096, 4096), fake_gfx950(), bad)
        assert e.value.status == g.GEMM_ERR_UNSUPPORTED, bad


@pytest.mark.parametrize("kw,status", [
    ({"K": 40}, g.GEMM_ERR_UNSUPPORTED),                       # K not a multiple of 16
    ({"K": 48, "fmt_a": "e2m1"}, g.GEMM_ERR_UNSUPPORTED),      # E2M1: K a multiple of 32
    ({"lda": 136}, g.GEMM_ERR_UNSUPPORTED),                    # row stride not a multiple of 16
    ({"ldsb": 6}, g.GEMM_ERR_UNSUPPORTED),                     # scale stride not a multiple of 4
    ({"ldsa": 0}, g.GEMM_ERR_INVALID_ARG),                     # below ceil(K/32)
    ({"lda": 64}, g.GEMM_ERR_INVALID_ARG),                     # below the row's bytes
    ({"ldd": 100}, g.GEMM_ERR_INVALID_ARG),                    # output rows overlap
    ({"K": 48, "fmt_a": "e4m3", "fmt_b": "e2m1"}, g.GEMM_ERR_UNSUPPORTED),   # mixed widths: K a multiple of 32
    ({"K": 80, "fmt_a": "e2m3", "fmt_b": "e2m3"}, g.GEMM_ERR_UNSUPPORTED),   # FP6: K a multiple of 32
    ({"out": 3}, g.GEMM_ERR_INVALID_ARG),
    ({"M": -1}, g.GEMM_ERR_INVALID_ARG),
])
def test_mx_validation_errors(kw, status):
    args = dict(M=256, N=128, K=128, fmt_a="e4m3", fmt_b=None)
    for k in ("M", "N", "K", "fmt_a", "fmt_b"):
        if k in kw:
            args[k] = kw.pop(k)
    p = mx.mx_problem(args["M"], args["N"], args["K"], args["fmt_a"], args["fmt_b"], **kw)
    with pytest.raises(g.GemmError) as e:
        mx.gemm_mx_plan_create_for(p, fake_gfx950())
    assert e.value.status == status
    assert g.gemm_last_error()


def test_mx_run_rejects_bad_pointers_without_launching():
    p = mx_plan(256, 128, 128)
    with pytest.raises(g.GemmError) as e:
        mx.gemm_mx_run(p, 0x1000, 0x2000, 0x3000, 0x4000, None, None)
    assert e.value.status == g.GEMM_ERR_INVALID_ARG            # D is NULL
    with pytest.raises(g.GemmError) as e:
        mx.gemm_mx_run(p, 0x1008, 0x20000, 0x30000, 0x40000, None, 0x100000)
    assert e.value.status == g.GEMM_ERR_UNSUPPORTED            # A not 16-byte aligned
    with pytest.raises(g.GemmError) as e:
        mx.gemm_mx_run(p, 0x10000, 0x20002, 0x30000, 0x40000, None, 0x100000)
    assert e.value.status == g.GEMM_ERR_UNSUPPORTED            # SA not 4-byte aligned
    with pytest.raises(g.GemmError) as e:
        mx.gemm_mx_run(p, 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x100000)
    assert e.value.status == g.GEMM_ERR_INVALID_ARG            # C given without has_c
    with pytest.raises(g.GemmError) as e:                      # D overlaps A
        mx.gemm_mx_run(p, 0x100000, 0x200000, 0x300000, 0x400000, None, 0x100100)
    assert e.value.status == g.GEMM_ERR_INVALID_ARG
    d = mx_plan(16, 8192, 8192, "e2m1")                        # needs a workspace
    with pytest.raises(g.GemmError) as e:
        mx.gemm_mx_run(d, 0x100000, 0x2000000, 0x3000000, 0x8000000, None, 0x9000000)
    assert e.value.status == g.GEMM_ERR_WORKSPACE
    with pytest.raises(g.GemmError) as e:
        mx.gemm_mx_run(d, 0x100000, 0x2000000, 0x3000000, 0x8000000, None, 0x9000000, 0xA000010, 1 << 24)
    assert e.value.status == g.GEMM_ERR_WORKSPACE              # not 256-byte aligned
    # an empty output launches nothing and succeeds without any pointer
    mx.gemm_mx_run(mx_plan(0, 128, 128), None, None, None, None, None, None)


def test_rows_of_k_with_short_row_stride_leave_the_direct_kernel():
    """The direct-to-LDS kernel zeroes the rows past K of a row-major B (or a
    K x M A) through the descriptor range, which needs the row stride to be at
    least N (M); overlapping rows go to the register-staged kernel."""
    ok = plan(512, 512, 512)
    assert ok.config.kernel == 3
    pr = g.problem(512, 512, 512, g.GEMM_BF16, ldb=256)     # B rows overlap (ldb < N)
    p = g.gemm_plan_create_for(pr, fake_gfx950())
    assert p.config.kernel == 1
    pr = g.problem(512, 512, 512, g.GEMM_BF16, ta=True, lda=256)   # A stored K x M, lda < M
    p = g.gemm_plan_create_for(pr, fake_gfx950())
    assert p.config.kernel == 1
    # a k-contiguous operand may overlap its rows: the K tail is masked per lane
    pr = g.problem(512, 512, 512, g.GEMM_BF16, lda=256)     # A row-major, lda < K
    assert g.gemm_plan_create_for(pr, fake_gfx950()).config.kernel == 3


def test_tile_choice_by_rounds_of_workgroups():
    """The 8-wave tile and its ring depth are chosen by rounds of workgroups
    (tiles / (CUs x workgroups resident per CU)) times the tile's relative
    cost per round (fitted to forced runs on the device): a 256 x 256 grid
    that leaves CUs idle loses to smaller tiles that fill them."""
    def tile(M, N, K):
        c = plan(M, N, K).config
        return (c.bm, c.bn, c.stages)
    assert tile(4096, 4096, 4096) == (256, 256, 2)     # 256 tiles: one full round
    assert tile(3072, 3072, 4096) == (192, 256, 2)     # 192 tiles in one round (256 x 256: 144)
    assert tile(3584, 3584, 4096) == (256, 256, 2)     # 192 x 256 would need a second round
    assert tile(4000, 3000, 1000) == (192, 256, 2)     # 252 tiles in one round (256 x 256: 192)
    assert tile(2560, 2560, 4096) == (256, 128, 3)     # 200 tiles, 3-stage ring
    assert tile(4096, 2048, 8192) == (256, 128, 3)
    assert tile(2048, 2048, 4096) == (128, 128, 4)     # 256 tiles, one per CU: 4-stage ring
    assert tile(1536, 1536, 8192) == (128, 128, 4)
    c = plan(1024, 1024, 1024).config                  # small: 256 tiles of the 4-wave 64 x 64, no slices
    assert (c.bm, c.bn, c.stages, c.splitk, c.waves_m, c.waves_n) == (64, 64, 4, 1, 2, 2)
    assert tile(512, 512, 512) == (64, 64, 4)
    c = plan(512, 512, 32768).config                   # few tiles, deep K: K slices of 128 x 128 tiles
    assert (c.bm, c.bn, c.splitk) == (128, 128, 16)
    assert c.stages == 4                               # slices run the 4-stage tile, one workgroup per CU
    for shape, s in (((1024, 1024, 16384), 4), ((1024, 1024, 4096), 4), ((256, 8192, 8192), 2),
                     ((768, 768, 8192), 7), ((192, 8192, 8192), 2)):
        c = plan(*shape).config                        # wide or deep problems with few 128 x 128 tiles
        assert (c.bm, c.bn, c.stages, c.splitk) == (128, 128, 4, s), shape
    for shape, s in (((64, 8192, 8192), 2), ((128, 4096, 4096), 2), ((64, 4096, 4096), 4)):
        c = plan(*shape).config                        # few slices of 128 x 128: 64 x 64 tiles slice K
        assert (c.bm, c.bn, c.stages, c.splitk, c.waves_m, c.waves_n) == (64, 64, 4, s, 2, 2), shape
    c = plan(768, 768, 2048).config                    # two slices would not pay for the reduce
    assert (c.bm, c.bn, c.splitk) == (64, 64, 1)
    for ta, tb in ((True, False), (False, True), (True, True)):   # every layout has the ladder's variants
        for shape in ((2560, 2560, 4096), (2048, 2048, 4096), (1024, 1024, 1024)):
            p = plan(*shape, ta=ta, tb=tb)
            assert p.config.kernel == 3 and (p.config.bm, p.config.bn, p.config.stages) == tile(*shape)
        # the 192 x 256 tile is compiled for row-major operands only: the
        # other layouts keep 256 x 256 there, on the direct-to-LDS kernel
        p = plan(3072, 3072, 4096, ta=ta, tb=tb)
        assert p.config.kernel == 3 and (p.config.bm, p.config.bn, p.config.stages) == (256, 256, 2)
    c = plan(3072, 3072, 4092).config                  # K not a multiple of 8: no vector path, no 192 x 256
    assert (c.bm, c.bn) != (192, 256)


def test_mx_tile_choice_by_rounds_of_workgroups():
    def cfg(M, N, K):
        c = mx_plan(M, N, K).config
        return (c.bm, c.bn, c.stages)
    assert cfg(4096, 4096, 4096) == (256, 256, 2)
    assert cfg(3072, 3072, 4096) == (192, 256, 2)     # 192 tiles in one round (256 x 256: 144)
    assert cfg(4000, 3000, 1024) == (192, 256, 2)
    assert cfg(3584, 3584, 4096) == (256, 256, 2)     # 192 x 256 would need a second round
    assert cfg(2048, 2048, 4096) == (128, 128, 3)
    # two K slices of the ladder's 128 x 128 tiles when both fit in one round
    # and each keeps >= 16 K steps; not with fewer steps, not for 64 x 64
    for (M, N, K, fmt), s in (((192, 8192, 8192, "e4m3"), 2), ((256, 8192, 16384, "e2m1"), 2),
                              ((256, 8192, 4096, "e2m1"), 1), ((2048, 2048, 4096, "e4m3"), 1),
                              ((256, 4096, 8192, "e4m3"), 1)):
        c = mx_plan(M, N, K, fmt).config
        assert c.splitk == s, (M, N, K, fmt, c.bm, c.bn, c.splitk)
    assert cfg(2560, 2560, 4096)[:2] in ((256, 128), (128, 256)) and cfg(2560, 2560, 4096)[2] == 3
    assert cfg(4096, 2048, 8192)[:2] in ((256, 128), (128, 256))
    assert cfg(1024, 1024, 4096) == (64, 64, 3)          # 256 small tiles beat 4 K slices of 128 x 128
    assert cfg(512, 512, 2048) == (64, 64, 3)            # too shallow for slices
    c = mx_plan(512, 512, 16384).config                  # few tiles, deep K: K slices
    assert (c.bm, c.bn, c.splitk) == (128, 128, 16)


def test_forced_group_m_is_clamped_to_the_grid():
    """A forced GROUP_M above the number of M tiles orders the tiles exactly as
    a band of the whole grid; the planners store the clamped value (the
    kernels' band arithmetic is 32-bit) and the exported tile order agrees."""
    huge = 1 << 30
    p = plan(1024, 1024, 1024, force={"group_m": huge})
    npm = -(-1024 // p.config.bm)
    assert p.config.group_m == npm
    q = mx.gemm_mx_plan_create_for(mx.mx_problem(1024, 1024, 1024, "e4m3"), fake_gfx950(), {"group_m": huge})
    assert q.config.group_m == -(-1024 // q.config.bm)
    npm, npn = 5, 7
    for w in range(npm * npn):
        assert g.gemm_tile_of_workgroup(w, npm, npn, huge, 8) == g.gemm_tile_of_workgroup(w, npm, npn, npm, 8)


def test_skinny_kernel_needs_its_offsets_in_32_bits():
    """The decode kernels address a chunk of B with 32-bit byte offsets: a row
    of B wider than ~1 GiB / (chunk rows), or a row stride that large, goes to
    another kernel instead of reading zeros past the descriptor's range."""
    assert "gemm_skinny_kernel" in plan(16, 8192, 8192).describe()
    wide = plan(16, 17_000_000, 64)                    # 64 rows x 34 MB of a chunk > 2 GiB
    assert "gemm_skinny_kernel" not in wide.describe(), wide.describe()
    strided = plan(16, 1024, 4096, ldb=1 << 25)        # B row stride of 64 MiB
    assert "gemm_skinny_kernel" not in strided.describe(), strided.describe()
    near = plan(16, 1024, 4096, ldb=1 << 20)           # 2 MiB row stride: chunk offsets fit
    assert "gemm_skinny_kernel" in near.describe(), near.describe()


def test_static_scratch_entry_point_rejects_large_workspaces_before_any_device_call():
    """gemm_run_static (for callers that cannot allocate) provides at most
    GEMM_STATIC_SCRATCH_BYTES of workspace; a plan needing more is refused with
    GEMM_ERR_WORKSPACE and a message naming both sizes, before any device call
    (so this runs without a GPU)."""
    hdr = open(os.path.join(ROOT, "include", "gemm.h")).read()
    m = re.search(r"#define GEMM_STATIC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", hdr)
    assert m and int(m.group(1)) << 20 == g.GEMM_STATIC_SCRATCH_BYTES
    big = plan(2048, 2048, 65536, force={"kernel": 3, "bm": 128, "bn": 128, "waves_m": 2, "waves_n": 4,
                                         "stages": 4, "splitk": 16})
    need = ctypes.c_size_t()
    assert g.lib().gemm_workspace_size(big.handle, ctypes.byref(need)) == 0
    assert need.value > g.GEMM_STATIC_SCRATCH_BYTES
    st = g.lib().gemm_run_static(big.handle, None, None, None, None, None)
    assert st == g.GEMM_ERR_WORKSPACE
    msg = g.gemm_last_error()
    assert str(need.value) in msg and str(g.GEMM_STATIC_SCRATCH_BYTES) in msg, msg


def test_mx_routes_every_pair_to_the_tile_kernel():
    """Every pair of formats runs the LDS-staged tile kernel (kernel 4): pairs
    of one width (8-bit, or E2M1) over the whole ladder, the others (an FP6
    operand, or 8-bit with 4-bit) over its square tiles and the decode slab,
    with K slices where the planner takes them; the register-direct kernel
    (kernel 5) only when forced, for any pair."""
    dev = fake_gfx950()
    for fa, fb in (("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e2m1", "e2m1")):
        assert mx.gemm_mx_plan_create_for(mx.mx_problem(4096, 4096, 4096, fa, fb), dev).config.kernel == 4
    for fa, fb in (("e2m3", "e2m3"), ("e3m2", "e2m3"), ("e4m3", "e2m1"), ("e2m1", "e5m2"), ("e3m2", "e4m3")):
        for (M, N, K), tile in (((4096, 4096, 4096), (256, 256)), ((1024, 1024, 4096), (64, 64)),
                                ((2048, 2048, 4096), (128, 128)), ((16, 8192, 8192), (32, 64))):
            pl = mx.gemm_mx_plan_create_for(mx.mx_problem(M, N, K, fa, fb), dev)
            c = pl.config
            assert (c.kernel, c.bm, c.bn) == (4, tile[0], tile[1]), (fa, fb, M, N, K, pl.describe())
            assert "gemm_mx_kernel<%d,%d," % tile in pl.describe()
            assert pl.describe().endswith("fmt=%d/%d out=1" % (mx.FORMATS[fa], mx.FORMATS[fb]))
            assert c.bk == 128
        # the decode slab slices K; deep K with few tiles slices 128 x 128 tiles
        assert mx.gemm_mx_plan_create_for(mx.mx_problem(16, 8192, 8192, fa, fb), dev).config.splitk == 2
        assert mx.gemm_mx_plan_create_for(mx.mx_problem(512, 512, 16384, fa, fb), dev).config.splitk >= 4
        # tiles of the one-width ladder only
        with pytest.raises(g.GemmError) as e:
            mx.gemm_mx_plan_create_for(mx.mx_problem(4096, 4096, 4096, fa, fb), dev, {"bm": 256, "bn": 128})
        assert e.value.status == g.GEMM_ERR_UNSUPPORTED
        pl = mx.gemm_mx_plan_create_for(mx.mx_problem(4096, 4096, 4096, fa, fb), dev, {"kernel": 5})
        assert (pl.config.kernel, pl.config.bm, pl.config.bn, pl.config.splitk) == (5, 128, 128, 1)
        assert "gemm_mx_direct_kernel<%d,%d>" % (mx.FORMATS[fa], mx.FORMATS[fb]) in pl.describe()
    assert mx.gemm_mx_plan_create_for(mx.mx_problem(4096, 4096, 4096, "e2m1", "e2m1"), dev).config.bk == 256
    forced = mx.gemm_mx_plan_create_for(mx.mx_problem(1024, 1024, 1024), dev, {"kernel": 5})
    assert forced.config.kernel == 5
    # FP6 rows: 3K/4 bytes, the default leading dimension
    p = mx.mx_problem(64, 64, 256, "e2m3", "e3m2")
    assert (p.lda, p.ldb) == (192, 192)


def test_library_binds_to_torchs_hip_runtime():
    """Loading libgemm before torch would put two HIP runtimes in one process
    (torch's libraries ask for libamdhip64.so, libgemm for .so.7): the binding
    imports torch first, so the process holds one runtime."""
    code = ("import sys; import dense_tiled_gemm_02_amd as g; assert 'torch' not in sys.modules; g.lib(); "
            "assert 'torch' in sys.modules; "
            "maps = open('/proc/self/maps').read(); "
            "paths = {l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}; "
            "print(len(paths)); assert len(paths) == 1, paths")
    subprocess.run([sys.executable, "-c", code], cwd=ROOT, check=True)
