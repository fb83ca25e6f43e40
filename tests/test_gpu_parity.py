"""Parity of the HIP path with the CPU oracle (GPU).

Every output must satisfy |d - ref| <= ulp_out(ref) + 2^-20 * sum_k |a_ik b_kj|
against the binary64 oracle on the same stored inputs; exact cases (identity,
integer inputs, dyadic rank-1) must match the correctly rounded exact result
bit for bit.  Sizes span several tiles and ragged tails; the large workloads
are checked in full where the oracle is fast and on sampled outputs otherwise,
in the launch configuration the benchmark times.
"""
import itertools

import numpy as np
import pytest
import torch

import dense_tiled_gemm_02_amd as g
import gemm_inputs
import oracle
from helpers import DT_CODE, check, gpu_run, sample_positions

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    torch.cuda.init()


def _inputs(M, N, K, dt, has_c, seed, dist="uniform", scale=1.0):
    A = gemm_inputs.draw((M, K), seed, dt, dist, scale)
    B = gemm_inputs.draw((K, N), seed + 1, dt, dist, scale)
    C = gemm_inputs.draw((M, N), seed + 2, dt, dist, scale) if has_c else None
    return A, B, C


# ---------------------------------------------------------------- workloads


@pytest.mark.parametrize("name", ["square_f16_256", "square_f16_1024", "skinny_bf16_16x8192",
                                  "tail_f16_4000x3000x1000_c", "deepk_bf16_512x512x32768"])
def test_workload_full_parity(name):
    w = gemm_inputs.WORKLOADS[name]
    A, B, C = gemm_inputs.make(w)
    print("case", name, flush=True)
    D = gpu_run(A, B, C)
    check(A, B, C, D, w.dtype, label=name)


def test_workload_4096_full_parity():
    """Every one of the 16.8 M outputs of the benchmark's workload, in the
    launch configuration the benchmark times (the planner's plan), against
    the full binary64 product (a few seconds of the oracle on the host)."""
    w = gemm_inputs.WORKLOADS["square_bf16_4096"]
    A, B, C = gemm_inputs.make(w)
    print("case", w.name, g.plan_for(A.cuda(), B.cuda(), None, None).describe(), flush=True)
    D = gpu_run(A, B, C)
    check(A, B, C, D, w.dtype, label=w.name)
    # every output finite and of the expected scale (property at any size)
    Df = D.float()
    assert torch.isfinite(Df).all()
    # A, B entries N(0,1)/64: each output has variance K * (1/64)^4, std 1/64
    assert 0.9 / 64 < Df.std().item() < 1.1 / 64


# ---------------------------------------------------------------- ragged shapes

ODD = [1, 2, 7, 15, 16, 17, 31, 33, 63, 65, 127, 129]


def _odd_cases():
    rng = np.random.default_rng(3)
    all_ = list(itertools.product(ODD, ODD, ODD))
    pick = rng.choice(len(all_), 40, replace=False)
    return [all_[i] for i in sorted(pick)] + [(1, 1, 1), (129, 129, 129), (1, 129, 1), (129, 1, 129)]


@pytest.mark.parametrize("mnk", _odd_cases())
def test_odd_shapes(mnk):
    M, N, K = mnk
    for dt, has_c in (("f16", True), ("bf16", False)):
        A, B, C = _inputs(M, N, K, dt, has_c, seed=M * 10007 + N * 101 + K)
        D = gpu_run(A, B, C)
        check(A, B, C, D, dt, label="%s %dx%dx%d c=%d" % (dt, M, N, K, has_c))


@pytest.mark.parametrize("shape", [(300, 200, 136), (520, 264, 1000), (96, 1000, 72)])
def test_every_compiled_variant(shape):
    """Each compiled tile variant (both kernel families), forced, passes on a
    ragged shape; variants with the same instruction shape agree bit for bit
    (same k-block summation order)."""
    M, N, K = shape
    for dt in ("f16", "bf16"):
        A, B, C = _inputs(M, N, K, dt, True, seed=M + N + K)
        by_mf = {}
        for cfg in _variants(dt):
            D = gpu_run(A, B, C, config=cfg)
            check(A, B, C, D, dt, label="%s %s %s" % (dt, shape, cfg))
            key = cfg["mfma"]
            if key in by_mf:
                assert torch.equal(by_mf[key][1].view(torch.int16), D.view(torch.int16)), (cfg, by_mf[key][0])
            else:
                by_mf[key] = (cfg, D)


def _variants(dt):
    import ctypes
    seen = []
    for bm, bn, bk, st, mf, wm, wn in [(256, 256, 64, 2, 32, 2, 4),
                                       (256, 128, 64, 2, 16, 2, 2), (256, 128, 64, 2, 32, 2, 2),
                                       (128, 256, 64, 2, 16, 2, 2), (128, 128, 64, 2, 16, 2, 2),
                                       (128, 128, 64, 2, 32, 2, 2), (128, 128, 64, 1, 16, 2, 2),
                                       (128, 128, 32, 2, 16, 2, 2), (64, 64, 64, 2, 16, 2, 2),
                                       (64, 64, 32, 2, 16, 2, 2), (64, 64, 32, 1, 16, 2, 2),
                                       (32, 32, 32, 2, 16, 2, 2), (16, 64, 64, 2, 16, 1, 4)]:
        seen.append(dict(bm=bm, bn=bn, bk=bk, stages=st, mfma=mf, waves_m=wm, waves_n=wn, kernel=1))
    for bm, bn, bk, st, mf, wm, wn in [(256, 256, 64, 2, 16, 2, 4), (256, 256, 32, 4, 16, 2, 4),
                                       (256, 256, 64, 2, 32, 2, 4), (256, 256, 32, 4, 32, 2, 4),
                                       (256, 128, 64, 3, 16, 2, 2), (256, 128, 64, 2, 16, 2, 2),
                                       (128, 256, 64, 2, 16, 2, 2), (128, 128, 64, 2, 16, 2, 2),
                                       (128, 128, 64, 4, 16, 2, 2), (128, 128, 64, 2, 32, 2, 2),
                                       (128, 128, 64, 2, 16, 2, 4), (256, 128, 64, 2, 16, 4, 2),
                                       (128, 256, 64, 2, 16, 2, 4), (256, 128, 64, 3, 16, 4, 2),
                                       (128, 256, 64, 3, 16, 2, 4), (64, 64, 64, 4, 16, 2, 2),
                                       (192, 256, 64, 2, 16, 2, 4),
                                       # one wave per SIMD, accumulators in AGPRs
                                       (256, 256, 64, 2, 32, 2, 2), (256, 256, 64, 2, 16, 2, 2)]:
        seen.append(dict(bm=bm, bn=bn, bk=bk, stages=st, mfma=mf, waves_m=wm, waves_n=wn, kernel=3))
    return seen


DMA_SPLIT = [(128, 128, 64, 2, 16, 2, 4), (128, 128, 64, 4, 16, 2, 4), (128, 128, 64, 2, 16, 2, 2),
             (128, 128, 64, 2, 32, 2, 2),
             (128, 128, 64, 4, 16, 2, 2), (256, 128, 64, 2, 16, 4, 2), (128, 256, 64, 2, 16, 2, 4),
             (64, 64, 64, 4, 16, 2, 2)]


@pytest.mark.parametrize("mnk", [(64, 4096, 4096), (128, 4096, 4096), (64, 8192, 8192), (96, 2000, 4136)])
def test_planned_k_slices_of_small_tiles(mnk):
    """Short, wide problems whose planned K slices run on 64 x 64 tiles: the
    planner's plan, full parity with the oracle, with an addend, and the same
    bits on a second run."""
    M, N, K = mnk
    A, B, C = _inputs(M, N, K, "bf16", True, seed=M + N + K)
    ref, S = oracle.gemm_f64(gemm_inputs.bits(A), gemm_inputs.bits(B), gemm_inputs.bits(C), "bf16")
    desc = g.plan_for(A.cuda(), B.cuda(), C.cuda()).describe()
    print("planned", mnk, desc, flush=True)
    D1 = gpu_run(A, B, C)
    D2 = gpu_run(A, B, C)
    n, worst, first = oracle.tol_check(gemm_inputs.bits(D1), ref, S, "bf16")
    assert n == 0, "%s %s: %d outside the bound (worst %.3g, first %d)" % (mnk, desc, n, worst, first)
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16)), (mnk, desc)


@pytest.mark.parametrize("N,K,splits", [(1024, 2048, 2), (520, 1000, 1), (2048, 4096, 4)])
def test_streamed_b_twin_is_bitwise_the_plain_kernel(N, K, splits):
    """One row of 64 x 64 tiles runs the streamed-B twin (non-temporal B
    loads); the same rows inside a two-row problem run the plain kernel.  The
    arithmetic is the same, so those rows agree bit for bit; the one-row
    result also passes the oracle."""
    cfg = dict(kernel=3, bm=64, bn=64, bk=64, stages=4, mfma=16, waves_m=2, waves_n=2, splitk=splits)
    A2, B, C2 = _inputs(128, N, K, "bf16", True, seed=N + K + splits)
    A1, C1 = A2[:64].contiguous(), C2[:64].contiguous()
    d1 = g.plan_for(A1.cuda(), B.cuda(), C1.cuda(), None, cfg).describe()
    d2 = g.plan_for(A2.cuda(), B.cuda(), C2.cuda(), None, cfg).describe()
    print("twin", d1, "|", d2, flush=True)
    assert "gemm_dma_sb_kernel" in d1 and "gemm_dma_sb_kernel" not in d2
    D1 = gpu_run(A1, B, C1, config=cfg)
    D2 = gpu_run(A2, B, C2, config=cfg)
    check(A1, B, C1, D1, "bf16", label="streamed-B %dx%dx%d" % (64, N, K))
    assert torch.equal(D1.view(torch.int16), D2[:64].view(torch.int16))


@pytest.mark.parametrize("mnk", [(300, 200, 1000), (130, 264, 2056), (128, 128, 4096), (520, 264, 200)])
def test_dma_split_k(mnk):
    """K slices across workgroups in the direct-to-LDS kernel (last arriver sums
    the fp32 partials in slice order): ragged M/N edges, a K tail inside the
    last slice, slices left without K steps (16 slices of a 4-step K), with
    and without C; every result inside the bound, and each config run twice
    gives the same bits whichever workgroup happened to arrive last."""
    M, N, K = mnk
    for dt, has_c in (("bf16", True), ("f16", False)):
        A, B, C = _inputs(M, N, K, dt, has_c, seed=3 * M + 5 * N + K)
        Ab, Bb = gemm_inputs.bits(A), gemm_inputs.bits(B)
        Cb = gemm_inputs.bits(C) if C is not None else None
        ref, S = oracle.gemm_f64(Ab, Bb, Cb, dt)
        for bm, bn, bk, st, mf, wm, wn in DMA_SPLIT:
            for sk in (2, 3, 5, 16):
                cfg = dict(kernel=3, bm=bm, bn=bn, bk=bk, stages=st, mfma=mf, waves_m=wm, waves_n=wn, splitk=sk)
                D1 = gpu_run(A, B, C, config=cfg)
                D2 = gpu_run(A, B, C, config=cfg)
                n, worst, first = oracle.tol_check(gemm_inputs.bits(D1), ref, S, dt)
                assert n == 0, "%s %s %s: %d outside the bound (worst %.3g, first %d)" % (dt, mnk, cfg, n, worst,
                                                                                         first)
                assert torch.equal(D1.view(torch.int16), D2.view(torch.int16)), (dt, mnk, cfg)


def test_split_plans_share_one_workspace():
    """A skinny split plan and a direct-to-LDS split plan take turns on one
    workspace (the counters sit in the same fixed region and every launch
    leaves them at zero): every result correct and repeatable."""
    A1, B1, C1 = _inputs(16, 2048, 2048, "bf16", True, seed=5)
    A2, B2, C2 = _inputs(384, 256, 3072, "bf16", True, seed=6)
    d1 = [t.cuda() for t in (A1, B1, C1)]
    d2 = [t.cuda() for t in (A2, B2, C2)]
    pa = g.plan_for(*d1, None, dict(kernel=2, bn=128, splitk=4))
    pb = g.plan_for(*d2, None, dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=4, splitk=6))
    need = max(g.gemm_workspace_size(pa), g.gemm_workspace_size(pb))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    g.gemm_workspace_init(pb, ws.data_ptr(), need, st)
    outs = []
    for i in range(6):
        pl, (a, b, c), (M, N) = (pa, d1, (16, 2048)) if i % 2 == 0 else (pb, d2, (384, 256))
        D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        g.gemm_run(pl, a.data_ptr(), b.data_ptr(), c.data_ptr(), D.data_ptr(), ws.data_ptr(), need, st)
        outs.append(D)
    torch.cuda.synchronize()
    for i, D in enumerate(outs):
        A, B, C = (A1, B1, C1) if i % 2 == 0 else (A2, B2, C2)
        check(A, B, C, D.cpu(), "bf16", label="shared workspace %d" % i)
        assert torch.equal(outs[i % 2].view(torch.int16), D.view(torch.int16))


SKINNY = [(256, 4, 32, 2), (128, 4, 32, 3), (128, 4, 32, 4), (128, 2, 32, 8), (128, 2, 32, 6), (128, 8, 32, 2), (64, 4, 64, 3), (64, 8, 64, 2), (32, 8, 64, 3), (16, 8, 64, 3)]


@pytest.mark.parametrize("mnk", [(16, 1000, 1000), (1, 520, 264), (5, 4096, 512), (16, 64, 64),
                                 (9, 136, 8), (16, 8192, 1032), (16, 1024, 4096)])
def test_skinny_variants(mnk):
    """The skinny-M kernels on ragged shapes (N and K tails, M < 16, K split over
    waves and over 1-8 workgroup slices, some slices and waves left without
    work); kernels with the same K partition (waves, chunk depth, slices, and
    chunk order: slabs of 128 columns or more walk their chunks rotated) agree
    bit for bit whatever their slab width."""
    M, N, K = mnk
    for dt, has_c in (("bf16", True), ("f16", False)):
        A, B, C = _inputs(M, N, K, dt, has_c, seed=M + 7 * N + 13 * K)
        by_part = {}
        for bn, nw, ck, st in SKINNY:
            for sk in (1, 2, 3, 8):
                cfg = dict(kernel=2, bn=bn, waves_n=nw, bk=ck, stages=st, splitk=sk)
                D = gpu_run(A, B, C, config=cfg)
                check(A, B, C, D, dt, label="%s %s %s" % (dt, mnk, cfg))
                key = (nw, ck, sk, bn >= 128)
                if key in by_part:
                    assert torch.equal(by_part[key].view(torch.int16), D.view(torch.int16)), cfg
                else:
                    by_part[key] = D


SKINNY32 = [(128, 8, 32, 2), (128, 4, 32, 3), (64, 8, 32, 3), (32, 8, 32, 3)]


@pytest.mark.parametrize("mnk", [(17, 1000, 1000), (24, 520, 264), (32, 4096, 512), (32, 64, 64),
                                 (20, 8, 1024)])
def test_skinny32_variants(mnk):
    """The 32-row skinny kernels (two MFMA row blocks) for 16 < M <= 32, with
    ragged N and K, over 1-8 workgroup slices; equal K partitions (with the
    chunk order: rotated for slabs of 128 columns or more) agree bit for bit
    whatever the slab width."""
    M, N, K = mnk
    for dt, has_c in (("bf16", True), ("f16", False)):
        A, B, C = _inputs(M, N, K, dt, has_c, seed=M + 11 * N + 3 * K)
        by_part = {}
        for bn, nw, ck, st in SKINNY32:
            for sk in (1, 2, 3, 8):
                cfg = dict(kernel=2, bm=32, bn=bn, waves_n=nw, bk=ck, stages=st, splitk=sk)
                D = gpu_run(A, B, C, config=cfg)
                check(A, B, C, D, dt, label="%s %s %s" % (dt, mnk, cfg))
                key = (nw, ck, sk, bn >= 128)
                if key in by_part:
                    assert torch.equal(by_part[key].view(torch.int16), D.view(torch.int16)), cfg
                else:
                    by_part[key] = D


@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 17, 24, 32])
def test_decode_buckets(m):
    """The planner's decode regime (M bucketed to 16- or 32-row slabs), with a
    workspace (K slices) and through the one-shot entry point (none)."""
    N, K = 4096, 4096
    A, B, C = _inputs(m, N, K, "bf16", m % 2 == 0, seed=700 + m, dist="normal", scale=1 / 64)
    D = gpu_run(A, B, C)
    check(A, B, C, D, "bf16", label="decode M=%d" % m)
    dA, dB = A.cuda(), B.cuda()
    dC = C.cuda() if C is not None else None
    pl = g.plan_for(dA, dB, dC, None)
    assert pl.config.kernel == 2 and pl.config.bm == (16 if m <= 16 else 32), pl.describe()
    D1 = torch.full((m, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    strides = [K, 1, N, 1, N if C is not None else 0, 1 if C is not None else 0, N, 1]
    g.gemm(dA.data_ptr(), dB.data_ptr(), dC.data_ptr() if dC is not None else None, D1.data_ptr(), m, N, K,
           strides, g.GEMM_BF16, 1 if C is not None else 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    check(A, B, C, D1.cpu(), "bf16", label="decode one-shot M=%d" % m)


@pytest.mark.parametrize("mnk", [(1, 4096, 11008), (16, 4096, 14336), (1, 4096, 8192), (16, 14336, 4096),
                                 (4, 6144, 4096)])
def test_decode_planned_shapes(mnk):
    """The planned decode plans of long-K and wide shapes (128-column slabs
    with 8 K slices, the tuned entries, unsliced 64-column slabs), every
    output against the oracle."""
    M, N, K = mnk
    A, B, C = _inputs(M, N, K, "bf16", M % 2 == 0, seed=M + N + K, dist="normal", scale=1 / 64)
    D = gpu_run(A, B, C)
    check(A, B, C, D, "bf16", label="decode %s" % (mnk,))


def test_skinny_workspace_reuse():
    """Slab counters reset themselves: many launches (and two plans) on one
    workspace all give the same, correct result."""
    M, N, K = 16, 2048, 2048
    A, B, C = _inputs(M, N, K, "bf16", True, seed=99)
    dA, dB, dC = A.cuda(), B.cuda(), C.cuda()
    pl4 = g.plan_for(dA, dB, dC, None, dict(kernel=2, bn=128, splitk=4))
    pl8 = g.plan_for(dA, dB, dC, None, dict(kernel=2, bn=64, splitk=8))
    need = max(g.gemm_workspace_size(pl4), g.gemm_workspace_size(pl8))
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    g.gemm_workspace_init(pl4, ws.data_ptr(), need, st)
    outs = []
    for i in range(6):
        pl = pl4 if i % 2 == 0 else pl8
        D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        g.gemm_run(pl, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), D.data_ptr(), ws.data_ptr(), need, st)
        outs.append(D)
    torch.cuda.synchronize()
    for i, D in enumerate(outs):
        check(A, B, C, D.cpu(), "bf16", label="reuse %d" % i)
        assert torch.equal(outs[i % 2].view(torch.int16), D.view(torch.int16))
    with pytest.raises(g.GemmError) as e:
        g.gemm_run(pl4, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), outs[0].data_ptr(), None, 0, st)
    assert e.value.status == g.GEMM_ERR_WORKSPACE


def test_skinny_rejects_tall_problems():
    with pytest.raises(g.GemmError) as e:
        g.gemm_plan_create(g.problem(32, 64, 64, g.GEMM_BF16), 0, dict(kernel=2))
    assert e.value.status == g.GEMM_ERR_UNSUPPORTED


@pytest.mark.parametrize("gm,xcd", [(1, 2), (4, 2), (8, 2), (8, 1), (3, 1)])
def test_group_and_xcd_orders_are_bitwise_identical(gm, xcd):
    A, B, C = _inputs(1000, 704, 256, "bf16", False, seed=77)
    base = gpu_run(A, B, C, config={"bm": 128, "bn": 128, "group_m": 1, "xcd_remap": 2})
    D = gpu_run(A, B, C, config={"bm": 128, "bn": 128, "group_m": gm, "xcd_remap": xcd})
    assert torch.equal(base.view(torch.int16), D.view(torch.int16))


# ---------------------------------------------------------------- exact cases


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_identity_with_subnormals_is_exact(dt):
    M, N = 200, 136
    rng = np.random.default_rng(5)
    x = rng.uniform(-1, 1, (M, N))
    tiny = 2.0 ** -20 if dt == "f16" else 2.0 ** -130
    x[rng.random((M, N)) < 0.2] *= tiny
    B = gemm_inputs.from_bits(oracle.encode_rne(x, dt), dt)
    I = torch.eye(M).to(gemm_inputs.TORCH_DTYPES[dt])
    D = gpu_run(I, B)
    # the exact result is B itself, except that 0 + (-0) = +0
    want = oracle.encode_rne(oracle.decode(gemm_inputs.bits(B), dt) + 0.0, dt)
    assert np.array_equal(gemm_inputs.bits(D), want)
    bv = np.abs(oracle.decode(gemm_inputs.bits(B), dt))
    assert np.count_nonzero((bv > 0) & (bv < (2.0 ** -14 if dt == "f16" else 2.0 ** -126))) > 100
    # with an addend: D = round(B + C), B + C exact in binary64
    C = gemm_inputs.draw((M, N), 9, dt)
    D = gpu_run(I, B, C)
    want = oracle.encode_rne(oracle.decode(gemm_inputs.bits(B), dt) + oracle.decode(gemm_inputs.bits(C), dt), dt)
    assert np.array_equal(gemm_inputs.bits(D), want)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_integer_inputs_are_exact(dt):
    M, N, K = 333, 250, 28          # |D| <= 9*28 + 3 = 255: exact in both types
    rng = np.random.default_rng(6)
    Ai, Bi, Ci = rng.integers(-3, 4, (M, K)), rng.integers(-3, 4, (K, N)), rng.integers(-3, 4, (M, N))
    T = gemm_inputs.TORCH_DTYPES[dt]
    A, B, C = (torch.from_numpy(x.astype(np.float32)).to(T) for x in (Ai, Bi, Ci))
    D = gpu_run(A, B, C)
    assert np.array_equal(D.float().numpy(), (Ai @ Bi + Ci).astype(np.float32))


def test_rank_one_dyadic_is_exact():
    M, N, K = 130, 90, 512
    rng = np.random.default_rng(8)
    u = 2.0 ** rng.integers(-4, 2, M) * rng.choice([-1, 1], M)
    v = 2.0 ** rng.integers(-4, 2, N)
    A = torch.from_numpy(np.repeat(u[:, None], K, 1)).to(torch.bfloat16)
    B = torch.from_numpy(np.repeat(v[None, :], K, 0)).to(torch.bfloat16)
    D = gpu_run(A, B)
    assert np.array_equal(D.double().numpy(), K * np.outer(u, v))


# ---------------------------------------------------------------- edges and invariants


def test_k_zero_gives_c_and_m_zero_is_a_no_op():
    C = gemm_inputs.draw((40, 24), 1, "f16")
    A = torch.empty((40, 0), dtype=torch.float16)
    B = torch.empty((0, 24), dtype=torch.float16)
    D = gpu_run(A, B, C)
    assert torch.equal(D.view(torch.int16), C.view(torch.int16))
    D = gpu_run(A, B)
    assert torch.equal(D, torch.zeros_like(D))
    out = torch.full((0, 24), 1.0, dtype=torch.float16, device="cuda")
    g.matmul(torch.empty((0, 8), dtype=torch.float16, device="cuda"),
             torch.ones((8, 24), dtype=torch.float16, device="cuda"), out=out)
    torch.cuda.synchronize()


def test_guard_band_untouched():
    M, N, K = 257, 129, 96
    A, B, C = _inputs(M, N, K, "f16", True, seed=11)
    big = torch.full((M + 64, N + 64), 7.0, dtype=torch.float16, device="cuda")
    D = big[32:32 + M, 16:16 + N]
    g.matmul(A.cuda(), B.cuda(), C.cuda(), out=D)
    torch.cuda.synchronize()
    host = big.cpu()
    mask = torch.ones_like(host, dtype=torch.bool)
    mask[32:32 + M, 16:16 + N] = False
    assert torch.all(host[mask] == 7.0)
    check(A, B, C, host[32:32 + M, 16:16 + N].contiguous(), "f16", label="strided D")


def test_in_place_addend():
    M, N, K = 300, 200, 64
    A, B, C = _inputs(M, N, K, "bf16", True, seed=12)
    dC = C.cuda()
    g.matmul(A.cuda(), B.cuda(), dC, out=dC)
    torch.cuda.synchronize()
    check(A, B, C, dC.cpu(), "bf16", label="in place")


def test_unaligned_base_uses_element_path():
    M, N, K = 190, 130, 200
    A0 = gemm_inputs.draw((M * K + 1,), 13, "f16")
    A = A0[1:].view(M, K)                 # base address 2 bytes past a 16-byte boundary
    B = gemm_inputs.draw((K, N), 15, "f16")
    dA = A0.cuda()[1:].view(M, K)
    D = g.matmul(dA, B.cuda())
    torch.cuda.synchronize()
    check(A, B, None, D.cpu(), "f16", label="unaligned")


def test_run_to_run_bitwise_identical():
    w = gemm_inputs.WORKLOADS["tail_f16_4000x3000x1000_c"]
    A, B, C = gemm_inputs.make(w)
    dA, dB, dC = A.cuda(), B.cuda(), C.cuda()
    D1 = g.matmul(dA, dB, dC)
    D2 = g.matmul(dA, dB, dC)
    torch.cuda.synchronize()
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))


def test_one_shot_entry_point():
    M, N, K = 100, 72, 40
    A, B, C = _inputs(M, N, K, "bf16", True, seed=16)
    dA, dB, dC = A.cuda(), B.cuda(), C.cuda()
    D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    g.gemm(dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), D.data_ptr(), M, N, K,
           [K, 1, N, 1, N, 1, N, 1], g.GEMM_BF16, 1, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    check(A, B, C, D.cpu(), "bf16", label="one-shot")


# ---------------------------------------------------------------- operand layouts


def _placed(X, transposed, pad):
    """X (CPU, rows x cols) on the GPU as a view with X's shape whose storage is
    row-major (rows x (cols + pad)) or, transposed, (cols x (rows + pad))."""
    r, c = X.shape
    if transposed:
        st = torch.zeros((c, r + pad), dtype=X.dtype)
        st[:, :r] = X.t()
        return st.cuda()[:, :r].t()
    st = torch.zeros((r, c + pad), dtype=X.dtype)
    st[:, :c] = X
    return st.cuda()[:, :c]


LAYOUT_TILES = [dict(kernel=3, bm=256, bn=256, waves_m=2, waves_n=4), dict(kernel=3, bm=256, bn=128, waves_m=4, waves_n=2),
                dict(kernel=3, bm=128, bn=256, waves_m=2, waves_n=4), dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=4),
                dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=4, splitk=3), None]


@pytest.mark.parametrize("mnk", [(520, 264, 200), (384, 640, 1000), (136, 1000, 520)])
def test_operand_layouts(mnk):
    """A stored K x M and / or B stored N x K (padded leading dimensions):
    the direct-to-LDS variants for each layout, and the planner's choice, all
    inside the bound; for a fixed tile every layout gives the same bits (the
    fragments, hence the accumulation order, do not depend on the layout)."""
    M, N, K = mnk
    for dt, has_c in (("bf16", True), ("f16", False)):
        A, B, C = _inputs(M, N, K, dt, has_c, seed=M + 2 * N + 5 * K)
        Ab, Bb = gemm_inputs.bits(A), gemm_inputs.bits(B)
        Cb = gemm_inputs.bits(C) if C is not None else None
        ref, S = oracle.gemm_f64(Ab, Bb, Cb, dt)
        dC = C.cuda() if C is not None else None
        for cfg in LAYOUT_TILES:
            outs = {}
            for ta in (False, True):
                for tb in (False, True):
                    dA, dB = _placed(A, ta, 8), _placed(B, tb, 16)
                    D = torch.full((M, N), float("nan"), dtype=A.dtype, device="cuda")
                    g.matmul(dA, dB, dC, out=D, config=cfg)
                    torch.cuda.synchronize()
                    Dh = D.cpu()
                    n, worst, first = oracle.tol_check(gemm_inputs.bits(Dh), ref, S, dt)
                    assert n == 0, "%s %s %s ta=%d tb=%d: %d outside (worst %.3g)" % (dt, mnk, cfg, ta, tb, n, worst)
                    outs[(ta, tb)] = Dh
            if cfg is not None:
                base = outs[(False, False)].view(torch.int16)
                for key, Dh in outs.items():
                    assert torch.equal(base, Dh.view(torch.int16)), (dt, mnk, cfg, key)


def test_general_strides_take_the_element_path():
    """Operands with neither stride 1 (every other row and column of a larger
    array) and odd extents: the element-wise kernel, inside the bound."""
    M, N, K = 70, 45, 33
    for dt in ("bf16", "f16"):
        A, B, C = _inputs(M, N, K, dt, True, seed=77)
        bigA = torch.zeros((2 * M, 3 * K), dtype=A.dtype)
        bigA[::2, ::3] = A
        bigB = torch.zeros((3 * K, 2 * N), dtype=B.dtype)
        bigB[::3, ::2] = B
        dA = bigA.cuda()[::2, ::3]
        dB = bigB.cuda()[::3, ::2]
        pl = g.plan_for(dA, dB, C.cuda(), None)
        assert "layout=-1" in pl.describe() and "vec=0" in pl.describe()
        D = g.matmul(dA, dB, C.cuda())
        torch.cuda.synchronize()
        check(A, B, C, D.cpu(), dt, label="general strides %s" % dt)


def test_overlapping_rows_of_k():
    """Operands whose rows of k overlap in memory (row-major B with row stride
    below N, A stored K x M with row stride below M): not the direct-to-LDS
    kernel, whose K tail relies on the descriptor range; the result is the
    product of the overlapping views, inside the bound.  A k-contiguous A with
    overlapping rows stays on the direct kernel (per-lane K-tail masks)."""
    M = N = K = 264
    for dt in ("bf16", "f16"):
        A, B, C = _inputs(M, N, K, dt, True, seed=91)
        bufB = gemm_inputs.draw(((K - 1) * 128 + N,), 93, dt).cuda()
        dB = torch.as_strided(bufB, (K, N), (128, 1))          # row k starts 128 elements after row k-1
        bufA = gemm_inputs.draw(((K - 1) * 136 + M,), 95, dt).cuda()
        dA_t = torch.as_strided(bufA, (M, K), (1, 136))         # A stored K x M, lda = 136 < M
        bufA2 = gemm_inputs.draw(((M - 1) * 200 + K,), 97, dt).cuda()
        dA_r = torch.as_strided(bufA2, (M, K), (200, 1))        # row-major A, lda = 200 < K
        for dA, dBx, want_dma in ((A.cuda(), dB, False), (dA_t, B.cuda(), False), (dA_r, B.cuda(), True)):
            pl = g.plan_for(dA, dBx, C.cuda(), None)
            assert ("gemm_dma_kernel" in pl.describe()) == want_dma, pl.describe()
            D = g.matmul(dA, dBx, C.cuda())
            torch.cuda.synchronize()
            check(dA.cpu(), dBx.cpu(), C, D.cpu(), dt, label="overlapping rows %s %s" % (dt, pl.describe()[:40]))


# ---------------------------------------------------------------- epilogue without an addend

DMA_TILES = [v for v in _variants("bf16") if v["kernel"] == 3]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_staged_epilogue_every_dma_variant(dt):
    """Without C the direct-to-LDS kernel writes D from a tile staged in LDS:
    every variant, forced, on ragged M / N / K (N a multiple of 8, as this
    kernel's B rows require).  D is written contiguous (16-byte stores), into
    a view of odd row stride 219 (element-wise stores) and into a view of row
    stride 224 (16-byte stores); the guard bands around the views must stay
    untouched."""
    M, N, K = 300, 200, 136
    A, B, _ = _inputs(M, N, K, dt, False, seed=71)
    dA, dB = A.cuda(), B.cuda()
    for cfg in DMA_TILES:
        D = torch.full((M, N), float("nan"), dtype=A.dtype, device="cuda")
        g.matmul(dA, dB, None, out=D, config=cfg)
        torch.cuda.synchronize()
        check(A, B, None, D.cpu(), dt, label="%s contiguous %s" % (dt, cfg))
        for pitch in (219, 224):
            big = torch.full((M + 16, pitch), 7.0, dtype=A.dtype, device="cuda")
            view = big[8:8 + M, 8:8 + N]
            g.matmul(dA, dB, None, out=view, config=cfg)
            torch.cuda.synchronize()
            host = big.cpu()
            mask = torch.ones_like(host, dtype=torch.bool)
            mask[8:8 + M, 8:8 + N] = False
            assert torch.all(host[mask] == 7.0), (cfg, pitch)
            check(A, B, None, host[8:8 + M, 8:8 + N].contiguous(), dt, label="%s pitch %d %s" % (dt, pitch, cfg))


def test_staged_epilogue_unaligned_output():
    """D based 2 bytes past a 16-byte boundary: element-wise stores only."""
    M, N, K = 260, 264, 192
    A, B, _ = _inputs(M, N, K, "bf16", False, seed=72)
    flat = torch.full((M * N + 1,), float("nan"), dtype=torch.bfloat16, device="cuda")
    view = flat[1:].view(M, N)
    gpu_run(A, B, None, config=dict(kernel=3, bm=256, bn=256), out=view)
    check(A, B, None, view.cpu(), "bf16", label="unaligned D")


@pytest.mark.parametrize("shape,ring", [((2048, 2048, 192), (128, 128, 4)), ((2560, 2560, 136), (256, 128, 3)),
                                        ((1000, 1024, 200), (64, 64, 4))])
def test_planned_ring_depths_every_layout(shape, ring):
    """Shapes whose planned tile is the 4-stage 128 x 128 or the 3-stage
    256 x 128 ring, in all four operand layouts: the plan is that tile, every
    sampled output is inside the bound, and the layouts agree bit for bit."""
    M, N, K = shape
    A, B, _ = _inputs(M, N, K, "bf16", False, seed=M + K)
    Ab, Bb = gemm_inputs.bits(A), gemm_inputs.bits(B)
    ii, jj = sample_positions(M, N, 4000, 5)
    ref, S = oracle.gemm_f64_at(Ab, Bb, None, ii, jj, "bf16")
    outs = {}
    for ta in (False, True):
        for tb in (False, True):
            dA, dB = _placed(A, ta, 8), _placed(B, tb, 16)
            D = torch.full((M, N), float("nan"), dtype=A.dtype, device="cuda")
            pl = g.plan_for(dA, dB, None, D)
            c = pl.config
            assert (c.kernel, c.bm, c.bn, c.stages) == (3,) + ring, (ta, tb, pl.describe())
            g.matmul(dA, dB, None, out=D)
            torch.cuda.synchronize()
            Dh = D.cpu()
            n, worst, _ = oracle.tol_check(gemm_inputs.bits(Dh)[ii, jj], ref, S, "bf16")
            assert n == 0, "%s ta=%d tb=%d: %d outside (worst %.3g)" % (shape, ta, tb, n, worst)
            assert not torch.isnan(Dh.float()).any()
            outs[(ta, tb)] = Dh.view(torch.int16)
    for key, Dh in outs.items():
        assert torch.equal(outs[(False, False)], Dh), key
