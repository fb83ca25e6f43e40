"""Parity of the block-scaled (MX) GEMM with the oracle (GPU).

Every case runs the HIP kernel through the C ABI (gemm_mx_plan_create /
gemm_mx_run) on seeded inputs from gemm_inputs.draw_mx and checks every
output (or, at the full 4096^3 size, sampled outputs) against the binary64
oracle with the MX acceptance rule
|d - ref| <= ulp_out(ref) + 2^-20 * S + 2^-10 * S8,
S = sum_k |scaled a * scaled b|, S8 = sum over runs of 8 consecutive k of
the largest such product (the scaled instruction's own rounding of a run).
Scale rows are padded with the NaN code 0xFF, so a read of a scale past
ceil(K/32) would show as a non-finite output.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_02_amd as g
import dense_tiled_gemm_02_amd.mx as mx
import gemm_inputs
import oracle

pytestmark = pytest.mark.gpu

PAIRS = [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e2m1", "e2m1")]
TILES = [(256, 256), (256, 128), (128, 256), (128, 128), (64, 64), (192, 256)]
OUT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    mx.mxlib()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _check(D, ref, S, S8, out, what):
    got = D.cpu().numpy() if out == "f32" else gemm_inputs.bits(D.cpu())
    n, worst, first = oracle.mx_tol_check(got, out, ref, S, S8)
    assert n == 0, "%s: %d outputs outside the bound (worst %.3g, first flat index %d)" % (what, n, worst, first)
    return worst


def _run(A, SA, B, SB, K, fa, fb, out="bf16", config=None):
    D = mx.mx_matmul(_dev(A), _dev(SA), _dev(B), _dev(SB), K, fa, fb, out_dtype=OUT[out], config=config)
    torch.cuda.synchronize()
    return D


def _case(M, N, K, fa, fb, seed):
    A, SA = gemm_inputs.draw_mx(M, K, fa, seed)
    B, SB = gemm_inputs.draw_mx(N, K, fb, seed + 1)
    return A, SA, B, SB


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("fa,fb", PAIRS)
def test_tiles_with_ragged_tails_match_oracle(fa, fb, tile):
    """M, N not tile multiples; K ends inside a K step and inside a scale block."""
    K = 1056 if fa != "e2m1" else 1088
    M, N = 520, 392
    A, SA, B, SB = _case(M, N, K, fa, fb, 31 + len(fa + fb) + tile[0] // 64)
    print("mx case", fa, fb, tile, M, N, K, flush=True)
    D = _run(A, SA, B, SB, K, fa, fb, config={"bm": tile[0], "bn": tile[1]})
    ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fa, fb, runs=True)
    _check(D, ref, S, S8, "bf16", "%s x %s tile %s" % (fa, fb, tile))


@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_output_types_and_addend(fmt, out):
    M, N, K = 300, 260, 512
    A, SA, B, SB = _case(M, N, K, fmt, fmt, 77)
    C = np.random.default_rng(5).uniform(-4, 4, (M, N)).astype(np.float32)
    Ct = torch.from_numpy(C).to(OUT[out])
    print("mx out", fmt, out, flush=True)
    D = mx.mx_matmul(_dev(A), _dev(SA), _dev(B), _dev(SB), K, fmt, fmt, C=Ct.cuda(), out_dtype=OUT[out])
    torch.cuda.synchronize()
    ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt, Ct.to(torch.float64).numpy(), runs=True)
    _check(D, ref, S, S8, out, "%s out %s + C" % (fmt, out))


@pytest.mark.parametrize("K", [768, 736])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e2m1"])
def test_padded_rows_and_scale_strides(fmt, K):
    """Row strides above the packed size (A, B, scales and D).  The bytes past
    K in every row of A and B are NaN codes (0x7F in both 8-bit formats;
    E2M1 has none, so its largest magnitude, 0x77), and K = 736 ends inside a
    K step: a K-tail mask missing on either operand shows as a non-finite or
    far-off output."""
    M, N = 200, 136
    A0, SA0, B0, SB0 = _case(M, N, K, fmt, fmt, 91)
    pad = lambda x, extra, fill: np.concatenate([x, np.full((x.shape[0], extra), fill, np.uint8)], 1)
    fill = 0x77 if fmt == "e2m1" else 0x7F
    A, B = pad(A0, 48, fill), pad(B0, 16, fill)
    SA, SB = pad(SA0, 8, 0xFF), pad(SB0, 4, 0xFF)
    Dbig = torch.full((M, N + 24), float("nan"), dtype=torch.bfloat16, device="cuda")
    D = Dbig[:, :N]
    print("mx padded", fmt, K, flush=True)
    mx.mx_matmul(_dev(A), _dev(SA), _dev(B), _dev(SB), K, fmt, fmt, out=D)
    torch.cuda.synchronize()
    ref, S, S8 = oracle.mx_gemm_f64(A0, SA0, B0, SB0, K, fmt, fmt, runs=True)
    assert torch.isfinite(D.float()).all()
    _check(D.contiguous(), ref, S, S8, "bf16", "padded %s K=%d" % (fmt, K))
    assert torch.isnan(Dbig[:, N:].float()).all()           # nothing written past N


def test_small_and_degenerate_shapes():
    for (M, N, K) in [(1, 1, 32), (7, 33, 64), (33, 7, 96), (129, 257, 160), (64, 64, 4096)]:
        for fmt in ("e4m3", "e2m1"):
            A, SA, B, SB = _case(M, N, K, fmt, fmt, M + N + K)
            print("mx small", fmt, M, N, K, flush=True)
            D = _run(A, SA, B, SB, K, fmt, fmt)
            ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt, runs=True)
            _check(D, ref, S, S8, "bf16", "%s %dx%dx%d" % (fmt, M, N, K))


def test_k_zero_writes_the_addend_and_empty_outputs_launch_nothing():
    M, N = 40, 24
    C = torch.randn(M, N, device="cuda").to(torch.bfloat16)
    e = torch.zeros((M, 0), dtype=torch.uint8, device="cuda")
    s = torch.zeros((M, 4), dtype=torch.uint8, device="cuda")
    eb = torch.zeros((N, 0), dtype=torch.uint8, device="cuda")
    sb = torch.zeros((N, 4), dtype=torch.uint8, device="cuda")
    p = mx.mx_problem(M, N, 0, "e4m3", has_c=True, lda=16, ldb=16, ldsa=4, ldsb=4)
    pl = mx.gemm_mx_plan_create(p, 0)
    D = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    mx.gemm_mx_run(pl, e.data_ptr(), s.data_ptr(), eb.data_ptr(), sb.data_ptr(), C.data_ptr(), D.data_ptr(),
                   stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(D, C)
    p0 = mx.mx_problem(0, N, 64, "e4m3")
    mx.gemm_mx_run(mx.gemm_mx_plan_create(p0, 0), None, None, None, None, None, None)


def test_runs_are_bitwise_reproducible():
    A, SA, B, SB = _case(512, 512, 2048, "e4m3", "e4m3", 5)
    D1 = _run(A, SA, B, SB, 2048, "e4m3", "e4m3")
    D2 = _run(A, SA, B, SB, 2048, "e4m3", "e4m3")
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))


@pytest.mark.parametrize("name", sorted(gemm_inputs.MX_WORKLOADS))
def test_full_size_workloads_sampled(name):
    """The benchmark's workloads at full size, in the launch configuration the
    benchmark times, on 3000 sampled outputs (all corners and edges included)."""
    w = gemm_inputs.MX_WORKLOADS[name]
    A, SA, B, SB, _ = gemm_inputs.make_mx(w)
    print("mx full", name, flush=True)
    D = _run(A, SA, B, SB, w.K, w.fmt_a, w.fmt_b, w.out)
    rng = np.random.default_rng(17)
    ii = np.concatenate([rng.integers(0, w.M, 3000), [0, 0, w.M - 1, w.M - 1]])
    jj = np.concatenate([rng.integers(0, w.N, 3000), [0, w.N - 1, 0, w.N - 1]])
    ref, S, S8 = oracle.mx_gemm_f64_at(A, SA, B, SB, w.K, w.fmt_a, w.fmt_b, None, ii, jj, runs=True)
    got = gemm_inputs.bits(D.cpu())[ii, jj]
    n, worst, first = oracle.mx_tol_check(got, w.out, ref, S, S8)
    assert n == 0, "%s: %d sampled outputs outside the bound (worst %.3g)" % (name, n, worst)
    assert torch.isfinite(D.float()).all()


@pytest.mark.parametrize("fmt,M,N,K", [("e4m3", 192, 8192, 4096), ("e2m1", 200, 8192, 8224)])
def test_wide_problems_take_two_k_slices(fmt, M, N, K):
    """Wide problems whose 128 x 128 tiles fill half the CUs or fewer run two
    K slices (planned, not forced); ragged M and K; sampled outputs, whole
    first / last rows and columns included, plus the result is repeatable."""
    A, SA, B, SB = _case(M, N, K, fmt, fmt, 91)
    p = mx.gemm_mx_plan_create(mx.mx_problem(M, N, K, fmt, fmt), 0, None)
    cfg = p.config
    print("mx wide", fmt, M, N, K, cfg.bm, cfg.bn, cfg.splitk, flush=True)
    assert (cfg.bm, cfg.bn, cfg.splitk) == (128, 128, 2)
    D = _run(A, SA, B, SB, K, fmt, fmt)
    D2 = _run(A, SA, B, SB, K, fmt, fmt)
    assert torch.equal(D.view(torch.int16), D2.view(torch.int16))
    from helpers import sample_positions
    ii, jj = sample_positions(M, N, 2000, 19)
    ref, S, S8 = oracle.mx_gemm_f64_at(A, SA, B, SB, K, fmt, fmt, None, ii, jj, runs=True)
    got = gemm_inputs.bits(D.cpu())[ii, jj]
    n, worst, first = oracle.mx_tol_check(got, "bf16", ref, S, S8)
    assert n == 0, "%s wide: %d sampled outputs outside the bound (worst %.3g)" % (fmt, n, worst)


def test_e2m1_products_are_exact_in_binary32():
    """Every E2M1 product has at most 4 significant bits and a run of 8 within one
    block spans few binades, so the instruction's run rounding never bites:
    with a binary32 output the result is the exact sum rounded once."""
    M, N, K = 256, 256, 1024
    A, SA, B, SB = _case(M, N, K, "e2m1", "e2m1", 21)
    D = _run(A, SA, B, SB, K, "e2m1", "e2m1", "f32")
    ref, S = oracle.mx_gemm_f64(A, SA, B, SB, K, "e2m1", "e2m1")
    n, worst, _ = oracle.mx_tol_check(D.cpu().numpy(), "f32", ref, S, None)
    assert n == 0


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("M", [1, 16, 32])
def test_decode_slabs_with_k_slices(fmt, M):
    """The decode regime (32-row slabs, K split over workgroups, fused
    deterministic reduce) against the oracle, with a ragged N and a K whose
    slices end inside a K step."""
    N, K = 1000, 3072 + 64
    A, SA, B, SB = _case(M, N, K, fmt, fmt, 40 + M)
    p = mx.mx_problem(M, N, K, fmt, lda=A.shape[1], ldb=B.shape[1], ldsa=SA.shape[1], ldsb=SB.shape[1])
    cfg = mx.gemm_mx_plan_create(p, 0).config
    assert (cfg.bm, cfg.bn) == (32, 64) and cfg.splitk > 1
    print("mx decode", fmt, M, cfg.splitk, flush=True)
    D = _run(A, SA, B, SB, K, fmt, fmt)
    ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt, runs=True)
    _check(D, ref, S, S8, "bf16", "decode %s M=%d" % (fmt, M))
    D2 = _run(A, SA, B, SB, K, fmt, fmt)          # the workspace is left ready for reuse
    assert torch.equal(D.view(torch.int16), D2.view(torch.int16))


@pytest.mark.parametrize("splits", [2, 3, 7])
def test_forced_k_slices_on_a_square_tile(splits):
    M, N, K = 300, 200, 2048
    A, SA, B, SB = _case(M, N, K, "e4m3", "e4m3", 60 + splits)
    print("mx split", splits, flush=True)
    D = _run(A, SA, B, SB, K, "e4m3", "e4m3", config={"bm": 128, "bn": 128, "splitk": splits})
    ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, "e4m3", "e4m3", runs=True)
    _check(D, ref, S, S8, "bf16", "split %d" % splits)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("M", [1, 16, 32])
@pytest.mark.parametrize("splits", [1, 4])
def test_decode_slab_with_forced_slices(fmt, M, splits):
    """The decode tile without K slices and with a forced count, ragged N and
    K ending inside a K step."""
    N, K = 1000, 3072 + 64
    A, SA, B, SB = _case(M, N, K, fmt, fmt, 50 + M + splits)
    print("mx decode forced", fmt, M, splits, flush=True)
    D = _run(A, SA, B, SB, K, fmt, fmt, config={"bm": 32, "bn": 64, "splitk": splits})
    ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt, runs=True)
    _check(D, ref, S, S8, "bf16", "decode %s M=%d splits=%d" % (fmt, M, splits))


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("tile", TILES + [(32, 64)])
def test_staged_epilogue_partial_chunks(fmt, tile):
    """16-bit output without an addend goes out as 16-byte row chunks: N = 203
    in a view of row stride 216 ends every row in a partial chunk, the guard
    band around the view stays untouched (NaN), and a contiguous D of odd row
    stride takes element-wise stores."""
    M, N, K = 200 if tile[0] > 32 else 24, 203, 512
    A, SA, B, SB = _case(M, N, K, fmt, fmt, 90 + tile[1] // 32)
    ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt, runs=True)
    cfg = {"bm": tile[0], "bn": tile[1]}
    print("mx staged", fmt, tile, flush=True)
    big = torch.full((M + 16, 216 + 8), float("nan"), dtype=torch.bfloat16, device="cuda")
    view = big[8:8 + M, 8:8 + N]
    mx.mx_matmul(_dev(A), _dev(SA), _dev(B), _dev(SB), K, fmt, fmt, out=view, config=cfg)
    torch.cuda.synchronize()
    host = big.cpu()
    mask = torch.ones_like(host, dtype=torch.bool)
    mask[8:8 + M, 8:8 + N] = False
    assert torch.isnan(host[mask].float()).all()
    _check(host[8:8 + M, 8:8 + N].contiguous(), ref, S, S8, "bf16", "strided %s %s" % (fmt, tile))
    D = _run(A, SA, B, SB, K, fmt, fmt, config=cfg)
    _check(D, ref, S, S8, "bf16", "contiguous %s %s" % (fmt, tile))


@pytest.mark.parametrize("out,has_c", [("f32", False), ("f32", True), ("bf16", True), ("f16", True)])
@pytest.mark.parametrize("tile", TILES + [(32, 64)])
def test_staged_epilogue_fp32_passes(tile, out, has_c):
    """An addend or an fp32 output stages the fp32 tile in row passes: C and D
    views of row stride 224 (16- or 32-byte accesses, a partial last run per
    row at N = 203), guard band untouched; contiguous C / D of odd row stride
    (element-wise accesses)."""
    fmt = "e4m3"
    M, N, K = 200 if tile[0] > 32 else 24, 203, 512
    A, SA, B, SB = _case(M, N, K, fmt, fmt, 120 + tile[1] // 32 + 7 * has_c)
    dt = OUT[out]
    Cf = np.random.default_rng(9).uniform(-4, 4, (M, N)).astype(np.float32)
    Ct = torch.from_numpy(Cf).to(dt)
    ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt, Ct.to(torch.float64).numpy() if has_c else None,
                                    runs=True)
    cfg = {"bm": tile[0], "bn": tile[1]}
    print("mx staged fp32", tile, out, has_c, flush=True)
    Cbig = torch.zeros((M + 16, 224), dtype=dt, device="cuda")
    Cbig[8:8 + M, 8:8 + N] = Ct.cuda()
    Cview = Cbig[8:8 + M, 8:8 + N] if has_c else None
    big = torch.full((M + 16, 224), float("nan"), dtype=dt, device="cuda")
    view = big[8:8 + M, 8:8 + N]
    mx.mx_matmul(_dev(A), _dev(SA), _dev(B), _dev(SB), K, fmt, fmt, C=Cview, out=view, config=cfg)
    torch.cuda.synchronize()
    host = big.cpu()
    mask = torch.ones_like(host, dtype=torch.bool)
    mask[8:8 + M, 8:8 + N] = False
    assert torch.isnan(host[mask].float()).all()
    _check(host[8:8 + M, 8:8 + N].contiguous(), ref, S, S8, out, "strided %s %s c=%d" % (tile, out, has_c))
    D = mx.mx_matmul(_dev(A), _dev(SA), _dev(B), _dev(SB), K, fmt, fmt, C=Ct.cuda() if has_c else None,
                     out_dtype=dt, config=cfg)
    torch.cuda.synchronize()
    _check(D, ref, S, S8, out, "contiguous %s %s c=%d" % (tile, out, has_c))


@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("splits", [2, 5])
def test_decode_slices_with_addend(out, splits):
    """K slices across workgroups with an addend and each output type: the last
    workgroup of a tile sums the fp32 partials in slice order, adds C and
    rounds once."""
    M, N, K, fmt = 20, 520, 2560 + 32, "e4m3"
    A, SA, B, SB = _case(M, N, K, fmt, fmt, 130 + splits)
    dt = OUT[out]
    Ct = torch.from_numpy(np.random.default_rng(11).uniform(-4, 4, (M, N)).astype(np.float32)).to(dt)
    ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt, Ct.to(torch.float64).numpy(), runs=True)
    print("mx decode addend", out, splits, flush=True)
    D = mx.mx_matmul(_dev(A), _dev(SA), _dev(B), _dev(SB), K, fmt, fmt, C=Ct.cuda(), out_dtype=dt,
                     config={"bm": 32, "bn": 64, "splitk": splits})
    torch.cuda.synchronize()
    _check(D, ref, S, S8, out, "decode + C %s splits %d" % (out, splits))


# ---------------------------------------------------------------- FP6 elements and mixed widths

MIXED_PAIRS = [("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e2m3", "e3m2"), ("e4m3", "e2m1"), ("e2m1", "e4m3"),
               ("e5m2", "e2m1"), ("e2m1", "e3m2"), ("e3m2", "e5m2"), ("e4m3", "e2m3")]
# the tile kernel's variants for these pairs, and the register-direct kernel
MIXED_TILES = [dict(kernel=4, bm=256, bn=256), dict(kernel=4, bm=256, bn=256, stages=2),
               dict(kernel=4, bm=128, bn=128), dict(kernel=4, bm=64, bn=64), dict(kernel=4, bm=32, bn=64),
               dict(kernel=5)]
# rows padded to a multiple of 16 bytes (an FP6 row is 3K/4 bytes) with 0xFF
_pad16 = lambda x: np.concatenate([x, np.full((x.shape[0], -x.shape[1] % 16), 0xFF, np.uint8)], 1)


@pytest.mark.parametrize("fa,fb", MIXED_PAIRS)
def test_fp6_and_mixed_widths_match_oracle(fa, fb):
    """FP6 operands and operands of different widths through the planner (the
    tile kernel, each operand staged in rows of its own width): ragged M / N,
    a K that ends inside a K step and inside a 16-byte chunk of FP6 bytes,
    every output type, with and without an addend."""
    for (M, N, K) in [(200, 136, 736), (129, 257, 160), (1, 1, 32), (64, 300, 4096), (300, 520, 1056)]:
        A, SA, B, SB = _case(M, N, K, fa, fb, M + N + K)
        A, B = _pad16(A), _pad16(B)
        for out in ("bf16", "f16", "f32"):
            C = torch.from_numpy(np.random.default_rng(K).standard_normal((M, N)).astype(np.float32)).to(OUT[out])
            for c in (None, C):
                print("mx pair", fa, fb, M, N, K, out, c is not None, flush=True)
                D = mx.mx_matmul(_dev(A), _dev(SA), _dev(B), _dev(SB), K, fa, fb, out_dtype=OUT[out],
                                 C=c.cuda() if c is not None else None)
                torch.cuda.synchronize()
                cref = c.to(torch.float64).numpy() if c is not None else None
                ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fa, fb, cref, runs=True)
                assert torch.isfinite(D.float()).all()
                _check(D, ref, S, S8, out, "%s x %s %dx%dx%d out %s c=%d" % (fa, fb, M, N, K, out, c is not None))


@pytest.mark.parametrize("fa,fb", MIXED_PAIRS)
def test_fp6_and_mixed_widths_every_variant(fa, fb):
    """Each compiled variant for these pairs, forced, on a ragged shape with
    several K steps and a K tail inside an FP6 chunk, with an addend; the tile
    variants of one K partition agree bit for bit."""
    M, N, K = 300, 200, 1056
    A, SA, B, SB = _case(M, N, K, fa, fb, 77)
    A, B = _pad16(A), _pad16(B)
    C = torch.from_numpy(np.random.default_rng(3).standard_normal((M, N)).astype(np.float32)).to(torch.bfloat16)
    ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fa, fb, C.to(torch.float64).numpy(), runs=True)
    bits = {}
    for cfg in MIXED_TILES:
        print("mx pair variant", fa, fb, cfg, flush=True)
        D = mx.mx_matmul(_dev(A), _dev(SA), _dev(B), _dev(SB), K, fa, fb, C=C.cuda(), out_dtype=torch.bfloat16,
                         config=cfg)
        torch.cuda.synchronize()
        _check(D, ref, S, S8, "bf16", "%s x %s %s" % (fa, fb, cfg))
        if cfg.get("kernel") == 4:
            bits[str(cfg)] = gemm_inputs.bits(D.cpu())
    vals = list(bits.values())
    assert all(np.array_equal(vals[0], v) for v in vals[1:])


@pytest.mark.parametrize("fa,fb", [("e2m3", "e2m3"), ("e4m3", "e2m1"), ("e3m2", "e2m1")])
@pytest.mark.parametrize("splits", [2, 5])
def test_fp6_and_mixed_widths_k_slices(fa, fb, splits):
    """K slices across workgroups for these pairs: the decode slab and the
    128 x 128 tile, with an addend, fp32 output."""
    for (M, N, K), cfg in (((20, 520, 2560 + 32), dict(kernel=4, bm=32, bn=64, splitk=splits)),
                           ((136, 264, 4096 + 96), dict(kernel=4, bm=128, bn=128, splitk=splits))):
        A, SA, B, SB = _case(M, N, K, fa, fb, 31 + splits)
        A, B = _pad16(A), _pad16(B)
        C = torch.from_numpy(np.random.default_rng(5).standard_normal((M, N)).astype(np.float32))
        ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fa, fb, C.to(torch.float64).numpy(), runs=True)
        print("mx pair slices", fa, fb, M, N, K, cfg, flush=True)
        D = mx.mx_matmul(_dev(A), _dev(SA), _dev(B), _dev(SB), K, fa, fb, C=C.cuda(), out_dtype=torch.float32,
                         config=cfg)
        torch.cuda.synchronize()
        _check(D, ref, S, S8, "f32", "%s x %s slices %s" % (fa, fb, cfg))


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e2m1", "e2m1"), ("e5m2", "e4m3")])
def test_direct_kernel_forced_on_single_width_pairs(fa, fb):
    """The register-direct kernel also runs the pairs the tile kernel takes:
    forced, inside the same bound on ragged shapes."""
    M, N, K = 200, 136, 736
    A, SA, B, SB = _case(M, N, K, fa, fb, 5)
    D = mx.mx_matmul(_dev(A), _dev(SA), _dev(B), _dev(SB), K, fa, fb, out_dtype=torch.bfloat16,
                     config={"kernel": 5})
    torch.cuda.synchronize()
    ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fa, fb, runs=True)
    _check(D, ref, S, S8, "bf16", "forced direct %s x %s" % (fa, fb))


@pytest.mark.parametrize("fa,fb", [("e2m3", "e3m2"), ("e4m3", "e2m1"), ("e2m3", "e2m3"), ("e3m2", "e4m3")])
@pytest.mark.parametrize("force", [None, {"kernel": 5}, {"kernel": 4, "bm": 32, "bn": 64}])
def test_padding_never_enters_a_sum(fa, fb, force):
    """Row bytes past K hold 0xFF (the most negative FP6 / FP4 magnitudes, a
    NaN in E4M3) and scale bytes past ceil(K/32) the NaN code: every output
    stays finite and inside the bound with K ending inside a K step and, for
    FP6 rows, inside a 16-byte chunk (the tile kernel loads that chunk whole
    and gives the block past K a zero scale)."""
    M, N, K = 136, 200, 736
    A0, SA0, B0, SB0 = _case(M, N, K, fa, fb, 9)
    pad = lambda x, extra, fill: np.concatenate([x, np.full((x.shape[0], extra), fill, np.uint8)], 1)
    A, B = pad(A0, 16 - A0.shape[1] % 16 + 32, 0xFF), pad(B0, 16 - B0.shape[1] % 16 + 16, 0xFF)
    SA, SB = pad(SA0, 8, 0xFF), pad(SB0, 4, 0xFF)
    p = mx.mx_problem(M, N, K, fa, fb, mx.GEMM_MX_OUT_BF16, lda=A.shape[1], ldb=B.shape[1], ldsa=SA.shape[1],
                      ldsb=SB.shape[1])
    pl = mx.gemm_mx_plan_create(p, 0, force)
    print("mx padded", fa, fb, pl.describe(), flush=True)
    D = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dA, dSA, dB, dSB = _dev(A), _dev(SA), _dev(B), _dev(SB)
    ws, wsb = mx._workspace(pl, 0, torch.cuda.current_stream().cuda_stream)
    st = mx.mxlib().gemm_mx_run(pl.handle, dA.data_ptr(), dSA.data_ptr(), dB.data_ptr(), dSB.data_ptr(), None,
                                D.data_ptr(), ws, wsb, torch.cuda.current_stream().cuda_stream)
    assert st == 0, g.gemm_last_error()
    torch.cuda.synchronize()
    assert torch.isfinite(D.float()).all()
    ref, S, S8 = oracle.mx_gemm_f64(A0, SA0, B0, SB0, K, fa, fb, runs=True)
    _check(D, ref, S, S8, "bf16", "padded %s x %s %s" % (fa, fb, force))


@pytest.mark.parametrize("name", ["mx_e2m3_4096", "mx_e4m3xe2m1_4096"])
def test_fp6_and_mixed_workloads_sampled(name):
    w = gemm_inputs.MX_WORKLOADS[name]
    A, SA, B, SB, _ = gemm_inputs.make_mx(w)
    D = mx.mx_matmul(_dev(A), _dev(SA), _dev(B), _dev(SB), w.K, w.fmt_a, w.fmt_b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    from helpers import sample_positions
    ii, jj = sample_positions(w.M, w.N, 3000, 23)
    ref, S, S8 = oracle.mx_gemm_f64_at(A, SA, B, SB, w.K, w.fmt_a, w.fmt_b, None, ii, jj, runs=True)
    got = gemm_inputs.bits(D.cpu())[ii, jj]
    n, worst, first = oracle.mx_tol_check(got, "bf16", ref, S, S8)
    assert n == 0, "%s: %d outside (worst %.3g)" % (name, n, worst)


ALL_FORMATS = ("e4m3", "e5m2", "e2m3", "e3m2", "e2m1")
_BITS = {"e4m3": 8, "e5m2": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4}


def _dyadic_rows(rows, K, fmt, rng):
    """Rows of element codes (stored as the format packs them) whose values
    are drawn from {0, +-1/2, +-1, +-2}, each code found by decoding every
    code of the format with the oracle."""
    n = 1 << _BITS[fmt]
    vals = oracle.mx_decode(np.arange(n, dtype=np.uint8), fmt)
    code = {}
    for c in range(n):
        v = float(vals[c])
        if v not in code and not (v == 0 and c != 0):
            code[v] = c
    pick = np.array([code[v] for v in (0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0)], dtype=np.uint8)
    c = pick[rng.integers(0, len(pick), (rows, K))]
    if _BITS[fmt] == 8:
        return np.ascontiguousarray(c)
    if _BITS[fmt] == 6:
        return gemm_inputs.pack_fp6(c)
    return np.ascontiguousarray((c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8))


@pytest.mark.parametrize("fa", ALL_FORMATS)
@pytest.mark.parametrize("fb", ALL_FORMATS)
def test_exact_dyadic_products_every_pair(fa, fb):
    """A pin of the block-scaled path by exact arithmetic, independent of the
    instruction's run rounding: with elements in {0, +-1/2, +-1, +-2} and
    power-of-two scales spanning 2^8, every product, every run of 8 and
    every fp32 partial sum is exact (K = 256: the sums need at most 20
    significant bits), so a binary32 output must equal the exact result and
    a bf16 output its round-to-nearest-even, bit for bit."""
    M, N, K = 96, 136, 256
    rng = np.random.default_rng(1000 + ALL_FORMATS.index(fa) * 5 + ALL_FORMATS.index(fb))
    A, B = _dyadic_rows(M, K, fa, rng), _dyadic_rows(N, K, fb, rng)
    nb = K // 32
    SA = (127 + rng.integers(-2, 3, (M, nb))).astype(np.uint8)
    SB = (127 + rng.integers(-2, 3, (N, nb))).astype(np.uint8)
    ref, _ = oracle.mx_gemm_f64(A, SA, B, SB, K, fa, fb)
    assert np.all(np.abs(ref) < 2.0 ** 16)
    D32 = _run(A, SA, B, SB, K, fa, fb, "f32").cpu().numpy().astype(np.float64)
    assert np.array_equal(D32, ref), "%s x %s: %d outputs differ from the exact sum" % (
        fa, fb, int(np.sum(D32 != ref)))
    D16 = gemm_inputs.bits(_run(A, SA, B, SB, K, fa, fb, "bf16").cpu())
    want = oracle.encode_rne(ref, "bf16")
    assert np.array_equal(D16, want), "%s x %s: %d bf16 outputs differ from RNE(exact)" % (
        fa, fb, int(np.sum(D16 != want)))
