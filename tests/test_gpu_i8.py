"""Parity of the int8 GEMM with the integer oracle (GPU): bit for bit.

D = A x B (+ C) with int8 A (M x K, row-major) and B stored N x K, int32 C
and D, through the C ABI (gemm_plan_create / gemm_run with dtype GEMM_I8).
Integer results have one correct value, the residue of the exact sum
modulo 2^32, so every output must equal the oracle's exactly: ragged shapes,
every compiled int8 tile, the full 4096^3 workload, a sum that wraps, the
extreme codes, an addend at the int32 limits, operands inside allocations
whose padding holds large codes, an in-place addend and the refusals.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_02_amd as g
import gemm_inputs
import oracle

pytestmark = pytest.mark.gpu

TILES = [None,
         dict(kernel=3, bm=256, bn=256, waves_m=2, waves_n=4, mfma=16, stages=2),
         dict(kernel=3, bm=256, bn=256, waves_m=2, waves_n=4, mfma=32, stages=2),
         dict(kernel=3, bm=256, bn=128, waves_m=4, waves_n=2, stages=3),
         dict(kernel=3, bm=128, bn=256, waves_m=2, waves_n=4, stages=3),
         dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=4, stages=4),
         dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=4, stages=2),
         dict(kernel=3, bm=64, bn=64, waves_m=2, waves_n=2, stages=4)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    torch.cuda.init()


def _gpu(A, Bt, C=None, config=None, out=None, dA=None, dBt=None):
    """D on the GPU; A M x K, Bt N x K numpy int8 (B = Bt^T), C int32 or None."""
    dA = torch.from_numpy(A).cuda() if dA is None else dA
    dBt = torch.from_numpy(Bt).cuda() if dBt is None else dBt
    dC = torch.from_numpy(C).cuda() if C is not None else None
    if out is None:
        out = torch.full((A.shape[0], Bt.shape[0]), -777, dtype=torch.int32, device="cuda")
    g.matmul(dA, dBt.t(), dC, out=out, config=config)
    torch.cuda.synchronize()
    return out


def _check(A, Bt, C, D, what):
    ref, _ = oracle.gemm_i8(A, Bt.T, C)
    got = D.cpu().numpy() if isinstance(D, torch.Tensor) else D
    bad = np.argwhere(got != ref)
    assert bad.size == 0, "%s: %d outputs differ, first at %s: %d != %d" % (
        what, len(bad), tuple(bad[0]), got[tuple(bad[0])], ref[tuple(bad[0])])


@pytest.mark.parametrize("mnk", [(300, 200, 1008), (520, 264, 4096), (96, 1000, 144), (17, 33, 16),
                                 (1, 1, 16), (129, 65, 48), (264, 136, 2064)])
def test_every_int8_tile(mnk):
    M, N, K = mnk
    A = gemm_inputs.draw_i8((M, K), M + K)
    Bt = gemm_inputs.draw_i8((N, K), N + K + 1)
    C = gemm_inputs.draw_i32((M, N), M + N)
    outs = {}
    for cfg in TILES:
        for c in (None, C):
            print("case", mnk, cfg, c is not None, flush=True)
            D = _gpu(A, Bt, c, cfg)
            _check(A, Bt, c, D, "%s %s c=%d" % (mnk, cfg, c is not None))
            outs[(str(cfg), c is not None)] = D.cpu()
    assert len(outs) == 2 * len(TILES)


def test_workload_4096_full_parity():
    """All 16.8 M outputs of the int8 benchmark workload, the planner's plan."""
    w = gemm_inputs.I8_WORKLOADS["square_i8_4096"]
    A, Bt, _ = gemm_inputs.make_i8(w)
    dA, dBt = torch.from_numpy(A).cuda(), torch.from_numpy(Bt).cuda()
    print("case", w.name, g.plan_for(dA, dBt.t()).describe(), flush=True)
    D = _gpu(A, Bt, dA=dA, dBt=dBt)
    _check(A, Bt, None, D, w.name)


def test_tail_workload_with_addend():
    w = gemm_inputs.I8_WORKLOADS["tail_i8_4000x3000x1008_c"]
    A, Bt, C = gemm_inputs.make_i8(w)
    D = _gpu(A, Bt, C)
    _check(A, Bt, C, D, w.name)


def test_sums_wrap_modulo_2_to_the_32():
    """127 x 127 x 140000 = 2258060000 > 2^31 - 1: the int32 accumulator wraps,
    and the result is the residue -2036907296 in every output."""
    K = 140000
    A = np.full((20, K), 127, np.int8)
    Bt = np.full((36, K), 127, np.int8)
    D = _gpu(A, Bt)
    assert (D.cpu().numpy() == -2036907296).all()
    _check(A, Bt, None, D, "wrap")


def test_extreme_codes_and_addend_limits():
    K = 64
    A = np.full((70, K), -128, np.int8)
    Bt = np.full((90, K), -128, np.int8)
    C = np.full((70, 90), 2 ** 31 - 1, np.int32)
    C[::2] = -2 ** 31
    D = _gpu(A, Bt, C)
    _check(A, Bt, C, D, "extremes")
    assert D.cpu().numpy()[1, 0] == oracle.wrap_i32(2 ** 31 - 1 + K * 16384)


def test_padding_never_enters_a_sum():
    """A and B as views of larger allocations whose elements past K (and past
    M, N) hold 127: any read of them would change the exact integer result."""
    M, N, K = 136, 264, 1040
    A = gemm_inputs.draw_i8((M, K), 5)
    Bt = gemm_inputs.draw_i8((N, K), 6)
    bigA = torch.full((M + 24, K + 48), 127, dtype=torch.int8)
    bigA[:M, :K] = torch.from_numpy(A)
    bigB = torch.full((N + 24, K + 16), 127, dtype=torch.int8)
    bigB[:N, :K] = torch.from_numpy(Bt)
    dA, dBt = bigA.cuda()[:M, :K], bigB.cuda()[:N, :K]
    for cfg in TILES:
        D = _gpu(A, Bt, None, cfg, dA=dA, dBt=dBt)
        _check(A, Bt, None, D, "padded %s" % cfg)


def test_in_place_addend_and_strided_output():
    M, N, K = 200, 136, 256
    A = gemm_inputs.draw_i8((M, K), 7)
    Bt = gemm_inputs.draw_i8((N, K), 8)
    C = gemm_inputs.draw_i32((M, N), 9)
    big = torch.full((M, N + 12), -5, dtype=torch.int32, device="cuda")
    big[:, :N] = torch.from_numpy(C).cuda()
    view = big[:, :N]
    g.matmul(torch.from_numpy(A).cuda(), torch.from_numpy(Bt).cuda().t(), view, out=view)
    torch.cuda.synchronize()
    _check(A, Bt, C, view.cpu().numpy(), "in place")
    assert (big[:, N:].cpu() == -5).all()


def test_refusals():
    dA = torch.zeros((64, 48), dtype=torch.int8, device="cuda")
    dB = torch.zeros((48, 64), dtype=torch.int8, device="cuda")          # row-major B: k not contiguous
    with pytest.raises(g.GemmError) as e:
        g.matmul(dA, dB)
    assert e.value.status == g.GEMM_ERR_UNSUPPORTED
    dBt = torch.zeros((64, 40), dtype=torch.int8, device="cuda")         # K = 40: not a multiple of 16
    with pytest.raises(g.GemmError) as e:
        g.matmul(torch.zeros((64, 40), dtype=torch.int8, device="cuda"), dBt.t())
    assert e.value.status == g.GEMM_ERR_UNSUPPORTED
    buf = torch.zeros(64 * 48 + 8, dtype=torch.int8, device="cuda")
    mis = buf[8:].view(64, 48)                                           # 8-byte aligned base
    with pytest.raises(g.GemmError) as e:
        g.matmul(mis, torch.zeros((64, 48), dtype=torch.int8, device="cuda").t())
    assert e.value.status == g.GEMM_ERR_UNSUPPORTED
