"""Masked tails against foreign data (GPU).

Reading of "Hopper Support in Triton", slides 15-16: both K-tail loads are
masked with zeros (`other = 0` on a and b), and so are loads past M and N.
Masking only one operand of a product would still multiply foreign data by
zero, and 0 x NaN = NaN.  So every operand here sits inside a larger
allocation whose elements outside the logical matrix are NaN:

* row-major A: NaN in columns K..lda of every row and in rows past M;
* A stored K x M: NaN in the rows past K and the columns past M;
* row-major B: NaN in the rows past K (same buffer) and the columns past N;
* B stored N x K: NaN in the columns past K and the rows past N.

Every kernel family runs on them with K not a multiple of the K step:
* the direct-to-LDS kernel in all four layouts, planned and forced tiles,
  with and without K slices;
* the register-staged kernel, vector and element-wise;
* the skinny kernel, with and without K slices.

Every output must be finite and inside the acceptance rule against the
oracle on the logical operands.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_02_amd as g
import gemm_inputs
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    torch.cuda.init()


def _poisoned(X, transposed, pad_inner, pad_outer):
    """X (CPU, rows x cols) on the GPU as a view with X's shape, inside a
    NaN-filled allocation.  Row-major: storage (rows + pad_outer) x
    (cols + pad_inner), X in the top-left corner.  Transposed: storage
    (cols + pad_outer) x (rows + pad_inner) holding X^T in its top-left
    corner; the view is its transpose."""
    r, c = X.shape
    if transposed:
        st = torch.full((c + pad_outer, r + pad_inner), float("nan"), dtype=X.dtype, device="cuda")
        st[:c, :r] = X.t().cuda()
        return st[:c, :r].t()
    st = torch.full((r + pad_outer, c + pad_inner), float("nan"), dtype=X.dtype, device="cuda")
    st[:r, :c] = X.cuda()
    return st[:r, :c]


def _check(A, B, C, D, dt, what):
    Dh = D.cpu()
    assert torch.isfinite(Dh.float()).all(), "%s: non-finite outputs (foreign NaN reached a product)" % what
    Cb = gemm_inputs.bits(C) if C is not None else None
    ref, S = oracle.gemm_f64(gemm_inputs.bits(A), gemm_inputs.bits(B), Cb, dt)
    n, worst, first = oracle.tol_check(gemm_inputs.bits(Dh), ref, S, dt)
    assert n == 0, "%s: %d outputs outside the bound (worst %.3g, first %d)" % (what, n, worst, first)


def _run(A, B, C, dt, ta, tb, cfg, what, pads=(8, 24)):
    """D = A x B (+C) with A, B poisoned in layout (ta, tb); returns the plan."""
    dA = _poisoned(A, ta, *pads)
    dB = _poisoned(B, tb, *pads)
    dC = C.cuda() if C is not None else None
    D = torch.full((A.shape[0], B.shape[1]), float("nan"), dtype=A.dtype, device="cuda")
    pl = g.plan_for(dA, dB, dC, D, cfg)
    g.matmul(dA, dB, dC, out=D, config=cfg)
    torch.cuda.synchronize()
    _check(A, B, C, D, dt, "%s %s" % (what, pl.describe()))
    return pl.describe()


DMA_TILES = [None,
             dict(kernel=3, bm=256, bn=256, waves_m=2, waves_n=4, stages=2),
             dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=4, stages=4),
             dict(kernel=3, bm=64, bn=64, waves_m=2, waves_n=2, stages=4),
             dict(kernel=3, bm=128, bn=128, waves_m=2, waves_n=4, stages=4, splitk=3)]


@pytest.mark.parametrize("mnk", [(136, 264, 200), (264, 136, 1000)])
def test_direct_kernel_every_layout(mnk):
    """K = 200 and 1000 end inside a 64-deep K step (8 and 40 k in the tail)."""
    M, N, K = mnk
    for dt, has_c in (("bf16", True), ("f16", False)):
        A = gemm_inputs.draw((M, K), M + K, dt)
        B = gemm_inputs.draw((K, N), N + K, dt)
        C = gemm_inputs.draw((M, N), M + N, dt) if has_c else None
        for cfg in DMA_TILES:
            for ta in (False, True):
                for tb in (False, True):
                    desc = _run(A, B, C, dt, ta, tb, cfg, "%s %s ta=%d tb=%d" % (dt, mnk, ta, tb))
                    assert "gemm_dma_kernel" in desc, desc


def test_direct_kernel_one_wave_per_simd_tiles():
    M, N, K = 264, 520, 200
    A = gemm_inputs.draw((M, K), 5, "bf16")
    B = gemm_inputs.draw((K, N), 6, "bf16")
    for mf in (16, 32):   # compiled for row-major operands
        cfg = dict(kernel=3, bm=256, bn=256, waves_m=2, waves_n=2, stages=2, mfma=mf)
        _run(A, B, None, "bf16", False, False, cfg, "4-wave mfma=%d" % mf)


def test_register_kernel_vector_and_element_paths():
    M, N, K = 136, 264, 200
    for dt in ("bf16", "f16"):
        A = gemm_inputs.draw((M, K), 11, dt)
        B = gemm_inputs.draw((K, N), 12, dt)
        C = gemm_inputs.draw((M, N), 13, dt)
        for cfg in (dict(kernel=1, bm=64, bn=64, bk=64, stages=2), dict(kernel=1, bm=128, bn=128, bk=64, stages=2)):
            desc = _run(A, B, C, dt, False, False, cfg, "register vector %s" % dt)
            assert "gemm_tile_kernel" in desc and "vec=1" in desc, desc
    # K and N not multiples of 8: the element-wise path, in every layout
    M, N, K = 70, 45, 203
    for dt in ("bf16", "f16"):
        A = gemm_inputs.draw((M, K), 21, dt)
        B = gemm_inputs.draw((K, N), 22, dt)
        C = gemm_inputs.draw((M, N), 23, dt)
        for ta in (False, True):
            for tb in (False, True):
                desc = _run(A, B, C, dt, ta, tb, None, "element-wise %s ta=%d tb=%d" % (dt, ta, tb),
                            pads=(5, 7))
                assert "vec=0" in desc, desc


@pytest.mark.parametrize("mnk", [(16, 1000, 1000), (5, 4096, 520), (32, 520, 1000)])
def test_skinny_kernel(mnk):
    """The decode kernels stream rows of B: NaN past K in B's buffer and past N
    in each row; with K slices (planner) and without (one-shot path: no
    workspace)."""
    M, N, K = mnk
    A = gemm_inputs.draw((M, K), M + 3, "bf16")
    B = gemm_inputs.draw((K, N), N + 3, "bf16")
    C = gemm_inputs.draw((M, N), K + 3, "bf16")
    desc = _run(A, B, C, "bf16", False, False, None, "skinny %s" % (mnk,))
    assert "gemm_skinny_kernel" in desc, desc
    for cfg in (dict(kernel=2, bn=32, waves_n=8, bk=64 if M <= 16 else 32, stages=3, splitk=1),
                dict(kernel=2, bn=128, waves_n=8, bk=32, stages=2, splitk=2)):
        cfg["bm"] = 16 if M <= 16 else 32
        desc = _run(A, B, C, "bf16", False, False, cfg, "skinny %s forced" % (mnk,))
        assert "gemm_skinny_kernel" in desc, desc


def test_foreign_data_is_really_there():
    """The poisoned views read NaN just outside the logical matrix (the test
    above would prove nothing if the padding were zeros)."""
    X = gemm_inputs.draw((6, 10), 1, "bf16")
    v = _poisoned(X, False, 8, 24)
    st = torch.as_strided(v, (7, 11), v.stride())
    assert torch.isnan(st[6, :].float()).all() and torch.isnan(st[:, 10].float()).all()
    t = _poisoned(X, True, 8, 24)
    st = torch.as_strided(t, (7, 11), t.stride())
    assert torch.isnan(st[6, :].float()).all() and torch.isnan(st[:, 10].float()).all()
    assert torch.equal(v.cpu(), X) and torch.equal(t.cpu(), X)
