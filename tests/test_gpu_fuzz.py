"""Seeded random problems through the automatic planner (GPU).

Each case draws M, N, K from one of four regimes (any size and alignment,
vector-friendly sizes with random operand layouts, short-M decode shapes,
deep K), a storage type and an optional addend, lets the planner choose
the kernel, and checks whole first / last rows and columns plus random
outputs against the binary64 oracle with the acceptance rule of the parity
tests.  The block-scaled cases do the same for random format pairs.
"""
import os

import numpy as np
import pytest
import torch

import dense_tiled_gemm_02_amd as g
import dense_tiled_gemm_02_amd.mx as mx
import gemm_inputs
import oracle
from helpers import check, sample_positions

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    torch.cuda.init()


# more cases, or other ones, on request (DTG_FUZZ_CASES=600 DTG_FUZZ_SEED=1 python -m pytest ...)
N_CASES = int(os.environ.get("DTG_FUZZ_CASES", "96"))
SEED = int(os.environ.get("DTG_FUZZ_SEED", "0"))


def _cases(n=N_CASES, seed=2024 + SEED):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = i % 4
        ta = tb = False
        if kind == 0:                                  # any size, any alignment
            M, N, K = (int(x) for x in rng.integers(1, 2500, 3))
        elif kind == 1:                                # vector path, random layouts
            M, N, K = (8 * int(x) for x in rng.integers(1, 512, 3))
            ta, tb = bool(rng.integers(2)), bool(rng.integers(2))
        elif kind == 2:                                # decode / skinny
            M = int(rng.integers(1, 65))
            N, K = (8 * int(x) for x in rng.integers(16, 1024, 2))
        else:                                          # deep K, few tiles
            M, N = (8 * int(x) for x in rng.integers(8, 128, 2))
            K = 8 * int(rng.integers(256, 2048))
        dt = "bf16" if rng.integers(2) else "f16"
        has_c = bool(rng.integers(2))
        out.append((M, N, K, dt, has_c, ta, tb))
    return out


def _dev(x, transposed):
    """x on the GPU, stored transposed (column-major) when asked."""
    return x.t().contiguous().cuda().t() if transposed else x.cuda()


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "%dx%dx%d-%s-c%d-t%d%d" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6]))
def test_random_problem_matches_oracle(case):
    M, N, K, dt, has_c, ta, tb = case
    seed = (M * 7919 + N * 104729 + K) % (1 << 31)
    A = gemm_inputs.draw((M, K), seed, dt, "uniform", 1.0)
    B = gemm_inputs.draw((K, N), seed + 1, dt, "uniform", 1.0)
    C = gemm_inputs.draw((M, N), seed + 2, dt, "uniform", 1.0) if has_c else None
    dA, dB = _dev(A, ta), _dev(B, tb)
    dC = C.cuda() if has_c else None
    D = torch.full((M, N), float("nan"), dtype=dA.dtype, device="cuda")
    plan = g.plan_for(dA, dB, dC, D)
    print("fuzz", case, plan.describe().split(" bm=")[0], "splitk=%d" % plan.config.splitk, flush=True)
    g.matmul(dA, dB, dC, out=D)
    torch.cuda.synchronize()
    check(A, B, C, D.cpu(), dt, sample=sample_positions(M, N, 600, seed % 1000), label="fuzz %s" % (case,))


def _mx_cases(n=max(8, N_CASES // 3), seed=77 + SEED):
    rng = np.random.default_rng(seed)
    fmts = ["e4m3", "e5m2", "e2m3", "e3m2", "e2m1"]
    pairs = [(a, b) for a in fmts for b in fmts]       # every pair of element formats
    out = []
    for i in range(n):
        fa, fb = pairs[int(rng.integers(len(pairs)))]
        if i % 2 == 0:
            M, N = (int(x) for x in rng.integers(1, 2500, 2))
        else:
            M, N = int(rng.integers(1, 300)), int(rng.integers(64, 8192))
        K = 32 * int(rng.integers(1, 256))
        out.append((M, N, K, fa, fb))
    return out


@pytest.mark.parametrize("case", _mx_cases(), ids=lambda c: "%dx%dx%d-%s-%s" % c)
def test_random_block_scaled_problem_matches_oracle(case):
    M, N, K, fa, fb = case
    seed = (M * 31 + N * 131 + K) % (1 << 31)
    A, SA = gemm_inputs.draw_mx(M, K, fa, seed)
    B, SB = gemm_inputs.draw_mx(N, K, fb, seed + 1)
    # rows to a multiple of 16 bytes (FP6 rows are 3K/4 bytes), padded with 0xFF
    pad16 = lambda x: np.concatenate([x, np.full((x.shape[0], -x.shape[1] % 16), 0xFF, np.uint8)], 1)
    A, B = pad16(A), pad16(B)
    dev = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (A, SA, B, SB)]
    print("fuzz mx", case, flush=True)
    D = mx.mx_matmul(dev[0], dev[1], dev[2], dev[3], K, fa, fb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ii, jj = sample_positions(M, N, 600, seed % 1000)
    ref, S, S8 = oracle.mx_gemm_f64_at(A, SA, B, SB, K, fa, fb, None, ii, jj, runs=True)
    got = gemm_inputs.bits(D.cpu())[ii, jj]
    n, worst, first = oracle.mx_tol_check(got, "bf16", ref, S, S8)
    assert n == 0, "fuzz mx %s: %d sampled outputs outside the bound (worst %.3g)" % (case, n, worst)
