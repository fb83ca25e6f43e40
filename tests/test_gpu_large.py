"""Operands larger than 4 GiB (GPU): the kernels address a tile or a chunk
with 32-bit offsets from descriptors rebased in 64 bits, so matrices far
beyond 2^32 bytes must come out right at every position checked.  Inputs are
drawn on the GPU (seeded), and the outputs of whole sampled rows and columns
are checked against the oracle on the gathered rows of A and columns of B
(the same sums, computed on the host in binary64)."""
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


def _draw(shape, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, generator=gen, device="cuda") / 64).to(torch.bfloat16)


def _check_sampled(A, B, D, rows, cols, label):
    ii = torch.tensor(sorted(set(rows)), dtype=torch.long, device="cuda")
    jj = torch.tensor(sorted(set(cols)), dtype=torch.long, device="cuda")
    Ab = gemm_inputs.bits(A.index_select(0, ii).cpu())
    Bb = gemm_inputs.bits(B.index_select(1, jj).cpu())
    got = gemm_inputs.bits(D.index_select(0, ii).index_select(1, jj).cpu())
    ref, S = oracle.gemm_f64(Ab, Bb, None, "bf16")
    n, worst, first = oracle.tol_check(got, ref, S, "bf16")
    assert n == 0, "%s: %d sampled outputs outside the bound (worst %.3g)" % (label, n, worst)


def test_a_of_4_gib():
    """A is 65536 x 32768 bf16 (4 GiB): the direct-to-LDS tiles of the far
    rows start 4 GiB past A's base."""
    M, N, K = 65536, 256, 32768
    A, B = _draw((M, K), 11), _draw((K, N), 12)
    D = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    print("plan", g.plan_for(A, B, None, D).describe(), flush=True)
    g.matmul(A, B, out=D)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = [0, 1, M // 2, M - 257, M - 2, M - 1] + rng.integers(0, M, 40).tolist()
    cols = [0, 1, 127, 128, N - 1] + rng.integers(0, N, 20).tolist()
    _check_sampled(A, B, D, rows, cols, "A 4 GiB")


def test_b_of_8_gib():
    """B is 1024 x 4194304 bf16 (8 GiB) under a decode-shaped product (M = 1):
    the skinny kernel's slabs of the far columns read 8 GiB past B's base."""
    M, N, K = 1, 1 << 22, 1024
    A, B = _draw((M, K), 21), _draw((K, N), 22)
    D = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    print("plan", g.plan_for(A, B, None, D).describe(), flush=True)
    g.matmul(A, B, out=D)
    torch.cuda.synchronize()
    assert torch.isfinite(D.float()).all()
    rng = np.random.default_rng(2)
    cols = [0, 1, 31, 32, N // 2, N - 33, N - 1] + rng.integers(0, N, 200).tolist()
    _check_sampled(A, B, D, [0], cols, "B 8 GiB")


def test_block_scaled_a_of_4_gib():
    """Block-scaled E4M3: A is 131072 rows of 32768 bytes (4 GiB), its
    scales 128 MiB; the tiles of the far rows start 4 GiB past A's base."""
    import dense_tiled_gemm_02_amd.mx as mx
    M, N, K = 131072, 256, 32768
    gen = torch.Generator(device="cuda").manual_seed(31)
    A = (torch.randn((M, K), generator=gen, device="cuda") * 8).to(torch.float8_e4m3fn).view(torch.uint8)
    B = (torch.randn((N, K), generator=gen, device="cuda") * 8).to(torch.float8_e4m3fn).view(torch.uint8)
    nb = K // 32
    SA = (124 + torch.randint(-2, 3, (M, nb), generator=gen, device="cuda")).to(torch.uint8)
    SB = (124 + torch.randint(-2, 3, (N, nb), generator=gen, device="cuda")).to(torch.uint8)
    D = mx.mx_matmul(A, SA, B, SB, K, "e4m3", "e4m3", out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = sorted(set([0, 1, M // 2, M - 257, M - 1] + rng.integers(0, M, 30).tolist()))
    cols = sorted(set([0, 1, 128, N - 1] + rng.integers(0, N, 20).tolist()))
    ii = torch.tensor(rows, dtype=torch.long, device="cuda")
    jj = torch.tensor(cols, dtype=torch.long, device="cuda")
    Ah, SAh = A.index_select(0, ii).cpu().numpy(), SA.index_select(0, ii).cpu().numpy()
    Bh, SBh = B.index_select(0, jj).cpu().numpy(), SB.index_select(0, jj).cpu().numpy()
    ref, S, S8 = oracle.mx_gemm_f64(Ah, SAh, Bh, SBh, K, "e4m3", "e4m3", runs=True)
    got = gemm_inputs.bits(D.index_select(0, ii).index_select(1, jj).cpu())
    n, worst, _ = oracle.mx_tol_check(got, "bf16", ref, S, S8)
    assert n == 0, "MX A 4 GiB: %d sampled outputs outside the bound (worst %.3g)" % (n, worst)
