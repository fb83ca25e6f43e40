"""Shared helpers of the GPU tests: run the HIP path, check it against the oracle."""
import numpy as np
import torch

import dense_tiled_gemm_02_amd as g
import gemm_inputs
import oracle

DT_CODE = {"f16": g.GEMM_F16, "bf16": g.GEMM_BF16}


def gpu_run(A, B, C=None, config=None, out=None):
    """D = A x B (+C) through libgemm.so; A, B, C are CPU tensors; returns CPU D."""
    dA, dB = A.cuda(), B.cuda()
    dC = C.cuda() if C is not None else None
    if out is None:
        # NaN-filled: an output the kernels fail to write cannot pass a check
        out = torch.full((A.shape[0], B.shape[1]), float("nan"), dtype=A.dtype, device="cuda")
    D = g.matmul(dA, dB, dC, out=out, config=config)
    torch.cuda.synchronize()
    return D.cpu()


def check(A, B, C, D, dtype, sample=None, label=""):
    """Apply the acceptance rule to D (CPU tensor) against the oracle.

    sample: None for every output, or (ii, jj) arrays of positions."""
    Ab, Bb = gemm_inputs.bits(A), gemm_inputs.bits(B)
    Cb = gemm_inputs.bits(C) if C is not None else None
    Db = gemm_inputs.bits(D)
    if sample is None:
        ref, S = oracle.gemm_f64(Ab, Bb, Cb, dtype)
        got = Db
    else:
        ii, jj = sample
        ref, S = oracle.gemm_f64_at(Ab, Bb, Cb, ii, jj, dtype)
        got = Db[ii, jj]
    n, worst, first = oracle.tol_check(got, ref, S, dtype)
    assert n == 0, "%s: %d outputs outside the bound (worst ratio %.3g, first flat index %d)" % (
        label, n, worst, first)
    return worst


def sample_positions(M, N, count, seed):
    """Whole first/last rows and columns plus random positions."""
    rng = np.random.default_rng(seed)
    ii = [np.zeros(N, np.int64), np.full(N, M - 1, np.int64), np.arange(M), np.arange(M),
          rng.integers(0, M, count)]
    jj = [np.arange(N), np.arange(N), np.zeros(M, np.int64), np.full(M, N - 1, np.int64),
          rng.integers(0, N, count)]
    return np.concatenate(ii), np.concatenate(jj)
