"""Launches captured in a HIP graph (GPU).

gemm_run and gemm_mx_run enqueue kernels only (no allocation, no memset, no
synchronization), so a caller may capture them.  Each case captures one run
on a side stream, then replays the graph several times with eager work and
synchronizations between the replays; every replay must equal the eager run
bit for bit (the kernels are deterministic, K slices included: their fused
reduce sums in slice order and returns the workspace counters to zero, which
is what lets a captured launch be replayed without re-initialising them).
After new inputs are written into the same buffers, a replay must equal an
eager run on them, and the eager result is checked against the oracle.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_02_amd as g
import dense_tiled_gemm_02_amd.mx as mx
import gemm_inputs
import oracle
from helpers import check

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    torch.cuda.init()


def _capture(launch):
    """A CUDAGraph holding launch(stream) recorded on a side stream."""
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        launch(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return graph


def _replays_equal(graph, D, ref, what):
    for r in range(REPLAYS):
        D.fill_(float("nan"))                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(D.view(torch.int16), ref.view(torch.int16)), "%s: replay %d differs" % (what, r)


# (M, N, K, forced config or None): 256 x 256 tiles with ragged edges, K
# slices of 128 x 128 tiles, the skinny kernel with K slices, a small ragged
# problem (64 x 64 tiles), stream-K over 37 workgroups (cut tiles exchanged)
CASES = [((1000, 1104, 520), dict(kernel=3, bm=256, bn=256, bk=64, stages=2, waves_m=2, waves_n=4)),
         ((512, 512, 8192), None),
         ((16, 8192, 2048), dict(kernel=2, bn=128, splitk=4)),
         ((200, 328, 136), None),
         ((1000, 1104, 1024), dict(kernel=6, bm=256, bn=256, splitk=37))]


@pytest.mark.parametrize("mnk,force", CASES)
def test_captured_run_replays_bitwise(mnk, force):
    M, N, K = mnk
    A, B, C = (gemm_inputs.draw(s, 70 + i, "bf16", "uniform", 1.0) for i, s in enumerate(((M, K), (K, N), (M, N))))
    dA, dB, dC = A.cuda(), B.cuda(), C.cuda()
    plan = g.gemm_plan_create(g.problem(M, N, K, g._dtype_code(dA), has_c=True), 0, force)
    print("graph", mnk, g.gemm_plan_describe(plan), flush=True)
    need = g.gemm_workspace_size(plan)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    if need:
        g.gemm_workspace_init(plan, ws.data_ptr(), need, st)
    wsp = ws.data_ptr() if need else None
    D_eager = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    D = torch.empty_like(D_eager)

    def run(out, stream):
        g.gemm_run(plan, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), out.data_ptr(), wsp, need, stream)

    run(D_eager, st)
    torch.cuda.synchronize()
    graph = _capture(lambda s: run(D, s))
    _replays_equal(graph, D, D_eager, "gemm %s" % (mnk,))

    # new inputs in the same buffers: the graph reads them
    A2 = gemm_inputs.draw((M, K), 90, "bf16", "uniform", 1.0)
    dA.copy_(A2.cuda())
    run(D_eager, st)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(D.view(torch.int16), D_eager.view(torch.int16))
    check(A2, B, C, D_eager.cpu(), "bf16", label="graph %s" % (mnk,))


@pytest.mark.parametrize("fmt,M,N,K", [("e2m1", 16, 4096, 4096), ("e4m3", 512, 512, 8192)])
def test_captured_mx_run_replays_bitwise(fmt, M, N, K):
    """The block-scaled kernel, in its decode regime (K slices) and with
    K slices of 128 x 128 tiles."""
    A, SA = gemm_inputs.draw_mx(M, K, fmt, 71)
    B, SB = gemm_inputs.draw_mx(N, K, fmt, 72)
    dA, dSA, dB, dSB = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (A, SA, B, SB))
    p = mx.mx_problem(M, N, K, fmt, fmt, mx.GEMM_MX_OUT_BF16, lda=A.shape[1], ldb=B.shape[1],
                      ldsa=SA.shape[1], ldsb=SB.shape[1])
    plan = mx.gemm_mx_plan_create(p, 0, None)
    print("graph mx", fmt, M, N, K, mx.gemm_mx_plan_describe(plan), flush=True)
    need = mx.gemm_mx_workspace_size(plan)
    assert need > 0, "expected a K-sliced plan"
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    mx.gemm_mx_workspace_init(plan, ws.data_ptr(), need, st)
    D_eager = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    D = torch.empty_like(D_eager)

    def run(out, stream):
        mx.gemm_mx_run(plan, dA.data_ptr(), dSA.data_ptr(), dB.data_ptr(), dSB.data_ptr(), None, out.data_ptr(),
                       ws.data_ptr(), need, stream)

    run(D_eager, st)
    torch.cuda.synchronize()
    graph = _capture(lambda s: run(D, s))
    _replays_equal(graph, D, D_eager, "mx %s" % fmt)
    ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt, runs=True)
    n, worst, first = oracle.mx_tol_check(gemm_inputs.bits(D.cpu()), "bf16", ref, S, S8)
    assert n == 0, "mx graph %s: %d outputs outside the bound (worst %.3g)" % (fmt, n, worst)
