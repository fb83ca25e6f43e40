"""Stream-K plans (kernel 6) on the GPU: parity with the CPU oracle for
ranges that cut tiles into 2..many parts, hold several whole tiles, or hold
one tile whole (then the result equals the data-parallel kernel's bit for
bit: the same accumulation), ragged edges, the addend, both 16-bit types;
run-to-run determinism; and 3072^2 x 4096 with one workgroup per CU, in
full."""
import pytest
import torch

import dense_tiled_gemm_02_amd as g
import gemm_inputs
from helpers import check, gpu_run

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


SK256 = dict(kernel=g.KERNEL_DMA_SK, bm=256, bn=256)
SK128 = dict(kernel=g.KERNEL_DMA_SK, bm=256, bn=128)


@pytest.mark.parametrize("mnk,tile,ws", [
    ((512, 512, 1024), SK256, (1, 3, 7, 16, 64)),        # 4 tiles x 16 K steps
    ((1000, 520, 1000), SK256, (2, 5, 11, 31)),          # ragged M, N and K (tail step of 40)
    ((1000, 520, 1000), SK128, (3, 13, 50)),             # 64 accumulators per lane
    ((768, 1024, 4096), SK256, (5, 24, 100)),            # 12 tiles x 64 K steps
])
def test_stream_k_parity(mnk, tile, ws):
    M, N, K = mnk
    for dt, has_c in (("bf16", True), ("f16", False)):
        A, B, C = _inputs(M, N, K, dt, has_c, seed=M + 3 * N + 7 * K)
        for w in ws:
            cfg = dict(tile, splitk=w)
            print("case %s %s %s" % (mnk, dt, cfg), flush=True)
            D = gpu_run(A, B, C, config=cfg)
            check(A, B, C, D, dt, label="stream-K %s %s W=%d" % (mnk, dt, w))


def test_one_range_equals_the_data_parallel_kernel():
    """W = 1: one range holds every tile whole, so no part is exchanged and
    each tile sums its K steps in the data-parallel kernel's order."""
    M, N, K = 600, 704, 520
    A, B, C = _inputs(M, N, K, "bf16", True, seed=5)
    D1 = gpu_run(A, B, C, config=dict(SK256, splitk=1))
    D0 = gpu_run(A, B, C, config=dict(kernel=3, bm=256, bn=256, bk=64, stages=2, mfma=16, waves_m=2,
                                       waves_n=4))
    check(A, B, C, D1, "bf16", label="stream-K W=1")
    assert torch.equal(D0.view(torch.int16), D1.view(torch.int16))


def test_stream_k_is_deterministic_and_reuses_its_workspace():
    M, N, K = 1024, 1024, 2048
    A, B, C = _inputs(M, N, K, "bf16", False, seed=9)
    outs = [gpu_run(A, B, C, config=dict(SK256, splitk=w)) for w in (37, 37, 5, 37)]
    check(A, B, C, outs[0], "bf16", label="stream-K W=37")
    check(A, B, C, outs[2], "bf16", label="stream-K W=5")
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[3].view(torch.int16))


def test_stream_k_3072_one_workgroup_per_cu():
    """3072^2 x 4096 (144 tiles of 256 x 256) dealt to 256 workgroups, every
    output against the oracle."""
    M = N = 3072
    K = 4096
    A, B, _ = _inputs(M, N, K, "bf16", False, seed=17, dist="normal", scale=1 / 64)
    cfg = dict(SK256, splitk=256)
    pl = g.plan_for(A.cuda(), B.cuda(), None, None, cfg)
    print("plan", pl.describe(), flush=True)
    assert pl.config.kernel == g.KERNEL_DMA_SK and pl.config.splitk == 256
    D = gpu_run(A, B, config=cfg)
    check(A, B, None, D, "bf16", label="stream-K 3072^2 x 4096")
