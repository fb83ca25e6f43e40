"""gemm_run_static, the entry point that allocates nothing (GPU).

Its K-slice workspace is a fixed device array of the library instead of a
caller's buffer.  Each call is checked against gemm_run with a workspace of
the caller's (the same plan, so the same kernels: bit for bit) and against
the oracle's acceptance rule.  The calls come in a row, on the one array:
* a K-sliced square plan (16 tiles x 16 slices, 16 MiB of partials);
* a smaller K-sliced decode plan;
* the first again, which needs the counters the earlier launches left at zero;
* a plan without a workspace;
* a forced stream-K plan (37 workgroups, ~19 MiB of parts) and the first again.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_02_amd as g
import gemm_inputs
from helpers import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    torch.cuda.init()


def _both(M, N, K, dt, has_c, seed, want_ws, config=None):
    A = gemm_inputs.draw((M, K), seed, dt)
    B = gemm_inputs.draw((K, N), seed + 1, dt)
    C = gemm_inputs.draw((M, N), seed + 2, dt) if has_c else None
    dA, dB = A.cuda(), B.cuda()
    dC = C.cuda() if C is not None else None
    pl = g.plan_for(dA, dB, dC, None, config)
    need = g.gemm_workspace_size(pl)
    print("case %dx%dx%d %s: %s, workspace %d" % (M, N, K, dt, pl.describe(), need), flush=True)
    assert (need > 0) == want_ws and need <= g.GEMM_STATIC_SCRATCH_BYTES
    ref = torch.full((M, N), float("nan"), dtype=A.dtype, device="cuda")
    g.matmul(dA, dB, dC, out=ref, config=config)           # gemm_run, caller's workspace
    out = torch.full((M, N), float("nan"), dtype=A.dtype, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = g.lib().gemm_run_static(pl.handle, dA.data_ptr(), dB.data_ptr(),
                                 dC.data_ptr() if dC is not None else None, out.data_ptr(), stream)
    assert st == g.GEMM_OK, g.gemm_last_error()
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), out.view(torch.int16))
    check(A, B, C, out.cpu(), dt, label="static scratch %dx%dx%d" % (M, N, K))


def test_static_scratch_matches_the_workspace_entry_point():
    _both(512, 512, 16384, "bf16", True, 11, True)
    _both(16, 4096, 4096, "bf16", False, 21, True)        # smaller
    _both(512, 512, 16384, "bf16", True, 31, True)        # the counters were left at zero
    _both(256, 256, 256, "f16", False, 41, False)         # no workspace: as gemm_run
    _both(1000, 1104, 1024, "bf16", True, 51, True, dict(kernel=g.KERNEL_DMA_SK, bm=256, bn=256, splitk=37))
    _both(512, 512, 16384, "bf16", True, 61, True)        # after the stream-K parts
