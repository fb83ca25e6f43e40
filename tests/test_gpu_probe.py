"""Lane-layout pins of the gfx950 matrix instructions the kernels rely on (GPU).

One wavefront runs one instruction on small integer matrices, packing the
operands with the lane layouts the tile kernel assumes and unpacking the result
with the assumed output layout; integer inputs make every product and sum
exact, so any layout mistake shows as a mismatch.
"""
import ctypes
import json
import os

import numpy as np
import pytest
import torch

import dense_tiled_gemm_02_amd as g
import gemm_inputs

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(g.LIB_PATH), "libgemm_probe.so")


@pytest.fixture(scope="module")
def probe():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    L = ctypes.CDLL(PROBE)
    L.probe_mfma.restype = ctypes.c_int
    L.probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_void_p, ctypes.c_void_p]
    L.probe_lds_read_tr.restype = ctypes.c_int
    L.probe_lds_read_tr.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return L


@pytest.mark.parametrize("mf", [16, 32])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_mfma_lane_layout(probe, mf, dt):
    ki = 32 if mf == 16 else 16
    rng = np.random.default_rng(mf * 10 + len(dt))
    Ai = rng.integers(-4, 5, (mf, ki))
    Bi = rng.integers(-4, 5, (ki, mf))
    A = torch.from_numpy(Ai.astype(np.float32)).to(gemm_inputs.TORCH_DTYPES[dt]).cuda()
    B = torch.from_numpy(Bi.astype(np.float32)).to(gemm_inputs.TORCH_DTYPES[dt]).cuda()
    D = torch.full((mf, mf), float("nan"), dtype=torch.float32, device="cuda")
    rc = probe.probe_mfma(mf, 1 if dt == "bf16" else 0, A.data_ptr(), B.data_ptr(), D.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert np.array_equal(D.cpu().numpy(), (Ai @ Bi).astype(np.float32))


def test_lds_transpose_read_lane_map(probe):
    """Records which LDS halfword each lane/element of the transposing 64-bit
    read returns (input halfword i holds the value i).  Written to
    gpurun_out/lds_read_tr_map.json; asserted only to be a permutation of the
    first 256 halfwords, the bytes the 64 lanes address."""
    src = torch.arange(512, dtype=torch.int32).to(torch.int16).cuda()
    out = torch.zeros(256, dtype=torch.int16, device="cuda")
    rc = probe.probe_lds_read_tr(src.data_ptr(), out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64).reshape(64, 4)
    os.makedirs("gpurun_out", exist_ok=True)
    with open(os.path.join("gpurun_out", "lds_read_tr_map.json"), "w") as f:
        json.dump(got.tolist(), f)
    assert sorted(got.ravel().tolist()) == list(range(256))
