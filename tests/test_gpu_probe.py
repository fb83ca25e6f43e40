"""Lane-layout pins of the gfx950 matrix instructions the kernels rely on (GPU).

One wavefront runs one instruction on small integer matrices, packing the
operands with the lane layouts the tile kernel assumes and unpacking the result
with the assumed output layout; integer inputs make every product and sum
exact, so any layout mistake shows as a mismatch.
"""
import ctypes
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
    L.probe_lds_dma.restype = ctypes.c_int
    L.probe_lds_dma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
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
    """The transposing 64-bit LDS read (ds_read_b64_tr_b16): within each group of
    16 lanes, the 16 addressed 8-byte pieces, taken in lane order, form a 4 x 16
    matrix of halfwords (lanes 4i..4i+3 supply row i); lane t of the group
    receives column t, rows 0..3.  Input halfword h holds the value h, and lane
    l addresses halfwords 4l..4l+3."""
    src = torch.arange(512, dtype=torch.int32).to(torch.int16).cuda()
    out = torch.zeros(256, dtype=torch.int16, device="cuda")
    rc = probe.probe_lds_read_tr(src.data_ptr(), out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64).reshape(64, 4)
    want = np.array([[64 * (l // 16) + 16 * i + (l % 16) for i in range(4)] for l in range(64)])
    assert np.array_equal(got, want)


def test_direct_lds_loads_place_lane_data_contiguously_and_zero_out_of_range(probe):
    """A 16-byte load into LDS puts lane l's data at LDS byte 16 l past the base
    (both the buffer and the global form), and the buffer form writes zeros for
    lanes whose offset is past the descriptor's range."""
    src = torch.arange(2048, dtype=torch.int32).to(torch.int16).cuda()   # 4096 bytes
    out = torch.zeros(1024, dtype=torch.int16, device="cuda")
    rc = probe.probe_lds_dma(src.data_ptr(), out.data_ptr(), 1024, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64).reshape(128, 8)
    for l in range(64):
        if l < 48:
            c = (7 * l) % 64
            assert list(got[l]) == list(range(8 * c, 8 * c + 8)), l
        else:
            assert list(got[l]) == [0] * 8, l
        c = (5 * l) % 64
        assert list(got[64 + l]) == list(range(8 * c, 8 * c + 8)), l
