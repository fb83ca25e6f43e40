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

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpu_probes", "libgemm_probe.so")


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


@pytest.mark.parametrize("mf", [16, 32])
def test_int8_mfma_lane_layout(probe, mf):
    """v_mfma_i32_16x16x64_i8 / 32x32x32_i8 with the operand layout the int8
    tile kernel assumes (lane l: row / column l % MF, k = 16 (l / MF) + 0..15)
    and the floating-point result layout; full-range codes, so the int32 sums
    are exact integers and the comparison is bit for bit."""
    L = probe
    L.probe_mfma_i8.restype = ctypes.c_int
    L.probe_mfma_i8.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    ki = 64 if mf == 16 else 32
    rng = np.random.default_rng(90 + mf)
    Ai = rng.integers(-128, 128, (mf, ki)).astype(np.int8)
    Bi = rng.integers(-128, 128, (ki, mf)).astype(np.int8)
    A, B = torch.from_numpy(Ai).cuda(), torch.from_numpy(Bi).cuda()
    D = torch.full((mf, mf), -7, dtype=torch.int32, device="cuda")
    rc = L.probe_mfma_i8(mf, A.data_ptr(), B.data_ptr(), D.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert np.array_equal(D.cpu().numpy(), Ai.astype(np.int64) @ Bi.astype(np.int64))


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


# Scaled matrix instruction: (mf, format of A, format of B, scale byte of A, of B)
SCALED = [(mf, fa, fb, oa, ob) for mf in (16, 32)
          for (fa, fb, oa, ob) in [(0, 0, 0, 0), (1, 1, 0, 0), (4, 4, 0, 0), (0, 1, 0, 0),
                                   (0, 0, 1, 2), (0, 0, 3, 1), (4, 4, 2, 3),
                                   # FP6 elements and operands of different widths
                                   (2, 2, 0, 0), (3, 3, 0, 0), (2, 3, 0, 0), (0, 4, 0, 0),
                                   (4, 0, 0, 0), (2, 4, 0, 0), (4, 3, 0, 0), (1, 2, 0, 0)]]
FMT_NAME = {0: "e4m3", 1: "e5m2", 2: "e2m3", 3: "e3m2", 4: "e2m1"}


def _small_codes(rng, shape, fmt):
    """Codes of small dyadic values (|v| <= 6), so every sum below is exact."""
    if fmt == "e2m1":
        return rng.integers(0, 16, shape).astype(np.uint8)
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -2, -3, -4, -6], dtype=np.float32)
    if fmt in ("e2m3", "e3m2"):                  # the codes of those values, looked up
        import oracle
        table = oracle.mx_decode(np.arange(64, dtype=np.uint8), fmt)
        lut = np.array([int(np.flatnonzero(table == v)[0]) for v in vals], np.uint8)
        return lut[rng.integers(0, len(vals), shape)]
    v = torch.from_numpy(vals[rng.integers(0, len(vals), shape)])
    dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    return v.to(dt).view(torch.uint8).numpy()


def _lane_bytes(codes_row, g, KI, fmt):
    """The 8 operand dwords of lane group g for one row (column) of the
    instruction's K = KI elements:
      8-bit formats: dwords 0-3 hold k = 16 g + 0..15, dwords 4-7 hold
        k = KI/2 + 16 g + 0..15 (one byte each);
      4-bit format: dwords 0-3 hold k = 32 g + 0..31, two per byte with the
        even k in the low nibble; dwords 4-7 are not read (nonzero filler);
      6-bit formats: dwords 0-5 hold k = 32 g + 0..31 as one little-endian
        bit string, k = 32 g + t in bits 6 t .. 6 t + 5; dwords 6-7 are not
        read (nonzero filler)."""
    if fmt in ("e2m3", "e3m2"):
        c = codes_row[32 * g:32 * g + 32].astype(object)
        bits = sum(int(v) << (6 * t) for t, v in enumerate(c))
        b = np.frombuffer(bits.to_bytes(24, "little"), np.uint8)
        b = np.concatenate([b, np.full(8, 0x5A, np.uint8)])
    elif fmt == "e2m1":
        c = codes_row[32 * g:32 * g + 32]
        b = (c[0::2] | (c[1::2] << 4)).astype(np.uint8)
        b = np.concatenate([b, np.full(16, 0x77, np.uint8)])
    else:
        b = np.concatenate([codes_row[16 * g:16 * g + 16], codes_row[KI // 2 + 16 * g:KI // 2 + 16 * g + 16]])
    return b.astype(np.uint8).view(np.uint32)


@pytest.mark.parametrize("mf,fa,fb,oa,ob", SCALED)
def test_scaled_mfma_lane_layout(probe, mf, fa, fb, oa, ob):
    """v_mfma_scale_f32_{16x16x128,32x32x64}_f8f6f4: lane l = r + MF g holds
    row (column) r of its operand, at the k positions given by _lane_bytes;
    byte `opsel` of its scale register is the E8M0 scale of row r and of the
    instruction's 32-k block number g (k = 32 g .. 32 g + 31), whichever lanes
    hold that block's elements; the result layout is that of the unscaled
    instructions of the same shape."""
    import oracle
    L = probe
    L.probe_mfma_scaled.restype = ctypes.c_int
    L.probe_mfma_scaled.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 6
    KI = 128 if mf == 16 else 64
    nb = KI // 32
    rng = np.random.default_rng(1000 * mf + 100 * fa + 10 * fb + 4 * oa + ob)
    fA, fB = FMT_NAME[fa], FMT_NAME[fb]
    Ac = _small_codes(rng, (mf, KI), fA)
    Bc = _small_codes(rng, (mf, KI), fB)           # row j = column j of B
    SA = rng.integers(125, 130, (mf, nb)).astype(np.uint8)
    SB = rng.integers(125, 130, (mf, nb)).astype(np.uint8)
    a = np.zeros((64, 8), np.uint32)
    b = np.zeros((64, 8), np.uint32)
    sa = rng.integers(100, 150, (64, 4)).astype(np.uint8)     # filler bytes
    sb = rng.integers(100, 150, (64, 4)).astype(np.uint8)
    for l in range(64):
        r, g = l % mf, l // mf
        a[l] = _lane_bytes(Ac[r], g, KI, fA)
        b[l] = _lane_bytes(Bc[r], g, KI, fB)
        sa[l, oa] = SA[r, g]
        sb[l, ob] = SB[r, g]
    Av = oracle.mx_decode(Ac, fA) * np.repeat(np.ldexp(1.0, SA.astype(np.int64) - 127), 32, 1)
    Bv = oracle.mx_decode(Bc, fB) * np.repeat(np.ldexp(1.0, SB.astype(np.int64) - 127), 32, 1)
    want = Av @ Bv.T
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int32)).cuda()
    ta, tb = dev(a), dev(b)
    tsa, tsb = dev(sa.view(np.uint32).reshape(64)), dev(sb.view(np.uint32).reshape(64))
    regs = 4 if mf == 16 else 16
    out = torch.full((64 * regs,), float("nan"), dtype=torch.float32, device="cuda")
    rc = L.probe_mfma_scaled(mf, fa, fb, oa, ob, ta.data_ptr(), tb.data_ptr(), tsa.data_ptr(), tsb.data_ptr(),
                             out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(64, regs).astype(np.float64)
    got = np.full((mf, mf), np.nan)
    for l in range(64):
        for r in range(regs):
            if mf == 16:
                got[4 * (l // 16) + r, l % 16] = o[l, r]
            else:
                got[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] = o[l, r]
    assert np.array_equal(got, want), (got - want)


def test_scaled_mfma_rounds_runs_of_eight_products():
    """The arithmetic behind the MX acceptance rule: the 32x32x64 scaled
    instruction (E4M3) adds each run of 8 consecutive products after aligning
    them to the largest, keeping 13 bits below its leading bit.  Row 0 of A
    holds 256 at k = 0 and a small value s at k = 1..63, B is all 1.0: the 7
    small products in the run of the large one are kept when s = 2^-5 (13
    binades below) and lost when s = 2^-6 (14 below); the other 56 are exact."""
    L = probe_lib_scaled()
    for small, code, kept in ((2.0 ** -5, 0x10, True), (2.0 ** -6, 0x08, False), (2.0 ** -9, 0x01, False)):
        a = np.zeros((64, 32), np.uint8)
        b = np.full((64, 32), 0x38, np.uint8)                  # 1.0
        a[0, :] = code
        a[32, :] = code
        a[0, 0] = 0x78                                         # 256
        s = np.full((64, 4), 127, np.uint8)
        o = _run_scaled(L, 32, 0, 0, a, b, s, s)
        want = 256.0 + (63 if kept else 56) * small
        assert o[0, 0] == np.float32(want), (small, o[0, 0], want)


def probe_lib_scaled():
    L = ctypes.CDLL(PROBE)
    L.probe_mfma_scaled.restype = ctypes.c_int
    L.probe_mfma_scaled.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 6
    return L


def _run_scaled(L, mf, fa, fb, a, b, sa, sb):
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int32).reshape(-1)).cuda()
    regs = 4 if mf == 16 else 16
    out = torch.full((64 * regs,), float("nan"), dtype=torch.float32, device="cuda")
    ta, tb, tsa, tsb = dev(a), dev(b), dev(sa), dev(sb)
    assert L.probe_mfma_scaled(mf, fa, fb, 0, 0, ta.data_ptr(), tb.data_ptr(), tsa.data_ptr(), tsb.data_ptr(),
                               out.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(64, regs)


def test_matrix_instruction_rates():
    """Back-to-back independent matrix instructions reach at least half of
    their nominal dense peak (the ceiling a kernel's instruction stream is
    read against; a mixed 8-bit x 4-bit pair runs at the 8-bit rate)."""
    import os
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpu_probes"))
    import rates
    for name, per_simd, tf, peak in rates.rates(grid=1024, iters=500):
        print("%s, %d wave(s) per SIMD: %.1f TFLOP/s (%.1f %% of %.1f)" % (name, per_simd, tf, 100 * tf / peak, peak))
        assert tf >= 0.5 * peak, (name, per_simd, tf)
