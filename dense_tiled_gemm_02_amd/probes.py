"""Rate probes of the gfx950 units the GEMM kernels lean on (needs the GPU).

    python -m dense_tiled_gemm_02_amd.probes

Runs the probe kernels of libgemm_probe.so on 256 workgroups of 8 waves
and prints one table each:
  * matrix-core rate: register-only MFMA loops (16x16x32 and 32x32x16 bf16),
    with the shader clock under that load (s_memtime against the 100 MHz
    s_memrealtime), and the same for the block-scaled instructions (E4M3 and
    E2M1 operands);
  * LDS fill rate: bytes per clock per CU that reach LDS from L2-resident
    data, by direct global -> LDS loads and by global -> VGPR loads plus LDS
    writes, alone and beside 16-byte LDS reads;
  * matrix-core rate under memory traffic: the same MFMA loop with 1..8 KiB
    of loads or LDS reads issued per 32 MFMAs per wave.
"""
import ctypes
import os
import statistics

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB = os.path.join(HERE, "libgemm_probe.so")


def _lib():
    L = ctypes.CDLL(PROBE_LIB)
    L.probe_mfma_rate.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    L.probe_lds_fill_rate.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.probe_mfma_scaled_rate.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 3
    L.probe_mfma_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return L


def _timed(fn):
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e)


def mfma_rate(L, stream):
    print("matrix-core rate, register operands, 8 waves per workgroup, 256 workgroups")
    grid, iters, waves = 256, 2000, 8
    out = torch.empty(grid * 64 * waves, device="cuda")
    clk = torch.zeros(2 * grid, dtype=torch.int64, device="cuda")
    for mf in (16, 32):
        assert L.probe_mfma_rate(mf, waves, 10, grid, out.data_ptr(), clk.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        ms = _timed(lambda: L.probe_mfma_rate(mf, waves, iters, grid, out.data_ptr(), clk.data_ptr(), stream))
        c = clk.cpu().view(-1, 2).double()
        ghz = (c[:, 0] / (c[:, 1] / 100e6) / 1e9).mean().item()
        flop = grid * waves * iters * 524288
        print("  %dx%d: %.0f TFLOP/s, shader clock %.2f GHz" % (mf, mf, flop / ms / 1e9, ghz))


def mfma_scaled_rate(L, stream):
    print("block-scaled matrix-core rate (v_mfma_scale_*_f8f6f4), register operands, 8 waves, 256 workgroups")
    grid, iters, waves = 256, 2000, 8
    out = torch.empty(grid * 64 * waves, device="cuda")
    clk = torch.zeros(2 * grid, dtype=torch.int64, device="cuda")
    for mf in (16, 32):
        for fmt, name in ((0, "E4M3"), (4, "E2M1")):
            assert L.probe_mfma_scaled_rate(mf, fmt, waves, 10, grid, out.data_ptr(), clk.data_ptr(), stream) == 0
            torch.cuda.synchronize()
            ms = _timed(lambda: L.probe_mfma_scaled_rate(mf, fmt, waves, iters, grid, out.data_ptr(),
                                                         clk.data_ptr(), stream))
            c = clk.cpu().view(-1, 2).double()
            ghz = (c[:, 0] / (c[:, 1] / 100e6) / 1e9).mean().item()
            per = 32 if mf == 16 else 16                          # instructions per iteration
            flop = grid * waves * iters * per * (2 * 16 * 16 * 128 if mf == 16 else 2 * 32 * 32 * 64)
            print("  %dx%d %s: %.0f TFLOP/s, shader clock %.2f GHz" % (mf, mf, name, flop / ms / 1e9, ghz))


def lds_fill(L, stream):
    print("LDS fill rate from L2-resident data (64 KiB per workgroup per pass), 256 workgroups")
    names = {0: "direct global->LDS loads", 1: "direct loads + 24 ds_read_b128/wave",
             2: "24 ds_read_b128/wave only", 3: "global->VGPR loads + ds_write_b128",
             4: "VGPR path + 24 ds_read_b128/wave"}
    grid, iters = 256, 400
    src = torch.randint(0, 30000, (grid * 32768,), dtype=torch.int16, device="cuda")
    cyc = torch.zeros(grid, dtype=torch.int32, device="cuda")
    sink = torch.zeros(512, dtype=torch.int32, device="cuda")
    for mode in range(5):
        assert L.probe_lds_fill_rate(mode, src.data_ptr(), grid * 65536, grid, 5, cyc.data_ptr(),
                                     sink.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        assert L.probe_lds_fill_rate(mode, src.data_ptr(), grid * 65536, grid, iters, cyc.data_ptr(),
                                     sink.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        per = statistics.median(cyc.cpu().tolist()) / iters
        rate = "%6.1f B/clk/CU into LDS" % (65536 / per) if mode != 2 else "(reads only)"
        print("  %-38s %7.1f cycles per pass  %s" % (names[mode], per, rate))


def mfma_mix(L, stream):
    print("matrix-core rate with memory instructions between the MFMAs (per 32 MFMAs per wave)")
    grid, iters = 256, 400
    src = torch.randint(0, 30000, (grid * 32768,), dtype=torch.int16, device="cuda")
    cyc = torch.zeros(grid, dtype=torch.int32, device="cuda")
    out = torch.zeros(grid * 512, dtype=torch.float32, device="cuda")
    names = {0: "direct global->LDS load", 1: "VGPR load + ds_write_b128", 2: "ds_read_b128", 3: "VGPR load only"}
    flop = grid * 8 * iters * 32 * 16384
    cases = [(0, 0)] + [(m, nl) for m in (0, 1, 3, 2) for nl in (1, 2, 4, 8)]
    res = {}
    for _ in range(3):
        for (m, nl) in cases:
            assert L.probe_mfma_mix(m, nl, src.data_ptr(), grid * 65536, grid, 5, cyc.data_ptr(), out.data_ptr(),
                                    stream) == 0
            torch.cuda.synchronize()
            ms = _timed(lambda: L.probe_mfma_mix(m, nl, src.data_ptr(), grid * 65536, grid, iters, cyc.data_ptr(),
                                                 out.data_ptr(), stream))
            res.setdefault((m, nl), []).append(ms)
    for (m, nl) in cases:
        ms = statistics.median(res[(m, nl)])
        label = "%s, %d KiB" % (names[m], nl) if nl else "MFMA only"
        print("  %-36s %6.0f TFLOP/s" % (label, flop / ms / 1e9))


def main():
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    L = _lib()
    stream = torch.cuda.current_stream().cuda_stream
    mfma_rate(L, stream)
    mfma_scaled_rate(L, stream)
    lds_fill(L, stream)
    mfma_mix(L, stream)


if __name__ == "__main__":
    main()
