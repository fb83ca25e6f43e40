"""Matrix-instruction throughput on this GPU (test infrastructure):

    python tests/gpu_probes/rates.py

Runs probe_mfma_rate (tests/gpu_probes/probe_layouts.hip) for each
instruction kind with one and two waves per SIMD and prints TFLOP/s next to
the nominal dense peak.  Needs tests/gpu_probes/libgemm_probe.so (build.py)."""
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
KINDS = [(0, "bf16 16x16x32", 2516.6), (1, "E4M3 scaled 32x32x64", 5033.2), (2, "E2M1 scaled 32x32x64", 10066.3),
         (3, "E2M3 (FP6) scaled 32x32x64", 10066.3), (4, "E4M3 x E2M1 scaled 32x32x64", 5033.2)]


def rates(grid=1024, iters=2000):
    import torch
    lib = ctypes.CDLL(os.path.join(HERE, "libgemm_probe.so"))
    lib.probe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    out = torch.empty(grid * 512, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    for waves in (4, 8):
        for kind, name, peak in KINDS:
            ms, flop = ctypes.c_float(), ctypes.c_double()
            st = lib.probe_mfma_rate(kind, grid, waves, iters, ctypes.c_void_p(out.data_ptr()),
                                     ctypes.c_void_p(stream), ctypes.byref(ms), ctypes.byref(flop))
            if st != 0:
                raise RuntimeError("probe_mfma_rate(%d) failed: %d" % (kind, st))
            tf = flop.value / (ms.value * 1e-3) / 1e12
            rows.append((name, waves // 4, tf, peak))
    return rows


if __name__ == "__main__":
    for name, per_simd, tf, peak in rates():
        print("%-30s %d wave(s) per SIMD  %8.1f TFLOP/s  %5.1f %% of the %.1f nominal" % (
            name, per_simd, tf, 100 * tf / peak, peak), flush=True)
    sys.exit(0)
