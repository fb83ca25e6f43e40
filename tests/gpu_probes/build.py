"""Build the single-instruction probe library (test infrastructure only).

    python tests/gpu_probes/build.py

Compiles probe_layouts.hip with hipcc for gfx950 (packed fp32 instructions
disabled, as for the GEMM library) into tests/gpu_probes/libgemm_probe.so.
The GPU tests in tests/test_gpu_probe.py load it to pin the lane layouts of
the matrix instructions, the transposing LDS read and the direct
global -> LDS loads that the kernels assume.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "probe_layouts.hip")
LIB = os.path.join(HERE, "libgemm_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wl,-z,defs",
           "-x", "hip", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe library build failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
