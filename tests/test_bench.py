"""Host logic of bench.py (CPU): the kernel-name mapping that ties the
committed counter runs to the plans the benchmark times, and the refusal of
more than one GPU."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_profiled_names_map_to_plan_names():
    assert bench.plan_kernel_name(
        "void dtg::(anonymous namespace)::gemm_dma_kernel<256, 256, 64, 2, 4, 16, 2, true, false, false>(dtg::KArgs)"
    ) == "gemm_dma_kernel<256,256,64,2,4,16,2,1,lay0>"
    assert bench.plan_kernel_name(
        "void dtg::(anonymous namespace)::gemm_dma_kernel<128, 128, 64, 2, 4, 16, 2, false, true, true>(dtg::KArgs)"
    ) == "gemm_dma_kernel<128,128,64,2,4,16,2,0,lay3>"
    assert bench.plan_kernel_name(
        "void dtg::(anonymous namespace)::gemm_skinny_kernel<128, 8, 32, 2, true, 16>(dtg::KArgs)"
    ) == "gemm_skinny_kernel<128,8,32,2,1,16>"
    assert bench.plan_kernel_name(
        "void dtg::(anonymous namespace)::gemm_mx_kernel<32, 64, 1, 2, 4, 4, 4>(dtg::MxArgs)"
    ) == "gemm_mx_kernel<32,64,1,2,4,4,4>"


def test_committed_traffic_names_resolve():
    """Every kernel of ours in the committed traffic files maps to a plan-style name."""
    for name in ("traffic.json", "traffic_mx.json"):
        kernels = json.load(open(os.path.join(ROOT, "profiles", name)))["kernels"]
        ours = [bench.plan_kernel_name(k) for k in kernels if "dtg::" in k]
        assert ours and all(n.startswith("gemm_") and n.endswith(">") for n in ours)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0 and "one GPU" in (r.stdout + r.stderr)
