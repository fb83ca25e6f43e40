"""Build the HIP library libgemm.so (gfx950) in-tree.

    python -m dense_tiled_gemm_02_amd.build [-j N]

Each HIP/C++ source is compiled with hipcc for gfx950 into an object under
_build/, then linked into dense_tiled_gemm_02_amd/libgemm.so.  Packed fp32
vector instructions are disabled for device code.  The compiler's resource
report of every kernel (VGPRs, AGPRs, scratch, spills, LDS, occupancy: its
kernel-resource-usage remarks) is written to _build/kernel_resources.json with
a digest of the sources, for the test that gates the compiled variant table
(tests/test_resources.py).  With DTG_ASM=1 (or -s) the gfx950 assembly of
every kernel source is also written to _build/*.s.
"""
import concurrent.futures as cf
import hashlib
import json
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgemm.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "api_mx.cpp", "gemm_tile.hip", "gemm_dma.hip", "gemm_dma_more.hip", "gemm_dma_layouts.hip", "gemm_dma_sk.hip",
           "gemm_mx.hip", "gemm_mx_pairs.hip",
           "gemm_skinny.hip", "gemm_static.hip", "gemm_i8.hip",
           "gemm_mx_direct.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + CSRC, "-I" + os.path.join(ROOT, "include"), "-Wall"]


REMARK = "-Rpass-analysis=kernel-resource-usage"
RESOURCES = os.path.join(BUILD, "kernel_resources.json")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [l for l in r.stdout.splitlines()
             if "packed-fp32-ops' is not a recognized feature" not in l
             and "argument unused during compilation: '--hip-link'" not in l]
    out = "\n".join(l for l in lines if REMARK not in l and not l.lstrip().startswith(("|", "^")) and
                    not re.match(r"^\s*\d+ \|", l))
    if r.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), out))
    if out.strip() and verbose:
        print(out, flush=True)
    return lines


def parse_resource_remarks(lines):
    """{kernel symbol: {field: value}} from the compiler's kernel-resource-usage
    remarks ("Function Name: ..." followed by "VGPRs: n", "AGPRs: n",
    "ScratchSize [bytes/lane]: n", "Occupancy [waves/SIMD]: n", ...)."""
    kernels, cur = {}, None
    for l in lines:
        if REMARK not in l:
            continue
        m = re.search(r"remark: Function Name: (\S+)", l)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\S+) \[", l)
        if m and cur is not None:
            v = m.group(2)
            cur[m.group(1)] = int(v) if v.lstrip("-").isdigit() else v
    return kernels


def _compile(src, verbose, asm=False):
    """Object file of one source; for HIP sources also the compiler's resource
    report of every kernel in it."""
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    lang = ["-x", "hip", REMARK] if src.endswith(".hip") else []
    lines = _run([HIPCC] + COMMON + lang + ["-c", path, "-o", obj], verbose)
    if asm and src.endswith(".hip"):
        asm = os.path.join(BUILD, src + ".s")
        _run([HIPCC] + COMMON + ["-x", "hip", "--cuda-device-only", "-S", path, "-o", asm], verbose)
    return obj, parse_resource_remarks(lines)


def source_digest():
    """sha256 over every source the library is built from."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)) + ["../../include/gemm.h", "../../include/gemm_mx.h"]:
        fp = os.path.normpath(os.path.join(CSRC, f))
        if os.path.isfile(fp) and fp.endswith((".hip", ".h", ".cpp")):
            h.update(os.path.basename(fp).encode())
            h.update(open(fp, "rb").read())
    return h.hexdigest()


def _link(objs, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    # -z defs: a symbol left undefined (e.g. a kernel stub the host pass did
    # not emit) fails the build instead of the first load of the library
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-Wl,-z,defs", "-o", tmp] + objs, verbose)
    os.replace(tmp, out)


def build(verbose=False, jobs=None, asm=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    if asm is None:
        asm = os.environ.get("DTG_ASM", "0") not in ("", "0")
    # the largest sources first, so they start at once
    srcs = sorted(SOURCES, key=lambda f: -os.path.getsize(os.path.join(CSRC, f)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        done = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose, asm), srcs)))
    _link([done[s][0] for s in SOURCES], LIB, verbose)
    report = {"sources_sha256": source_digest(), "arch": ARCH,
              "kernels": {k: v for s in SOURCES for k, v in done[s][1].items()}}
    with open(RESOURCES + ".tmp", "w") as f:
        json.dump(report, f, indent=1, sort_keys=True)
    os.replace(RESOURCES + ".tmp", RESOURCES)
    return LIB


if __name__ == "__main__":
    j = None
    if "-j" in sys.argv:
        j = int(sys.argv[sys.argv.index("-j") + 1])
    print(build(verbose="-v" in sys.argv, jobs=j, asm=True if "-s" in sys.argv else None))
