"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random matrices and rounds them to fp16/bf16; it holds none
of the matrix-product arithmetic, so both the HIP path and the CPU oracle can
take their inputs from it without sharing any computation.

Values are drawn in float64 with numpy's PCG64 generator (default_rng(seed)),
then rounded to the storage type with torch on the CPU.  Both sides read the
same stored bits, so the rounding route does not affect any comparison.

Workloads (all row-major: A is M x K, B is K x N, C and D are M x N; the
distributions apply to every operand):
  square_f16_256      fp16 256^3, U[-1,1]
  square_f16_1024     fp16 1024^3, U[-1,1]  (the tile-size sweep shape of
                      "Hopper Support in Triton", slide 6: M=N=K=1024)
  square_bf16_4096    bf16 4096^3, N(0,1)/sqrt(K)  (the 4096^3 bf16 shape of
                      "Tuning Triton", section 1)
  skinny_bf16_16x8192 bf16 M=16, N=K=8192, N(0,1)*0.02  (decode-like shape,
                      "Tuning Triton", section 4 regime split)
  tail_f16_4000x3000x1000_c  fp16 4000x3000x1000 plus addend C, U[-1,1]
"""
import numpy as np
import torch

TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


class Workload:
    def __init__(self, name, M, N, K, dtype, dist, scale, seeds, has_c=False):
        self.name = name
        self.M, self.N, self.K = M, N, K
        self.dtype = dtype
        self.dist = dist          # "uniform" (U[-1,1]) or "normal" (N(0,1) * scale)
        self.scale = scale
        self.seeds = seeds        # (seed_A, seed_B, seed_C)
        self.has_c = has_c

    def flops(self):
        return 2.0 * self.M * self.N * self.K

    def bytes(self):
        n = self.M * self.K + self.K * self.N + self.M * self.N
        if self.has_c:
            n += self.M * self.N
        return 2.0 * n

    def describe(self):
        d = {"workload": self.name, "M": self.M, "N": self.N, "K": self.K,
             "dtype": self.dtype, "layout": "row-major A (MxK), B (KxN), D (MxN)",
             "has_c": self.has_c}
        if self.dist == "uniform":
            d["values"] = "U[-1,1] rounded to %s" % self.dtype
        else:
            d["values"] = "N(0,1)*%.6g rounded to %s" % (self.scale, self.dtype)
        d["seeds"] = list(self.seeds[: 3 if self.has_c else 2])
        return d


WORKLOADS = {
    w.name: w for w in [
        Workload("square_f16_256", 256, 256, 256, "f16", "uniform", 1.0, (101, 102, 103)),
        Workload("square_f16_1024", 1024, 1024, 1024, "f16", "uniform", 1.0, (201, 202, 203)),
        Workload("square_bf16_4096", 4096, 4096, 4096, "bf16", "normal", 1.0 / 64.0,
                 (301, 302, 303)),
        Workload("skinny_bf16_16x8192", 16, 8192, 8192, "bf16", "normal", 0.02,
                 (401, 402, 403)),
        Workload("tail_f16_4000x3000x1000_c", 4000, 3000, 1000, "f16", "uniform", 1.0,
                 (501, 502, 503), has_c=True),
        # decode: one row, the pages' M = 1, N = K = 4096 case
        Workload("decode_bf16_1x4096x4096", 1, 4096, 4096, "bf16", "normal", 1.0 / 64.0, (701, 702, 703)),
        # few output tiles, deep K: the K-split regime (entries N(0,1)/sqrt(K))
        Workload("deepk_bf16_512x512x32768", 512, 512, 32768, "bf16", "normal", 1.0 / 181.0193359837562,
                 (601, 602, 603)),
    ]
}


def draw(shape, seed, dtype, dist="uniform", scale=1.0):
    """A CPU torch tensor of the given storage dtype ('f16'/'bf16')."""
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "normal":
        x = rng.standard_normal(size=shape) * scale
    elif dist == "int":
        lo, hi = scale
        x = rng.integers(lo, hi + 1, size=shape).astype(np.float64)
    else:
        raise ValueError("unknown distribution %r" % (dist,))
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DTYPES[dtype])


def make(workload, with_c=None):
    """(A, B, C) CPU tensors for a Workload (C is None unless the workload has one)."""
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    has_c = w.has_c if with_c is None else with_c
    A = draw((w.M, w.K), w.seeds[0], w.dtype, w.dist, w.scale)
    B = draw((w.K, w.N), w.seeds[1], w.dtype, w.dist, w.scale)
    C = draw((w.M, w.N), w.seeds[2], w.dtype, w.dist, w.scale) if has_c else None
    return A, B, C


def bits(t):
    """Raw 16-bit patterns of a CPU fp16/bf16 tensor, as a numpy uint16 array."""
    if t is None:
        return None
    t = t.detach()
    if t.device.type != "cpu":
        t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16)


def from_bits(b, dtype):
    """CPU torch tensor of dtype 'f16'/'bf16' holding the given uint16 bit patterns."""
    arr = np.ascontiguousarray(b, dtype=np.uint16)
    return torch.from_numpy(arr.view(np.int16).copy()).view(TORCH_DTYPES[dtype])
