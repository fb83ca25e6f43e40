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
                      "Tuning Triton kernels", section 1)
  skinny_bf16_16x8192 bf16 M=16, N=K=8192, N(0,1)*0.02  (decode-like shape,
                      "Tuning Triton kernels", section 4 regime split)
  tail_f16_4000x3000x1000_c  fp16 4000x3000x1000 plus addend C, U[-1,1]

Block-scaled (MX) workloads draw element codes and E8M0 scale codes directly
(MX_WORKLOADS, draw_mx): 8-bit elements are N(0,1)*8 rounded to the format by
torch's float8 conversion; E2M1 codes are drawn with a fixed probability per
magnitude code (a bell shape, peak at the middle codes) and a fair sign; each
32-k block gets a scale code of base + U{-2..2} (base 124 for 8-bit
elements, 126 for E2M1).  Scale rows are padded to a multiple of 4 bytes with
0xFF (the NaN code), which the library must never use.  Nothing here decodes
a code: both sides take the same stored bytes.

Integer workloads (I8_WORKLOADS, draw_i8): int8 codes uniform over [-128, 127],
A row-major M x K and B stored N x K, int32 addends uniform over
[-2^20, 2^20].  The pages measure no integer GEMM; the shapes are the 4096^3
and ragged tail shapes of the 16-bit workloads.
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


# ---------------------------------------------------------------- block-scaled (MX)

MX_ELEMENT_BITS = {"e4m3": 8, "e5m2": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4}
MX_SCALE_BASE = {"e2m3": 125, "e3m2": 124, "e4m3": 124, "e5m2": 124, "e2m1": 126}
_E2M1_MAG_P = np.array([0.08, 0.14, 0.17, 0.17, 0.15, 0.13, 0.10, 0.06])   # magnitude codes 0..7


class MxWorkload:
    def __init__(self, name, M, N, K, fmt_a, fmt_b, out, seeds, has_c=False):
        self.name = name
        self.M, self.N, self.K = M, N, K
        self.fmt_a, self.fmt_b = fmt_a, fmt_b
        self.out = out            # "bf16", "f16" or "f32"
        self.seeds = seeds        # (A, B, C)
        self.has_c = has_c

    def flops(self):
        return 2.0 * self.M * self.N * self.K

    def bytes(self):
        nb = (self.K + 31) // 32
        osz = 4 if self.out == "f32" else 2
        n = (self.M * self.K * MX_ELEMENT_BITS[self.fmt_a] + self.N * self.K * MX_ELEMENT_BITS[self.fmt_b]) / 8.0
        n += (self.M + self.N) * nb + self.M * self.N * osz * (2 if self.has_c else 1)
        return n

    def describe(self):
        return {"workload": self.name, "M": self.M, "N": self.N, "K": self.K,
                "elements": "%s x %s" % (self.fmt_a, self.fmt_b), "scales": "E8M0 per 32 k",
                "out": self.out, "layout": "A M x K, B stored N x K (k contiguous), D M x N row-major",
                "has_c": self.has_c, "seeds": list(self.seeds[: 3 if self.has_c else 2])}


MX_WORKLOADS = {
    w.name: w for w in [
        # the pages' microscaled GEMM is FP4 x FP4 ("afp4wfp4"); 4096^3 as the square bf16 case
        MxWorkload("mx_e2m1_4096", 4096, 4096, 4096, "e2m1", "e2m1", "bf16", (801, 802, 803)),
        MxWorkload("mx_e4m3_4096", 4096, 4096, 4096, "e4m3", "e4m3", "bf16", (811, 812, 813)),
        # the decode shape at which the pages split K for the FP4 kernel (M = 16)
        MxWorkload("mx_e2m1_16x8192x8192", 16, 8192, 8192, "e2m1", "e2m1", "bf16", (821, 822, 823)),
        # FP6 elements, and an FP8 x FP4 pair of different widths (register-direct kernel)
        MxWorkload("mx_e2m3_4096", 4096, 4096, 4096, "e2m3", "e2m3", "bf16", (831, 832, 833)),
        MxWorkload("mx_e4m3xe2m1_4096", 4096, 4096, 4096, "e4m3", "e2m1", "bf16", (841, 842, 843)),
    ]
}


def draw_mx(rows, K, fmt, seed):
    """(codes, scales) numpy uint8 arrays for `rows` rows of K elements: codes
    rows of K bytes (8-bit formats), 3K/4 bytes (FP6, packed by pack_fp6;
    codes uniform over the 64 values) or K/2 bytes (E2M1, even k in the low
    nibble); scales rows of ceil(K/32) codes padded with 0xFF to a multiple of 4."""
    rng = np.random.default_rng(seed)
    if fmt in ("e4m3", "e5m2"):
        x = torch.from_numpy(rng.standard_normal((rows, K)).astype(np.float32) * 8.0)
        dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
        codes = x.to(dt).view(torch.uint8).numpy()
    elif fmt == "e2m1":
        if K % 2:
            raise ValueError("E2M1 rows need an even K")
        mag = rng.choice(8, size=(rows, K), p=_E2M1_MAG_P).astype(np.uint8)
        nib = mag | (rng.integers(0, 2, (rows, K)).astype(np.uint8) << 3)
        codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    elif fmt in ("e2m3", "e3m2"):
        codes = pack_fp6(rng.integers(0, 64, (rows, K)).astype(np.uint8))
    else:
        raise ValueError("unknown MX element format %r" % (fmt,))
    nb = (K + 31) // 32
    ld = -(-nb // 4) * 4
    scales = np.full((rows, ld), 0xFF, dtype=np.uint8)
    scales[:, :nb] = (MX_SCALE_BASE[fmt] + rng.integers(-2, 3, (rows, nb))).astype(np.uint8)
    return np.ascontiguousarray(codes), scales


def pack_fp6(codes):
    """Rows of 6-bit codes (numpy uint8, K a multiple of 4) packed four per
    three bytes: each row is one little-endian bit string, code k in bits
    6k .. 6k + 5."""
    c = np.asarray(codes, dtype=np.uint32)
    rows, K = c.shape
    if K % 4:
        raise ValueError("FP6 rows need K a multiple of 4")
    q = c.reshape(rows, K // 4, 4)
    v = q[:, :, 0] | (q[:, :, 1] << 6) | (q[:, :, 2] << 12) | (q[:, :, 3] << 18)
    out = np.stack([v & 0xFF, (v >> 8) & 0xFF, (v >> 16) & 0xFF], axis=2).astype(np.uint8)
    return np.ascontiguousarray(out.reshape(rows, 3 * K // 4))


def make_mx(workload):
    """(A, SA, B, SB, C) numpy arrays for an MxWorkload (C: float64 values
    already in the output type, or None)."""
    w = MX_WORKLOADS[workload] if isinstance(workload, str) else workload
    A, SA = draw_mx(w.M, w.K, w.fmt_a, w.seeds[0])
    B, SB = draw_mx(w.N, w.K, w.fmt_b, w.seeds[1])
    C = None
    if w.has_c:
        dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.out]
        C = draw((w.M, w.N), w.seeds[2], "f16", "uniform").to(dt)
    return A, SA, B, SB, C


# ---------------------------------------------------------------- 8-bit integers

class I8Workload:
    """int8 A (M x K, row-major) and B stored N x K (k contiguous), int32 C and
    D; entries uniform over the full int8 range [-128, 127] (C, where present,
    uniform over [-2^20, 2^20])."""

    def __init__(self, name, M, N, K, seeds, has_c=False):
        self.name = name
        self.M, self.N, self.K = M, N, K
        self.seeds = seeds
        self.has_c = has_c

    def flops(self):          # integer operations, counted like flops: 2 per multiply-add
        return 2.0 * self.M * self.N * self.K

    def bytes(self):
        return float(self.M * self.K + self.N * self.K + 4 * self.M * self.N * (2 if self.has_c else 1))

    def describe(self):
        return {"workload": self.name, "M": self.M, "N": self.N, "K": self.K, "dtype": "int8 -> int32",
                "layout": "row-major A (MxK), B stored NxK (k contiguous), int32 D (MxN)", "has_c": self.has_c,
                "values": "uniform integers in [-128, 127]", "seeds": list(self.seeds[: 3 if self.has_c else 2])}


I8_WORKLOADS = {
    w.name: w for w in [
        I8Workload("square_i8_4096", 4096, 4096, 4096, (901, 902, 903)),
        I8Workload("tail_i8_4000x3000x1008_c", 4000, 3000, 1008, (911, 912, 913), has_c=True),
    ]
}


def draw_i8(shape, seed):
    """A numpy int8 array of uniform codes in [-128, 127]."""
    return np.random.default_rng(seed).integers(-128, 128, shape).astype(np.int8)


def draw_i32(shape, seed, bound=1 << 20):
    """A numpy int32 array of uniform integers in [-bound, bound]."""
    return np.random.default_rng(seed).integers(-bound, bound + 1, shape).astype(np.int32)


def make_i8(workload):
    """(A, Bt, C) numpy arrays of an I8Workload: A M x K, Bt N x K (B's
    columns as rows), C int32 M x N or None."""
    w = I8_WORKLOADS[workload] if isinstance(workload, str) else workload
    A = draw_i8((w.M, w.K), w.seeds[0])
    Bt = draw_i8((w.N, w.K), w.seeds[1])
    C = draw_i32((w.M, w.N), w.seeds[2]) if w.has_c else None
    return A, Bt, C
