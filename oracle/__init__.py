"""CPU oracle for D = A x B (+ C) on fp16/bf16 inputs.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library and does not import it.

The arithmetic lives in oracle.c (plain C, binary64).  This module only
marshals numpy arrays into it:

  gemm_f64(A, B, C, dtype)         -> (ref, S)  full M x N reference and
                                      S = sum_k |a_ik b_kj|
  gemm_f64_at(A, B, C, ii, jj, dt) -> (ref, S)  the same at chosen positions
  decode / encode_rne / ulp_out    exact fp16/bf16 <-> binary64 conversions
  tol_check(got, ref, S, dtype)    acceptance rule |g-ref| <= ulp_out(ref) + 2^-20 S
  grouped_order                    the grouped tile visiting order, enumerated
                                   plainly (FlagGems "Hygon optimization",
                                   section "Grouped scheduling")

Inputs are numpy uint16 arrays holding the raw fp16/bf16 bit patterns (any
element strides); dtype is "f16" or "bf16".

Block-scaled (MX) operands, arithmetic in oracle_mx.c:

  mx_decode(codes, fmt) / e8m0_decode(codes)  exact element and scale values
  mx_gemm_f64(A, SA, B, SB, K, fa, fb, C)     (ref, S) of the scaled product
  mx_gemm_f64_at(..., ii, jj)                 the same at chosen positions
  ulp_f32 / tol_check_f32                     acceptance rule for binary32 outputs
  mx_tol_check(got, out, ref, S, S8)          the MX acceptance rule (run term 2^-10 S8)

MX operands are numpy uint8 arrays of raw bytes, one row per output row
(A: M rows) or column (B: N rows, k along the row), with unit stride along
the row; fmt is "e4m3", "e5m2", "e2m3", "e3m2" (FP6: four elements per
three bytes, element k in bits 6k .. 6k + 5 of the row read as a
little-endian bit string) or "e2m1" (two elements per byte, even k in the low
nibble); scales are uint8 arrays of E8M0 exponents, one per 32 k.

Integer operands, arithmetic in oracle_i8.c:

  gemm_i8(A, B, C)                 -> (D, exact)  int8 A (M x K) and B (K x N),
                                      optional int32 C; exact int64 sums and D,
                                      their residues modulo 2^32 as int32
  wrap_i32(x)                      the residue of one int64 modulo 2^32

Every function here is pinned by tests/test_oracle.py, tests/test_oracle_i8.py
and tests/test_oracle_mx.py against exhaustive library conversions, exact
rational arithmetic, BLAS in float64 and closed forms (identity, permutation,
rank-1, integer-valued inputs, single scaled blocks).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_DT = {"f16": 0, "bf16": 1}
_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_decode_f16.restype = ctypes.c_double
    lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bf16.restype = ctypes.c_double
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_ulp_out.restype = ctypes.c_double
    lib.oracle_ulp_out.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.oracle_encode_rne.restype = ctypes.c_uint16
    lib.oracle_encode_rne.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.oracle_decode_array.restype = None
    lib.oracle_decode_array.argtypes = [_p, _p, _i64, ctypes.c_int]
    lib.oracle_encode_array.restype = None
    lib.oracle_encode_array.argtypes = [_p, _p, _i64, ctypes.c_int]
    lib.oracle_ulp_array.restype = ctypes.c_double
    lib.oracle_ulp_array.argtypes = [_p, _p, _i64, ctypes.c_int]
    lib.oracle_gemm_f64.restype = ctypes.c_int
    lib.oracle_gemm_f64.argtypes = [_i64, _i64, _i64, ctypes.c_int,
                                    _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _p]
    lib.oracle_gemm_f64_at.restype = ctypes.c_int
    lib.oracle_gemm_f64_at.argtypes = [_i64, ctypes.c_int,
                                       _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64,
                                       _i64, _p, _p, _p, _p]
    lib.oracle_tol_check.restype = _i64
    lib.oracle_tol_check.argtypes = [_i64, _p, _p, _p, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]
    for f in ("e4m3", "e5m2", "e2m3", "e3m2", "e2m1", "e8m0"):
        fn = getattr(lib, "oracle_decode_" + f)
        fn.restype = ctypes.c_double
        fn.argtypes = [ctypes.c_uint8]
    lib.oracle_fp6_code.restype = ctypes.c_uint8
    lib.oracle_fp6_code.argtypes = [_p, _i64]
    lib.oracle_mx_gemm_f64.restype = ctypes.c_int
    lib.oracle_mx_gemm_f64.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                       _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _p, _p, _p]
    lib.oracle_mx_gemm_f64_at.restype = ctypes.c_int
    lib.oracle_mx_gemm_f64_at.argtypes = [_i64, ctypes.c_int, ctypes.c_int,
                                          _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _i64,
                                          _i64, _p, _p, _p, _p, _p]
    lib.oracle_mx_tol_check.restype = _i64
    lib.oracle_mx_tol_check.argtypes = [_i64, _p, ctypes.c_int, _p, _p, _p, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(_i64)]
    lib.oracle_ulp_f32.restype = ctypes.c_double
    lib.oracle_ulp_f32.argtypes = [ctypes.c_double]
    lib.oracle_tol_check_f32.restype = _i64
    lib.oracle_tol_check_f32.argtypes = [_i64, _p, _p, _p, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(_i64)]
    lib.oracle_gemm_i8.restype = ctypes.c_int
    lib.oracle_gemm_i8.argtypes = [_i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _p]
    lib.oracle_wrap_i32.restype = ctypes.c_int32
    lib.oracle_wrap_i32.argtypes = [_i64]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _dt(dtype):
    try:
        return _DT[dtype]
    except KeyError:
        raise ValueError("dtype must be 'f16' or 'bf16', got %r" % (dtype,))


def _bits(x, name):
    if not isinstance(x, np.ndarray) or x.dtype != np.uint16:
        raise TypeError("%s must be a numpy uint16 array of raw fp16/bf16 bits" % name)
    if x.ndim != 2:
        raise ValueError("%s must be 2-D" % name)
    return x


def _estrides(x):
    """Element strides of a uint16 array (numpy reports bytes)."""
    return x.strides[0] // 2, x.strides[1] // 2


def num_threads() -> int:
    return _load().oracle_num_threads()


def decode(bits, dtype):
    """Exact binary64 value of each fp16/bf16 bit pattern."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_decode_array(b.ctypes.data, out.ctypes.data, b.size, _dt(dtype))
    return out


def encode_rne(x, dtype):
    """Bit patterns of x rounded to fp16/bf16, nearest with ties to even."""
    v = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_encode_array(v.ctypes.data, out.ctypes.data, v.size, _dt(dtype))
    return out


def ulp_out(x, dtype):
    """One ulp of the output format in the binade of |x| (subnormal quantum at least)."""
    v = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    _load().oracle_ulp_array(v.ctypes.data, out.ctypes.data, v.size, _dt(dtype))
    return out


def gemm_f64(A, B, C=None, dtype="f16"):
    """ref = A x B (+ C) and S = sum_k |a_ik b_kj|, in binary64, from exact inputs."""
    A = _bits(A, "A")
    B = _bits(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ: A is %dx%d, B is %dx%d" % (M, K, K2, N))
    sam, sak = _estrides(A)
    sbk, sbn = _estrides(B)
    if C is not None:
        C = _bits(C, "C")
        if C.shape != (M, N):
            raise ValueError("C must be %dx%d" % (M, N))
        scm, scn = _estrides(C)
        cptr = C.ctypes.data
    else:
        scm = scn = 0
        cptr = None
    ref = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_f64(M, N, K, _dt(dtype), A.ctypes.data, sam, sak,
                                 B.ctypes.data, sbk, sbn, cptr, scm, scn,
                                 ref.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_gemm_f64 failed (%d)" % rc)
    return ref, S


def gemm_f64_at(A, B, C, ii, jj, dtype="f16"):
    """ref and S at output positions (ii[t], jj[t])."""
    A = _bits(A, "A")
    B = _bits(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape or ii.ndim != 1:
        raise ValueError("ii and jj must be 1-D and of equal length")
    if ii.size and (ii.min() < 0 or ii.max() >= M or jj.min() < 0 or jj.max() >= N):
        raise IndexError("sample position outside the output")
    sam, sak = _estrides(A)
    sbk, sbn = _estrides(B)
    if C is not None:
        C = _bits(C, "C")
        scm, scn = _estrides(C)
        cptr = C.ctypes.data
    else:
        scm = scn = 0
        cptr = None
    ref = np.empty(ii.shape, dtype=np.float64)
    S = np.empty(ii.shape, dtype=np.float64)
    rc = _load().oracle_gemm_f64_at(K, _dt(dtype), A.ctypes.data, sam, sak,
                                    B.ctypes.data, sbk, sbn, cptr, scm, scn,
                                    ii.size, ii.ctypes.data, jj.ctypes.data,
                                    ref.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_gemm_f64_at failed (%d)" % rc)
    return ref, S


def tol_check(got, ref, S, dtype):
    """Apply the acceptance rule to computed output bits.

    Returns (n_fail, worst, first_bad): worst is max |g-ref|/(ulp_out(ref)+2^-20 S)
    (inf when some g is not finite); first_bad the flat index of the first
    failure or -1.
    """
    g = np.ascontiguousarray(got, dtype=np.uint16).ravel()
    r = np.ascontiguousarray(ref, dtype=np.float64).ravel()
    s = np.ascontiguousarray(S, dtype=np.float64).ravel()
    if not (g.size == r.size == s.size):
        raise ValueError("got, ref and S differ in size")
    worst = ctypes.c_double(0.0)
    first = ctypes.c_int64(-1)
    n = _load().oracle_tol_check(g.size, g.ctypes.data, r.ctypes.data, s.ctypes.data,
                                 _dt(dtype), ctypes.byref(worst), ctypes.byref(first))
    return int(n), float(worst.value), int(first.value)


def grouped_order(num_pid_m, num_pid_n, group_m):
    """Order in which a grouped launch visits the output tiles (FlagGems
    "Hygon optimization", section "Grouped scheduling: improve L2 data reuse").

    The M tiles are cut into bands of group_m consecutive tiles (the last band
    keeps only the tiles that remain).  Bands are visited one after another;
    inside a band the walk goes down the band's M tiles for one N tile, then
    moves to the next N tile, so consecutive programs share a K x N panel of B.
    Returns the list of (pid_m, pid_n); program id p computes entry p.
    """
    order = []
    for first in range(0, num_pid_m, group_m):
        band = range(first, min(first + group_m, num_pid_m))
        for n in range(num_pid_n):
            for m in band:
                order.append((m, n))
    return order


# ---------------------------------------------------------------------------
# Block-scaled (MX) operands

MX_FORMATS = {"e4m3": 0, "e5m2": 1, "e2m3": 2, "e3m2": 3, "e2m1": 4}
MX_ELEMENT_BITS = {"e4m3": 8, "e5m2": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4}


def _mxf(fmt):
    try:
        return MX_FORMATS[fmt]
    except KeyError:
        raise ValueError("MX element format must be one of %s, got %r" % (sorted(MX_FORMATS), fmt))


def fp6_codes(row, K):
    """The K element codes of one stored FP6 row (numpy uint8 bytes), as the
    oracle reads them (oracle_fp6_code: element k in bits 6k .. 6k + 5 of the
    row read as a little-endian bit string)."""
    row = np.ascontiguousarray(row, dtype=np.uint8)
    fn = _load().oracle_fp6_code
    return np.array([fn(row.ctypes.data, k) for k in range(K)], dtype=np.uint8)


def mx_decode(codes, fmt):
    """Exact binary64 value of each element code (for e2m1 the low 4 bits,
    for e2m3 / e3m2 the low 6)."""
    _mxf(fmt)
    fn = getattr(_load(), "oracle_decode_" + fmt)
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([fn(int(x)) for x in c.ravel()], dtype=np.float64).reshape(c.shape)


def e8m0_decode(codes):
    """Exact binary64 value of each E8M0 scale code (NaN for 255)."""
    fn = _load().oracle_decode_e8m0
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([fn(int(x)) for x in c.ravel()], dtype=np.float64).reshape(c.shape)


def _rows(x, name):
    if not isinstance(x, np.ndarray) or x.dtype != np.uint8 or x.ndim != 2:
        raise TypeError("%s must be a 2-D numpy uint8 array" % name)
    if x.size and x.shape[1] > 1 and x.strides[1] != 1:
        raise ValueError("%s must have unit stride along its rows" % name)
    return x


def _mx_args(A, SA, B, SB, K, fmt_a, fmt_b, C, M, N):
    A, SA, B, SB = _rows(A, "A"), _rows(SA, "SA"), _rows(B, "B"), _rows(SB, "SB")
    if A.shape[0] != M or SA.shape[0] != M or B.shape[0] != N or SB.shape[0] != N:
        raise ValueError("row counts of A/SA (M) and B/SB (N) disagree")
    nblk = (K + 31) // 32
    for x, f, nm in ((A, fmt_a, "A"), (B, fmt_b, "B")):
        if x.shape[1] * 8 < K * MX_ELEMENT_BITS[f]:
            raise ValueError("%s rows hold fewer than K elements" % nm)
    if SA.shape[1] < nblk or SB.shape[1] < nblk:
        raise ValueError("scale rows hold fewer than ceil(K/32) scales")
    if C is not None:
        C = np.asarray(C, dtype=np.float64)
        cs = (C.strides[0] // 8, C.strides[1] // 8)
        cptr = C.ctypes.data
    else:
        cs, cptr = (0, 0), None
    return A, SA, B, SB, C, cs, cptr


def mx_gemm_f64(A, SA, B, SB, K, fmt_a, fmt_b, C=None, runs=False):
    """ref = A x B (+ C) and S = sum_k |a_ik b_kj| on MX operands, binary64;
    with runs=True also S8 = sum over runs of 8 consecutive k of the largest
    |product| (the run term of the MX acceptance rule).

    A: M rows of element bytes, SA: M rows of scales; B: N rows (the columns
    of B, k along the row), SB: N rows; C: optional M x N binary64 addend."""
    M, N = A.shape[0], B.shape[0]
    A, SA, B, SB, C, cs, cptr = _mx_args(A, SA, B, SB, K, fmt_a, fmt_b, C, M, N)
    ref = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    S8 = np.empty((M, N), dtype=np.float64) if runs else None
    rc = _load().oracle_mx_gemm_f64(M, N, K, _mxf(fmt_a), _mxf(fmt_b),
                                    A.ctypes.data, A.strides[0], SA.ctypes.data, SA.strides[0],
                                    B.ctypes.data, B.strides[0], SB.ctypes.data, SB.strides[0],
                                    cptr, cs[0], cs[1], ref.ctypes.data, S.ctypes.data,
                                    S8.ctypes.data if runs else None)
    if rc != 0:
        raise RuntimeError("oracle_mx_gemm_f64 failed (%d)" % rc)
    return (ref, S, S8) if runs else (ref, S)


def mx_gemm_f64_at(A, SA, B, SB, K, fmt_a, fmt_b, C, ii, jj, runs=False):
    """ref and S (and S8 with runs=True) of the MX product at output positions (ii[t], jj[t])."""
    M, N = A.shape[0], B.shape[0]
    A, SA, B, SB, C, cs, cptr = _mx_args(A, SA, B, SB, K, fmt_a, fmt_b, C, M, N)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape or ii.ndim != 1:
        raise ValueError("ii and jj must be 1-D and of equal length")
    if ii.size and (ii.min() < 0 or ii.max() >= M or jj.min() < 0 or jj.max() >= N):
        raise IndexError("sample position outside the output")
    ref = np.empty(ii.shape, dtype=np.float64)
    S = np.empty(ii.shape, dtype=np.float64)
    S8 = np.empty(ii.shape, dtype=np.float64) if runs else None
    rc = _load().oracle_mx_gemm_f64_at(K, _mxf(fmt_a), _mxf(fmt_b),
                                       A.ctypes.data, A.strides[0], SA.ctypes.data, SA.strides[0],
                                       B.ctypes.data, B.strides[0], SB.ctypes.data, SB.strides[0],
                                       cptr, cs[0], cs[1], ii.size, ii.ctypes.data, jj.ctypes.data,
                                       ref.ctypes.data, S.ctypes.data, S8.ctypes.data if runs else None)
    if rc != 0:
        raise RuntimeError("oracle_mx_gemm_f64_at failed (%d)" % rc)
    return (ref, S, S8) if runs else (ref, S)


def ulp_f32(x):
    """One ulp of binary32 in the binade of |x| (2^-149 below 2^-126)."""
    fn = _load().oracle_ulp_f32
    v = np.asarray(x, dtype=np.float64)
    return np.array([fn(float(t)) for t in v.ravel()], dtype=np.float64).reshape(v.shape)


def tol_check_f32(got, ref, S):
    """Acceptance rule for binary32 outputs: (n_fail, worst, first_bad) as tol_check."""
    g = np.ascontiguousarray(got, dtype=np.float32).ravel()
    r = np.ascontiguousarray(ref, dtype=np.float64).ravel()
    s = np.ascontiguousarray(S, dtype=np.float64).ravel()
    if not (g.size == r.size == s.size):
        raise ValueError("got, ref and S differ in size")
    worst = ctypes.c_double(0.0)
    first = ctypes.c_int64(-1)
    n = _load().oracle_tol_check_f32(g.size, g.ctypes.data, r.ctypes.data, s.ctypes.data,
                                     ctypes.byref(worst), ctypes.byref(first))
    return int(n), float(worst.value), int(first.value)


_OUT_KIND = {"f16": 0, "bf16": 1, "f32": 2}


def mx_tol_check(got, out, ref, S, S8):
    """MX acceptance rule |g - ref| <= ulp_out(ref) + 2^-20 S + 2^-10 S8 for
    outputs of type out ("f16", "bf16": raw uint16 bits; "f32": float32
    values).  S8=None drops the run term.  Returns (n_fail, worst, first_bad)."""
    kind = _OUT_KIND[out]
    g = np.ascontiguousarray(got, dtype=np.float32 if kind == 2 else np.uint16).ravel()
    r = np.ascontiguousarray(ref, dtype=np.float64).ravel()
    s = np.ascontiguousarray(S, dtype=np.float64).ravel()
    s8 = None if S8 is None else np.ascontiguousarray(S8, dtype=np.float64).ravel()
    if not (g.size == r.size == s.size) or (s8 is not None and s8.size != r.size):
        raise ValueError("got, ref, S and S8 differ in size")
    worst = ctypes.c_double(0.0)
    first = ctypes.c_int64(-1)
    n = _load().oracle_mx_tol_check(g.size, g.ctypes.data, kind, r.ctypes.data, s.ctypes.data,
                                    s8.ctypes.data if s8 is not None else None,
                                    ctypes.byref(worst), ctypes.byref(first))
    return int(n), float(worst.value), int(first.value)


# ---------------------------------------------------------------- integer operands


def _i8(x, name):
    x = np.asarray(x)
    if x.dtype != np.int8 or x.ndim != 2:
        raise TypeError("%s must be a 2-D int8 array" % name)
    return x


def gemm_i8(A, B, C=None):
    """(D, exact) of D = A x B (+ C): A int8 M x K, B int8 K x N (any element
    strides: a B stored N x K is passed as its transposed view), C int32 M x N
    or None.  exact: int64 sums (+ c); D: their residues modulo 2^32 as int32
    (oracle_i8.c)."""
    A, B = _i8(A, "A"), _i8(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if C is not None:
        C = np.asarray(C)
        if C.dtype != np.int32 or C.shape != (M, N):
            raise TypeError("C must be an int32 M x N array")
    exact = np.zeros((M, N), np.int64)
    D = np.zeros((M, N), np.int32)
    sa, sb = A.strides, B.strides
    sc = C.strides if C is not None else (0, 0)
    rc = _load().oracle_gemm_i8(M, N, K, A.ctypes.data, sa[0], sa[1], B.ctypes.data, sb[0], sb[1],
                                C.ctypes.data if C is not None else None, sc[0] // 4, sc[1] // 4,
                                exact.ctypes.data, D.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_gemm_i8 failed (%d)" % rc)
    return D, exact


def wrap_i32(x):
    """x (a Python or numpy integer) modulo 2^32 as a two's-complement int32."""
    return int(_load().oracle_wrap_i32(int(x)))
