"""Python binding of the block-scaled (MX) entry points of libgemm.so.

Argument marshalling only, like the package's gemm_* functions: the product
runs in the HIP kernels (include/gemm_mx.h holds the contract).  Operands are
raw bytes: A (M rows) and B (N rows, the columns of B) with k along each row,
8-bit elements one per byte or E2M1 elements two per byte (even k in the low
nibble); SA / SB hold one E8M0 scale byte per 32 k of each row.
"""
import ctypes
import threading

from . import (GemmError, _check, _force, _i32, _i64, _p, gemm_config, gemm_device_info, gemm_last_error,
               lib)

GEMM_MX_E4M3 = 0
GEMM_MX_E5M2 = 1
GEMM_MX_E2M3 = 2
GEMM_MX_E3M2 = 3
GEMM_MX_E2M1 = 4
GEMM_MX_OUT_F16 = 0
GEMM_MX_OUT_BF16 = 1
GEMM_MX_OUT_F32 = 2
KERNEL_MX = 4           # the LDS-staged tile kernel (pairs of one width: 8-bit or E2M1)
KERNEL_MX_DIRECT = 5    # the register-direct kernel (every pair of formats)
FORMATS = {"e4m3": GEMM_MX_E4M3, "e5m2": GEMM_MX_E5M2, "e2m3": GEMM_MX_E2M3, "e3m2": GEMM_MX_E3M2,
           "e2m1": GEMM_MX_E2M1}
ELEMENT_BITS = {GEMM_MX_E4M3: 8, GEMM_MX_E5M2: 8, GEMM_MX_E2M3: 6, GEMM_MX_E3M2: 6, GEMM_MX_E2M1: 4}


class gemm_mx_problem(ctypes.Structure):
    _fields_ = [("M", _i64), ("N", _i64), ("K", _i64),
                ("lda", _i64), ("ldb", _i64), ("ldsa", _i64), ("ldsb", _i64), ("ldc", _i64), ("ldd", _i64),
                ("fmt_a", ctypes.c_int), ("fmt_b", ctypes.c_int), ("out", ctypes.c_int), ("has_c", _i32)]


# (name, restype, argtypes) of every entry point declared in include/gemm_mx.h
MX_SIGNATURES = [
    ("gemm_mx_plan_create", ctypes.c_int,
     [ctypes.POINTER(gemm_mx_problem), ctypes.c_int, ctypes.POINTER(gemm_config), ctypes.POINTER(_p)]),
    ("gemm_mx_plan_create_for", ctypes.c_int,
     [ctypes.POINTER(gemm_mx_problem), ctypes.POINTER(gemm_device_info), ctypes.POINTER(gemm_config),
      ctypes.POINTER(_p)]),
    ("gemm_mx_plan_destroy", None, [_p]),
    ("gemm_mx_plan_config", ctypes.c_int, [_p, ctypes.POINTER(gemm_config)]),
    ("gemm_mx_plan_launch", ctypes.c_int, [_p, ctypes.POINTER(_i64), ctypes.POINTER(_i32), ctypes.POINTER(_i64)]),
    ("gemm_mx_plan_describe", ctypes.c_int, [_p, ctypes.c_char_p, ctypes.c_size_t]),
    ("gemm_mx_workspace_size", ctypes.c_int, [_p, ctypes.POINTER(ctypes.c_size_t)]),
    ("gemm_mx_workspace_init", ctypes.c_int, [_p, _p, ctypes.c_size_t, _p]),
    ("gemm_mx_run", ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]),
]

_ready = False
_lock = threading.Lock()


def mxlib():
    """libgemm.so with the MX entry points typed (raises if it is not built)."""
    global _ready
    L = lib()
    if not _ready:
        with _lock:
            for name, res, args in MX_SIGNATURES:
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _ready = True
    return L


class MxPlan:
    """Owns one gemm_mx_plan*; destroyed with the object."""

    def __init__(self, handle, problem):
        self.handle = handle
        self.problem = problem

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _ready:
            lib().gemm_mx_plan_destroy(h)

    @property
    def config(self):
        return gemm_mx_plan_config(self)

    def describe(self):
        return gemm_mx_plan_describe(self)


def gemm_mx_plan_create(problem, device=0, force=None):
    h = _p()
    _check(mxlib().gemm_mx_plan_create(ctypes.byref(problem), device, _force(force), ctypes.byref(h)))
    return MxPlan(h, problem)


def gemm_mx_plan_create_for(problem, info, force=None):
    h = _p()
    _check(mxlib().gemm_mx_plan_create_for(ctypes.byref(problem), ctypes.byref(info), _force(force),
                                           ctypes.byref(h)))
    return MxPlan(h, problem)


def gemm_mx_plan_destroy(plan):
    h, plan.handle = plan.handle, None
    if h:
        mxlib().gemm_mx_plan_destroy(h)


def gemm_mx_plan_config(plan):
    c = gemm_config()
    _check(mxlib().gemm_mx_plan_config(plan.handle, ctypes.byref(c)))
    return c


def gemm_mx_plan_launch(plan):
    g, t, l = _i64(), _i32(), _i64()
    _check(mxlib().gemm_mx_plan_launch(plan.handle, ctypes.byref(g), ctypes.byref(t), ctypes.byref(l)))
    return g.value, t.value, l.value


def gemm_mx_plan_describe(plan):
    buf = ctypes.create_string_buffer(1024)
    _check(mxlib().gemm_mx_plan_describe(plan.handle, buf, len(buf)))
    return buf.value.decode()


def gemm_mx_workspace_size(plan):
    n = ctypes.c_size_t()
    _check(mxlib().gemm_mx_workspace_size(plan.handle, ctypes.byref(n)))
    return n.value


def gemm_mx_workspace_init(plan, workspace, workspace_bytes, stream=None):
    _check(mxlib().gemm_mx_workspace_init(plan.handle, workspace, workspace_bytes, stream))


def gemm_mx_run(plan, A, SA, B, SB, C, D, workspace=None, workspace_bytes=0, stream=None):
    """Device addresses (integers or None) and a hipStream_t (or None)."""
    _check(mxlib().gemm_mx_run(plan.handle, A, SA, B, SB, C, D, workspace, workspace_bytes, stream))


# ---------------------------------------------------------------- torch convenience

def mx_problem(M, N, K, fmt_a="e4m3", fmt_b=None, out=GEMM_MX_OUT_BF16, has_c=False, lda=None, ldb=None,
               ldsa=None, ldsb=None, ldc=None, ldd=None):
    """A gemm_mx_problem with packed rows by default: lda = ldb = bytes of K
    elements, ldsa = ldsb = ceil(K/32) rounded up to 4, ldc = ldd = N."""
    fa = FORMATS[fmt_a] if isinstance(fmt_a, str) else fmt_a
    fb = fa if fmt_b is None else (FORMATS[fmt_b] if isinstance(fmt_b, str) else fmt_b)
    kba, kbb = K * ELEMENT_BITS[fa] // 8, K * ELEMENT_BITS[fb] // 8
    ns = -(-((K + 31) // 32) // 4) * 4
    p = gemm_mx_problem()
    p.M, p.N, p.K = M, N, K
    p.lda = kba if lda is None else lda
    p.ldb = kbb if ldb is None else ldb
    p.ldsa = ns if ldsa is None else ldsa
    p.ldsb = ns if ldsb is None else ldsb
    p.ldc = (N if ldc is None else ldc) if has_c else 0
    p.ldd = N if ldd is None else ldd
    p.fmt_a, p.fmt_b, p.out = fa, fb, out
    p.has_c = 1 if has_c else 0
    return p


def _out_code(dtype):
    import torch
    m = {torch.float16: GEMM_MX_OUT_F16, torch.bfloat16: GEMM_MX_OUT_BF16, torch.float32: GEMM_MX_OUT_F32}
    if dtype not in m:
        raise TypeError("output dtype must be float16, bfloat16 or float32, got %s" % dtype)
    return m[dtype]


_plans = {}
_cache_lock = threading.Lock()   # guards _plans and _ws (callers on several threads)


def mx_matmul(A, SA, B, SB, K, fmt_a="e4m3", fmt_b=None, C=None, out=None, out_dtype=None, config=None,
              stream=None):
    """D = A x B (+ C) on MX operands through libgemm.so; returns D.

    A: uint8 tensor of M rows (k along the row), B: uint8 tensor of N rows
    (the columns of B), SA / SB: uint8 scale tensors of M / N rows; row
    strides are taken from the tensors (unit stride along a row).  C / out:
    M x N tensors of the output dtype (float16, bfloat16 or float32)."""
    import torch
    for name, t in (("A", A), ("SA", SA), ("B", B), ("SB", SB)):
        if t.dtype != torch.uint8 or t.dim() != 2 or not t.is_cuda:
            raise ValueError("%s must be a 2-D uint8 GPU tensor" % name)
        if t.shape[1] > 1 and t.stride(1) != 1:
            raise ValueError("%s must have unit stride along its rows" % name)
    M, N = A.shape[0], B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or (C.dtype if C is not None else torch.bfloat16),
                          device=A.device)
    code = _out_code(out.dtype)
    p = mx_problem(M, N, K, fmt_a, fmt_b, code, C is not None, lda=A.stride(0), ldb=B.stride(0),
                   ldsa=SA.stride(0), ldsb=SB.stride(0), ldc=C.stride(0) if C is not None else None,
                   ldd=out.stride(0))
    dev = A.device.index if A.device.index is not None else 0
    key = (dev, tuple(getattr(p, f) for f, _ in gemm_mx_problem._fields_),
           tuple(sorted(config.items())) if isinstance(config, dict) else None)
    with _cache_lock:
        pl = _plans.get(key)
        if pl is None:
            pl = _plans[key] = gemm_mx_plan_create(p, dev, config)
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    ws, ws_bytes = _workspace(pl, dev, stream)
    gemm_mx_run(pl, A.data_ptr(), SA.data_ptr(), B.data_ptr(), SB.data_ptr(),
                C.data_ptr() if C is not None else None, out.data_ptr(), ws, ws_bytes, stream)
    return out


_ws = {}


def _workspace(plan, device, stream):
    """A zero-filled workspace of at least the plan's size, one per (device,
    stream), grown on demand (launches leave it ready for reuse)."""
    import torch
    need = gemm_mx_workspace_size(plan)
    if need == 0:
        return None, 0
    with _cache_lock:
        buf = _ws.get((device, stream))
        if buf is None or buf.numel() < need:
            buf = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device="cuda:%d" % device)
            _ws[(device, stream)] = buf
    return buf.data_ptr(), buf.numel()


__all__ = ["GemmError", "gemm_last_error"] + [n for n, _, _ in MX_SIGNATURES]
