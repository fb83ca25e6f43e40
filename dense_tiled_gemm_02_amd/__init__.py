"""Python binding of libgemm.so, the gfx950 tiled GEMM  D = A x B (+ C).

Argument marshalling only: every step of the product runs in the HIP kernels
of libgemm.so (see include/gemm.h for the contract).  The functions named
gemm_* mirror the C entry points one to one; `matmul` is a convenience that
takes torch tensors, which are used here only as device memory and streams.

There is no fallback: if libgemm.so is missing or cannot be loaded, every call
raises.  Build it with  python -m dense_tiled_gemm_02_amd.build.
"""
import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemm.so")

GEMM_F16 = 0
GEMM_BF16 = 1
GEMM_I8 = 2     # int8 A and B (k contiguous), int32 C and D
GEMM_OK = 0
GEMM_ERR_INVALID_ARG = 1
GEMM_ERR_UNSUPPORTED = 2
GEMM_ERR_HIP = 3
GEMM_ERR_WORKSPACE = 4
GEMM_XCD_ON = 1
GEMM_XCD_OFF = 2
GEMM_STATIC_SCRATCH_BYTES = 24 << 20   # include/gemm.h: the workspace gemm_run_static provides
KERNEL_TILE = 1
KERNEL_SKINNY = 2
KERNEL_DMA = 3
KERNEL_DMA_SK = 6   # stream-K: config.splitk is the workgroup count

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_p = ctypes.c_void_p


class gemm_problem(ctypes.Structure):
    _fields_ = [("M", _i64), ("N", _i64), ("K", _i64),
                ("sa_m", _i64), ("sa_k", _i64), ("sb_k", _i64), ("sb_n", _i64),
                ("sc_m", _i64), ("sc_n", _i64), ("sd_m", _i64), ("sd_n", _i64),
                ("dtype", ctypes.c_int), ("has_c", _i32)]


class gemm_config(ctypes.Structure):
    _fields_ = [("bm", _i32), ("bn", _i32), ("bk", _i32), ("stages", _i32), ("mfma", _i32),
                ("waves_m", _i32), ("waves_n", _i32), ("group_m", _i32), ("splitk", _i32),
                ("xcd_remap", _i32), ("kernel", _i32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class gemm_device_info(ctypes.Structure):
    _fields_ = [("arch", _i32), ("cu_count", _i32), ("xcd_count", _i32), ("clock_khz", _i32),
                ("lds_per_cu", _i64), ("lds_per_wg", _i64), ("wave_size", _i32)]


class GemmError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        self.detail = detail
        super().__init__("%s: %s" % (_status_name(status), detail))


_lib = None
_lib_lock = threading.Lock()

# (name, restype, argtypes) of every entry point declared in include/gemm.h
SIGNATURES = [
    ("gemm_device_query", ctypes.c_int, [ctypes.c_int, ctypes.POINTER(gemm_device_info)]),
    ("gemm_plan_create", ctypes.c_int,
     [ctypes.POINTER(gemm_problem), ctypes.c_int, ctypes.POINTER(gemm_config), ctypes.POINTER(_p)]),
    ("gemm_plan_create_for", ctypes.c_int,
     [ctypes.POINTER(gemm_problem), ctypes.POINTER(gemm_device_info), ctypes.POINTER(gemm_config),
      ctypes.POINTER(_p)]),
    ("gemm_plan_destroy", None, [_p]),
    ("gemm_plan_config", ctypes.c_int, [_p, ctypes.POINTER(gemm_config)]),
    ("gemm_plan_launch", ctypes.c_int, [_p, ctypes.POINTER(_i64), ctypes.POINTER(_i32), ctypes.POINTER(_i64)]),
    ("gemm_plan_describe", ctypes.c_int, [_p, ctypes.c_char_p, ctypes.c_size_t]),
    ("gemm_workspace_size", ctypes.c_int, [_p, ctypes.POINTER(ctypes.c_size_t)]),
    ("gemm_workspace_init", ctypes.c_int, [_p, _p, ctypes.c_size_t, _p]),
    ("gemm_run", ctypes.c_int, [_p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]),
    ("gemm_run_static", ctypes.c_int, [_p, _p, _p, _p, _p, _p]),
    ("gemm", ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, ctypes.POINTER(_i64), ctypes.c_int, _i32, _p]),
    ("gemm_cache_clear", None, []),
    ("gemm_lds_bytes", _i64, [_i32, _i32, _i32, _i32, ctypes.c_int]),
    ("gemm_tile_of_workgroup", ctypes.c_int,
     [_i64, _i64, _i64, _i32, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    ("gemm_streamk_pieces", ctypes.c_int,
     [_i32, _i32, _i32, _i32, ctypes.POINTER(_i32), _i32, ctypes.POINTER(_i32)]),
    ("gemm_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("gemm_last_error", ctypes.c_char_p, []),
]


def lib():
    """The loaded libgemm.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libgemm.so is not built (%s); run "
                                   "'python -m dense_tiled_gemm_02_amd.build'" % LIB_PATH)
            # torch's HIP runtime first: libgemm then binds to that same
            # runtime (it provides libgemm's libamdhip64.so.7), so torch's
            # streams and device pointers are valid in libgemm.  Loaded the
            # other way round, torch loads a second runtime of its own, and
            # the one initialised second finds no device.
            import torch  # noqa: F401
            L = ctypes.CDLL(LIB_PATH)
            for name, res, args in SIGNATURES:
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def _status_name(s):
    try:
        return lib().gemm_status_string(s).decode()
    except Exception:
        return "status %d" % s


def _check(status):
    if status != GEMM_OK:
        raise GemmError(status, gemm_last_error())


def gemm_status_string(status):
    return lib().gemm_status_string(status).decode()


def gemm_last_error():
    return lib().gemm_last_error().decode()


def gemm_device_query(device=0):
    info = gemm_device_info()
    _check(lib().gemm_device_query(device, ctypes.byref(info)))
    return info


class Plan:
    """Owns one gemm_plan*; destroyed with the object."""

    def __init__(self, handle, problem):
        self.handle = handle
        self.problem = problem

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.gemm_plan_destroy(h)

    @property
    def config(self):
        return gemm_plan_config(self)

    def describe(self):
        return gemm_plan_describe(self)


def _force(force):
    if force is None:
        return None
    if isinstance(force, gemm_config):
        return ctypes.byref(force)
    c = gemm_config()
    for k, v in dict(force).items():
        setattr(c, k, int(v))
    return ctypes.byref(c)


def gemm_plan_create(problem, device=0, force=None):
    h = _p()
    _check(lib().gemm_plan_create(ctypes.byref(problem), device, _force(force), ctypes.byref(h)))
    return Plan(h, problem)


def gemm_plan_create_for(problem, info, force=None):
    h = _p()
    _check(lib().gemm_plan_create_for(ctypes.byref(problem), ctypes.byref(info), _force(force),
                                      ctypes.byref(h)))
    return Plan(h, problem)


def gemm_plan_destroy(plan):
    h, plan.handle = plan.handle, None
    if h:
        lib().gemm_plan_destroy(h)


def gemm_plan_config(plan):
    c = gemm_config()
    _check(lib().gemm_plan_config(plan.handle, ctypes.byref(c)))
    return c


def gemm_plan_launch(plan):
    g, t, l = _i64(), _i32(), _i64()
    _check(lib().gemm_plan_launch(plan.handle, ctypes.byref(g), ctypes.byref(t), ctypes.byref(l)))
    return g.value, t.value, l.value


def gemm_plan_describe(plan):
    buf = ctypes.create_string_buffer(1024)
    _check(lib().gemm_plan_describe(plan.handle, buf, len(buf)))
    return buf.value.decode()


def gemm_workspace_size(plan):
    n = ctypes.c_size_t()
    _check(lib().gemm_workspace_size(plan.handle, ctypes.byref(n)))
    return n.value


def gemm_workspace_init(plan, workspace, workspace_bytes, stream=None):
    _check(lib().gemm_workspace_init(plan.handle, workspace, workspace_bytes, stream))


def gemm_run(plan, A, B, C, D, workspace=None, workspace_bytes=0, stream=None):
    """A, B, C, D, workspace, stream: integer device addresses / hipStream_t (or None)."""
    _check(lib().gemm_run(plan.handle, A, B, C, D, workspace, workspace_bytes, stream))


def gemm(A, B, C, D, M, N, K, strides, dtype, has_c, stream=None):
    arr = (_i64 * 8)(*[int(s) for s in strides])
    _check(lib().gemm(A, B, C, D, M, N, K, arr, dtype, has_c, stream))


def gemm_cache_clear():
    lib().gemm_cache_clear()


def gemm_lds_bytes(bm, bn, bk, stages, dtype):
    return lib().gemm_lds_bytes(bm, bn, bk, stages, dtype)


def gemm_tile_of_workgroup(wg, num_pid_m, num_pid_n, group_m, xcd_count):
    pm, pn = _i64(), _i64()
    _check(lib().gemm_tile_of_workgroup(wg, num_pid_m, num_pid_n, group_m, xcd_count,
                                        ctypes.byref(pm), ctypes.byref(pn)))
    return pm.value, pn.value


def gemm_streamk_pieces(tiles, k_steps, workgroups, wg):
    """The pieces of stream-K range `wg`: (tile, kt0, kt1, part, nparts, slot) each."""
    n = _i32()
    _check(lib().gemm_streamk_pieces(tiles, k_steps, workgroups, wg, None, 0, ctypes.byref(n)))
    buf = (_i32 * (6 * max(n.value, 1)))()
    _check(lib().gemm_streamk_pieces(tiles, k_steps, workgroups, wg, buf, n.value, ctypes.byref(n)))
    return [tuple(buf[6 * i:6 * i + 6]) for i in range(n.value)]


# ---------------------------------------------------------------- torch convenience

def problem(M, N, K, dtype, has_c=False, lda=None, ldb=None, ldc=None, ldd=None, ta=False, tb=False):
    """A gemm_problem with row-major C, D and, unless ta / tb, row-major A, B.
    ta: A stored K x M (element (m, k) at m + k * lda); tb: B stored N x K
    (element (k, n) at k + n * ldb)."""
    p = gemm_problem()
    p.M, p.N, p.K = M, N, K
    if ta:
        p.sa_m, p.sa_k = 1, (M if lda is None else lda)
    else:
        p.sa_m, p.sa_k = (K if lda is None else lda), 1
    if tb:
        p.sb_k, p.sb_n = 1, (K if ldb is None else ldb)
    else:
        p.sb_k, p.sb_n = (N if ldb is None else ldb), 1
    p.sc_m, p.sc_n = ((N if ldc is None else ldc), 1) if has_c else (0, 0)
    p.sd_m, p.sd_n = (N if ldd is None else ldd), 1
    p.dtype = dtype
    p.has_c = 1 if has_c else 0
    return p


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return GEMM_F16
    if t.dtype == torch.bfloat16:
        return GEMM_BF16
    if t.dtype == torch.int8:
        return GEMM_I8
    raise TypeError("only float16, bfloat16 and int8 operands are supported, got %s" % t.dtype)


def out_dtype(t):
    """The dtype of C and D for operands of t's dtype (int32 for int8 operands)."""
    import torch
    return torch.int32 if t.dtype == torch.int8 else t.dtype


def problem_for(A, B, C=None, D=None):
    """gemm_problem for torch tensors A (MxK), B (KxN), optional C and D (MxN)."""
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ: %s x %s" % (tuple(A.shape), tuple(B.shape)))
    dt = _dtype_code(A)
    od = out_dtype(A)
    for name, t, want in (("B", B, A.dtype), ("C", C, od), ("D", D, od)):
        if t is not None and t.dtype != want:
            raise TypeError("%s has dtype %s, expected %s for %s operands" % (name, t.dtype, want, A.dtype))
    for name, t in (("C", C), ("D", D)):
        if t is not None and tuple(t.shape) != (M, N):
            raise ValueError("%s must be %dx%d" % (name, M, N))
    p = gemm_problem()
    p.M, p.N, p.K = M, N, K
    p.sa_m, p.sa_k = A.stride()
    p.sb_k, p.sb_n = B.stride()
    if C is not None:
        p.sc_m, p.sc_n = C.stride()
    p.sd_m, p.sd_n = D.stride() if D is not None else (N, 1)
    p.dtype = dt
    p.has_c = 1 if C is not None else 0
    return p


_plan_cache = {}
_plan_lock = threading.Lock()
_ws_cache = {}


def workspace_for(plan, device, stream):
    """A zero-filled workspace of at least the plan's size, one per (device,
    stream), grown on demand and reused (launches leave it ready for reuse).
    Returns (address, bytes) or (None, 0)."""
    import torch
    need = gemm_workspace_size(plan)
    if need == 0:
        return None, 0
    key = (device, stream)
    with _plan_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < need:
            # 256-byte aligned by the caching allocator; zero-filled on creation
            buf = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device="cuda:%d" % device)
            _ws_cache[key] = buf
    return buf.data_ptr(), buf.numel()


def plan_for(A, B, C=None, D=None, config=None):
    """Cached plan for these operand shapes, strides and dtype on A's device."""
    p = problem_for(A, B, C, D)
    dev = A.device.index if A.device.index is not None else 0
    key = (dev, tuple(getattr(p, f) for f, _ in gemm_problem._fields_),
           tuple(sorted(config.items())) if isinstance(config, dict) else None)
    with _plan_lock:
        pl = _plan_cache.get(key)
        if pl is None:
            pl = gemm_plan_create(p, dev, config)
            _plan_cache[key] = pl
    return pl


def matmul(A, B, C=None, out=None, config=None, stream=None):
    """D = A x B (+ C) on the GPU through libgemm.so; returns D (torch tensor).

    A, B, C, out: CUDA (HIP) torch tensors of one dtype (float16 / bfloat16),
    or int8 A and B with int32 C and out (B k-contiguous: the transposed view
    of an N x K tensor).
    config: optional dict of gemm_config fields to force.  The call is
    asynchronous on `stream` (default: torch's current stream)."""
    import torch
    for name, t in (("A", A), ("B", B), ("C", C), ("out", out)):
        if t is not None and not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
    if out is None:
        out = torch.empty((A.shape[0], B.shape[1]), dtype=out_dtype(A), device=A.device)
    pl = plan_for(A, B, C, out, config)
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    dev = A.device.index if A.device.index is not None else 0
    ws, ws_bytes = workspace_for(pl, dev, stream)
    gemm_run(pl, A.data_ptr(), B.data_ptr(), C.data_ptr() if C is not None else None,
             out.data_ptr(), ws, ws_bytes, stream)
    return out
