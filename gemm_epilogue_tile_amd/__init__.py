"""Python binding of ``libgemm_epi.so``, the fused GEMM + epilogue engine for MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/gemm_epi.h``.  PyTorch
provides device memory and the current stream; nothing here computes.

The binding raises ``GemmEpiError`` on a nonzero status and
``RuntimeError`` when the HIP library has not been built -- there is no
fallback path.
"""
from __future__ import annotations

import collections
import ctypes
import os
import threading

__all__ = [
    "GemmEpiError", "Desc", "Plan", "lib", "lib_path", "plan", "gemm_epilogue", "swiglu", "w4_gemm",
    "gemm_epilogue_unfused", "swiglu_unfused", "w4_gemm_unfused", "w4_dequant", "add_rmsnorm",
    "F32", "BF16", "U4X2", "ACTS", "Prepared", "prepare_gemm_epilogue", "prepare_swiglu", "prepare_w4_gemm",
    "w4_prepack", "b_prepack", "U8", "FP8E4M3", "WEIGHT_FORMATS", "rope_qk", "rope", "prepare_rope_qk",
    "prepare_rope", "gemm_epilogue_noalloc", "add_rmsnorm_unfused", "prepare_add_rmsnorm", "swiglu_prepack",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libgemm_epi.so")

# status codes, types, layouts, activations, kinds, flags (mirror gemm_epi.h)
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_NO_DEVICE, ERR_HIP, ERR_ALIGN = range(6)
F32, BF16, U4X2, U8, FP8E4M3 = 0, 1, 2, 3, 4
LAYOUT_KN, LAYOUT_NK = 0, 1
ROPE_INTERLEAVED, ROPE_EXACT = 1, 2
ACTS = {"none": 0, "relu": 1, "gelu_tanh": 2, "silu": 3}
KIND_GENERIC, KIND_SWIGLU, KIND_W4 = 0, 1, 2
FLAG_BIAS, FLAG_C, FLAG_RESIDUAL, FLAG_NIBBLE_LO_FIRST, FLAG_W4_PREPACKED, FLAG_B_PREPACKED = 1, 2, 4, 8, 16, 32
FLAG_NO_SCRATCH = 64

EXPORTS = [
    "ge_desc_init", "gemm_epi_plan", "gemm_epi_plan_destroy", "gemm_epi_plan_kernel", "gemm_epi_plan_scratch_bytes", "gemm_epi_run",
    "gemm_epi_run_noalloc",
    "gemm_swiglu_run", "gemm_w4_run", "gemm_epi_unfused_workspace_bytes", "gemm_epi_run_unfused",
    "gemm_swiglu_run_unfused", "gemm_w4_run_unfused", "gemm_w4_dequant_run", "gemm_w4_prepack", "gemm_b_prepack",
    "ge_add_rmsnorm_run", "ge_add_rmsnorm_run_unfused", "ge_rope_qk_run", "ge_rope_run",
    "ge_status_string", "ge_last_error", "ge_version",
]


class GemmEpiError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({_status_name(status)}): {detail}")


class Desc(ctypes.Structure):
    """Mirror of ``ge_desc``."""
    _fields_ = [
        ("M", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
        ("a_type", ctypes.c_int32), ("b_type", ctypes.c_int32),
        ("c_type", ctypes.c_int32), ("d_type", ctypes.c_int32),
        ("bias_type", ctypes.c_int32), ("r_type", ctypes.c_int32), ("scale_type", ctypes.c_int32),
        ("b_layout", ctypes.c_int32),
        ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64),
        ("ldd", ctypes.c_int64), ("ldr", ctypes.c_int64),
        ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
        ("act", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("group_size", ctypes.c_int32), ("zero_point", ctypes.c_int32),
    ]


_lib = None
_lib_lock = threading.Lock()


def lib():
    """Load the HIP library (raises if it was never built)."""
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(lib_path):
                raise RuntimeError(f"{lib_path} is missing: build it first "
                                   "(python -c 'import __graft_entry__ as g; g.build()')")
            L = ctypes.CDLL(lib_path)
            P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
            L.ge_desc_init.argtypes = [ctypes.POINTER(Desc)]
            L.ge_desc_init.restype = None
            L.gemm_epi_plan.argtypes = [ctypes.POINTER(Desc), I, ctypes.POINTER(P)]
            L.gemm_epi_plan.restype = I
            L.gemm_epi_plan_destroy.argtypes = [P]
            L.gemm_epi_plan_destroy.restype = I
            L.gemm_epi_plan_kernel.argtypes = [P]
            L.gemm_epi_plan_kernel.restype = ctypes.c_char_p
            L.gemm_epi_plan_scratch_bytes.argtypes = [P]
            L.gemm_epi_plan_scratch_bytes.restype = ctypes.c_size_t
            L.gemm_epi_run.argtypes = [P] * 8
            L.gemm_epi_run.restype = I
            L.gemm_epi_run_noalloc.argtypes = [P] * 8
            L.gemm_epi_run_noalloc.restype = I
            L.gemm_swiglu_run.argtypes = [P] * 6
            L.gemm_swiglu_run.restype = I
            L.gemm_w4_run.argtypes = [P] * 9
            L.gemm_w4_run.restype = I
            L.gemm_epi_unfused_workspace_bytes.argtypes = [P, ctypes.POINTER(S)]
            L.gemm_epi_unfused_workspace_bytes.restype = I
            L.gemm_epi_run_unfused.argtypes = [P] * 9
            L.gemm_epi_run_unfused.restype = I
            L.gemm_swiglu_run_unfused.argtypes = [P] * 7
            L.gemm_swiglu_run_unfused.restype = I
            L.gemm_w4_run_unfused.argtypes = [P] * 10
            L.gemm_w4_run_unfused.restype = I
            L.gemm_w4_dequant_run.argtypes = [P] * 5
            L.gemm_w4_dequant_run.restype = I
            L.gemm_w4_prepack.argtypes = [P] * 4
            L.gemm_w4_prepack.restype = I
            L.gemm_b_prepack.argtypes = [P] * 4
            L.gemm_b_prepack.restype = I
            L.ge_add_rmsnorm_run.argtypes = [I, I, P, P, P, ctypes.c_float, P, P, P]
            L.ge_add_rmsnorm_run.restype = I
            L.ge_add_rmsnorm_run_unfused.argtypes = [I, I, P, P, P, ctypes.c_float, P, P, P]
            L.ge_add_rmsnorm_run_unfused.restype = I
            L.ge_rope_qk_run.argtypes = [I, I, I, I, P, P, P, P, I, I, I, I, ctypes.c_float, I, P, P]
            L.ge_rope_qk_run.restype = I
            L.ge_rope_run.argtypes = [I, I, I, P, P, P, I, I, I, P, P]
            L.ge_rope_run.restype = I
            L.ge_status_string.argtypes = [I]
            L.ge_status_string.restype = ctypes.c_char_p
            L.ge_last_error.argtypes = []
            L.ge_last_error.restype = ctypes.c_char_p
            L.ge_version.argtypes = []
            L.ge_version.restype = ctypes.c_char_p
            _lib = L
    return _lib


def _status_name(s: int) -> str:
    try:
        return lib().ge_status_string(s).decode()
    except Exception:  # noqa: BLE001 - only used to format an error
        return str(s)


def _check(status: int, where: str):
    if status != OK:
        raise GemmEpiError(status, where, lib().ge_last_error().decode())


# --------------------------------------------------------------------------
# torch marshalling
# --------------------------------------------------------------------------

def _torch():
    import torch  # plumbing: device memory and streams
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.uint8:
        return U4X2
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ld(t) -> int:
    """Leading dimension (row stride in elements) of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


class Plan:
    """Owner of a ``ge_plan*``."""

    def __init__(self, desc: Desc, kind: int):
        self.desc = desc
        self.kind = kind
        h = ctypes.c_void_p()
        _check(lib().gemm_epi_plan(ctypes.byref(desc), kind, ctypes.byref(h)), "gemm_epi_plan")
        self.handle = h

    @property
    def kernel(self) -> str:
        return lib().gemm_epi_plan_kernel(self.handle).decode()

    @property
    def scratch_bytes(self) -> int:
        """Device scratch the plan owns (a plan with scratch runs on one stream at a time)."""
        return int(lib().gemm_epi_plan_scratch_bytes(self.handle))

    def workspace_bytes(self) -> int:
        n = ctypes.c_size_t()
        _check(lib().gemm_epi_unfused_workspace_bytes(self.handle, ctypes.byref(n)),
               "gemm_epi_unfused_workspace_bytes")
        return n.value

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _lib is not None:
            _lib.gemm_epi_plan_destroy(h)
            self.handle = None


class Prepared:
    """A run call with every argument already converted: ``call()`` only crosses
    the C ABI.  For timing loops and graph capture, where per-call Python work
    would otherwise dominate small kernels.  The tensors passed at preparation
    must stay alive (they are referenced here)."""

    def __init__(self, fn, where, plan_obj, tensors, args):
        self._fn = fn
        self._where = where
        self._plan = plan_obj
        self._tensors = tensors
        self._args = args

    def __call__(self):
        s = self._fn(*self._args)
        if s != OK:
            raise GemmEpiError(s, self._where, lib().ge_last_error().decode())

    def with_stream(self, stream=None) -> "Prepared":
        """The same call bound to another stream (default: the current one), e.g.
        the capture stream inside ``torch.cuda.graph``.  The runs allocate nothing
        and never synchronise, so they can be captured into a HIP graph.  The call
        keeps its plan: when that plan owns device scratch, the two bindings must
        not run at the same time (prepare the call again with ``stream=`` for that)."""
        return Prepared(self._fn, self._where, self._plan, self._tensors, self._args[:-1] + (_stream(stream),))


# Plans by descriptor (and device).  A plan that owns device scratch serves one stream at a time,
# so such plans are cached per stream as well; the cache keeps the most recently used plans only.
_plan_cache: "collections.OrderedDict" = collections.OrderedDict()
_PLAN_CACHE_MAX = 256
_cache_lock = threading.Lock()


def _stream_key(stream) -> int:
    if stream is None:
        return int(_torch().cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def plan(kind: int, M: int, N: int, K: int, *, a_type=BF16, b_type=None, d_type=BF16, c_type=None,
         bias_type=None, r_type=None, b_layout=LAYOUT_KN, lda=0, ldb=0, ldc=0, ldd=0, ldr=0,
         alpha=1.0, beta=0.0, act="none", bias=False, C=False, R=False, group=128, zero_point=8,
         lo_first=False, prepacked=False, b_prepacked=False, no_scratch=False, stream=None) -> Plan:
    """Build (or fetch from a cache) the plan of one problem descriptor on the current device.

    Calls with equal descriptors share one plan, except that a plan owning device scratch
    (``Plan.scratch_bytes > 0``: bf16 decode shapes whose K is split over workgroups, quantised weights
    with a K split: at M <= 16, or on the tile kernel when its tiles leave CUs idle; SwiGLU at M <= 32,
    whose gate and up blocks run on workgroup pairs) is made once per
    ``stream`` (default: the current stream), since it must not run on two streams at once.
    ``no_scratch``: a plan that allocates no device memory (for ``gemm_epilogue_noalloc``).  The cache
    holds the 256 most recently used plans."""
    d = Desc()
    lib().ge_desc_init(ctypes.byref(d))
    d.M, d.N, d.K = M, N, K
    d.a_type = a_type
    d.b_type = a_type if b_type is None else b_type
    d.d_type = d_type
    d.c_type = d_type if c_type is None else c_type
    d.bias_type = d_type if bias_type is None else bias_type
    d.r_type = d_type if r_type is None else r_type
    d.b_layout = b_layout
    d.lda, d.ldb, d.ldc, d.ldd, d.ldr = lda, ldb, ldc, ldd, ldr
    d.alpha, d.beta = alpha, beta
    d.act = ACTS[act] if isinstance(act, str) else int(act)
    d.flags = ((FLAG_BIAS if bias else 0) | (FLAG_C if C else 0) | (FLAG_RESIDUAL if R else 0)
               | (FLAG_NIBBLE_LO_FIRST if lo_first else 0) | (FLAG_W4_PREPACKED if prepacked else 0)
               | (FLAG_B_PREPACKED if b_prepacked else 0) | (FLAG_NO_SCRATCH if no_scratch else 0))
    d.group_size, d.zero_point = group, zero_point
    torch = _torch()
    base = (kind, bytes(d), torch.cuda.current_device() if torch.cuda.is_available() else -1)
    skey = base + (_stream_key(stream),) if torch.cuda.is_available() else base + (0,)
    with _cache_lock:
        for key in (base, skey):
            p = _plan_cache.get(key)
            if p is not None:
                _plan_cache.move_to_end(key)
                return p
    p = Plan(d, kind)
    with _cache_lock:
        _plan_cache[skey if p.scratch_bytes > 0 else base] = p
        while len(_plan_cache) > _PLAN_CACHE_MAX:
            _plan_cache.popitem(last=False)
    return p


def _out(M, N, dtype, device, out):
    if out is not None:
        return out
    return _torch().empty((M, N), dtype=dtype, device=device)


def _generic_plan(A, B, b_layout, C, bias, R, out, alpha, beta, act, prepacked=False, stream=None,
                  no_scratch=False):
    M, K = A.shape
    N = B.shape[1] if b_layout == LAYOUT_KN else B.shape[0]
    return plan(KIND_GENERIC, M, N, K, a_type=_dtype_code(A), b_type=_dtype_code(B),
                d_type=_dtype_code(out), c_type=_dtype_code(C) if C is not None else None,
                bias_type=_dtype_code(bias) if bias is not None else None,
                r_type=_dtype_code(R) if R is not None else None, b_layout=b_layout,
                lda=_ld(A), ldb=_ld(B), ldc=_ld(C) if C is not None else 0, ldd=_ld(out),
                ldr=_ld(R) if R is not None else 0, alpha=alpha, beta=beta, act=act,
                bias=bias is not None, C=C is not None and beta != 0.0, R=R is not None, b_prepacked=prepacked,
                no_scratch=no_scratch, stream=stream)


def gemm_epilogue(A, B, *, bias=None, C=None, R=None, alpha=1.0, beta=0.0, act="none",
                  b_layout="KN", out=None, out_dtype=None, stream=None, prepacked=False):
    """D = act(alpha * A @ B + beta * C + bias) + R on the GPU (fused kernel).

    ``prepacked``: B is the [K, N] tensor ``b_prepack`` returned (decode shapes, M <= 32)."""
    lay = LAYOUT_KN if b_layout == "KN" else LAYOUT_NK
    M = A.shape[0]
    N = B.shape[1] if lay == LAYOUT_KN else B.shape[0]
    out = _out(M, N, out_dtype or A.dtype, A.device, out)
    p = _generic_plan(A, B, lay, C, bias, R, out, alpha, beta, act, prepacked, stream)
    _check(lib().gemm_epi_run(p.handle, _ptr(A), _ptr(B), _ptr(C), _ptr(bias), _ptr(R), _ptr(out),
                              _stream(stream)), "gemm_epi_run")
    return out


def gemm_epilogue_noalloc(A, B, *, out, bias=None, C=None, R=None, alpha=1.0, beta=0.0, act="none",
                          b_layout="KN", stream=None, prepacked=False):
    """``gemm_epilogue`` through ``gemm_epi_run_noalloc``: the plan allocates no device memory and the
    run uses the library's static per-GPU scratch (calls that overlap on one GPU race).  ``out`` is
    required, so the call allocates nothing either."""
    lay = LAYOUT_KN if b_layout == "KN" else LAYOUT_NK
    p = _generic_plan(A, B, lay, C, bias, R, out, alpha, beta, act, prepacked, stream, no_scratch=True)
    _check(lib().gemm_epi_run_noalloc(p.handle, _ptr(A), _ptr(B), _ptr(C), _ptr(bias), _ptr(R), _ptr(out),
                                      _stream(stream)), "gemm_epi_run_noalloc")
    return out


def gemm_epilogue_unfused(A, B, *, bias=None, C=None, R=None, alpha=1.0, beta=0.0, act="none",
                          b_layout="KN", out=None, out_dtype=None, workspace=None, stream=None):
    """Same result as ``gemm_epilogue`` from the unfused chain of kernels."""
    lay = LAYOUT_KN if b_layout == "KN" else LAYOUT_NK
    M = A.shape[0]
    N = B.shape[1] if lay == LAYOUT_KN else B.shape[0]
    out = _out(M, N, out_dtype or A.dtype, A.device, out)
    p = _generic_plan(A, B, lay, C, bias, R, out, alpha, beta, act, stream=stream)
    ws = workspace if workspace is not None else _workspace(p, A.device)
    _check(lib().gemm_epi_run_unfused(p.handle, _ptr(A), _ptr(B), _ptr(C), _ptr(bias), _ptr(R), _ptr(out),
                                      _ptr(ws), _stream(stream)), "gemm_epi_run_unfused")
    return out


def _workspace(p: Plan, device):
    torch = _torch()
    return torch.empty(max(p.workspace_bytes(), 256), dtype=torch.uint8, device=device)


def _swiglu_plan(X, Wg, out, stream=None, prepacked=False, no_scratch=False):
    M, K = X.shape
    N = Wg.shape[1]
    return plan(KIND_SWIGLU, M, N, K, a_type=BF16, b_type=BF16, d_type=BF16, lda=_ld(X), ldb=_ld(Wg),
                ldd=_ld(out), b_prepacked=prepacked, no_scratch=no_scratch, stream=stream)


def swiglu(X, Wg, Wu, *, out=None, prepacked=False, no_scratch=False, stream=None):
    """D = silu(X @ Wg) * (X @ Wu) (fused dual GEMM).

    ``prepacked``: Wg and Wu were converted by ``swiglu_prepack`` (M <= 32, N % 128 == 0, K % 32 == 0):
    each column block of the gate and of the up weight streams on a workgroup of its own through the
    prepacked decode loop, and the second of the two to finish combines silu(gate) * up for the
    block (fp32 tiles in the plan's scratch).  ``no_scratch``: a plan that allocates no device memory
    (raw weights only: the tile kernel at every M)."""
    if Wg.stride() != Wu.stride() or Wg.shape != Wu.shape:
        raise ValueError("Wg and Wu must have the same shape and strides")
    out = _out(X.shape[0], Wg.shape[1], X.dtype, X.device, out)
    p = _swiglu_plan(X, Wg, out, stream, prepacked, no_scratch)
    _check(lib().gemm_swiglu_run(p.handle, _ptr(X), _ptr(Wg), _ptr(Wu), _ptr(out), _stream(stream)),
           "gemm_swiglu_run")
    return out


def swiglu_unfused(X, Wg, Wu, *, out=None, workspace=None, prepacked=False, stream=None):
    out = _out(X.shape[0], Wg.shape[1], X.dtype, X.device, out)
    p = _swiglu_plan(X, Wg, out, stream, prepacked)
    ws = workspace if workspace is not None else _workspace(p, X.device)
    _check(lib().gemm_swiglu_run_unfused(p.handle, _ptr(X), _ptr(Wg), _ptr(Wu), _ptr(out), _ptr(ws),
                                         _stream(stream)), "gemm_swiglu_run_unfused")
    return out


WEIGHT_FORMATS = {"u4": U4X2, "u8": U8, "fp8": FP8E4M3}
_DEFAULT_ZP = {"u4": 8, "u8": 128, "fp8": 0}


def _zp(fmt, zero_point):
    if fmt not in WEIGHT_FORMATS:
        raise ValueError(f"weight format {fmt!r} not in {sorted(WEIGHT_FORMATS)}")
    return _DEFAULT_ZP[fmt] if zero_point is None else zero_point


def _w4_plan(X, Wq, scales, C, bias, R, out, alpha, beta, act, group, zero_point, lo_first, prepacked=False,
             fmt="u4", stream=None):
    M, K = X.shape
    N = scales.shape[1]
    return plan(KIND_W4, M, N, K, a_type=BF16, b_type=WEIGHT_FORMATS[fmt], d_type=_dtype_code(out),
                c_type=_dtype_code(C) if C is not None else None,
                bias_type=_dtype_code(bias) if bias is not None else None,
                r_type=_dtype_code(R) if R is not None else None, lda=_ld(X),
                ldb=_ld(Wq) if Wq.dim() == 2 else 0,
                ldc=_ld(C) if C is not None else 0, ldd=_ld(out), ldr=_ld(R) if R is not None else 0,
                alpha=alpha, beta=beta, act=act, bias=bias is not None, C=C is not None and beta != 0.0,
                R=R is not None, group=group, zero_point=_zp(fmt, zero_point), lo_first=lo_first,
                prepacked=prepacked, stream=stream)


def w4_gemm(X, Wq, scales, *, bias=None, C=None, R=None, alpha=1.0, beta=0.0, act="none", group=128,
            zero_point=None, lo_first=False, prepacked=False, out=None, out_dtype=None, stream=None, fmt="u4"):
    """D = act(alpha * X @ deq(Wq, scales) + beta * C + bias) + R with quantised weights (fused).

    ``fmt``: "u4" (packed pairs, Wq [K, N/2]), "u8" or "fp8" (E4M3; Wq [K, N] bytes).
    ``zero_point``: default 8 (u4), 128 (u8), 0 (fp8).
    ``prepacked``: Wq came from ``w4_prepack`` with the same ``fmt`` (kernel-native layout, same byte count)."""
    out = _out(X.shape[0], scales.shape[1], out_dtype or X.dtype, X.device, out)
    p = _w4_plan(X, Wq, scales, C, bias, R, out, alpha, beta, act, group, zero_point, lo_first, prepacked, fmt,
                 stream)
    _check(lib().gemm_w4_run(p.handle, _ptr(X), _ptr(Wq), _ptr(scales), _ptr(C), _ptr(bias), _ptr(R),
                             _ptr(out), _stream(stream)), "gemm_w4_run")
    return out


def w4_gemm_unfused(X, Wq, scales, *, bias=None, C=None, R=None, alpha=1.0, beta=0.0, act="none",
                    group=128, zero_point=None, lo_first=False, prepacked=False, out=None, out_dtype=None,
                    workspace=None, stream=None, fmt="u4"):
    out = _out(X.shape[0], scales.shape[1], out_dtype or X.dtype, X.device, out)
    p = _w4_plan(X, Wq, scales, C, bias, R, out, alpha, beta, act, group, zero_point, lo_first, prepacked, fmt,
                 stream)
    ws = workspace if workspace is not None else _workspace(p, X.device)
    _check(lib().gemm_w4_run_unfused(p.handle, _ptr(X), _ptr(Wq), _ptr(scales), _ptr(C), _ptr(bias),
                                     _ptr(R), _ptr(out), _ptr(ws), _stream(stream)), "gemm_w4_run_unfused")
    return out


def w4_dequant(Wq, scales, *, M=1, group=128, zero_point=None, lo_first=False, out=None, stream=None, fmt="u4"):
    """bf16 W[k][n] = rne(value(code) * s[k // group][n]) (the unfused chain's first step)."""
    torch = _torch()
    K = Wq.shape[0]
    N = Wq.shape[1] * 2 if fmt == "u4" else Wq.shape[1]
    out = out if out is not None else torch.empty((K, N), dtype=torch.bfloat16, device=Wq.device)
    p = plan(KIND_W4, M, N, K, a_type=BF16, b_type=WEIGHT_FORMATS[fmt], d_type=BF16, ldb=_ld(Wq), group=group,
             zero_point=_zp(fmt, zero_point), lo_first=lo_first)
    _check(lib().gemm_w4_dequant_run(p.handle, _ptr(Wq), _ptr(scales), _ptr(out), _stream(stream)),
           "gemm_w4_dequant_run")
    return out


def _add_rmsnorm_args(a, x, w, eps, resid, out, stream):
    torch = _torch()
    M, N = a.shape
    resid = resid if resid is not None else torch.empty_like(a)
    out = out if out is not None else torch.empty_like(a)
    for t in (a, x, resid, out):
        if not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError("add_rmsnorm takes dense bf16 rows")
    return resid, out, (M, N, _ptr(a), _ptr(x), _ptr(w), float(eps), _ptr(resid), _ptr(out), _stream(stream))


def add_rmsnorm(a, x, w, *, eps=1e-6, resid=None, out=None, stream=None):
    """resid = a + x; out = resid * rsqrt(mean(resid^2) + eps) * w (fused row kernel, bf16)."""
    resid, out, args = _add_rmsnorm_args(a, x, w, eps, resid, out, stream)
    _check(lib().ge_add_rmsnorm_run(*args), "ge_add_rmsnorm_run")
    return resid, out


def add_rmsnorm_unfused(a, x, w, *, eps=1e-6, resid=None, out=None, stream=None):
    """The same step as two kernels (add, then RMSNorm over the stored bf16 residual); measurement only."""
    resid, out, args = _add_rmsnorm_args(a, x, w, eps, resid, out, stream)
    _check(lib().ge_add_rmsnorm_run_unfused(*args), "ge_add_rmsnorm_run_unfused")
    return resid, out


def prepare_add_rmsnorm(a, x, w, *, resid, out, eps=1e-6, unfused=False, stream=None) -> Prepared:
    """``add_rmsnorm`` (or its unfused chain) bound to fixed tensors and stream."""
    resid, out, args = _add_rmsnorm_args(a, x, w, eps, resid, out, stream)
    name = "ge_add_rmsnorm_run_unfused" if unfused else "ge_add_rmsnorm_run"
    return Prepared(getattr(lib(), name), name, None, [a, x, w, resid, out], args)


def prepare_gemm_epilogue(A, B, *, out, bias=None, C=None, R=None, alpha=1.0, beta=0.0, act="none",
                          b_layout="KN", unfused=False, workspace=None, stream=None, prepacked=False) -> Prepared:
    """Bind one fused (or unfused) generic call to fixed tensors and stream."""
    lay = LAYOUT_KN if b_layout == "KN" else LAYOUT_NK
    p = _generic_plan(A, B, lay, C, bias, R, out, alpha, beta, act, prepacked, stream)
    ts = [A, B, C, bias, R, out]
    if unfused:
        ws = workspace if workspace is not None else _workspace(p, A.device)
        ts.append(ws)
        args = (p.handle, _ptr(A), _ptr(B), _ptr(C), _ptr(bias), _ptr(R), _ptr(out), _ptr(ws), _stream(stream))
        return Prepared(lib().gemm_epi_run_unfused, "gemm_epi_run_unfused", p, ts, args)
    args = (p.handle, _ptr(A), _ptr(B), _ptr(C), _ptr(bias), _ptr(R), _ptr(out), _stream(stream))
    return Prepared(lib().gemm_epi_run, "gemm_epi_run", p, ts, args)


def prepare_swiglu(X, Wg, Wu, *, out, unfused=False, workspace=None, prepacked=False, stream=None) -> Prepared:
    p = _swiglu_plan(X, Wg, out, stream, prepacked)
    ts = [X, Wg, Wu, out]
    if unfused:
        ws = workspace if workspace is not None else _workspace(p, X.device)
        ts.append(ws)
        args = (p.handle, _ptr(X), _ptr(Wg), _ptr(Wu), _ptr(out), _ptr(ws), _stream(stream))
        return Prepared(lib().gemm_swiglu_run_unfused, "gemm_swiglu_run_unfused", p, ts, args)
    args = (p.handle, _ptr(X), _ptr(Wg), _ptr(Wu), _ptr(out), _stream(stream))
    return Prepared(lib().gemm_swiglu_run, "gemm_swiglu_run", p, ts, args)


def prepare_w4_gemm(X, Wq, scales, *, out, bias=None, C=None, R=None, alpha=1.0, beta=0.0, act="none",
                    group=128, zero_point=None, lo_first=False, prepacked=False, unfused=False, workspace=None,
                    stream=None, fmt="u4") -> Prepared:
    p = _w4_plan(X, Wq, scales, C, bias, R, out, alpha, beta, act, group, zero_point, lo_first, prepacked, fmt,
                 stream)
    ts = [X, Wq, scales, C, bias, R, out]
    if unfused:
        ws = workspace if workspace is not None else _workspace(p, X.device)
        ts.append(ws)
        args = (p.handle, _ptr(X), _ptr(Wq), _ptr(scales), _ptr(C), _ptr(bias), _ptr(R), _ptr(out), _ptr(ws),
                _stream(stream))
        return Prepared(lib().gemm_w4_run_unfused, "gemm_w4_run_unfused", p, ts, args)
    args = (p.handle, _ptr(X), _ptr(Wq), _ptr(scales), _ptr(C), _ptr(bias), _ptr(R), _ptr(out), _stream(stream))
    return Prepared(lib().gemm_w4_run, "gemm_w4_run", p, ts, args)


def w4_prepack(Wq, *, lo_first=False, fmt="u4", out=None, stream=None):
    """Raw quantised weights -> the fused decode kernels' layout (same bytes, one-time).

    ``fmt`` "u4": packed int4 [K, N/2]; "u8" / "fp8": 8-bit codes [K, N] (N % 128 == 0, M <= 16 plans)."""
    torch = _torch()
    if fmt == "u4":
        K, N = Wq.shape[0], Wq.shape[1] * 2
        out = out if out is not None else torch.empty(K * N // 2, dtype=torch.uint8, device=Wq.device)
        p = plan(KIND_W4, 1, N, K, a_type=BF16, b_type=U4X2, d_type=BF16, ldb=_ld(Wq), lo_first=lo_first)
    else:
        K, N = Wq.shape
        out = out if out is not None else torch.empty(K * N, dtype=torch.uint8, device=Wq.device)
        p = plan(KIND_W4, 1, N, K, a_type=BF16, b_type=WEIGHT_FORMATS[fmt], d_type=BF16, ldb=_ld(Wq), group=32,
                 zero_point=_DEFAULT_ZP[fmt])
    _check(lib().gemm_w4_prepack(p.handle, _ptr(Wq), _ptr(out), _stream(stream)), "gemm_w4_prepack")
    return out


def b_prepack(B, *, out=None, stream=None):
    """bf16 weights [K, N] -> the prepacked decode layout (same bytes, one-time), returned as a
    [K, N] tensor whose contents only the prepacked kernels read (``prepacked=True``)."""
    torch = _torch()
    K, N = B.shape
    out = out if out is not None else torch.empty((K, N), dtype=torch.bfloat16, device=B.device)
    p = plan(KIND_GENERIC, 1, N, K, a_type=BF16, b_type=BF16, d_type=BF16, ldb=_ld(B))
    _check(lib().gemm_b_prepack(p.handle, _ptr(B), _ptr(out), _stream(stream)), "gemm_b_prepack")
    return out


def swiglu_prepack(Wg, Wu, *, stream=None):
    """SwiGLU weights [K, N] (bf16) -> the prepacked layout ``swiglu(..., prepacked=True)`` reads
    (one-time): the decode layout of ``b_prepack`` with the column-block width chosen so that the
    gate and up blocks, one workgroup each, fill the GPU."""
    torch = _torch()
    if Wg.shape != Wu.shape:
        raise ValueError("Wg and Wu must have the same shape")
    K, N = Wg.shape
    outs = []
    for W in (Wg, Wu):
        out = torch.empty((K, N), dtype=torch.bfloat16, device=W.device)
        p = plan(KIND_SWIGLU, 1, N, K, a_type=BF16, b_type=BF16, d_type=BF16, ldb=_ld(W))
        _check(lib().gemm_b_prepack(p.handle, _ptr(W), _ptr(out), _stream(stream)), "gemm_b_prepack")
        outs.append(out)
    return tuple(outs)


def _rope_flags(interleaved, exact):
    return (ROPE_INTERLEAVED if interleaved else 0) | (ROPE_EXACT if exact else 0)


def rope_qk(Q, K, cos=None, sin=None, *, q_pos0=0, k_pos0=0, alpha=1.0, interleaved=False, exact=False, out=None,
            out_dtype=None, stream=None):
    """S[b] = alpha * rope(Q[b]) @ rope(K[b])^T with the rotation applied at tile load (one kernel).

    Q [B, Sq, D], K [B, Sk, D] bf16; cos, sin float32 [P, D/2] (None: no rotation).  exact: each rotated
    coordinate is the exact rotation rounded once to bf16 (else fp32, within one bf16 unit of it)."""
    torch = _torch()
    B, Sq, D = Q.shape
    Sk = K.shape[1]
    out = out if out is not None else torch.empty((B, Sq, Sk), dtype=out_dtype or torch.float32, device=Q.device)
    n_pos = cos.shape[0] if cos is not None else 0
    _check(lib().ge_rope_qk_run(B, Sq, Sk, D, _ptr(Q), _ptr(K), _ptr(cos), _ptr(sin), n_pos, q_pos0, k_pos0,
                                _rope_flags(interleaved, exact), float(alpha), _dtype_code(out), _ptr(out), _stream(stream)),
           "ge_rope_qk_run")
    return out


def rope(X, cos, sin, *, pos0=0, interleaved=False, exact=False, out=None, stream=None):
    """The rotation alone: rope(X) for X [B, S, D] bf16, row s at position pos0 + s (``exact`` as in
    ``rope_qk``)."""
    torch = _torch()
    B, S, D = X.shape
    out = out if out is not None else torch.empty_like(X)
    _check(lib().ge_rope_run(B, S, D, _ptr(X), _ptr(cos), _ptr(sin), cos.shape[0], pos0, _rope_flags(interleaved, exact),
                             _ptr(out), _stream(stream)), "ge_rope_run")
    return out


def prepare_rope_qk(Q, K, cos=None, sin=None, *, out, q_pos0=0, k_pos0=0, alpha=1.0, interleaved=False, exact=False,
                    stream=None) -> Prepared:
    """``rope_qk`` bound to fixed tensors and stream (for timing loops and graph capture)."""
    B, Sq, D = Q.shape
    args = (B, Sq, K.shape[1], D, _ptr(Q), _ptr(K), _ptr(cos), _ptr(sin), cos.shape[0] if cos is not None else 0,
            q_pos0, k_pos0, _rope_flags(interleaved, exact), float(alpha), _dtype_code(out), _ptr(out), _stream(stream))
    return Prepared(lib().ge_rope_qk_run, "ge_rope_qk_run", None, [Q, K, cos, sin, out], args)


def prepare_rope(X, cos, sin, *, out, pos0=0, interleaved=False, exact=False, stream=None) -> Prepared:
    """``rope`` bound to fixed tensors and stream."""
    B, S, D = X.shape
    args = (B, S, D, _ptr(X), _ptr(cos), _ptr(sin), cos.shape[0], pos0, _rope_flags(interleaved, exact), _ptr(out),
            _stream(stream))
    return Prepared(lib().ge_rope_run, "ge_rope_run", None, [X, cos, sin, out], args)
