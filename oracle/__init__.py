"""CPU fp64 oracle for the fused GEMM + epilogue path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product package.
It shares no code with the GPU library.  The arithmetic lives in
``oracle.c`` (plain C, fp64, one pass per step); this module only moves
numpy arrays in and out of it and chains the passes in the pages' order:

    D = act(alpha * (A @ B) + beta * C + bias) + R          generic
    D = silu(X @ Wg) * (X @ Wu)                              SwiGLU
    D = act(alpha * (X @ dequant(Wq, s)) + beta*C + bias) + R    W4

Storage types: ``"f32"`` (float32 arrays), ``"bf16"`` (uint16 bit patterns),
``"f64"`` (float64).  Results are float64 with no final rounding.

Readings of points the pages leave open (see the design notes): beta*C sits
inside the activation and the residual is added after it; the int4 nibble
order is high nibble first unless ``lo_first``; dequantisation is exact.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_DT = {"f32": 0, "bf16": 1, "f64": 2}
_ACT = {"none": 0, "relu": 1, "gelu_tanh": 2, "silu": 3}


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (plain C, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-D_GNU_SOURCE", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
            lib.oracle_gemm.argtypes = [I, I, I, P, I, L, P, I, I, L, P]
            lib.oracle_gemm.restype = I
            lib.oracle_scale.argtypes = [L, P, D]
            lib.oracle_scale.restype = None
            lib.oracle_add_matrix.argtypes = [I, I, P, P, I, L, D]
            lib.oracle_add_matrix.restype = I
            lib.oracle_add_bias.argtypes = [I, I, P, P, I]
            lib.oracle_add_bias.restype = I
            lib.oracle_activation.argtypes = [L, P, I]
            lib.oracle_activation.restype = I
            lib.oracle_mul.argtypes = [L, P, P, P]
            lib.oracle_mul.restype = None
            lib.oracle_w4_unpack.argtypes = [I, I, P, L, I, P]
            lib.oracle_w4_unpack.restype = I
            lib.oracle_w4_dequant.argtypes = [I, I, P, P, I, L, I, I, P]
            lib.oracle_w4_dequant.restype = I
            lib.oracle_w8_dequant.argtypes = [I, I, P, L, I, I, P, I, L, I, P]
            lib.oracle_w8_dequant.restype = I
            lib.oracle_add_rmsnorm.argtypes = [I, I, P, I, P, I, P, I, D, P, P]
            lib.oracle_add_rmsnorm.restype = I
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = I
            _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


_NP = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}


def _as(a, dtype: str) -> np.ndarray:
    want = _NP[dtype]
    a = np.asarray(a)
    if a.dtype != want:
        raise TypeError(f"expected {np.dtype(want)} storage for {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad argument")


# --------------------------------------------------------------------------
# single passes
# --------------------------------------------------------------------------

def gemm(A, B, a_dtype: str, b_dtype: str, b_layout: str = "KN") -> np.ndarray:
    """acc = A @ B in fp64.  A is [M, K]; B is [K, N] ("KN") or [N, K] ("NK")."""
    lib = _load()
    A = _as(A, a_dtype)
    B = _as(B, b_dtype)
    M, K = A.shape
    if b_layout == "KN":
        K2, N = B.shape
        lay = 0
    elif b_layout == "NK":
        N, K2 = B.shape
        lay = 1
    else:
        raise ValueError(b_layout)
    if K2 != K:
        raise ValueError("inner dimensions differ")
    acc = np.empty((M, N), dtype=np.float64)
    _check(lib.oracle_gemm(M, N, K, _ptr(A), _DT[a_dtype], K, _ptr(B), _DT[b_dtype], lay,
                           B.shape[1], _ptr(acc)), "gemm")
    return acc


def epilogue(acc: np.ndarray, *, alpha=1.0, beta=0.0, C=None, c_dtype=None, bias=None,
             bias_dtype=None, act="none", R=None, r_dtype=None) -> np.ndarray:
    """Apply the epilogue passes, in order, to a copy of ``acc`` (fp64 [M, N])."""
    lib = _load()
    t = np.array(acc, dtype=np.float64, order="C", copy=True)
    M, N = t.shape
    lib.oracle_scale(t.size, _ptr(t), float(alpha))
    if beta != 0.0:
        if C is None:
            raise ValueError("beta != 0 needs C")
        C = _as(C, c_dtype)
        _check(lib.oracle_add_matrix(M, N, _ptr(t), _ptr(C), _DT[c_dtype], C.shape[1], float(beta)), "C")
    if bias is not None:
        bias = _as(bias, bias_dtype)
        _check(lib.oracle_add_bias(M, N, _ptr(t), _ptr(bias), _DT[bias_dtype]), "bias")
    _check(lib.oracle_activation(t.size, _ptr(t), _ACT[act]), "activation")
    if R is not None:
        R = _as(R, r_dtype)
        _check(lib.oracle_add_matrix(M, N, _ptr(t), _ptr(R), _DT[r_dtype], R.shape[1], 1.0), "residual")
    return t


def activation(x, act: str) -> np.ndarray:
    lib = _load()
    t = np.array(x, dtype=np.float64, order="C", copy=True)
    _check(lib.oracle_activation(t.size, _ptr(t), _ACT[act]), "activation")
    return t


def gemm_epilogue(A, B, dtype: str, *, b_layout="KN", alpha=1.0, beta=0.0, C=None, bias=None,
                  act="none", R=None, out_dtype=None) -> np.ndarray:
    """Generic path: act(alpha * A @ B + beta * C + bias) + R, all inputs stored as ``dtype``."""
    acc = gemm(A, B, dtype, dtype, b_layout)
    return epilogue(acc, alpha=alpha, beta=beta, C=C, c_dtype=dtype, bias=bias, bias_dtype=dtype,
                    act=act, R=R, r_dtype=dtype)


def swiglu(X, Wg, Wu, dtype: str = "bf16") -> np.ndarray:
    """silu(X @ Wg) * (X @ Wu): two GEMM passes, the SiLU pass, the product pass."""
    lib = _load()
    g = gemm(X, Wg, dtype, dtype)
    u = gemm(X, Wu, dtype, dtype)
    _check(lib.oracle_activation(g.size, _ptr(g), _ACT["silu"]), "silu")
    out = np.empty_like(g)
    lib.oracle_mul(g.size, _ptr(out), _ptr(g), _ptr(u))
    return out


def w4_unpack(Wq, N: int, lo_first: bool = False) -> np.ndarray:
    """Codes [K, N] (uint8) of packed int4 weights Wq [K, N/2]."""
    lib = _load()
    Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
    K = Wq.shape[0]
    if Wq.shape[1] * 2 != N:
        raise ValueError("Wq must be [K, N/2]")
    codes = np.empty((K, N), dtype=np.uint8)
    _check(lib.oracle_w4_unpack(K, N, _ptr(Wq), Wq.shape[1], int(bool(lo_first)), _ptr(codes)), "unpack")
    return codes


def w4_dequant(Wq, scales, N: int, *, group=128, zero_point=8, lo_first=False,
               s_dtype="bf16") -> np.ndarray:
    """Exact fp64 weights W[k][n] = (code - zero_point) * s[k // group][n]."""
    lib = _load()
    codes = w4_unpack(Wq, N, lo_first)
    K = codes.shape[0]
    scales = _as(scales, s_dtype)
    if scales.shape != (K // group, N):
        raise ValueError("scales must be [K/group, N]")
    W = np.empty((K, N), dtype=np.float64)
    _check(lib.oracle_w4_dequant(K, N, _ptr(codes), _ptr(scales), _DT[s_dtype], N, group, zero_point,
                                 _ptr(W)), "dequant")
    return W


def w4_gemm(X, Wq, scales, N: int, dtype: str = "bf16", *, group=128, zero_point=8, lo_first=False,
            alpha=1.0, beta=0.0, C=None, bias=None, act="none", R=None) -> np.ndarray:
    """W4 path: unpack pass, dequant pass, GEMM pass, then the epilogue passes."""
    W = w4_dequant(Wq, scales, N, group=group, zero_point=zero_point, lo_first=lo_first)
    acc = gemm(X, W, dtype, "f64")
    return epilogue(acc, alpha=alpha, beta=beta, C=C, c_dtype=dtype, bias=bias, bias_dtype=dtype,
                    act=act, R=R, r_dtype=dtype)


W8_FORMATS = {"u8": 1, "fp8": 2}


def w8_dequant(Wq, scales, fmt: str, *, group=128, zero_point=0, s_dtype="bf16") -> np.ndarray:
    """Exact fp64 weights of 8-bit codes Wq [K, N]: (q - zero_point) * s (u8) or
    e4m3(q) * s (fp8), s = scales[k // group][n]."""
    lib = _load()
    Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
    K, N = Wq.shape
    scales = _as(scales, s_dtype)
    if scales.shape != (K // group, N):
        raise ValueError("scales must be [K/group, N]")
    W = np.empty((K, N), dtype=np.float64)
    _check(lib.oracle_w8_dequant(K, N, _ptr(Wq), N, W8_FORMATS[fmt], int(zero_point), _ptr(scales),
                                 _DT[s_dtype], N, group, _ptr(W)), "w8 dequant")
    return W


def w8_gemm(X, Wq, scales, fmt: str, dtype: str = "bf16", *, group=128, zero_point=0, alpha=1.0, beta=0.0,
            C=None, bias=None, act="none", R=None, s_dtype="bf16") -> np.ndarray:
    """8-bit weight path: dequant pass, GEMM pass, then the epilogue passes."""
    W = w8_dequant(Wq, scales, fmt, group=group, zero_point=zero_point, s_dtype=s_dtype)
    acc = gemm(X, W, dtype, "f64")
    return epilogue(acc, alpha=alpha, beta=beta, C=C, c_dtype=dtype, bias=bias, bias_dtype=dtype,
                    act=act, R=R, r_dtype=dtype)


def add_rmsnorm(a, x, w, dtype: str = "bf16", eps: float = 1e-6):
    """Residual add then RMSNorm per row: returns (resid, normed) in fp64."""
    lib = _load()
    a = _as(a, dtype)
    x = _as(x, dtype)
    w = _as(w, dtype)
    M, N = a.shape
    resid = np.empty((M, N), dtype=np.float64)
    out = np.empty((M, N), dtype=np.float64)
    _check(lib.oracle_add_rmsnorm(M, N, _ptr(a), _DT[dtype], _ptr(x), _DT[dtype], _ptr(w), _DT[dtype],
                                  float(eps), _ptr(resid), _ptr(out)), "add_rmsnorm")
    return resid, out


def reference(inputs: dict, rows=None) -> np.ndarray:
    """Oracle output for a ``workloads.make_inputs`` dict, optionally for a subset of rows only."""
    kind, dt = inputs["kind"], inputs["dtype"]

    def sel(name):
        a = inputs.get(name)
        if a is None or rows is None:
            return a
        return np.ascontiguousarray(a[rows])

    if kind == "generic":
        return gemm_epilogue(sel("A"), inputs["B"], dt, alpha=inputs["alpha"], beta=inputs["beta"],
                             C=sel("C"), bias=inputs.get("bias"), act=inputs["act"], R=sel("R"))
    if kind == "swiglu":
        return swiglu(sel("X"), inputs["Wg"], inputs["Wu"], dt)
    if kind == "w4":
        return w4_gemm(sel("X"), inputs["Wq"], inputs["scales"], inputs["N"], dt,
                       group=inputs["group"], zero_point=inputs["zero_point"],
                       alpha=inputs["alpha"], beta=inputs["beta"], C=sel("C"),
                       bias=inputs.get("bias"), act=inputs["act"], R=sel("R"))
    if kind == "w8":
        return w8_gemm(sel("X"), inputs["Wq"], inputs["scales"], inputs["fmt"], dt, group=inputs["group"],
                       zero_point=inputs["zero_point"], alpha=inputs["alpha"], beta=inputs["beta"],
                       C=sel("C"), bias=inputs.get("bias"), act=inputs["act"], R=sel("R"))
    raise ValueError(kind)


# --------------------------------------------------------------------------
# rotary position embedding at operand load ("Fusion Thinking", Pattern 4)
# --------------------------------------------------------------------------

def _bf16_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(y) -> np.ndarray:
    """float64 values -> bf16 bit patterns, round to nearest, ties to even (the storage step of a
    bf16 result).  The value is scaled by a power of two so that the bf16 grid becomes the integers
    (steps of 2^(e - 8) for |y| in [2^(e - 1), 2^e), 2^-133 below 2^-126, the subnormal spacing),
    rounded with numpy's rint (half to even), and scaled back: every step is exact in float64.
    Magnitudes beyond the largest bf16 become infinities."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("round_bf16 takes finite values")
    _, e = np.frexp(y)
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(y / step) * step
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)  # exact: r lies on the bf16 grid (or overflows to inf)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _round_sum_bf16(p, q) -> np.ndarray:
    """bf16 bits of the exact value p + q (p, q float64 arrays holding exact products), rounded to
    nearest, ties to even.  The float64 sum is exact or within 2^-53 of p + q; where that rounding
    could decide the bf16 rounding (the sum lies within 2^-40 of a bf16 rounding point, in units of
    the bf16 spacing), the element is recomputed with exact rational arithmetic."""
    from fractions import Fraction
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    y = p + q
    bits = round_bf16(y)
    _, e = np.frexp(y)
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    t = np.abs(y) / step
    near = np.abs(t - np.floor(t) - 0.5) <= 2.0 ** -40
    for idx in zip(*np.nonzero(near)):
        exact = Fraction(float(p[idx])) + Fraction(float(q[idx]))
        sgn = -1 if exact < 0 else 1
        mag = abs(exact)
        if mag == 0:
            bits[idx] = 0
            continue
        # exponent of the exact value: 2^(ex - 1) <= mag < 2^ex
        ex = mag.numerator.bit_length() - mag.denominator.bit_length()
        while Fraction(2) ** ex <= mag:
            ex += 1
        while Fraction(2) ** (ex - 1) > mag:
            ex -= 1
        stp = Fraction(2) ** max(ex - 8, -133)
        n = mag / stp
        fl = n.numerator // n.denominator
        rem = n - fl
        up = rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1)
        val = float((fl + up) * stp) * sgn
        bits[idx] = round_bf16(np.array([val]))[0]
    return bits


def rope(X, cos, sin, pos0: int = 0, interleaved: bool = False) -> np.ndarray:
    """Rotary position embedding of the rows of X (bf16 bits, [..., S, D]; row s sits at position
    pos0 + s), the rope(q, cos, sin) step of page "Fusion Thinking", Pattern 4.

    cos, sin: float32 [P, D/2], row p holding cos(p theta_i), sin(p theta_i).  Pair i of a row is
    (i, i + D/2) (rotate-half, the Llama layout) or (2i, 2i + 1) (``interleaved``), rotated by the
    angle of its position:  x'_a = x_a cos - x_b sin,  x'_b = x_a sin + x_b cos.  The plain
    definition: the exact rotated value (each product of a bf16 and a float32 number is exact in
    float64), stored as bf16 with one rounding to nearest, ties to even, as the unfused chain
    writes q' and k' before the product.  Returns bf16 bit patterns of X's shape."""
    x = _bf16_to_f32(X).astype(np.float64)
    S, D = x.shape[-2], x.shape[-1]
    if D % 2:
        raise ValueError("D must be even")
    c = np.asarray(cos, dtype=np.float32)[pos0:pos0 + S].astype(np.float64)
    s = np.asarray(sin, dtype=np.float32)[pos0:pos0 + S].astype(np.float64)
    if c.shape != (S, D // 2) or s.shape != (S, D // 2):
        raise ValueError("cos / sin tables do not cover the positions")
    if interleaved:
        a, b = x[..., 0::2], x[..., 1::2]
    else:
        a, b = x[..., :D // 2], x[..., D // 2:]
    ya = _round_sum_bf16(a * c, -(b * s))
    yb = _round_sum_bf16(a * s, b * c)
    y = np.empty(x.shape, dtype=np.uint16)
    if interleaved:
        y[..., 0::2], y[..., 1::2] = ya, yb
    else:
        y[..., :D // 2], y[..., D // 2:] = ya, yb
    return y


def rope_qk(Q, K, cos, sin, *, q_pos0: int = 0, k_pos0: int = 0, alpha: float = 1.0,
            interleaved: bool = False, rotate: bool = True) -> np.ndarray:
    """Scores S[b] = alpha * rope(Q[b]) @ rope(K[b])^T in fp64, as separate passes: the two
    rotations, the product (fp64, index order), the scale.  Q [B, Sq, D], K [B, Sk, D] bf16 bits.
    ``rotate=False`` gives the plain product of Q and K."""
    Q = _as(Q, "bf16")
    K = _as(K, "bf16")
    q = rope(Q, cos, sin, q_pos0, interleaved) if rotate else Q
    k = rope(K, cos, sin, k_pos0, interleaved) if rotate else K
    return np.stack([epilogue(gemm(q[b], k[b], "bf16", "bf16", "NK"), alpha=alpha) for b in range(Q.shape[0])])
