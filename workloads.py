"""Seeded synthetic inputs for the fused GEMM + epilogue workloads.

This module is shared by the CPU oracle tests and the GPU path.  It draws
random numbers, rounds them to their storage type and names the workload
shapes; it holds none of the method's arithmetic (no product, no epilogue,
no int4 unpacking).

Recipe (one generator per tensor):
  * ``numpy.random.default_rng([workload_id, tensor_id, seed])`` (PCG64);
  * normal tensors are drawn in float32 with the stated standard deviation,
    uniform tensors in float32 on the stated interval;
  * bf16 tensors are the float32 draw rounded to nearest-even bf16 and kept as
    raw ``uint16`` bit patterns, so both sides read exactly the same values;
  * packed int4 weights are uniform bytes U{0..255}: each nibble of a byte is
    then an independent U{0..15} code.

Distributions follow the workloads of the fusion pages (Llama-3-8B MLP
shape for SwiGLU, a 4096^3 square GEMM, a 16-row decode GEMM and a W4A16
GEMM with 128-row K groups).  The second parameter of N(0, s) is the
standard deviation.
"""
from __future__ import annotations

import dataclasses
import numpy as np

# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------

def _rng(workload_id: int, tensor_id: int, seed: int) -> np.random.Generator:
    return np.random.default_rng([int(workload_id), int(tensor_id), int(seed)])


def normal(shape, std, dtype, *, wid, tid, seed=0):
    g = _rng(wid, tid, seed)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return _store(x, dtype)


def uniform(shape, lo, hi, dtype, *, wid, tid, seed=0):
    g = _rng(wid, tid, seed)
    x = g.random(size=shape, dtype=np.float32)
    x *= np.float32(hi - lo)
    x += np.float32(lo)
    return _store(x, dtype)


def lattice_bf16(rows: int, cols: int, *, seed: int = 0) -> np.ndarray:
    """bf16 bits of ((17 i + 29 j + seed) mod 251 - 125) / 256 at row i, column j.

    Deterministic, exact in bf16 (at most 7 significant bits), never periodic
    along a row over fewer than 251 columns, and cheap at any size: for
    matrices too large to draw element by element (several GiB)."""
    table = f32_to_bf16_bits((np.arange(502, dtype=np.float32) % 251 - 125) / 256)
    cj = ((29 * np.arange(cols, dtype=np.int64) + seed) % 251).astype(np.int16)
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, 512):
        ri = ((17 * np.arange(r0, min(rows, r0 + 512), dtype=np.int64)) % 251).astype(np.int16)
        np.take(table, ri[:, None] + cj[None, :], out=out[r0:r0 + len(ri)])
    return out


def uniform_bytes(shape, *, wid, tid, seed=0) -> np.ndarray:
    g = _rng(wid, tid, seed)
    return g.integers(0, 256, size=shape, dtype=np.uint8)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    kind: str            # "generic" | "swiglu" | "w4" | "w8"
    M: int
    N: int
    K: int
    dtype: str           # storage type of A, B, C, bias, R and D ("f32" | "bf16")
    alpha: float = 1.0
    beta: float = 0.0
    act: str = "none"    # none | relu | gelu_tanh | silu
    bias: bool = False
    C: bool = False
    R: bool = False
    group: int = 128
    zero_point: int = 8
    fmt: str = "u4"      # weight code format: u4 (packed pairs), u8, fp8 (OCP E4M3)

    def with_shape(self, M=None, N=None, K=None) -> "Workload":
        return dataclasses.replace(self, M=M or self.M, N=N or self.N, K=K or self.K)


WORKLOADS = {
    # alpha*A*B + beta*C + bias under ReLU, all fp32, U[-1,1]
    "tiny_fp32": Workload("tiny_fp32", 0, "generic", 64, 64, 128, "f32",
                          alpha=1.5, beta=0.5, act="relu", bias=True, C=True),
    # GELU(tanh)(A*B + bias) + R, bf16 storage, fp32 accumulation
    "square_bf16": Workload("square_bf16", 1, "generic", 4096, 4096, 4096, "bf16",
                            act="gelu_tanh", bias=True, R=True),
    # silu(x*Wg) * (x*Wu), Llama-3-8B MLP shape
    "swiglu_8b": Workload("swiglu_8b", 2, "swiglu", 2048, 14336, 4096, "bf16"),
    # 16-row decode GEMM + bias + residual
    "skinny_decode": Workload("skinny_decode", 3, "generic", 16, 28672, 8192, "bf16",
                              bias=True, R=True),
    # W4A16 GEMM + bias, two batch sizes
    "w4a16_m16": Workload("w4a16_m16", 4, "w4", 16, 8192, 8192, "bf16", bias=True),
    "w4a16_m512": Workload("w4a16_m512", 5, "w4", 512, 8192, 8192, "bf16", bias=True),
    # 8-bit weight formats on the same decode shape (beyond the five configurations)
    "w8a16_u8_m16": Workload("w8a16_u8_m16", 6, "w8", 16, 8192, 8192, "bf16", bias=True, zero_point=128,
                             fmt="u8"),
    "w8a16_fp8_m16": Workload("w8a16_fp8_m16", 7, "w8", 16, 8192, 8192, "bf16", bias=True, zero_point=0,
                              fmt="fp8"),
    # and on the W4A16 M=512 shape
    "w8a16_u8_m512": Workload("w8a16_u8_m512", 8, "w8", 512, 8192, 8192, "bf16", bias=True, zero_point=128,
                              fmt="u8"),
    "w8a16_fp8_m512": Workload("w8a16_fp8_m512", 9, "w8", 512, 8192, 8192, "bf16", bias=True, zero_point=0,
                               fmt="fp8"),
    # the SwiGLU MLP shape at 16 rows (decode), beyond the five configurations
    "swiglu_decode": Workload("swiglu_decode", 11, "swiglu", 16, 14336, 4096, "bf16"),
}


def fp8_codes(shape, *, wid, tid, seed=0) -> np.ndarray:
    """E4M3 codes with random sign, exponent field 0..9 (so |value| < 4, subnormals
    included, never NaN) and mantissa field 0..7."""
    r = _rng(wid, tid, seed)
    sign = r.integers(0, 2, size=shape, dtype=np.uint8)
    e = r.integers(0, 10, size=shape, dtype=np.uint8)
    f = r.integers(0, 8, size=shape, dtype=np.uint8)
    return ((sign << 7) | (e << 3) | f).astype(np.uint8)


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """Draw every input tensor of workload ``w`` (row-major, dense).

    Returned dict: numpy arrays (bf16 as uint16 bits, f32 as float32, packed
    int4 as uint8) plus the scalar parameters.
    """
    M, N, K, dt = w.M, w.N, w.K, w.dtype
    out = dict(alpha=w.alpha, beta=w.beta, act=w.act, dtype=dt, kind=w.kind,
               M=M, N=N, K=K, group=w.group, zero_point=w.zero_point)
    wid = w.wid
    if w.kind == "generic":
        if dt == "f32":
            out["A"] = uniform((M, K), -1.0, 1.0, dt, wid=wid, tid=0, seed=seed)
            out["B"] = uniform((K, N), -1.0, 1.0, dt, wid=wid, tid=1, seed=seed)
            if w.C:
                out["C"] = uniform((M, N), -1.0, 1.0, dt, wid=wid, tid=2, seed=seed)
            if w.bias:
                out["bias"] = uniform((N,), -1.0, 1.0, dt, wid=wid, tid=3, seed=seed)
            if w.R:
                out["R"] = uniform((M, N), -1.0, 1.0, dt, wid=wid, tid=4, seed=seed)
        else:
            out["A"] = normal((M, K), 1.0, dt, wid=wid, tid=0, seed=seed)
            out["B"] = normal((K, N), 1.0 / np.sqrt(K), dt, wid=wid, tid=1, seed=seed)
            if w.C:
                out["C"] = normal((M, N), 1.0, dt, wid=wid, tid=2, seed=seed)
            if w.bias:
                out["bias"] = normal((N,), 0.1, dt, wid=wid, tid=3, seed=seed)
            if w.R:
                out["R"] = normal((M, N), 1.0, dt, wid=wid, tid=4, seed=seed)
    elif w.kind == "swiglu":
        out["X"] = normal((M, K), 1.0, dt, wid=wid, tid=0, seed=seed)
        out["Wg"] = normal((K, N), 1.0 / np.sqrt(K), dt, wid=wid, tid=1, seed=seed)
        out["Wu"] = normal((K, N), 1.0 / np.sqrt(K), dt, wid=wid, tid=2, seed=seed)
    elif w.kind == "w4":
        if K % w.group or N % 2:
            raise ValueError("w4 workload needs K % group == 0 and even N")
        out["X"] = normal((M, K), 1.0, dt, wid=wid, tid=0, seed=seed)
        out["Wq"] = uniform_bytes((K, N // 2), wid=wid, tid=1, seed=seed)
        out["scales"] = uniform((K // w.group, N), 0.005, 0.02, "bf16", wid=wid, tid=2, seed=seed)
        if w.bias:
            out["bias"] = normal((N,), 0.1, dt, wid=wid, tid=3, seed=seed)
        if w.R:
            out["R"] = normal((M, N), 1.0, dt, wid=wid, tid=4, seed=seed)
        if w.C:
            out["C"] = normal((M, N), 1.0, dt, wid=wid, tid=5, seed=seed)
    elif w.kind == "w8":
        if K % w.group:
            raise ValueError("w8 workload needs K % group == 0")
        out["X"] = normal((M, K), 1.0, dt, wid=wid, tid=0, seed=seed)
        if w.fmt == "fp8":
            out["Wq"] = fp8_codes((K, N), wid=wid, tid=1, seed=seed)
            out["scales"] = uniform((K // w.group, N), 0.005, 0.02, "bf16", wid=wid, tid=2, seed=seed)
        else:
            out["Wq"] = uniform_bytes((K, N), wid=wid, tid=1, seed=seed)
            out["scales"] = uniform((K // w.group, N), 0.0003, 0.0012, "bf16", wid=wid, tid=2, seed=seed)
        out["fmt"] = w.fmt
        if w.bias:
            out["bias"] = normal((N,), 0.1, dt, wid=wid, tid=3, seed=seed)
        if w.R:
            out["R"] = normal((M, N), 1.0, dt, wid=wid, tid=4, seed=seed)
        if w.C:
            out["C"] = normal((M, N), 1.0, dt, wid=wid, tid=5, seed=seed)
    else:
        raise ValueError(w.kind)
    return out


# --------------------------------------------------------------------------
# rotary position embedding at operand load: scores S = alpha * rope(Q) rope(K)^T per head
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class RopeWorkload:
    name: str
    wid: int
    heads: int
    Sq: int
    Sk: int
    D: int
    q_pos0: int = 0
    k_pos0: int = 0
    base: float = 500000.0   # Llama-3's rotary base
    interleaved: bool = False
    out: str = "f32"          # score storage type

    def with_shape(self, **kw) -> "RopeWorkload":
        return dataclasses.replace(self, **kw)


ROPE_WORKLOADS = {
    # prefill of one layer's attention scores, 32 heads of 128, 1024 queries x 1024 keys
    "rope_qk_prefill": RopeWorkload("rope_qk_prefill", 8, 32, 1024, 1024, 128),
}


def rope_tables(P: int, D: int, base: float):
    """cos, sin as float32 [P, D/2]: angle p * base^(-2i/D) for position p and pair i, computed in
    float64 and rounded once (the tables are inputs of the rotation, as in rope(q, cos, sin))."""
    i = np.arange(D // 2, dtype=np.float64)
    ang = np.arange(P, dtype=np.float64)[:, None] * (base ** (-2.0 * i / D))[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def make_rope_inputs(w: RopeWorkload, seed: int = 0) -> dict:
    """Q [heads, Sq, D], K [heads, Sk, D] ~N(0,1) as bf16 bits; the tables cover every position."""
    Q = normal((w.heads, w.Sq, w.D), 1.0, "bf16", wid=w.wid, tid=0, seed=seed)
    K = normal((w.heads, w.Sk, w.D), 1.0, "bf16", wid=w.wid, tid=1, seed=seed)
    cos, sin = rope_tables(max(w.q_pos0 + w.Sq, w.k_pos0 + w.Sk), w.D, w.base)
    return dict(Q=Q, K=K, cos=cos, sin=sin, q_pos0=w.q_pos0, k_pos0=w.k_pos0, interleaved=w.interleaved,
                alpha=float(1.0 / np.sqrt(w.D)), out=w.out)
