"""Algorithmic work of each workload: FLOPs of the products and the bytes a
perfect kernel must move (every input read once, the output written once),
for the fused kernel and for the unfused chain of one-op kernels.

Fusion leaves the FLOPs unchanged and removes the intermediate round trips
(pages "Kernel fusion" (Check yourself) and "kernel fusion" wiki: fusion
saves bytes, not operations).  The epilogue's few FLOPs per output are not
counted.
"""
from __future__ import annotations

PEAK_BF16_FLOPS = 2.5e15
PEAK_HBM_BYTES = 8.0e12
RIDGE = PEAK_BF16_FLOPS / PEAK_HBM_BYTES  # FLOP per byte where the bf16 roofline bends


def _es(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def swiglu_intermediate_bytes_per_token(d_intermediate: int, elem_bytes: int = 2) -> int:
    """Bytes of the gate and up activations one token writes out when the
    SwiGLU product is not fused into the GEMMs."""
    return 2 * d_intermediate * elem_bytes


def w4_bits_per_weight(group: int = 128, scale_bits: int = 16) -> float:
    """Storage cost of a packed int4 weight including its share of the group scale."""
    return 4.0 + scale_bits / group


def work(w) -> dict:
    """FLOPs, fused bytes, unfused bytes and the roofline bound of workload ``w``
    (a ``workloads.Workload``)."""
    M, N, K = w.M, w.N, w.K
    es = _es(w.dtype)
    mn = M * N
    out_b = mn * es
    epi_in = (mn * es if w.C and w.beta != 0 else 0) + (N * es if w.bias else 0) + (mn * es if w.R else 0)
    if w.kind == "generic":
        flops = 2.0 * M * N * K
        a_b, b_b = M * K * es, K * N * es
        fused = a_b + b_b + epi_in + out_b
        # plain GEMM writes T0; each epilogue op reads T and writes T' (plus its own operand)
        unfused = a_b + b_b + out_b
        steps = [(w.alpha != 1.0, 0), (w.C and w.beta != 0, mn * es), (w.bias, N * es),
                 (w.act != "none", 0), (w.R, mn * es)]
        for used, extra in steps:
            if used:
                unfused += 2 * out_b + extra
    elif w.kind == "swiglu":
        flops = 4.0 * M * N * K
        x_b, w_b = M * K * es, K * N * es
        fused = x_b + 2 * w_b + out_b
        # gate GEMM, up GEMM, sigmoid(g), g * s, h * u
        unfused = 2 * (x_b + w_b + out_b) + 2 * out_b + 3 * out_b + 3 * out_b
    elif w.kind in ("w4", "w8"):
        flops = 2.0 * M * N * K
        x_b = M * K * 2
        wq_b = K * N // 2 if w.kind == "w4" else K * N
        s_b = (K // w.group) * N * 2
        fused = x_b + wq_b + s_b + epi_in + out_b
        # dequant writes bf16 W; the GEMM reads it back
        unfused = (wq_b + s_b + K * N * 2) + (x_b + K * N * 2 + out_b)
        steps = [(w.alpha != 1.0, 0), (w.C and w.beta != 0, mn * es), (w.bias, N * es),
                 (w.act != "none", 0), (w.R, mn * es)]
        for used, extra in steps:
            if used:
                unfused += 2 * out_b + extra
    else:
        raise ValueError(w.kind)
    intensity = flops / fused
    return {"flops": flops, "bytes": fused, "unfused_bytes": unfused, "intensity": intensity,
            "bound": "mfma" if intensity >= RIDGE else "hbm"}
