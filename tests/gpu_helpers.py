"""Helpers shared by the GPU test modules (moving seeded host arrays to the
device and comparing device results with the oracle)."""
import numpy as np
import torch

import workloads

DEV = torch.device("cuda:0")

TOL_BF16 = 1e-2   # max |gpu - ref| / (1 + |ref|) for bf16 outputs
TOL_F32 = 1e-4    # ... for fp32 outputs


def to_dev(a, dtype=None):
    """numpy (bf16 as uint16 bits, f32, uint8) -> device tensor of the storage type."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16 or dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_host(t) -> np.ndarray:
    """device tensor -> float64 numpy (exact widening of bf16 / fp32)."""
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return workloads.bf16_bits_to_f32(bits).astype(np.float64)
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    return np.abs(gpu - ref) / (1.0 + np.abs(ref))


def assert_close(gpu_t, ref, tol, what=""):
    g = to_host(gpu_t) if isinstance(gpu_t, torch.Tensor) else gpu_t
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    e = rel_err(g, ref)
    i = np.unravel_index(np.argmax(e), e.shape)
    assert e[i] <= tol, f"{what}: max err {e[i]:.3e} at {i}: gpu {g[i]!r} ref {ref[i]!r} (tol {tol})"
    return float(e[i])


def dev_inputs(inp: dict) -> dict:
    """Device copies of every array in a workloads.make_inputs dict."""
    out = {}
    for k, v in inp.items():
        if isinstance(v, np.ndarray):
            out[k] = to_dev(v)
    return out


def w4_tile_cols(M, N):
    """Columns per workgroup of the quantised tile kernel: 256 (8 waves) where N % 256 == 0 and its
    64 x 256 tiles still give every CU one, else 128 (4 waves)."""
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    return 256 if N % 256 == 0 and (M + 63) // 64 * (N // 256) >= cu else 128


def w4_tile_kernel(fmt, M, N, K):
    """Kernel name the plan gives the quantised tile path: split over K (64 x 128 tiles x S slices,
    S in 2, 4, 8 dividing the K / 128 groups with 2 or more per slice) when the tiles do not fill
    the CUs, else w4_tile_cols."""
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    prefix = {"u4": "tile_w4_bf16", "u8": "tile_w8_u8", "fp8": "tile_w8_fp8"}[fmt]
    tiles, ngt, s = (M + 63) // 64 * (N // 128), K // 128, 1
    for c in (2, 4, 8):
        if tiles * c <= cu and ngt % c == 0 and ngt // c >= 2:
            s = c
    if s > 1:
        return f"{prefix}_64x128x32_split{s}"
    return f"{prefix}_64x{w4_tile_cols(M, N)}x32"
