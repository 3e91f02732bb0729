"""GPU parity at operand sizes past the 32-bit offset range.

The streaming and tile kernels address operands through 32-bit buffer
offsets.  The decode kernels start a weight's range where a wave's (raw
layout) or a column block's (prepacked layout) share begins, so only that
share has to span less than 2^31 bytes; a problem no fast kernel can address
runs on the general kernel, which uses 64-bit offsets.  Here a decode product
with an LM-head-sized weight (a 152064-token vocabulary: 16 x 152064 x 8192
bf16, 2.3 GiB) runs on the raw-layout and on the prepacked streaming kernel;
one with an odd vocabulary (152063 columns, rows not 16-byte aligned) on the
general kernel; and one just under 2 GiB (16 x 131064 x 8192) on the
raw-layout streaming kernel;
output columns at both ends and in between are checked against the oracle,
computed on the same columns."""
import numpy as np
import pytest

import gemm_epilogue_tile_amd as ge
import oracle
import workloads
from gpu_helpers import TOL_BF16, assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu

K = 8192
WID = 20  # seed stream of these inputs


@pytest.mark.parametrize("N,prepacked,kernel", [(152064, False, "skinny_bf16_m16"),
                                                (152064, True, "skinny_bf16_m16_128col_prepacked"),
                                                (152063, False, "general_64x64"),
                                                (131064, False, "skinny_bf16_m16")])
def test_weights_past_and_below_2gib(N, prepacked, kernel):
    M = 16
    assert (K * N * 2 >= 1 << 31) == (N > 131064)
    A = workloads.normal((M, K), 1.0, "bf16", wid=WID, tid=0)
    B = workloads.lattice_bf16(K, N, seed=N)
    bias = workloads.normal((N,), 0.1, "bf16", wid=WID, tid=3)
    R = workloads.normal((M, N), 1.0, "bf16", wid=WID, tid=4)
    assert ge.plan(ge.KIND_GENERIC, M, N, K, bias=True, R=True, b_prepacked=prepacked).kernel.startswith(kernel)
    print(f"limits: 16x{N}x{K}, B {K * N * 2 / 2**30:.3f} GiB, kernel {kernel}", flush=True)
    Bd = to_dev(B)
    if prepacked:
        Bd = ge.b_prepack(Bd)
    out = to_host(ge.gemm_epilogue(to_dev(A), Bd, bias=to_dev(bias), R=to_dev(R), prepacked=prepacked))
    rng = np.random.default_rng(N)
    cols = np.unique(np.concatenate([np.arange(64), np.arange(N - 256, N), rng.choice(N, 256, replace=False)]))
    ref = oracle.gemm_epilogue(A, np.ascontiguousarray(B[:, cols]), "bf16", bias=bias[cols],
                               R=np.ascontiguousarray(R[:, cols]))
    assert_close(out[:, cols], ref, TOL_BF16, f"16x{N}x{K}")
    assert np.all(np.isfinite(out))
