"""The entry point that allocates nothing (gemm_epi_run_noalloc), for callers
that cannot allocate device memory: its plans (GE_FLAG_NO_SCRATCH) own no
device memory and its stream-K decode launches hand partial tiles off
through the library's static per-GPU scratch.  Its outputs equal those of
gemm_epi_run on a plan that owns scratch (the same kernel, deterministic),
on two calls in a row with the second one smaller, and match the oracle."""
import numpy as np
import pytest
import torch

import gemm_epilogue_tile_amd as ge
import oracle
import workloads
from gpu_helpers import DEV, TOL_BF16, assert_close, to_dev

pytestmark = pytest.mark.gpu


def _case(M, N, K, wid, prepacked=False):
    w = workloads.Workload("noalloc", wid, "generic", M, N, K, "bf16", act="gelu_tanh", bias=True, R=True)
    inp = workloads.make_inputs(w)
    A, B, bias, R = (to_dev(inp[k]) for k in ("A", "B", "bias", "R"))
    if prepacked:
        B = ge.b_prepack(B)
    return inp, A, B, bias, R


@pytest.mark.parametrize("prepacked", [False, True])
def test_noalloc_matches_the_scratch_owning_entry_point(prepacked):
    # 16 x 8192 x 4096 then the smaller 16 x 8192 x 2048: both take the stream-K decode kernel, whose
    # counters and partial tiles sit at fixed places in the static scratch, so the second call reuses
    # what the first left behind
    for M, N, K, wid in [(16, 8192, 4096, 60), (16, 8192, 2048, 61)]:
        inp, A, B, bias, R = _case(M, N, K, wid, prepacked)
        kw = dict(bias=bias, R=R, act="gelu_tanh", prepacked=prepacked)
        p = ge.plan(ge.KIND_GENERIC, M, N, K, lda=K, ldb=N, ldd=N, ldr=N, bias=True, R=True, act="gelu_tanh",
                    b_prepacked=prepacked)
        assert p.scratch_bytes > 0 and p.kernel.endswith("streamk")
        q = ge.plan(ge.KIND_GENERIC, M, N, K, lda=K, ldb=N, ldd=N, ldr=N, bias=True, R=True, act="gelu_tanh",
                    b_prepacked=prepacked, no_scratch=True)
        assert q.scratch_bytes == 0 and not q.kernel.endswith("streamk")
        want = ge.gemm_epilogue(A, B, **kw)
        got = torch.empty_like(want)
        for _ in range(2):  # the counters re-arm: a second call on the same buffer gives the same result
            got.fill_(0)
            ge.gemm_epilogue_noalloc(A, B, out=got, **kw)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{M}x{N}x{K}"
        assert_close(got, oracle.reference(inp), TOL_BF16, f"noalloc {M}x{N}x{K}")


def test_noalloc_plan_without_scratch_on_the_plain_entry_point():
    # gemm_epi_run on a GE_FLAG_NO_SCRATCH plan launches the variant without a K split
    M, N, K = 16, 4096, 2048
    inp, A, B, bias, R = _case(M, N, K, 62)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    p = ge.plan(ge.KIND_GENERIC, M, N, K, lda=K, ldb=N, ldd=N, ldr=N, bias=True, R=True, act="gelu_tanh",
                no_scratch=True)
    rc = ge.lib().gemm_epi_run(p.handle, ge._ptr(A), ge._ptr(B), None, ge._ptr(bias), ge._ptr(R), ge._ptr(out),
                               ge._stream(None))
    assert rc == ge.OK
    assert_close(out, oracle.reference(inp), TOL_BF16, "plain kernel of a no-scratch plan")


def test_noalloc_shapes_without_scratch_and_graph_capture():
    # a tile-kernel shape (no scratch needed) and the stream-K shape captured in a graph and replayed
    inp1, A1, B1, b1, R1 = _case(256, 512, 1024, 63)
    inp2, A2, B2, b2, R2 = _case(16, 8192, 4096, 64)
    o1 = torch.empty((256, 512), dtype=torch.bfloat16, device=DEV)
    o2 = torch.empty((16, 8192), dtype=torch.bfloat16, device=DEV)
    kw = dict(act="gelu_tanh")
    ge.gemm_epilogue_noalloc(A1, B1, out=o1, bias=b1, R=R1, **kw)
    ge.gemm_epilogue_noalloc(A2, B2, out=o2, bias=b2, R=R2, **kw)  # plans made before capture
    torch.cuda.synchronize()
    assert_close(o1, oracle.reference(inp1), TOL_BF16, "tile shape")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ge.gemm_epilogue_noalloc(A2, B2, out=o2, bias=b2, R=R2, **kw)
    for _ in range(3):
        o2.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert_close(o2, oracle.reference(inp2), TOL_BF16, "graph replay")
