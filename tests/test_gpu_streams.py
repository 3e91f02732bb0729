"""Calls on several HIP streams: a plan holds no per-call state (apart from
the device scratch of the plans that own one, which serve one stream at a
time), so calls of different plans may run concurrently on different streams,
and every call is ordered by the stream it is given.  The kernels used here
are deterministic, so concurrent results must equal sequential ones bit for
bit."""
import numpy as np
import pytest
import torch

import gemm_epilogue_tile_amd as ge
import oracle
import workloads
from gpu_helpers import DEV, TOL_BF16, assert_close, to_dev

pytestmark = pytest.mark.gpu


def _inputs(M, N, K, wid):
    w = workloads.Workload("streams", wid, "generic", M, N, K, "bf16", act="gelu_tanh", bias=True, R=True)
    return w, workloads.make_inputs(w)


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def test_two_plans_on_two_streams_match_sequential_bitwise():
    # a tile-kernel product and a prepacked decode product, interleaved on two side streams
    _, sq = _inputs(512, 1024, 768, 31)
    _, dc = _inputs(16, 4096, 2048, 32)
    a1, b1, bias1, r1 = (to_dev(sq[k]) for k in ("A", "B", "bias", "R"))
    a2, b2, bias2, r2 = (to_dev(dc[k]) for k in ("A", "B", "bias", "R"))
    b2p = ge.b_prepack(b2)

    def tile(out, stream=None):
        return ge.gemm_epilogue(a1, b1, bias=bias1, R=r1, act="gelu_tanh", out=out, stream=stream)

    def decode(out, stream=None):
        return ge.gemm_epilogue(a2, b2p, bias=bias2, R=r2, act="gelu_tanh", out=out, prepacked=True, stream=stream)

    ref1 = tile(torch.empty((512, 1024), dtype=torch.bfloat16, device=DEV))
    ref2 = decode(torch.empty((16, 4096), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    outs1 = [torch.empty_like(ref1) for _ in range(6)]
    outs2 = [torch.empty_like(ref2) for _ in range(6)]
    torch.cuda.synchronize()
    for o1, o2 in zip(outs1, outs2):
        tile(o1, s1)
        decode(o2, s2)
    s1.synchronize()
    s2.synchronize()
    for o in outs1:
        assert np.array_equal(_bits(o), _bits(ref1))
    for o in outs2:
        assert np.array_equal(_bits(o), _bits(ref2))
    assert_close(ref2, oracle.reference(dc), TOL_BF16, "decode")


def test_call_is_ordered_by_its_stream():
    # on a side stream: overwrite A, then the product; the product must see the new A
    w, inp = _inputs(256, 512, 1024, 33)
    _, other = _inputs(256, 512, 1024, 34)
    A, B, bias, R = (to_dev(inp[k]) for k in ("A", "B", "bias", "R"))
    A_new = to_dev(other["A"])
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        big = torch.empty(64 << 20, dtype=torch.float32, device=DEV)
        big.fill_(1.0)  # keeps the stream busy ahead of the copy
        A.copy_(A_new)
        out = ge.gemm_epilogue(A, B, bias=bias, R=R, act="gelu_tanh")
    s.synchronize()
    want = dict(inp, A=other["A"])
    assert_close(out, oracle.reference(want), TOL_BF16, "stream order")


@pytest.mark.parametrize("shape,kernel", [((16, 4096, 2048), "skinny_bf16_m16_128col_streamk"),
                                          ((16, 8192, 4096), "skinny_bf16_m16_128col_streamk")])
def test_scratch_owning_shape_on_two_streams_at_once(shape, kernel):
    # the stream-K decode kernel hands partial tiles off through its plan's scratch: the same
    # descriptor issued on two streams gets one plan (and scratch) per stream, so interleaved calls
    # on both streams, with no synchronisation between them, each match the oracle
    M, N, K = shape
    _, i1 = _inputs(M, N, K, 35)
    _, i2 = _inputs(M, N, K, 36)
    B, bias, R = (to_dev(i1[k]) for k in ("B", "bias", "R"))
    A1, A2 = to_dev(i1["A"]), to_dev(i2["A"])
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    kw = dict(bias=True, R=True, act="gelu_tanh", lda=K, ldb=N, ldd=N, ldr=N)  # the descriptor gemm_epilogue makes
    p1 = ge.plan(ge.KIND_GENERIC, M, N, K, stream=s1, **kw)
    p2 = ge.plan(ge.KIND_GENERIC, M, N, K, stream=s2, **kw)
    assert p1.kernel == kernel and p1.scratch_bytes > 0
    assert p1 is not p2 and p1 is ge.plan(ge.KIND_GENERIC, M, N, K, stream=s1, **kw)
    outs1 = [torch.empty((M, N), dtype=torch.bfloat16, device=DEV) for _ in range(8)]
    outs2 = [torch.empty((M, N), dtype=torch.bfloat16, device=DEV) for _ in range(8)]
    torch.cuda.synchronize()
    for o1, o2 in zip(outs1, outs2):
        ge.gemm_epilogue(A1, B, bias=bias, R=R, act="gelu_tanh", out=o1, stream=s1)
        ge.gemm_epilogue(A2, B, bias=bias, R=R, act="gelu_tanh", out=o2, stream=s2)
    s1.synchronize()
    s2.synchronize()
    ref1 = oracle.reference(i1)
    ref2 = oracle.reference(dict(i1, A=i2["A"]))
    for o in outs1:
        assert_close(o, ref1, TOL_BF16, "stream 1")
    for o in outs2:
        assert_close(o, ref2, TOL_BF16, "stream 2")
