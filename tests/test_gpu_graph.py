"""A decode chain of fused calls captured in a HIP graph and replayed (the
runs allocate nothing and do not synchronise, so they are capture-safe).

Every replay is checked against the oracle on the replay's own inputs (the
bf16 or fp32 tolerance) and bitwise against the eager result of the same
inputs, with eager work and synchronisations between replays; the inputs
change between replays (the graph must read the current contents)."""
import numpy as np
import pytest
import torch

import gemm_epilogue_tile_amd as ge
import oracle
import workloads
from gpu_helpers import DEV, TOL_BF16, TOL_F32, assert_close

pytestmark = pytest.mark.gpu


def _np(t):
    """host copy of a tensor: bf16 as uint16 bit patterns, other types as they are"""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _chain_inputs(seed):
    g = torch.Generator().manual_seed(seed)
    M, K, N1, N2, N3 = 16, 1024, 2048, 1024, 512
    x = torch.randn(M, K, generator=g).bfloat16()
    W1 = (torch.randn(K, N1, generator=g) / 32).bfloat16()
    b1 = (torch.randn(N1, generator=g) * 0.1).bfloat16()
    R1 = torch.randn(M, N1, generator=g).bfloat16()
    Wq = torch.randint(0, 256, (N1, N2 // 2), generator=g, dtype=torch.uint8)
    sc = workloads.f32_to_bf16_bits(np.full((N1 // 128, N2), 0.01, np.float32))
    W3 = (torch.randn(N2, N3, generator=g) / 32).bfloat16()
    return [t.to(DEV) for t in (x, W1, b1, R1, Wq)] + [torch.from_numpy(sc.view(np.int16)).to(DEV).view(torch.bfloat16), W3.to(DEV)]


def _prepare(x, W1, b1, R1, Wp, sc, W3, h, y, z):
    # h = gelu(x W1 + b1) + R1 ; y = h deq(Wq) ; z = silu(y W3)
    return [ge.prepare_gemm_epilogue(x, W1, out=h, bias=b1, R=R1, act="gelu_tanh"),
            ge.prepare_w4_gemm(h, Wp, sc, out=y, prepacked=True),
            ge.prepare_gemm_epilogue(y, W3, out=z, act="silu")]


def test_decode_chain_graph_replays_match_eager():
    x, W1, b1, R1, Wq, sc, W3 = _chain_inputs(1)
    Wp = ge.w4_prepack(Wq)
    M, N1, N2, N3 = x.shape[0], W1.shape[1], sc.shape[1], W3.shape[1]
    bufs_e = [torch.empty(M, n, dtype=torch.bfloat16, device=DEV) for n in (N1, N2, N3)]
    bufs_g = [torch.empty(M, n, dtype=torch.bfloat16, device=DEV) for n in (N1, N2, N3)]
    eager = _prepare(x, W1, b1, R1, Wp, sc, W3, *bufs_e)
    graph_calls = _prepare(x, W1, b1, R1, Wp, sc, W3, *bufs_g)
    for f in eager + graph_calls:   # plans and kernels set up before capture
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in graph_calls:
            f.with_stream()()
    W1n, b1n, R1n, Wqn, scn, W3n = (_np(t) for t in (W1, b1, R1, Wq, sc, W3))
    for rep in range(4):
        x.copy_(_chain_inputs(100 + rep)[0])   # new activations each step
        for f in eager:
            f()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for be, bg in zip(bufs_e, bufs_g):
            assert torch.equal(be, bg), f"replay {rep} differs from the eager chain"
        # the oracle chain from the replay's inputs, each stage stored as bf16 like the chain's buffers
        h = oracle.gemm_epilogue(_np(x), W1n, "bf16", bias=b1n, act="gelu_tanh", R=R1n)
        y = oracle.w4_gemm(oracle.round_bf16(h), Wqn, scn, N2, "bf16")
        z = oracle.gemm_epilogue(oracle.round_bf16(y), W3n, "bf16", act="silu")
        for got, ref, name in zip(bufs_g, (h, y, z), ("h", "y", "z")):
            assert_close(got, ref, TOL_BF16, f"replay {rep}: {name}")


def _scratch_inputs(seed):
    g = torch.Generator().manual_seed(seed)
    x8 = torch.randn(16, 4096, generator=g).bfloat16()
    x4 = torch.randn(256, 1024, generator=g).bfloat16()
    xs = torch.randn(512, 256, generator=g).bfloat16()
    xw = torch.randn(16, 512, generator=g).bfloat16()
    return [t.to(DEV) for t in (x8, x4, xs, xw)]


def test_scratch_using_calls_replay_in_a_graph():
    # calls whose plans own device scratch (the 8-bit K split: tile handoff, counters that re-arm
    # themselves; the stream-K decode kernel), the int4 tile kernel (per-group partial products and
    # the correction product through LDS), the SwiGLU launch whose partial last round is peeled
    # into 128 x 128 tiles, and SwiGLU on prepacked weights (gate / up workgroup pairs, per-block
    # counters that re-arm themselves)
    g = torch.Generator().manual_seed(9)
    x8, x4, xs, xw = _scratch_inputs(2)
    Wq8 = torch.randint(0, 256, (4096, 4096), generator=g, dtype=torch.uint8).to(DEV)
    s8 = torch.full((32, 4096), 0.001).bfloat16().to(DEV)
    Wq4 = torch.randint(0, 256, (1024, 512), generator=g, dtype=torch.uint8).to(DEV)
    Wp4 = ge.w4_prepack(Wq4)
    s4 = torch.full((8, 1024), 0.01).bfloat16().to(DEV)
    Wg = (torch.randn(256, 136 * 128, generator=g) / 16).bfloat16().to(DEV)
    Wu = (torch.randn(256, 136 * 128, generator=g) / 16).bfloat16().to(DEV)

    xd = (torch.randn(16, 2048, generator=g)).bfloat16().to(DEV)
    Wd = (torch.randn(2048, 4096, generator=g) / 16).bfloat16().to(DEV)
    bd = (torch.randn(4096, generator=g) * 0.1).bfloat16().to(DEV)
    Wgd = (torch.randn(512, 14336, generator=g) / 16).bfloat16().to(DEV)
    Wud = (torch.randn(512, 14336, generator=g) / 16).bfloat16().to(DEV)
    Wgp, Wup = ge.swiglu_prepack(Wgd, Wud)

    def outs():
        return [torch.empty(16, 4096, dtype=torch.bfloat16, device=DEV),
                torch.empty(256, 1024, dtype=torch.bfloat16, device=DEV),
                torch.empty(512, 136 * 128, dtype=torch.bfloat16, device=DEV),
                torch.empty(16, 4096, dtype=torch.bfloat16, device=DEV),
                torch.empty(16, 14336, dtype=torch.bfloat16, device=DEV)]

    def prepare(o):
        return [ge.prepare_w4_gemm(x8, Wq8, s8, out=o[0], zero_point=128, fmt="u8"),
                ge.prepare_w4_gemm(x4, Wp4, s4, out=o[1], prepacked=True),
                ge.prepare_swiglu(xs, Wg, Wu, out=o[2]),
                ge.prepare_gemm_epilogue(xd, Wd, bias=bd, out=o[3]),
                ge.prepare_swiglu(xw, Wgp, Wup, out=o[4], prepacked=True)]

    oe, og = outs(), outs()
    eager, graph_calls = prepare(oe), prepare(og)
    kernels = [f._plan.kernel for f in eager]
    assert kernels[0] == "skinny_u8_m16_128col_split4" and kernels[1] == "tile_w4_bf16_64x128x32_split4"
    assert kernels[2] == "tile_swiglu_256x128x32+128x128x32"
    assert kernels[3] == "skinny_bf16_m16_128col_streamk"
    assert kernels[4] == "skinny_bf16p_swiglu_112col_pairs"
    assert all(eager[i]._plan.scratch_bytes > 0 for i in (0, 1, 3, 4))
    for f in eager + graph_calls:
        f()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for f in graph_calls:
            f.with_stream()()
    Wq4n = _np(Wq4)
    for rep in range(4):
        for dst, src in zip((x8, x4, xs, xw), _scratch_inputs(200 + rep)):
            dst.copy_(src)
        for f in eager:
            f()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for be, bg in zip(oe, og):
            assert torch.equal(be, bg), f"replay {rep} differs from the eager calls"
        refs = [oracle.w8_gemm(_np(x8), _np(Wq8), _np(s8), "u8", "bf16", group=128, zero_point=128),
                oracle.w4_gemm(_np(x4), Wq4n, _np(s4), 1024, "bf16"),
                oracle.swiglu(_np(xs), _np(Wg), _np(Wu), "bf16"),
                oracle.gemm_epilogue(_np(xd), _np(Wd), "bf16", bias=_np(bd)),
                oracle.swiglu(_np(xw), _np(Wgd), _np(Wud), "bf16")]
        for got, ref, name in zip(og, refs, ("u8 split", "int4 tile", "swiglu", "stream-k", "swiglu prepacked")):
            assert_close(got, ref, TOL_BF16, f"replay {rep}: {name}")


def test_prepacked_decode_and_rope_calls_replay_in_a_graph():
    # prepacked bf16 decode (plain and stream-K, whose plan scratch holds self-re-arming counters),
    # prepacked 8-bit codes with the K split, and the RoPE scores kernel, captured once and replayed
    # with new activations each time; every replay bitwise equal to the eager calls
    g = torch.Generator().manual_seed(13)

    def acts(seed):
        h = torch.Generator().manual_seed(seed)
        return [t.bfloat16().to(DEV) for t in (torch.randn(16, 1024, generator=h), torch.randn(16, 256, generator=h),
                                               torch.randn(16, 4096, generator=h),
                                               torch.randn(2, 256, 128, generator=h),
                                               torch.randn(2, 384, 128, generator=h))]

    xs, xp, x8, Q, K = acts(3)
    Wsr = (torch.randn(1024, 8192, generator=g) / 32).bfloat16().to(DEV)
    Wpr = (torch.randn(256, 16512, generator=g) / 16).bfloat16().to(DEV)
    Wq8r = torch.randint(0, 256, (4096, 4096), generator=g, dtype=torch.uint8).to(DEV)
    Ws, Wp, Wq8 = ge.b_prepack(Wsr), ge.b_prepack(Wpr), ge.w4_prepack(Wq8r, fmt="u8")
    s8 = torch.full((32, 4096), 0.001).bfloat16().to(DEV)
    cos, sin = (torch.from_numpy(t).to(DEV) for t in workloads.rope_tables(384, 128, 500000.0))

    def outs():
        return [torch.empty(16, 8192, dtype=torch.bfloat16, device=DEV),
                torch.empty(16, 16512, dtype=torch.bfloat16, device=DEV),
                torch.empty(16, 4096, dtype=torch.bfloat16, device=DEV),
                torch.empty(2, 256, 384, dtype=torch.float32, device=DEV)]

    def prepare(o):
        return [ge.prepare_gemm_epilogue(xs, Ws, out=o[0], prepacked=True),
                ge.prepare_gemm_epilogue(xp, Wp, out=o[1], prepacked=True),
                ge.prepare_w4_gemm(x8, Wq8, s8, out=o[2], zero_point=128, fmt="u8", prepacked=True),
                ge.prepare_rope_qk(Q, K, cos, sin, out=o[3], q_pos0=128, alpha=0.125, exact=True)]

    oe, og = outs(), outs()
    eager, graph_calls = prepare(oe), prepare(og)
    kernels = [f._plan.kernel for f in eager[:3]]
    assert kernels == ["skinny_bf16_m16_prepacked_streamk", "skinny_bf16_m16_128col_prepacked",
                       "skinny_u8_m16_128col_split4_prepacked"]
    for f in eager + graph_calls:
        f()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for f in graph_calls:
            f.with_stream()()
    cosn, sinn = cos.cpu().numpy(), sin.cpu().numpy()
    for rep in range(4):
        for dst, src in zip((xs, xp, x8, Q, K), acts(300 + rep)):
            dst.copy_(src)
        for f in eager:
            f()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for be, bg in zip(oe, og):
            assert torch.equal(be, bg), f"replay {rep} differs from the eager calls"
        refs = [oracle.gemm_epilogue(_np(xs), _np(Wsr), "bf16"),
                oracle.gemm_epilogue(_np(xp), _np(Wpr), "bf16"),
                oracle.w8_gemm(_np(x8), _np(Wq8r), _np(s8), "u8", "bf16", group=128, zero_point=128)]
        for got, ref, name in zip(og[:3], refs, ("bf16 stream-k", "bf16 prepacked", "u8 prepacked")):
            assert_close(got, ref, TOL_BF16, f"replay {rep}: {name}")
        sref = oracle.rope_qk(_np(Q), _np(K), cosn, sinn, q_pos0=128, alpha=0.125)
        assert_close(og[3], sref, TOL_F32, f"replay {rep}: rope scores")
