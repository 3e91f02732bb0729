"""GPU parity: every fused entry point against the CPU oracle, element by
element, on seeded inputs (small and ragged shapes spanning several tiles,
edge cases, strides, aliasing, misalignment, the unfused chains)."""
import numpy as np
import pytest
import torch

import gemm_epilogue_tile_amd as ge
import oracle
import workloads
from gpu_helpers import DEV, TOL_BF16, TOL_F32, assert_close, dev_inputs, to_dev, to_host, w4_tile_cols, w4_tile_kernel

pytestmark = pytest.mark.gpu

SQ = workloads.WORKLOADS["square_bf16"]


def _generic(inp, act=None, **kw):
    d = dev_inputs(inp)
    return ge.gemm_epilogue(d["A"], d["B"], bias=d.get("bias"), C=d.get("C"), R=d.get("R"),
                            alpha=inp["alpha"], beta=inp["beta"], act=act or inp["act"], **kw)


def test_tiny_fp32_config():
    w = workloads.WORKLOADS["tiny_fp32"]
    inp = workloads.make_inputs(w)
    out = _generic(inp)
    assert out.dtype == torch.float32
    assert_close(out, oracle.reference(inp), TOL_F32, "tiny_fp32")


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (1, 8, 8), (7, 13, 5), (64, 64, 32), (65, 63, 33),
                                   (128, 256, 512), (200, 136, 264), (257, 520, 96), (16, 1000, 776),
                                   (300, 17, 1024), (513, 264, 136)])
def test_bf16_gelu_bias_residual_ragged(M, N, K):
    w = SQ.with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M * 7 + N)
    assert_close(_generic(inp), oracle.reference(inp), TOL_BF16, f"bf16 {M}x{N}x{K}")


def _random_cases(n=32, seed=20261202):
    rng = np.random.default_rng(seed)
    acts, flag_sets = ["none", "relu", "gelu_tanh", "silu"], ["", "b", "c", "r", "bcr"]
    return [(int(M), int(N), int(K), acts[c % 4], flag_sets[(c * 3) % 5])
            for c, (M, N, K) in enumerate(rng.integers(1, 301, size=(n, 3)))]


@pytest.mark.parametrize("M,N,K,act,flags", _random_cases())
def test_random_ragged_shapes_through_the_generic_path(M, N, K, act, flags):
    # seeded sweep over M, N, K in [1, 300] with every activation and epilogue term
    import dataclasses
    w = dataclasses.replace(SQ, M=M, N=N, K=K, alpha=0.75 if "c" in flags else 1.0,
                            beta=-0.5 if "c" in flags else 0.0, act=act, bias="b" in flags, C="c" in flags,
                            R="r" in flags)
    inp = workloads.make_inputs(w, seed=M * 1000 + N)
    assert_close(_generic(inp), oracle.reference(inp), TOL_BF16, f"random {M}x{N}x{K} {act}/{flags}")


@pytest.mark.parametrize("act", ["none", "relu", "gelu_tanh", "silu"])
@pytest.mark.parametrize("flags", ["", "b", "c", "r", "bcr"])
def test_bf16_every_activation_and_flag(act, flags):
    import dataclasses
    w = dataclasses.replace(SQ, M=192, N=264, K=320, alpha=0.75 if "c" in flags else 1.0,
                            beta=-0.5 if "c" in flags else 0.0, act=act, bias="b" in flags,
                            C="c" in flags, R="r" in flags)
    inp = workloads.make_inputs(w, seed=5)
    assert_close(_generic(inp), oracle.reference(inp), TOL_BF16, f"{act}/{flags}")


@pytest.mark.parametrize("M,N,K", [(64, 64, 128), (33, 71, 130), (256, 256, 256)])
def test_fp32_operands_all_epilogue_terms(M, N, K):
    w = workloads.WORKLOADS["tiny_fp32"].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=2)
    assert_close(_generic(inp), oracle.reference(inp), TOL_F32, f"fp32 {M}x{N}x{K}")


# Plain products take 128 x 128 tiles when those fit in one round over the CUs, else 256 x 256
# tiles; both sizes, both B layouts, ragged edges.
@pytest.mark.parametrize("M,N,K,layout,kernel", [
    (48, 28672, 256, "KN", "tile_kn_128x128x32"),      # batched decode rows: 224 tiles of 128
    (100, 3000, 520, "NK", "tile_nk_128x128x32"),
    (2100, 2056, 200, "KN", "tile_kn_256x256x32"),     # 289 tiles of 128 would take two rounds
    (2100, 2056, 200, "NK", "tile_nk_256x256x32"),
])
def test_tile_size_choice_and_parity(M, N, K, layout, kernel):
    w = SQ.with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M + N)
    lay = ge.LAYOUT_KN if layout == "KN" else ge.LAYOUT_NK
    assert ge.plan(ge.KIND_GENERIC, M, N, K, bias=True, R=True, act="gelu_tanh", b_layout=lay).kernel == kernel
    d = dev_inputs(inp)
    B = d["B"] if layout == "KN" else to_dev(np.ascontiguousarray(inp["B"].T))
    out = ge.gemm_epilogue(d["A"], B, bias=d["bias"], R=d["R"], act="gelu_tanh", b_layout=layout)
    assert_close(out, oracle.reference(inp), TOL_BF16, f"{kernel} {M}x{N}x{K}")


# SwiGLU at decode sizes (M <= 32) on raw weights: gate / up workgroup pairs over the raw decode loop
# (128- or 64-column blocks); shapes the raw decode kernel cannot read (N % 8 != 0) take the tile or
# general kernel
@pytest.mark.parametrize("M,N,K,kernel", [(1, 14336, 256, "skinny_bf16_swiglu_128col_pairs"),
                                          (16, 1000, 520, "skinny_bf16_swiglu_64col_pairs"),
                                          (31, 3000, 136, "skinny_bf16_swiglu_64col_pairs"),
                                          (8, 1001, 256, None)])
def test_swiglu_few_rows(M, N, K, kernel):
    w = workloads.Workload("swiglu_rows", 2, "swiglu", M, N, K, "bf16")
    inp = workloads.make_inputs(w, seed=M)
    pl = ge.plan(ge.KIND_SWIGLU, M, N, K)
    if kernel is not None:
        assert pl.kernel == kernel, pl.kernel
        assert pl.scratch_bytes > 0
    else:
        assert not pl.kernel.startswith("skinny"), pl.kernel
    d = dev_inputs(inp)
    out = ge.swiglu(d["X"], d["Wg"], d["Wu"])
    assert_close(out, oracle.reference(inp), TOL_BF16, f"swiglu {M}x{N}x{K}")
    assert torch.equal(out, ge.swiglu(d["X"], d["Wg"], d["Wu"])), "repeat calls must agree bitwise"


def test_swiglu_few_rows_without_scratch():
    # a plan that may not allocate keeps the tile kernel; prepacked weights need the pairs' scratch
    M, N, K = 16, 1024, 256
    pl = ge.plan(ge.KIND_SWIGLU, M, N, K, no_scratch=True)
    assert pl.scratch_bytes == 0 and pl.kernel.startswith("tile_swiglu"), pl.kernel
    w = workloads.Workload("swiglu_rows", 2, "swiglu", M, N, K, "bf16")
    inp = workloads.make_inputs(w, seed=4)
    d = dev_inputs(inp)
    assert_close(ge.swiglu(d["X"], d["Wg"], d["Wu"], no_scratch=True), oracle.reference(inp), TOL_BF16,
                 "swiglu without scratch")
    with pytest.raises(ge.GemmEpiError) as e:
        ge.plan(ge.KIND_SWIGLU, M, N, K, b_prepacked=True, no_scratch=True)
    assert e.value.status == ge.ERR_UNSUPPORTED


def test_swiglu_pairs_fall_back_on_misaligned_operands():
    # X one element off 16-byte alignment: the plan's pairs cannot read it, the call takes the tile
    # or general kernel instead, same results within the tolerance
    M, N, K = 16, 1024, 256
    w = workloads.Workload("swiglu_rows", 2, "swiglu", M, N, K, "bf16")
    inp = workloads.make_inputs(w, seed=3)
    d = dev_inputs(inp)
    flat = torch.zeros(M * K + 1, dtype=torch.bfloat16, device=DEV)
    flat[1:] = d["X"].reshape(-1)
    X = flat[1:].view(M, K)
    assert X.data_ptr() % 16 != 0
    assert_close(ge.swiglu(X, d["Wg"], d["Wu"]), oracle.reference(inp), TOL_BF16, "swiglu misaligned X")


# SwiGLU at decode sizes on prepacked weights: each column block of W_gate and of W_up streams on a
# workgroup of its own through the prepacked decode loop; the second of a pair to finish combines
# silu(gate) * up (112-column blocks where 2 N / 112 fills the CUs, 128 otherwise)
@pytest.mark.parametrize("M,N,K,cols", [(1, 14336, 4096, 112), (16, 14336, 4096, 112), (5, 1024, 256, 128),
                                        (32, 2048, 512, 128), (17, 384, 96, 128), (16, 28672, 128, 112)])
def test_swiglu_prepacked_decode(M, N, K, cols):
    w = workloads.WORKLOADS["swiglu_8b"].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M + N + K)
    d = dev_inputs(inp)
    pl = ge.plan(ge.KIND_SWIGLU, M, N, K, b_prepacked=True)
    assert pl.kernel == f"skinny_bf16p_swiglu_{cols}col_pairs", pl.kernel
    ncb = N // cols
    assert pl.scratch_bytes == 2 * ncb * (16 if M <= 16 else 32) * cols * 4 + ncb * 4
    Wgp, Wup = ge.swiglu_prepack(d["Wg"], d["Wu"])
    out = ge.swiglu(d["X"], Wgp, Wup, prepacked=True)
    assert_close(out, oracle.reference(inp), TOL_BF16, f"swiglu prepacked {M}x{N}x{K} ({pl.kernel})")
    again = ge.swiglu(d["X"], Wgp, Wup, prepacked=True)
    assert torch.equal(out, again), "repeat calls must agree bitwise"


def test_swiglu_prepacked_refusals():
    for M, N, ldb in [(33, 1024, 0), (16, 1000, 0), (16, 1024, 1152)]:
        with pytest.raises(ge.GemmEpiError) as e:
            ge.plan(ge.KIND_SWIGLU, M, N, 256, b_prepacked=True, ldb=ldb)
        assert e.value.status == ge.ERR_UNSUPPORTED, (M, N, ldb)
    # the unfused chain reads raw weights
    X = torch.zeros(4, 256, dtype=torch.bfloat16, device=DEV)
    W = torch.zeros(256, 1024, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ge.GemmEpiError) as e:
        ge.swiglu_unfused(X, W, W, prepacked=True)
    assert e.value.status == ge.ERR_UNSUPPORTED


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (100, 72, 200), (512, 512, 1024)])
def test_nk_layout(M, N, K):
    w = SQ.with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=4)
    d = dev_inputs(inp)
    Bt = to_dev(np.ascontiguousarray(inp["B"].T))
    out = ge.gemm_epilogue(d["A"], Bt, bias=d["bias"], R=d["R"], act="gelu_tanh", b_layout="NK")
    assert_close(out, oracle.reference(inp), TOL_BF16, "NK")


def test_fp32_output_with_mixed_epilogue_types():
    w = SQ.with_shape(M=130, N=200, K=256)
    inp = workloads.make_inputs(w, seed=6)
    d = dev_inputs(inp)
    bias32 = d["bias"].float()
    out = ge.gemm_epilogue(d["A"], d["B"], bias=bias32, R=d["R"], act="gelu_tanh", out_dtype=torch.float32)
    # the product is bf16 x bf16 with fp32 accumulation: fp32-level agreement
    assert_close(out, oracle.reference(inp), TOL_F32, "fp32 out")


def test_strided_operands_and_output():
    M, N, K = 96, 136, 200
    w = SQ.with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=8)
    d = dev_inputs(inp)
    Abig = torch.zeros((M, K + 24), dtype=torch.bfloat16, device=DEV)
    Abig[:, :K] = d["A"]
    Bbig = torch.zeros((K, N + 8), dtype=torch.bfloat16, device=DEV)
    Bbig[:, :N] = d["B"]
    Rbig = torch.zeros((M, N + 16), dtype=torch.bfloat16, device=DEV)
    Rbig[:, :N] = d["R"]
    Dbig = torch.full((M, N + 40), 7.0, dtype=torch.bfloat16, device=DEV)
    ge.gemm_epilogue(Abig[:, :K], Bbig[:, :N], bias=d["bias"], R=Rbig[:, :N], act="gelu_tanh",
                     out=Dbig[:, :N])
    assert_close(Dbig[:, :N], oracle.reference(inp), TOL_BF16, "strided")
    assert torch.all(Dbig[:, N:] == 7.0), "wrote outside the output view"


def test_misaligned_pointers_take_the_general_kernel():
    M, N, K = 70, 90, 101
    w = SQ.with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=9)
    d = dev_inputs(inp)
    flatA = torch.zeros(M * K + 1, dtype=torch.bfloat16, device=DEV)
    flatA[1:] = d["A"].reshape(-1)
    A = flatA[1:].view(M, K)
    assert A.data_ptr() % 16 != 0
    out = ge.gemm_epilogue(A, d["B"], bias=d["bias"], R=d["R"], act="gelu_tanh")
    assert_close(out, oracle.reference(inp), TOL_BF16, "misaligned")


# The general kernel takes 32 x 32 tiles when 64 x 64 ones would fill fewer than half of the 256
# CUs, 64 x 64 tiles otherwise; both sizes against the oracle, for fp32 operands, misaligned bf16
# operands (which the tile kernels refuse), the dual product and raw int4 weights.
@pytest.mark.parametrize("case,M,N,K,tile", [
    ("f32", 64, 64, 128, 32),       # the tiny config's shape: one 64 x 64 tile, four of 32 x 32
    ("f32", 300, 200, 70, 32),      # 5 x 4 tiles of 64
    ("f32", 700, 1200, 96, 64),     # 11 x 19 = 209 tiles of 64
    ("bf16_misaligned", 70, 90, 101, 32),
    ("bf16_misaligned", 700, 1200, 101, 64),
    ("swiglu_k_ragged", 100, 300, 100, 32),
    ("swiglu_k_ragged", 900, 1100, 100, 64),
    ("w4_raw", 40, 256, 256, 32),
    ("w4_raw", 600, 1024, 256, 64),
])
def test_general_tile_size_choice_and_parity(case, M, N, K, tile):
    name = f"general_{tile}x{tile}"
    if case == "f32":
        w = workloads.WORKLOADS["tiny_fp32"].with_shape(M=M, N=N, K=K)
        inp = workloads.make_inputs(w, seed=M + K)
        assert ge.plan(ge.KIND_GENERIC, M, N, K, a_type=ge.F32, b_type=ge.F32, d_type=ge.F32, c_type=ge.F32,
                       bias_type=ge.F32, bias=True, C=True, beta=0.5, act="relu").kernel == name
        assert_close(_generic(inp), oracle.reference(inp), TOL_F32, f"f32 {M}x{N}x{K}")
    elif case == "bf16_misaligned":
        w = SQ.with_shape(M=M, N=N, K=K)
        inp = workloads.make_inputs(w, seed=M + 1)
        d = dev_inputs(inp)
        flatA = torch.zeros(M * K + 1, dtype=torch.bfloat16, device=DEV)
        flatA[1:] = d["A"].reshape(-1)
        A = flatA[1:].view(M, K)
        out = ge.gemm_epilogue(A, d["B"], bias=d["bias"], R=d["R"], act="gelu_tanh")
        assert_close(out, oracle.reference(inp), TOL_BF16, f"misaligned {M}x{N}x{K}")
    elif case == "swiglu_k_ragged":
        assert ge.plan(ge.KIND_SWIGLU, M, N, K).kernel == name
        w = workloads.WORKLOADS["swiglu_8b"].with_shape(M=M, N=N, K=K)
        inp = workloads.make_inputs(w, seed=M + N)
        d = dev_inputs(inp)
        assert_close(ge.swiglu(d["X"], d["Wg"], d["Wu"]), oracle.reference(inp), TOL_BF16, f"swiglu {M}x{N}x{K}")
    else:
        assert ge.plan(ge.KIND_W4, M, N, K, b_type=ge.U4X2, bias=True).kernel == name
        w = workloads.WORKLOADS["w4a16_m16"].with_shape(M=M, N=N, K=K)
        inp = workloads.make_inputs(w, seed=M + K)
        assert_close(_w4(inp), oracle.reference(inp), TOL_BF16, f"w4 raw {M}x{N}x{K}")


def test_output_aliases_residual():
    w = SQ.with_shape(M=128, N=128, K=256)
    inp = workloads.make_inputs(w, seed=10)
    d = dev_inputs(inp)
    R = d["R"].clone()
    ge.gemm_epilogue(d["A"], d["B"], bias=d["bias"], R=R, act="gelu_tanh", out=R)
    assert_close(R, oracle.reference(inp), TOL_BF16, "D == R")


def test_output_aliases_C():
    w = workloads.WORKLOADS["tiny_fp32"]
    inp = workloads.make_inputs(w)
    d = dev_inputs(inp)
    C = d["C"].clone()
    ge.gemm_epilogue(d["A"], d["B"], C=C, bias=d["bias"], alpha=w.alpha, beta=w.beta, act="relu", out=C)
    assert_close(C, oracle.reference(inp), TOL_F32, "D == C")


def test_identity_B_returns_A():
    K = 256
    A = workloads.normal((96, K), 1.0, "bf16", wid=97, tid=0)
    I = workloads.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    out = ge.gemm_epilogue(to_dev(A), to_dev(I))
    assert np.array_equal(to_host(out), workloads.bf16_bits_to_f32(A).astype(np.float64))


def test_repeat_runs_are_bitwise_identical():
    w = SQ.with_shape(M=512, N=384, K=640)
    inp = workloads.make_inputs(w, seed=11)
    a = _generic(inp)
    b = _generic(inp)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# --------------------------------------------------------------------------
# SwiGLU
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (16, 64, 64), (64, 128, 256), (130, 200, 264),
                                   (256, 512, 512), (512, 1024, 640)])
def test_swiglu_ragged(M, N, K):
    w = workloads.WORKLOADS["swiglu_8b"].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M + N)
    d = dev_inputs(inp)
    out = ge.swiglu(d["X"], d["Wg"], d["Wu"])
    assert_close(out, oracle.reference(inp), TOL_BF16, f"swiglu {M}x{N}x{K}")


def test_swiglu_peeled_last_round():
    # 2 x 136 tiles of 256 x 128 leave a partial round on 256 CUs: the last 8 column blocks run
    # as 128 x 128 tiles in a second launch; every column is checked against the oracle
    M, N, K = 512, 136 * 128, 256
    p = ge.plan(ge.KIND_SWIGLU, M, N, K)
    assert p.kernel == "tile_swiglu_256x128x32+128x128x32"
    w = workloads.WORKLOADS["swiglu_8b"].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=7)
    d = dev_inputs(inp)
    assert_close(ge.swiglu(d["X"], d["Wg"], d["Wu"]), oracle.reference(inp), TOL_BF16, "swiglu peeled")
    assert ge.plan(ge.KIND_SWIGLU, 2048, 14336, 4096).kernel == "tile_swiglu_256x128x32+128x128x32"
    assert ge.plan(ge.KIND_SWIGLU, 2048, 16384, 4096).kernel == "tile_swiglu_256x128x32"  # 1024 tiles


# --------------------------------------------------------------------------
# W4A16
# --------------------------------------------------------------------------

def _w4(inp, **kw):
    d = dev_inputs(inp)
    return ge.w4_gemm(d["X"], torch.from_numpy(inp["Wq"]).to(DEV), d["scales"], bias=d.get("bias"),
                      group=inp["group"], zero_point=inp["zero_point"], **kw)


@pytest.mark.parametrize("M,N,K", [(1, 2, 128), (16, 256, 512), (16, 1000, 1024), (33, 264, 384),
                                   (128, 512, 1024), (512, 512, 256), (200, 136, 640)])
def test_w4_ragged(M, N, K):
    w = workloads.WORKLOADS["w4a16_m16"].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M + K)
    assert_close(_w4(inp), oracle.reference(inp), TOL_BF16, f"w4 {M}x{N}x{K}")


@pytest.mark.parametrize("group", [32, 64, 256])
def test_w4_group_sizes(group):
    import dataclasses
    w = dataclasses.replace(workloads.WORKLOADS["w4a16_m16"], M=32, N=256, K=512, group=group)
    inp = workloads.make_inputs(w, seed=group)
    assert_close(_w4(inp), oracle.reference(inp), TOL_BF16, f"group {group}")


def test_w4_lo_first_and_zero_point():
    w = workloads.WORKLOADS["w4a16_m16"].with_shape(M=16, N=128, K=256)
    inp = workloads.make_inputs(w, seed=3)
    ref = oracle.w4_gemm(inp["X"], inp["Wq"], inp["scales"], w.N, "bf16", zero_point=5, lo_first=True,
                         bias=inp["bias"])
    d = dev_inputs(inp)
    out = ge.w4_gemm(d["X"], torch.from_numpy(inp["Wq"]).to(DEV), d["scales"], bias=d["bias"],
                     zero_point=5, lo_first=True)
    assert_close(out, ref, TOL_BF16, "lo_first zp5")


@pytest.mark.parametrize("M", [16, 512])
def test_w4_unpack_bit_exact_with_one_hot_rows(M):
    # X row m is one-hot at k_m and scales are 2^-6: D[m][n] = (code - 8) * 2^-6 exactly
    K, N = 1024, 512
    Wq = workloads.uniform_bytes((K, N // 2), wid=98, tid=1)
    scales = workloads.f32_to_bf16_bits(np.full((K // 128, N), 2.0 ** -6, np.float32))
    ks = np.arange(M) * 37 % K
    X = np.zeros((M, K), np.float32)
    X[np.arange(M), ks] = 1.0
    Xb = workloads.f32_to_bf16_bits(X)
    out = to_host(ge.w4_gemm(to_dev(Xb), torch.from_numpy(Wq).to(DEV), to_dev(scales)))
    codes = oracle.w4_unpack(Wq, N).astype(np.int64)
    want = (codes[ks] - 8) * 2.0 ** -6
    assert np.array_equal(out, want)


def test_w4_dequant_kernel_bit_exact():
    K, N = 256, 384
    Wq = workloads.uniform_bytes((K, N // 2), wid=99, tid=1)
    scales = workloads.uniform((K // 128, N), 0.005, 0.02, "bf16", wid=99, tid=2)
    W = ge.w4_dequant(torch.from_numpy(Wq).to(DEV), to_dev(scales))
    exact = oracle.w4_dequant(Wq, scales, N)  # products of <= 12 significant bits: exact in fp32
    want = workloads.f32_to_bf16_bits(exact.astype(np.float32))
    got = W.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# unfused chains (measurement baselines)
# --------------------------------------------------------------------------

def _unfused_tol(ref_t, ref, extra_roundings):
    # each extra bf16 rounding of an intermediate of size |t| adds <= 2^-9 |t|
    return TOL_BF16 * (1 + np.abs(ref)) + extra_roundings * 2.0 ** -9 * (1 + np.abs(ref_t)) * 1.2


def test_unfused_generic_matches_oracle():
    w = SQ.with_shape(M=256, N=264, K=320)
    inp = workloads.make_inputs(w, seed=12)
    d = dev_inputs(inp)
    out = to_host(ge.gemm_epilogue_unfused(d["A"], d["B"], bias=d["bias"], R=d["R"], act="gelu_tanh"))
    ref = oracle.reference(inp)
    t = oracle.gemm(inp["A"], inp["B"], "bf16", "bf16")
    assert np.all(np.abs(out - ref) <= _unfused_tol(t, ref, 3))


def test_unfused_fp32_alpha_beta_chain():
    w = workloads.WORKLOADS["tiny_fp32"]
    inp = workloads.make_inputs(w)
    d = dev_inputs(inp)
    out = ge.gemm_epilogue_unfused(d["A"], d["B"], C=d["C"], bias=d["bias"], alpha=w.alpha, beta=w.beta,
                                   act="relu")
    assert_close(out, oracle.reference(inp), TOL_F32, "unfused fp32")


def test_unfused_swiglu_matches_oracle():
    w = workloads.WORKLOADS["swiglu_8b"].with_shape(M=128, N=256, K=512)
    inp = workloads.make_inputs(w, seed=13)
    d = dev_inputs(inp)
    out = to_host(ge.swiglu_unfused(d["X"], d["Wg"], d["Wu"]))
    ref = oracle.reference(inp)
    assert np.all(np.abs(out - ref) <= TOL_BF16 * (1 + np.abs(ref)) + 5 * 2.0 ** -9 * np.abs(ref))


def test_unfused_w4_matches_oracle():
    w = workloads.WORKLOADS["w4a16_m16"].with_shape(M=16, N=512, K=1024)
    inp = workloads.make_inputs(w, seed=14)
    d = dev_inputs(inp)
    out = to_host(ge.w4_gemm_unfused(d["X"], torch.from_numpy(inp["Wq"]).to(DEV), d["scales"],
                                     bias=d["bias"]))
    ref = oracle.reference(inp)
    # the chain rounds every dequantised weight to bf16: random error per product <= 2^-9 |x w|
    X = workloads.bf16_bits_to_f32(inp["X"]).astype(np.float64)
    W = oracle.w4_dequant(inp["Wq"], inp["scales"], w.N)
    spread = np.sqrt((X ** 2) @ (W ** 2))
    tol = TOL_BF16 * (1 + np.abs(ref)) + 6 * 2.0 ** -9 * spread / np.sqrt(3) + 2 * 2.0 ** -9 * np.abs(ref)
    assert np.all(np.abs(out - ref) <= tol)


# --------------------------------------------------------------------------
# fused residual add + RMSNorm
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N", [(1, 8), (4, 100), (16, 4096), (33, 8192), (7, 16384),
                                 # one wave per row: ragged chunk counts, rows not a multiple of
                                 # four, more rows than one launch of workgroups covers
                                 (5, 1000), (9, 2056), (300000, 8)])
def test_add_rmsnorm(M, N):
    a = workloads.normal((M, N), 1.0, "bf16", wid=100, tid=0, seed=N)
    x = workloads.normal((M, N), 1.0, "bf16", wid=100, tid=1, seed=N)
    wt = workloads.normal((N,), 1.0, "bf16", wid=100, tid=2, seed=N)
    resid, out = ge.add_rmsnorm(to_dev(a), to_dev(x), to_dev(wt), eps=1e-6)
    rr, ro = oracle.add_rmsnorm(a, x, wt, "bf16", eps=1e-6)
    assert_close(resid, rr, TOL_BF16, "resid")
    assert_close(out, ro, TOL_BF16, "normed")


@pytest.mark.parametrize("N", [4096, 1000, 8192])  # one wave per row; a workgroup per row (unaligned, long)
@pytest.mark.parametrize("scale,eps", [(1e-3, 1e-6), (1.0, 4.0)])
def test_add_rmsnorm_eps_changes_the_result(N, scale, eps):
    # mean(r^2) of the same order as eps, so eps moves rrms by 18-60% and its placement (inside
    # the root, added to the mean) is visible at the bf16 tolerance; row 0 is all zeros (finite
    # only through eps)
    M = 6
    a = workloads.normal((M, N), scale, "bf16", wid=102, tid=0, seed=N)
    x = workloads.normal((M, N), scale, "bf16", wid=102, tid=1, seed=N)
    a[0] = 0
    x[0] = 0
    wt = workloads.normal((N,), 1.0, "bf16", wid=102, tid=2, seed=N)
    resid, out = ge.add_rmsnorm(to_dev(a), to_dev(x), to_dev(wt), eps=eps)
    rr, ro = oracle.add_rmsnorm(a, x, wt, "bf16", eps=eps)
    _, ro_no_eps = oracle.add_rmsnorm(a[1:], x[1:], wt, "bf16", eps=0.0)
    assert np.max(np.abs(ro[1:] - ro_no_eps) / (1 + np.abs(ro_no_eps))) > 0.1  # eps is not negligible here
    assert_close(resid, rr, TOL_BF16, "resid")
    assert_close(out, ro, TOL_BF16, f"normed eps={eps}")


def test_add_rmsnorm_in_place_residual():
    M, N = 8, 2048
    a = workloads.normal((M, N), 1.0, "bf16", wid=101, tid=0)
    x = workloads.normal((M, N), 1.0, "bf16", wid=101, tid=1)
    wt = workloads.normal((N,), 1.0, "bf16", wid=101, tid=2)
    ad = to_dev(a)
    ge.add_rmsnorm(ad, to_dev(x), to_dev(wt), resid=ad)
    rr, _ = oracle.add_rmsnorm(a, x, wt, "bf16")
    assert_close(ad, rr, TOL_BF16, "resid in place")


# the same step unfused (measurement only): add kernel, then the RMSNorm over the stored residual,
# on both row kernels (one wave per row: aligned rows of at most 4096; a workgroup per row otherwise)
@pytest.mark.parametrize("M,N,eps", [(4, 100, 1e-6), (16, 4096, 1e-6), (33, 8192, 1e-6), (5, 1000, 1e-6),
                                     (300000, 8, 1e-6), (6, 4096, 4.0), (6, 8192, 4.0)])
def test_add_rmsnorm_unfused(M, N, eps):
    a = workloads.normal((M, N), 1.0, "bf16", wid=103, tid=0, seed=N)
    x = workloads.normal((M, N), 1.0, "bf16", wid=103, tid=1, seed=N)
    wt = workloads.normal((N,), 1.0, "bf16", wid=103, tid=2, seed=N)
    ad, xd, wd = to_dev(a), to_dev(x), to_dev(wt)
    resid, out = ge.add_rmsnorm_unfused(ad, xd, wd, eps=eps)
    fresid, _ = ge.add_rmsnorm(ad, xd, wd, eps=eps)
    rr, ro = oracle.add_rmsnorm(a, x, wt, "bf16", eps=eps)
    assert torch.equal(resid, fresid), "both paths store bf16(a + x)"
    assert_close(resid, rr, TOL_BF16, "resid")
    # the norm is taken over the rounded residual: one more bf16 rounding than the fused kernel,
    # far inside the tolerance
    assert_close(out, ro, TOL_BF16, f"normed unfused eps={eps}")


# --------------------------------------------------------------------------
# small-M weight-streaming kernels
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (3, 136, 96), (16, 1000, 1000), (16, 2048, 4096),
                                   (17, 264, 520), (32, 512, 2048), (5, 4104, 136),
                                   # wide N: 128-column workgroups
                                   (16, 32768, 64), (16, 28672, 96), (32, 28680, 64)])
def test_skinny_bf16_bias_residual_gelu(M, N, K):
    w = workloads.WORKLOADS["skinny_decode"].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M + N + K)
    d = dev_inputs(inp)
    out = ge.gemm_epilogue(d["A"], d["B"], bias=d["bias"], R=d["R"], act="gelu_tanh")
    ref = oracle.gemm_epilogue(inp["A"], inp["B"], "bf16", bias=inp["bias"], act="gelu_tanh", R=inp["R"])
    assert_close(out, ref, TOL_BF16, f"skinny {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(16, 4096, 2048), (7, 8104, 2040), (1, 4096, 4096)])
def test_skinny_streamk_bias_residual_gelu(M, N, K):
    # too few column blocks for the CUs: the (column block, 32-row block) units are dealt evenly to
    # one workgroup per CU, each workgroup one K piece of one column block, partial tiles handed
    # off through the plan's scratch (4 or 8 pieces per block here)
    p = ge.plan(ge.KIND_GENERIC, M, N, K, bias=True, R=True, act="gelu_tanh")
    assert p.kernel == "skinny_bf16_m16_128col_streamk" and p.scratch_bytes > 0
    w = workloads.WORKLOADS["skinny_decode"].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M + K)
    d = dev_inputs(inp)
    out = ge.gemm_epilogue(d["A"], d["B"], bias=d["bias"], R=d["R"], act="gelu_tanh")
    ref = oracle.gemm_epilogue(inp["A"], inp["B"], "bf16", bias=inp["bias"], act="gelu_tanh", R=inp["R"])
    assert_close(out, ref, TOL_BF16, f"streamk {M}x{N}x{K}")


def test_skinny_streamk_plan_and_repeat_calls():
    p = ge.plan(ge.KIND_GENERIC, 16, 8192, 8192, bias=True, R=True)
    # 64 column blocks x 256 row blocks over 256 workgroups: 64 units each, 4 workgroups per block
    assert p.kernel == "skinny_bf16_m16_128col_streamk"
    assert p.scratch_bytes == 64 * 4 * 16 * 128 * 4 + 64 * 4
    # a range that would straddle two column blocks keeps the plain kernel
    for N in (28672, 32768):
        assert ge.plan(ge.KIND_GENERIC, 16, N, 8192, bias=True, R=True).kernel == "skinny_bf16_m16_128col"
    w = workloads.WORKLOADS["skinny_decode"].with_shape(M=16, N=4096, K=2048)
    inp = workloads.make_inputs(w, seed=4)
    d = dev_inputs(inp)
    outs = [torch.empty(16, 4096, dtype=torch.bfloat16, device=DEV) for _ in range(200)]
    for o in outs:
        ge.gemm_epilogue(d["A"], d["B"], bias=d["bias"], R=d["R"], out=o)
    torch.cuda.synchronize()
    first = outs[0].view(torch.int16)
    assert all(torch.equal(o.view(torch.int16), first) for o in outs[1:])
    ref = oracle.gemm_epilogue(inp["A"], inp["B"], "bf16", bias=inp["bias"], R=inp["R"])
    assert_close(outs[0], ref, TOL_BF16, "streamk 16x4096x2048")


def test_skinny_plan_picks_the_streaming_kernel():
    p = ge.plan(ge.KIND_GENERIC, 16, 28672, 8192, bias=True, R=True)
    assert p.kernel.startswith("skinny_bf16")
    q16 = ge.plan(ge.KIND_GENERIC, 16, 4096, 1024, bias=True, R=True)
    assert q16.kernel == "skinny_bf16_m16_64col"  # 64 workgroups of 64 columns beat 32 of 128
    # at K = 8192 there is enough work to split each column block's K range over 8 workgroups
    assert ge.plan(ge.KIND_GENERIC, 16, 4096, 8192, bias=True, R=True).kernel.endswith("_streamk")
    q = ge.plan(ge.KIND_W4, 16, 8192, 8192, b_type=ge.U4X2, bias=True, prepacked=True)
    assert q.kernel.startswith("skinny_w4")


def _w4_packed(inp, **kw):
    d = dev_inputs(inp)
    Wq = torch.from_numpy(inp["Wq"]).to(DEV)
    Wp = ge.w4_prepack(Wq, lo_first=kw.get("lo_first", False))
    return ge.w4_gemm(d["X"], Wp, d["scales"], bias=d.get("bias"), group=inp["group"],
                      zero_point=inp["zero_point"], prepacked=True, **kw)


@pytest.mark.parametrize("M,N,K,kernel", [(1, 16, 128, "skinny_w4_m16_32col"), (7, 256, 512, "skinny_w4_m16_128col"),
                                          (16, 1008, 1024, "skinny_w4_m16_32col"),
                                          (16, 4096, 2048, "skinny_w4_m16_128col_split2"),
                                          (17, 1008, 1024, "skinny_w4_m32_32col"), (25, 272, 512, "skinny_w4_m32_32col"),
                                          (32, 4096, 2048, "skinny_w4_m32_32col")])
def test_w4_prepacked_ragged(M, N, K, kernel):
    # 17 <= M <= 32: two 16-row tiles of X per weight fragment; M <= 16 with N a multiple of 128:
    # 128-column workgroups, K split over workgroups where the column blocks leave CUs idle
    w = workloads.WORKLOADS["w4a16_m16"].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M + N)
    assert ge.plan(ge.KIND_W4, M, N, K, b_type=ge.U4X2, bias=True, prepacked=True).kernel == kernel
    assert_close(_w4_packed(inp), oracle.reference(inp), TOL_BF16, f"w4 packed {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,kernel", [
    (16, 128, 1024, "skinny_w4_m16_128col"),           # one workgroup, one group per wave
    (9, 640, 2944, "skinny_w4_m16_128col_split2"),     # 23 groups: a wave with one, waves with none
    (3, 1024, 4096, "skinny_w4_m16_128col_split4"),    # one group per wave
    (16, 2048, 16384, "skinny_w4_m16_128col_split8"),
    (16, 128, 24576, "skinny_w4_m16_128col_split8"),   # three groups per wave
])
def test_w4_prepacked_128col_split(M, N, K, kernel):
    w = workloads.WORKLOADS["w4a16_m16"].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M + K)
    pl = ge.plan(ge.KIND_W4, M, N, K, b_type=ge.U4X2, bias=True, prepacked=True)
    assert pl.kernel == kernel and (pl.scratch_bytes > 0) == ("split" in kernel)
    ref = oracle.reference(inp)
    for rep in range(3):  # the split counters re-arm themselves: repeated calls agree
        assert_close(_w4_packed(inp), ref, TOL_BF16, f"w4 128col {M}x{N}x{K} call {rep}")
    # a plan without device scratch takes the 32-column kernel
    assert ge.plan(ge.KIND_W4, M, N, K, b_type=ge.U4X2, bias=True, prepacked=True,
                   no_scratch=True).kernel in ("skinny_w4_m16_32col", "skinny_w4_m16_128col")


@pytest.mark.parametrize("M", [16, 17, 32])
@pytest.mark.parametrize("group", [32, 64])
def test_w4_prepacked_group_sizes(group, M):
    # M 17 .. 32: each weight fragment feeds two 16-row tiles of X (the group-32 variant included)
    import dataclasses
    w = dataclasses.replace(workloads.WORKLOADS["w4a16_m16"], M=M, N=256, K=512, group=group)
    inp = workloads.make_inputs(w, seed=group + M)
    assert_close(_w4_packed(inp), oracle.reference(inp), TOL_BF16, f"w4 packed group {group}")


@pytest.mark.parametrize("M", [16, 17, 32, 96])
def test_w4_prepacked_lo_first_and_zero_point(M):
    w = workloads.WORKLOADS["w4a16_m16"].with_shape(M=M, N=128, K=256)
    inp = workloads.make_inputs(w, seed=7)
    ref = oracle.w4_gemm(inp["X"], inp["Wq"], inp["scales"], w.N, "bf16", zero_point=3, lo_first=True,
                         bias=inp["bias"])
    inp["zero_point"] = 3
    assert_close(_w4_packed(inp, lo_first=True), ref, TOL_BF16, "packed lo_first zp3")


def _host_w4_prepack(Wq: np.ndarray, N: int, lo_first: bool) -> np.ndarray:
    """The documented int4 prepacked layout, built on the host from the unpacked codes: 128-column
    blocks, then 128-row groups, then the block's 16-column tiles (the last block holds the
    remaining tiles), each 64 lanes x 16 bytes; lane l, dword q holds the codes of column
    16 t + l % 16 at k = 128 g + 32 q + 8 (l // 16) + j, code j at bit 4 (j // 2) + 16 (j % 2)."""
    codes = oracle.w4_unpack(Wq, N, lo_first).astype(np.uint32)  # [K, N]
    K = codes.shape[0]
    ngroups, ntiles = K // 128, N // 16
    out = np.zeros(K * N // 2, np.uint8)
    lanes = np.arange(64)
    shifts = np.array([4 * (j // 2) + 16 * (j % 2) for j in range(8)], np.uint32)
    for t in range(ntiles):
        b, nb = t // 8, min(8, ntiles - 8 * (t // 8))
        for g in range(ngroups):
            frag = np.zeros((64, 4), np.uint32)
            for q in range(4):
                ks = 128 * g + 32 * q + 8 * (lanes // 16)[:, None] + np.arange(8)[None, :]  # [64, 8]
                c = codes[ks, (16 * t + lanes % 16)[:, None]]
                frag[:, q] = np.bitwise_or.reduce(c << shifts[None, :], axis=1)
            off = (b * ngroups * 8 + g * nb + t % 8) * 1024
            out[off:off + 1024] = frag.view(np.uint8).reshape(-1)
    return out


@pytest.mark.parametrize("N,K,lo_first", [(256, 256, False), (48, 384, True), (400, 128, False)])
def test_w4_prepack_layout_matches_the_documented_one(N, K, lo_first):
    # N = 48 and 400: a last block of three and of one 16-column tiles
    Wq = workloads.uniform_bytes((K, N // 2), wid=104, tid=N)
    got = ge.w4_prepack(torch.from_numpy(Wq).to(DEV), lo_first=lo_first).cpu().numpy()
    assert np.array_equal(got, _host_w4_prepack(Wq, N, lo_first))


@pytest.mark.parametrize("M", [16, 32])
def test_w4_prepacked_one_hot_rows_bit_exact(M):
    K, N = 1024, 512
    Wq = workloads.uniform_bytes((K, N // 2), wid=102, tid=1)
    scales = workloads.f32_to_bf16_bits(np.full((K // 128, N), 2.0 ** -6, np.float32))
    ks = np.arange(M) * 61 % K
    X = np.zeros((M, K), np.float32)
    X[np.arange(M), ks] = 1.0
    Wp = ge.w4_prepack(torch.from_numpy(Wq).to(DEV))
    out = to_host(ge.w4_gemm(to_dev(workloads.f32_to_bf16_bits(X)), Wp, to_dev(scales), prepacked=True))
    codes = oracle.w4_unpack(Wq, N).astype(np.int64)
    assert np.array_equal(out, (codes[ks] - 8) * 2.0 ** -6)


def test_w4_prepacked_rejected_by_unfused_chain():
    p = ge.plan(ge.KIND_W4, 16, 256, 256, b_type=ge.U4X2, prepacked=True)
    n = ge.ctypes.c_size_t()
    assert ge.lib().gemm_epi_unfused_workspace_bytes(p.handle, ge.ctypes.byref(n)) == 0
    with pytest.raises(ge.GemmEpiError):
        X = torch.zeros((16, 256), dtype=torch.bfloat16, device=DEV)
        ge.w4_gemm_unfused(X, torch.zeros(256 * 128, dtype=torch.uint8, device=DEV),
                           torch.zeros((2, 256), dtype=torch.bfloat16, device=DEV), prepacked=True)


@pytest.mark.parametrize("M,N,K", [(33, 128, 128), (128, 256, 512), (200, 384, 1024), (512, 512, 2048),
                                   (100, 32768, 256), (130, 22016, 384)])
def test_w4_prepacked_tile_path(M, N, K):
    w = workloads.WORKLOADS["w4a16_m512"].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M + N)
    p = ge.plan(ge.KIND_W4, M, N, K, b_type=ge.U4X2, bias=True, prepacked=True)
    # 8 waves and 256 columns per workgroup where those tiles fill the CUs, else 4 waves and 128,
    # split over K where the 64 x 128 tiles leave CUs idle and the groups allow
    assert p.kernel == w4_tile_kernel("u4", M, N, K)
    assert_close(_w4_packed(inp), oracle.reference(inp), TOL_BF16, f"w4 tile {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(200, 384, 1024), (512, 8192, 1024)])
def test_w4_tile_plan_scratch_and_repeats_bitwise(M, N, K):
    # the int4 tile kernel reads X directly (bf16) and keeps its per-group partial products and the
    # zero-point correction on chip; only the K split (12 tiles of 64 x 128 here) owns plan scratch:
    # partial tiles and per-tile counters that the kernel re-arms.  A second X on the same plan,
    # then the first again, bitwise as before (the slices are summed in a fixed order)
    w = workloads.WORKLOADS["w4a16_m512"].with_shape(M=M, N=N, K=K)
    p = ge.plan(ge.KIND_W4, M, N, K, b_type=ge.U4X2, bias=True, prepacked=True)
    assert p.kernel == w4_tile_kernel("u4", M, N, K)
    assert (p.scratch_bytes > 0) == ("split" in p.kernel)
    a, b = workloads.make_inputs(w, seed=31), workloads.make_inputs(w, seed=32)
    b["Wq"], b["scales"], b["bias"] = a["Wq"], a["scales"], a["bias"]
    oa = _w4_packed(a)
    ob = _w4_packed(b)
    assert_close(oa, oracle.reference(a), TOL_BF16, "first X")
    assert_close(ob, oracle.reference(b), TOL_BF16, "second X")
    assert torch.equal(_w4_packed(a).view(torch.int16), oa.view(torch.int16))


@pytest.mark.parametrize("M,N,K", [(33, 128, 128), (64, 256, 8576), (100, 128, 4224), (65, 384, 12288)])
def test_w4_tile_path_k_chunks(M, N, K):
    # the zero-point correction product runs once per 32 groups: one group; 67 groups (two full
    # chunks and a partial one, an odd group count); 33 groups; 96 groups
    w = workloads.WORKLOADS["w4a16_m512"].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M + K)
    assert ge.plan(ge.KIND_W4, M, N, K, b_type=ge.U4X2, bias=True, prepacked=True).kernel == w4_tile_kernel("u4", M, N, K)
    assert_close(_w4_packed(inp), oracle.reference(inp), TOL_BF16, f"w4 tile {M}x{N}x{K}")


@pytest.mark.parametrize("xmag,smag", [(1e5, 0.01), (3e4, 0.01), (1e-6, 0.01), (1.0, 3e4), (1.0, 1e-7),
                                       (1e-30, 1e20), (1e25, 1e-20)])
def test_w4_tile_path_any_finite_range(xmag, smag):
    # activations and scales far outside the fp16 range (or below its normal range): the tile
    # kernel works in bf16 with fp32 accumulation, so every finite input gives the oracle's result
    # within the bf16 tolerance; the sign pattern and magnitudes vary per element
    M, N, K = 96, 256, 1024
    w = workloads.WORKLOADS["w4a16_m512"].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=int(abs(np.log10(xmag * smag))) + 7)
    x = workloads.bf16_bits_to_f32(inp["X"]).astype(np.float64) * xmag
    sc = workloads.bf16_bits_to_f32(inp["scales"]).astype(np.float64) / 0.0125 * smag
    inp["X"] = workloads.f32_to_bf16_bits(x.astype(np.float32))
    inp["scales"] = workloads.f32_to_bf16_bits(sc.astype(np.float32))
    inp["bias"] = None
    ref = oracle.reference(inp)
    out = to_host(_w4_packed(inp))
    assert np.all(np.isfinite(out))
    scale = np.max(np.abs(ref))
    # compared on the scale of the result (bf16 tolerance relative to the largest output)
    assert np.max(np.abs(out - ref)) <= 1e-2 * scale, (np.max(np.abs(out - ref)), scale)
    assert_close(out / scale, ref / scale, TOL_BF16, f"x ~ {xmag}, s ~ {smag}")


@pytest.mark.parametrize("M", [33, 96, 130])
def test_w4_tile_path_one_hot_rows_bit_exact(M):
    # one-hot rows of X select single codes: (128 + c) * 2^-6 from the product, -(128 + 8) * 2^-6 from
    # the correction, both exact, so D = (c - 8) * 2^-6 exactly
    K, N = 1024, 256
    Wq = workloads.uniform_bytes((K, N // 2), wid=103, tid=1)
    scales = workloads.f32_to_bf16_bits(np.full((K // 128, N), 2.0 ** -6, np.float32))
    ks = np.arange(M) * 61 % K
    X = np.zeros((M, K), np.float32)
    X[np.arange(M), ks] = 1.0
    p = ge.plan(ge.KIND_W4, M, N, K, b_type=ge.U4X2, prepacked=True)
    assert p.kernel.startswith("tile_w4")
    Wp = ge.w4_prepack(torch.from_numpy(Wq).to(DEV))
    out = to_host(ge.w4_gemm(to_dev(workloads.f32_to_bf16_bits(X)), Wp, to_dev(scales), prepacked=True))
    codes = oracle.w4_unpack(Wq, N).astype(np.int64)
    assert np.array_equal(out, (codes[ks] - 8) * 2.0 ** -6)


def test_w4_prepacked_tile_one_hot_rows_bit_exact():
    K, N, M = 512, 256, 160
    Wq = workloads.uniform_bytes((K, N // 2), wid=103, tid=1)
    scales = workloads.f32_to_bf16_bits(np.full((K // 128, N), 2.0 ** -6, np.float32))
    ks = np.arange(M) * 37 % K
    X = np.zeros((M, K), np.float32)
    X[np.arange(M), ks] = 1.0
    Wp = ge.w4_prepack(torch.from_numpy(Wq).to(DEV))
    out = to_host(ge.w4_gemm(to_dev(workloads.f32_to_bf16_bits(X)), Wp, to_dev(scales), prepacked=True))
    codes = oracle.w4_unpack(Wq, N).astype(np.int64)
    assert np.array_equal(out, (codes[ks] - 8) * 2.0 ** -6)


def test_w4_prepacked_tile_needs_group_128():
    with pytest.raises(ge.GemmEpiError):
        ge.plan(ge.KIND_W4, 64, 256, 512, b_type=ge.U4X2, group=64, prepacked=True)
