"""GPU parity of the 8-bit weight formats (unsigned codes with a zero point,
OCP fp8 E4M3) against the oracle: the streaming kernel (M <= 16), the general
kernel (larger M, ragged N), every group size and epilogue term, bit-exact
decoding through one-hot activation rows, the dequantisation kernel, and the
unfused chain."""
import dataclasses

import numpy as np
import pytest
import torch

import gemm_epilogue_tile_amd as ge
import oracle
import workloads
from gpu_helpers import DEV, TOL_BF16, assert_close, dev_inputs, to_dev, to_host, w4_tile_cols, w4_tile_kernel

pytestmark = pytest.mark.gpu

BASE = {"u8": workloads.WORKLOADS["w8a16_u8_m16"], "fp8": workloads.WORKLOADS["w8a16_fp8_m16"]}
FMTS = ["u8", "fp8"]


def _w8(inp, **kw):
    d = dev_inputs(inp)
    return ge.w4_gemm(d["X"], torch.from_numpy(inp["Wq"]).to(DEV), d["scales"], bias=d.get("bias"),
                      C=d.get("C"), R=d.get("R"), alpha=inp["alpha"], beta=inp["beta"], act=inp["act"],
                      group=inp["group"], zero_point=inp["zero_point"], fmt=inp["fmt"], **kw)


def _plan_kernel(fmt, M, N, K, **kw):
    return ge.plan(ge.KIND_W4, M, N, K, b_type=ge.WEIGHT_FORMATS[fmt], bias=True,
                   zero_point=128 if fmt == "u8" else 0, **kw).kernel


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(1, 8, 128), (16, 256, 512), (16, 1000, 1024), (7, 4104, 2048),
                                   (16, 8192, 1024), (3, 13, 128), (33, 264, 384), (128, 512, 1024),
                                   (200, 136, 640)])
def test_w8_ragged(fmt, M, N, K):
    w = BASE[fmt].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M + N + K)
    assert_close(_w8(inp), oracle.reference(inp), TOL_BF16, f"{fmt} {M}x{N}x{K}")


def test_w8_plans_pick_the_streaming_kernel_for_small_M():
    assert _plan_kernel("u8", 16, 8192, 8192).startswith("skinny_u8_m16_128col")
    assert _plan_kernel("fp8", 1, 4096, 1024).startswith("skinny_fp8_m16_128col")
    assert not _plan_kernel("u8", 17, 8192, 8192).startswith("skinny")
    assert not _plan_kernel("fp8", 16, 13, 128).startswith("skinny")  # N % 8 != 0


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(17, 128, 128), (64, 256, 1024), (100, 384, 4224), (512, 1024, 2048)])
def test_w8_tile_kernel(fmt, M, N, K):
    # M > 16 with N % 128 == 0, K % 128 == 0 and 128-row groups: the tile kernel on raw codes (4 waves,
    # 128 columns per workgroup at these sizes, split over K where the groups allow); K = 4224 is 33
    # groups, not a whole number of the kernel's two-group loop trips
    w = BASE[fmt].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=3 * M + K)
    assert _plan_kernel(fmt, M, N, K) == w4_tile_kernel(fmt, M, N, K)
    assert_close(_w8(inp), oracle.reference(inp), TOL_BF16, f"{fmt} tile {M}x{N}x{K}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(100, 32768, 256), (130, 22016, 384)])
def test_w8_tile_kernel_eight_waves(fmt, M, N, K):
    # enough 64 x 256 tiles for every CU: the 8-wave workgroups, ragged M (two and three row tiles)
    w = BASE[fmt].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M + K)
    assert _plan_kernel(fmt, M, N, K) == w4_tile_kernel(fmt, M, N, K) == f"tile_w8_{fmt}_64x{w4_tile_cols(M, N)}x32"
    assert_close(_w8(inp), oracle.reference(inp), TOL_BF16, f"{fmt} 8-wave tile {M}x{N}x{K}")


@pytest.mark.parametrize("zp", [0, 77, 255])
def test_w8_tile_u8_zero_points(zp):
    w = dataclasses.replace(BASE["u8"], M=96, N=256, K=1024, zero_point=zp)
    inp = workloads.make_inputs(w, seed=zp)
    assert_close(_w8(inp), oracle.reference(inp), TOL_BF16, f"u8 tile zero point {zp}")


@pytest.mark.parametrize("fmt", FMTS)
def test_w8_tile_strided_operands(fmt):
    # X with a row stride of K + 8 elements, codes with a row stride of N + 16 bytes
    M, N, K = 80, 256, 512
    w = BASE[fmt].with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=11)
    d = dev_inputs(inp)
    Xf = torch.zeros((M, K + 8), dtype=torch.bfloat16, device=DEV)
    Xf[:, :K] = d["X"]
    Wf = torch.zeros((K, N + 16), dtype=torch.uint8, device=DEV)
    Wf[:, :N] = torch.from_numpy(inp["Wq"]).to(DEV)
    out = ge.w4_gemm(Xf[:, :K], Wf[:, :N], d["scales"], bias=d.get("bias"), group=inp["group"],
                     zero_point=inp["zero_point"], fmt=fmt)
    assert _plan_kernel(fmt, M, N, K, lda=K + 8, ldb=N + 16) == w4_tile_kernel(fmt, M, N, K)
    assert_close(out, oracle.reference(inp), TOL_BF16, f"{fmt} tile strided")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [16, 40])
@pytest.mark.parametrize("group", [32, 64, 128, 256])
def test_w8_group_sizes(fmt, M, group):
    w = dataclasses.replace(BASE[fmt], M=M, N=384, K=1024, group=group)
    inp = workloads.make_inputs(w, seed=group + M)
    assert_close(_w8(inp), oracle.reference(inp), TOL_BF16, f"{fmt} M{M} group {group}")


@pytest.mark.parametrize("M", [16, 40])
@pytest.mark.parametrize("zp", [0, 77, 255])
def test_u8_zero_points(M, zp):
    w = dataclasses.replace(BASE["u8"], M=M, N=256, K=512, zero_point=zp)
    inp = workloads.make_inputs(w, seed=zp)
    assert_close(_w8(inp), oracle.reference(inp), TOL_BF16, f"u8 M{M} zp {zp}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [9, 64])
@pytest.mark.parametrize("act", ["relu", "gelu_tanh", "silu"])
def test_w8_every_epilogue_term(fmt, M, act):
    w = dataclasses.replace(BASE[fmt], M=M, N=520, K=256, alpha=0.75, beta=-0.5, act=act, C=True, R=True)
    inp = workloads.make_inputs(w, seed=M)
    assert_close(_w8(inp), oracle.reference(inp), TOL_BF16, f"{fmt} M{M} {act}")


def _non_nan_codes(shape, wid):
    q = workloads.uniform_bytes(shape, wid=wid, tid=1)
    q[(q & 0x7F) == 0x7F] = 0  # E4M3 has NaN at S.1111.111 only; every other code is finite
    return q


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [16, 48, 130])
def test_w8_decode_bit_exact_with_one_hot_rows(fmt, M):
    # X row m is one-hot at k_m and scales are 2^-6, so D[m][n] = value(code) * 2^-6 exactly:
    # at most 9 significant bits for u8, 4 for fp8 (subnormals and 448 included)
    K, N, zp = 1024, 512, (128 if fmt == "u8" else 0)
    Wq = _non_nan_codes((K, N), 97) if fmt == "fp8" else workloads.uniform_bytes((K, N), wid=97, tid=1)
    scales = workloads.f32_to_bf16_bits(np.full((K // 128, N), 2.0 ** -6, np.float32))
    ks = np.arange(M) * 37 % K
    X = np.zeros((M, K), np.float32)
    X[np.arange(M), ks] = 1.0
    out = to_host(ge.w4_gemm(to_dev(workloads.f32_to_bf16_bits(X)), torch.from_numpy(Wq).to(DEV),
                             to_dev(scales), zero_point=zp, fmt=fmt))
    ones = workloads.f32_to_bf16_bits(np.ones((K // 128, N), np.float32))
    want = oracle.w8_dequant(Wq, ones, fmt, zero_point=zp)[ks] * 2.0 ** -6
    assert np.array_equal(out, want)


@pytest.mark.parametrize("fmt", FMTS)
def test_w8_dequant_kernel_bit_exact(fmt):
    K, N = 512, 392
    w = dataclasses.replace(BASE[fmt], M=1, N=N, K=K, group=64)
    inp = workloads.make_inputs(w, seed=11)
    W = ge.w4_dequant(torch.from_numpy(inp["Wq"]).to(DEV), to_dev(inp["scales"]), group=64,
                      zero_point=inp["zero_point"], fmt=fmt)
    # code values carry <= 9 significant bits and scales 8: every product is exact in fp32
    exact = oracle.w8_dequant(inp["Wq"], inp["scales"], fmt, group=64, zero_point=inp["zero_point"])
    want = workloads.f32_to_bf16_bits(exact.astype(np.float32))
    got = W.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [16, 96])
def test_unfused_w8_matches_oracle(fmt, M):
    w = BASE[fmt].with_shape(M=M, N=512, K=1024)
    inp = workloads.make_inputs(w, seed=15)
    d = dev_inputs(inp)
    out = to_host(ge.w4_gemm_unfused(d["X"], torch.from_numpy(inp["Wq"]).to(DEV), d["scales"],
                                     bias=d["bias"], zero_point=inp["zero_point"], fmt=fmt))
    ref = oracle.reference(inp)
    # the chain rounds every dequantised weight to bf16: random error per product <= 2^-9 |x w|
    X = workloads.bf16_bits_to_f32(inp["X"]).astype(np.float64)
    W = oracle.w8_dequant(inp["Wq"], inp["scales"], fmt, zero_point=inp["zero_point"])
    spread = np.sqrt((X ** 2) @ (W ** 2))
    tol = TOL_BF16 * (1 + np.abs(ref)) + 6 * 2.0 ** -9 * spread / np.sqrt(3) + 2 * 2.0 ** -9 * np.abs(ref)
    assert np.all(np.abs(out - ref) <= tol)


def test_w8_strided_and_misaligned_weights_take_the_general_kernel():
    # ldb > N and a weight pointer off the 8-byte grid: same values as the packed call
    w = BASE["u8"].with_shape(M=16, N=256, K=512)
    inp = workloads.make_inputs(w, seed=21)
    d = dev_inputs(inp)
    Wq = torch.from_numpy(inp["Wq"]).to(DEV)
    big = torch.zeros((512, 256 + 40), dtype=torch.uint8, device=DEV)
    big[:, 3:259] = Wq
    out = ge.w4_gemm(d["X"], big[:, 3:259], d["scales"], bias=d["bias"], zero_point=128, fmt="u8")
    assert_close(out, oracle.reference(inp), TOL_BF16, "u8 strided misaligned")


def test_w8_split_plans_own_scratch():
    # 64 column blocks of 128 do not fill 256 CUs: K is split 4 ways, with
    # 4 x 64 fp32 tiles of 16 x 128 and 64 counters of scratch
    p = ge.plan(ge.KIND_W4, 16, 8192, 8192, b_type=ge.U8, bias=True, zero_point=128)
    assert p.kernel == "skinny_u8_m16_128col_split4"
    assert p.scratch_bytes == 4 * 64 * 16 * 128 * 4 + 64 * 4
    q = ge.plan(ge.KIND_W4, 16, 28672, 8192, b_type=ge.FP8E4M3, bias=True, zero_point=0)
    assert q.kernel == "skinny_fp8_m16_128col_split2"
    # 40 rows take the tile kernel: 64 tiles of 64 x 128 split 4 ways over K, 4 x 64 partial tiles of
    # 4 waves x 8 fragments of 1 KiB and 64 counters
    r = ge.plan(ge.KIND_W4, 40, 8192, 8192, b_type=ge.U8, bias=True, zero_point=128)
    assert r.kernel == w4_tile_kernel("u8", 40, 8192, 8192)
    if r.kernel.endswith("split4"):
        assert r.scratch_bytes == 4 * 64 * 4 * 8 * 1024 + 64 * 4


@pytest.mark.parametrize("fmt", FMTS)
def test_w8_split_repeat_calls_are_bitwise_identical(fmt):
    # the split counters re-arm themselves: repeated and interleaved calls on
    # one plan give the same bits, and each matches the oracle
    w = BASE[fmt].with_shape(M=16, N=4096, K=4096)
    outs = []
    for seed in (1, 2, 1, 2, 1):
        inp = workloads.make_inputs(w, seed=seed)
        o = _w8(inp)
        if seed == 1 and not outs:
            assert_close(o, oracle.reference(inp), TOL_BF16, f"{fmt} split seed 1")
        outs.append((seed, o.view(torch.int16).clone()))
    assert ge.plan(ge.KIND_W4, 16, 4096, 4096, b_type=ge.WEIGHT_FORMATS[fmt], bias=True,
                   zero_point=128 if fmt == "u8" else 0).kernel.endswith("_split4")
    ref = {s: o for s, o in outs[:2]}
    for s, o in outs[2:]:
        assert torch.equal(o, ref[s])


@pytest.mark.parametrize("fmt", FMTS)
def test_w8_split_handoff_is_stable_over_many_calls(fmt):
    # 300 back-to-back calls through the cross-workgroup handoff (device-scope loads and stores,
    # counters re-armed by the last workgroup): every output bitwise equal to the first
    w = BASE[fmt]
    inp = workloads.make_inputs(w, seed=3)
    d = dev_inputs(inp)
    Wq = torch.from_numpy(inp["Wq"]).to(DEV)
    outs = [torch.empty(w.M, w.N, dtype=torch.bfloat16, device=DEV) for _ in range(300)]
    f = [ge.prepare_w4_gemm(d["X"], Wq, d["scales"], bias=d["bias"], out=o, zero_point=w.zero_point, fmt=fmt)
         for o in outs]
    assert f[0]._plan.kernel.endswith("_split4")
    for g in f:
        g()
    torch.cuda.synchronize()
    first = outs[0].view(torch.int16)
    bad = [i for i, o in enumerate(outs) if not torch.equal(o.view(torch.int16), first)]
    assert not bad, f"calls {bad[:10]} differ from the first"



# ---------------------------------------------------------------------------
# prepacked 8-bit codes (gemm_w4_prepack on an 8-bit plan)
# ---------------------------------------------------------------------------

def _host_prepack8(Wq: np.ndarray) -> np.ndarray:
    """The documented layout, with numpy: block (cb, kb), load q, lane l holds rows 32 kb + 8 (l // 16)
    + 2q and + 2q + 1 (8 bytes each), columns 128 cb + 8 (l % 16) .. + 7."""
    K, N = Wq.shape
    v = Wq.reshape(K // 32, 4, 4, 2, N // 128, 16, 8)  # kb, l//16, q, r%2, cb, l%16, byte
    return np.ascontiguousarray(v.transpose(4, 0, 2, 1, 5, 3, 6)).reshape(-1)  # cb, kb, q, l//16, l%16, r%2, byte


def _w8_packed(inp, **kw):
    d = dev_inputs(inp)
    Wp = ge.w4_prepack(torch.from_numpy(inp["Wq"]).to(DEV), fmt=inp["fmt"])
    return ge.w4_gemm(d["X"], Wp, d["scales"], bias=d.get("bias"), C=d.get("C"), R=d.get("R"), alpha=inp["alpha"],
                      beta=inp["beta"], act=inp["act"], group=inp["group"], zero_point=inp["zero_point"],
                      fmt=inp["fmt"], prepacked=True, **kw)


@pytest.mark.parametrize("fmt", FMTS)
def test_w8_prepack_layout_matches_the_documented_one(fmt):
    K, N = 96, 384
    Wq = workloads.uniform_bytes((K, N), wid=95, tid=1)
    got = ge.w4_prepack(torch.from_numpy(Wq).to(DEV), fmt=fmt).cpu().numpy()
    assert np.array_equal(got, _host_prepack8(Wq))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K,group", [(16, 8192, 4096, 128), (1, 128, 32, 32), (7, 1024, 2048, 64),
                                         (16, 2048, 8192, 256), (13, 384, 1024, 32)])
def test_w8_prepacked_matches_the_oracle(fmt, M, N, K, group):
    w = dataclasses.replace(BASE[fmt], M=M, N=N, K=K, group=group)
    inp = workloads.make_inputs(w, seed=M + N + group)
    p = ge.plan(ge.KIND_W4, M, N, K, b_type=ge.WEIGHT_FORMATS[fmt], bias=True, group=group,
                zero_point=inp["zero_point"], prepacked=True)
    assert p.kernel.startswith(f"skinny_{fmt}_m16_128col")
    for seed in (0, 1):  # two calls on one plan: the split counters re-arm themselves
        if seed:
            inp = workloads.make_inputs(w, seed=M + N + group + 100)
        assert_close(_w8_packed(inp), oracle.reference(inp), TOL_BF16, f"{fmt} packed {M}x{N}x{K} g{group} #{seed}")


@pytest.mark.parametrize("fmt", FMTS)
def test_w8_prepacked_every_epilogue_term(fmt):
    w = dataclasses.replace(BASE[fmt], M=16, N=256, K=512, alpha=0.5, beta=-1.0, act="gelu_tanh", bias=True,
                            C=True, R=True)
    inp = workloads.make_inputs(w, seed=17)
    assert_close(_w8_packed(inp), oracle.reference(inp), TOL_BF16, f"{fmt} packed b/c/r gelu")


@pytest.mark.parametrize("fmt", FMTS)
def test_w8_prepacked_refusals(fmt):
    bt = ge.WEIGHT_FORMATS[fmt]
    zp = 128 if fmt == "u8" else 0
    for M, N, K in [(17, 256, 256), (16, 200, 256), (16, 256, 48)]:
        with pytest.raises(ge.GemmEpiError):
            ge.plan(ge.KIND_W4, M, N, K, b_type=bt, zero_point=zp, group=16 if K == 48 else 128, prepacked=True)
    with pytest.raises(ge.GemmEpiError):
        ge.w4_prepack(torch.zeros((64, 200), dtype=torch.uint8, device=DEV), fmt=fmt)
