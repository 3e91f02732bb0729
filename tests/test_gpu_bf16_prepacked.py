"""GPU parity of the prepacked bf16 decode path (M <= 16): gemm_b_prepack's
layout against a host rearrangement of the same bytes, the fused kernel
against the oracle on ragged shapes with every epilogue term, bit-exact
one-hot rows, and the requests the path must refuse."""
import dataclasses

import numpy as np
import pytest
import torch

import gemm_epilogue_tile_amd as ge
import oracle
import workloads
from gpu_helpers import DEV, TOL_BF16, assert_close, dev_inputs, to_dev, to_host

pytestmark = pytest.mark.gpu

DEC = workloads.WORKLOADS["skinny_decode"]


def _block_tiles(N: int) -> int:
    """Tiles per column block the header documents: 7 where N / 112 is a multiple of the CU count
    and N / 128 is not, else 8."""
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    even112 = N % 112 == 0 and (N // 112) % cu == 0
    even128 = N % 128 == 0 and (N // 128) % cu == 0
    return 7 if even112 and not even128 else 8


def _host_prepack(B: np.ndarray) -> np.ndarray:
    """The layout gemm_epi.h documents, written with numpy: piece (cb, kb), tile t, lane l holds
    column 16 T cb + 16 t + l % 16 at k = 32 kb + 8 (l // 16) + j, j = 0..7 (T tiles per block)."""
    K, N = B.shape
    T = _block_tiles(N)
    v = B.reshape(K // 32, 4, 8, N // (16 * T), T, 16)     # kb, l//16, j, cb, t, l%16
    v = v.transpose(3, 0, 4, 1, 5, 2)                       # cb, kb, t, l//16, l%16, j
    return np.ascontiguousarray(v).reshape(K, N)


def _prepacked(inp, **kw):
    d = dev_inputs(inp)
    Bp = ge.b_prepack(d["B"])
    return ge.gemm_epilogue(d["A"], Bp, bias=d.get("bias"), C=d.get("C"), R=d.get("R"), alpha=inp["alpha"],
                            beta=inp["beta"], act=kw.pop("act", inp["act"]), prepacked=True, **kw)


@pytest.mark.parametrize("K,N", [(32, 128), (96, 256), (1024, 384), (64, 28672)])
def test_prepack_layout_matches_the_documented_one(K, N):
    # N = 28672 on 256 CUs: 112-column blocks (256 of them, against 224 of 128 columns)
    B = workloads.f32_to_bf16_bits(np.random.default_rng(K + N).standard_normal((K, N)).astype(np.float32))
    got = ge.b_prepack(to_dev(B)).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, _host_prepack(B))


def test_prepack_reads_a_strided_source():
    K, N, ldb = 64, 256, 264
    full = workloads.f32_to_bf16_bits(np.random.default_rng(3).standard_normal((K, ldb)).astype(np.float32))
    src = to_dev(full)[:, :N]
    got = ge.b_prepack(src).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, _host_prepack(np.ascontiguousarray(full[:, :N])))


@pytest.mark.parametrize("M,N,K", [(1, 128, 32), (7, 256, 96), (16, 384, 1056), (13, 1024, 8192),
                                   (16, 2048, 4096), (17, 384, 1056), (29, 1024, 8192), (32, 28672, 512),
                                   (16, 28672, 512), (5, 28672, 96)])
def test_prepacked_decode_ragged(M, N, K):
    # M <= 16: one 16-row tile of X per weight fragment; 17 <= M <= 32: two
    w = DEC.with_shape(M=M, N=N, K=K)
    inp = workloads.make_inputs(w, seed=M + N + K)
    p = ge.plan(ge.KIND_GENERIC, M, N, K, bias=True, R=True, b_prepacked=True)
    cols = 16 * _block_tiles(N)
    want = f"skinny_bf16_m16_{cols}col_prepacked" if M <= 16 else f"skinny_bf16_m32_{cols}col_prepacked"
    assert p.kernel == want and p.scratch_bytes == 0
    assert_close(_prepacked(inp), oracle.reference(inp), TOL_BF16, f"prepacked {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(16, 12288, 8192), (16, 8192, 2048), (9, 5120, 4096), (3, 14336, 1024)])
def test_prepacked_streamk_ranges_across_column_blocks(M, N, K):
    # few column blocks (at most half the CU count): the (block, 32-row block) pieces are dealt
    # to one workgroup per CU in equal contiguous ranges, which straddle blocks in all but the
    # second shape; partial tiles meet in the plan's scratch.  Two calls on one plan: the arrival
    # counters must re-arm themselves.
    w = DEC.with_shape(M=M, N=N, K=K)
    p = ge.plan(ge.KIND_GENERIC, M, N, K, bias=True, R=True, b_prepacked=True)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    if 2 * (N // 128) <= ncu:
        assert p.kernel == "skinny_bf16_m16_prepacked_streamk" and p.scratch_bytes > 0
    for seed in (1, 2):
        inp = workloads.make_inputs(w, seed=seed + N)
        assert_close(_prepacked(inp), oracle.reference(inp), TOL_BF16, f"prepacked stream-K {M}x{N}x{K} #{seed}")


@pytest.mark.parametrize("act", ["none", "relu", "gelu_tanh", "silu"])
def test_prepacked_every_epilogue_term(act):
    w = dataclasses.replace(DEC, M=16, N=256, K=512, alpha=0.75, beta=-0.5, act=act, bias=True, C=True, R=True)
    inp = workloads.make_inputs(w, seed=11)
    assert_close(_prepacked(inp), oracle.reference(inp), TOL_BF16, f"prepacked {act} b/c/r")


def test_prepacked_fp32_output():
    w = DEC.with_shape(M=5, N=256, K=256)
    inp = workloads.make_inputs(w, seed=4)
    d = dev_inputs(inp)
    out = ge.gemm_epilogue(d["A"], ge.b_prepack(d["B"]), prepacked=True, out_dtype=torch.float32)
    ref = oracle.gemm(inp["A"], inp["B"], "bf16", "bf16")
    assert_close(out, ref, 1e-4, "prepacked fp32 out")


def test_prepacked_one_hot_rows_bit_exact():
    # row m of X selects weight row k_m: D = B[k_m, :] exactly (one product per sum), so a
    # misplaced column, k or lane in the layout shows up as a wrong value
    M, N, K = 16, 512, 1024
    B = workloads.f32_to_bf16_bits(np.random.default_rng(9).standard_normal((K, N)).astype(np.float32))
    ks = np.arange(M) * 67 % K
    X = np.zeros((M, K), np.float32)
    X[np.arange(M), ks] = 1.0
    out = to_host(ge.gemm_epilogue(to_dev(workloads.f32_to_bf16_bits(X)), ge.b_prepack(to_dev(B)), prepacked=True))
    assert np.array_equal(out, workloads.bf16_bits_to_f32(B[ks]).astype(np.float64))


def test_prepacked_matches_the_raw_layout_path():
    w = DEC.with_shape(M=16, N=1024, K=2048)
    inp = workloads.make_inputs(w, seed=21)
    d = dev_inputs(inp)
    raw = to_host(ge.gemm_epilogue(d["A"], d["B"], bias=d["bias"], R=d["R"]))
    packed = to_host(_prepacked(inp))
    assert np.max(np.abs(raw - packed) / (1 + np.abs(raw))) <= TOL_BF16


@pytest.mark.parametrize("M,N,K", [(33, 128, 64), (16, 200, 64), (16, 128, 48)])
def test_prepacked_plan_refuses_shapes_outside_the_layout(M, N, K):
    with pytest.raises(ge.GemmEpiError) as ei:
        ge.plan(ge.KIND_GENERIC, M, N, K, b_prepacked=True)
    assert ei.value.status == ge.ERR_UNSUPPORTED


def test_prepacked_rejected_by_the_unfused_chain_and_other_kinds():
    X = torch.zeros((16, 256), dtype=torch.bfloat16, device=DEV)
    Bp = ge.b_prepack(torch.zeros((256, 256), dtype=torch.bfloat16, device=DEV))
    p = ge.plan(ge.KIND_GENERIC, 16, 256, 256, b_prepacked=True)
    out = torch.empty((16, 256), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    st = ge.lib().gemm_epi_run_unfused(p.handle, ge._ptr(X), ge._ptr(Bp), None, None, None, ge._ptr(out),
                                       ge._ptr(ws), None)
    assert st == ge.ERR_UNSUPPORTED
    with pytest.raises(ge.GemmEpiError):
        ge.plan(ge.KIND_W4, 16, 256, 256, b_type=ge.U4X2, b_prepacked=True)
    with pytest.raises(ge.GemmEpiError):
        ge.b_prepack(torch.zeros((48, 256), dtype=torch.bfloat16, device=DEV))
