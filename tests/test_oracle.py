"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties one pass of the oracle to something it cannot agree with by
construction: exact rational arithmetic, hand-worked fixtures, closed-form
identities, or an independent library routine (numpy BLAS, scipy, math.erf).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

import oracle
import workloads
from conftest import GOLDEN

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _bf16_values(bits):
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


# --------------------------------------------------------------------------
# GEMM pass
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (8, 8, 8), (2, 9, 4), (7, 1, 9)])
def test_gemm_exact_integers_match_rational_sum(M, N, K):
    rng = np.random.default_rng([11, M, N, K])
    A = rng.integers(-16, 17, size=(M, K)).astype(np.float32)
    B = rng.integers(-16, 17, size=(K, N)).astype(np.float32)
    got = oracle.gemm(A, B, "f32", "f32")
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(int(A[m, k])) * Fraction(int(B[k, n])) for k in range(K))
            assert got[m, n] == float(exact)


@pytest.mark.parametrize("M,N,K", [(4, 3, 16), (5, 6, 33)])
def test_gemm_bf16_values_within_fp64_bound_of_exact(M, N, K):
    A = workloads.normal((M, K), 1.0, "bf16", wid=90, tid=0)
    B = workloads.normal((K, N), 0.3, "bf16", wid=90, tid=1)
    got = oracle.gemm(A, B, "bf16", "bf16")
    Av, Bv = _bf16_values(A), _bf16_values(B)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(Av[m, k])) * Fraction(float(Bv[k, n])) for k in range(K))
            mag = sum(abs(float(Av[m, k]) * float(Bv[k, n])) for k in range(K))
            # recursive summation in fp64: |err| <= K * 2^-53 * sum |a_k b_k| (first order)
            assert abs(got[m, n] - float(exact)) <= K * 2.0 ** -53 * mag * 1.01 + 1e-300


@pytest.mark.parametrize("M,N,K", [(37, 53, 129), (64, 64, 128), (1, 300, 17)])
def test_gemm_matches_numpy_blas(M, N, K):
    A = workloads.uniform((M, K), -1, 1, "f32", wid=91, tid=0)
    B = workloads.uniform((K, N), -1, 1, "f32", wid=91, tid=1)
    got = oracle.gemm(A, B, "f32", "f32")
    ref = A.astype(np.float64) @ B.astype(np.float64)
    assert np.max(np.abs(got - ref)) <= 1e-12 * (1 + np.max(np.abs(ref)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_B_returns_A_bitwise(dtype):
    K = 48
    A = workloads.normal((13, K), 1.0, dtype, wid=92, tid=0)
    eye = np.eye(K, dtype=np.float32)
    I = eye if dtype == "f32" else workloads.f32_to_bf16_bits(eye)
    got = oracle.gemm_epilogue(A, I, dtype)
    Av = A.astype(np.float64) if dtype == "f32" else _bf16_values(A)
    assert np.array_equal(got, Av)
    got_nk = oracle.gemm_epilogue(A, I, dtype, b_layout="NK")
    assert np.array_equal(got_nk, Av)


def test_nk_layout_equals_kn_bitwise():
    A = workloads.normal((9, 40), 1.0, "bf16", wid=93, tid=0)
    B = workloads.normal((40, 11), 1.0, "bf16", wid=93, tid=1)
    kn = oracle.gemm(A, B, "bf16", "bf16", "KN")
    nk = oracle.gemm(A, np.ascontiguousarray(B.T), "bf16", "bf16", "NK")
    assert np.array_equal(kn, nk)


# --------------------------------------------------------------------------
# epilogue passes against hand-worked cases
# --------------------------------------------------------------------------

def _floats(s):
    s = s.strip()
    return None if s == "-" else np.array([float(v) for v in s.split()], dtype=np.float32)


def _golden_cases(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([p.strip() for p in line.split("|")])
    return rows


@pytest.mark.parametrize("row", _golden_cases("epilogue_worked.txt"), ids=lambda r: r[0])
def test_epilogue_worked_examples(row):
    name, dims, A, B, ab, C, bias, act, R, D = row
    M, N, K = (int(v) for v in dims.split())
    alpha, beta = (float(v) for v in ab.split())
    A = _floats(A).reshape(M, K)
    B = _floats(B).reshape(K, N)
    C = _floats(C)
    R = _floats(R)
    got = oracle.gemm_epilogue(A, B, "f32", alpha=alpha, beta=beta,
                               C=None if C is None else C.reshape(M, N), bias=_floats(bias),
                               act=act, R=None if R is None else R.reshape(M, N))
    assert np.array_equal(got, _floats(D).astype(np.float64).reshape(M, N))


def test_beta_zero_never_reads_C():
    A = np.ones((2, 3), np.float32)
    B = np.ones((3, 2), np.float32)
    got = oracle.gemm_epilogue(A, B, "f32", beta=0.0, C=np.full((2, 2), np.nan, np.float32))
    assert np.array_equal(got, np.full((2, 2), 3.0))


def test_zero_A_reduces_to_epilogue_of_C_bias_R():
    # A = 0: D = act(beta*C + bias) + R for any B
    M, N, K = 5, 7, 9
    A = np.zeros((M, K), np.float32)
    B = workloads.uniform((K, N), -1, 1, "f32", wid=94, tid=1)
    C = np.arange(M * N, dtype=np.float32).reshape(M, N) - 17.0
    bias = np.linspace(-4, 4, N).astype(np.float32)
    R = np.full((M, N), 0.25, np.float32)
    got = oracle.gemm_epilogue(A, B, "f32", alpha=3.0, beta=0.5, C=C, bias=bias, act="relu", R=R)
    want = np.maximum(0.5 * C.astype(np.float64) + bias.astype(np.float64), 0.0) + 0.25
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# activations
# --------------------------------------------------------------------------

def test_relu_is_exact():
    x = np.array([-3.5, -0.0, 0.0, 1e-300, 2.25, -1e300], np.float64)
    got = oracle.activation(x, "relu")
    assert list(got) == [0.0, 0.0, 0.0, 1e-300, 2.25, 0.0]


def test_gelu_tanh_tracks_exact_gelu_within_published_error():
    # The tanh form approximates x * Phi(x); its largest deviation is about 4.7e-4
    # (near |x| = 2.7).  A wrong constant (e.g. 0.04715 or 0.79) pushes it past 1e-3.
    x = np.linspace(-10, 10, 400001)
    got = oracle.activation(x, "gelu_tanh")
    exact = np.array([v * 0.5 * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x[::50]])
    dev = np.abs(got[::50] - exact)
    assert dev.max() <= 5.0e-4
    assert dev.max() >= 4.0e-4  # the approximation is not the exact function


def test_gelu_tanh_identities():
    x = np.linspace(-6, 6, 1201)
    f = oracle.activation(x, "gelu_tanh")
    fm = oracle.activation(-x, "gelu_tanh")
    assert np.max(np.abs((f - fm) - x)) <= 1e-14 * (1 + np.abs(x)).max()
    assert oracle.activation(np.array([0.0]), "gelu_tanh")[0] == 0.0
    big = oracle.activation(np.array([12.0, -12.0]), "gelu_tanh")
    assert big[0] == 12.0 and abs(big[1]) < 1e-300 + 1e-30
    # slope 1/2 at the origin, curvature sqrt(2/pi)
    h = 1e-4
    f_h = oracle.activation(np.array([h, -h]), "gelu_tanh")
    assert abs((f_h[0] - f_h[1]) / (2 * h) - 0.5) < 1e-9
    assert abs((f_h[0] + f_h[1]) / h ** 2 - math.sqrt(2 / math.pi)) < 1e-5


def test_silu_matches_scipy_expit_and_identities():
    x = np.linspace(-30, 30, 6001)
    got = oracle.activation(x, "silu")
    ref = x * expit(x)
    assert np.max(np.abs(got - ref) / (1 + np.abs(ref))) <= 4e-16
    neg = oracle.activation(-x, "silu")
    assert np.max(np.abs((got - neg) - x)) <= 1e-14 * 31
    assert oracle.activation(np.array([0.0]), "silu")[0] == 0.0


# --------------------------------------------------------------------------
# SwiGLU
# --------------------------------------------------------------------------

def test_swiglu_worked_example():
    (row,) = _golden_cases("swiglu_worked.txt")
    X, Wg, Wu, out = (_floats(p).reshape(2, 2) for p in row)
    got = oracle.swiglu(X, Wg, Wu, "f32")
    assert np.max(np.abs(got - out.astype(np.float64))) <= 1e-6
    # the fixture's values carry 16 digits; recheck them against scipy directly
    assert np.max(np.abs(got - Wg * expit(Wg.astype(np.float64)) * Wu)) <= 1e-15 * 6


# --------------------------------------------------------------------------
# int4 unpack + dequant
# --------------------------------------------------------------------------

def _w4_fixture():
    rows = []
    with open(os.path.join(GOLDEN, "w4_unpack.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                b, ce, co, we, wo = line.split()
                rows.append((int(b, 16), int(ce), int(co), float(we), float(wo)))
    return rows


def test_w4_unpack_and_dequant_hand_computed():
    rows = _w4_fixture()
    Wq = np.array([[r[0] for r in rows]], dtype=np.uint8)  # K = 1 row, N = 2 * len
    N = 2 * len(rows)
    codes = oracle.w4_unpack(Wq, N)
    assert list(codes[0, 0::2]) == [r[1] for r in rows]
    assert list(codes[0, 1::2]) == [r[2] for r in rows]
    # K = 128 rows (one group), scale 2^-4 everywhere
    Wq128 = np.repeat(Wq, 128, axis=0)
    scales = np.full((1, N), 0.0625, np.float64)
    W = oracle.w4_dequant(Wq128, scales, N, s_dtype="f64")
    assert list(W[0, 0::2]) == [r[3] for r in rows]
    assert list(W[0, 1::2]) == [r[4] for r in rows]
    assert np.array_equal(W, np.repeat(W[:1], 128, axis=0))


def test_w4_lo_first_swaps_nibbles():
    Wq = np.array([[0x8F, 0x07]], np.uint8)
    assert list(oracle.w4_unpack(Wq, 4, lo_first=True)[0]) == [15, 8, 7, 0]


def test_w4_scale_groups_broadcast_along_k():
    K, N, G = 256, 4, 128
    Wq = np.full((K, N // 2), 0x9B, np.uint8)  # codes 9 and 11 -> +1 and +3
    scales = np.array([[1.0, 2.0, 4.0, 8.0], [0.5, 0.25, 0.125, 0.0625]], np.float64)
    W = oracle.w4_dequant(Wq, scales, N, group=G, s_dtype="f64")
    assert np.array_equal(W[:G], np.tile([1.0, 6.0, 4.0, 24.0], (G, 1)))
    assert np.array_equal(W[G:], np.tile([0.5, 0.75, 0.125, 0.1875], (G, 1)))


def test_w4_gemm_one_hot_rows_select_weights_exactly():
    # X row m is one-hot at k_m, so D[m] = (code[k_m] - 8) * s[k_m // 128] exactly
    K, N = 256, 16
    Wq = workloads.uniform_bytes((K, N // 2), wid=95, tid=1)
    scales = workloads.f32_to_bf16_bits(np.full((K // 128, N), 2.0 ** -6, np.float32))
    ks = [0, 1, 127, 128, 200, 255]
    X = np.zeros((len(ks), K), np.float32)
    for m, k in enumerate(ks):
        X[m, k] = 1.0
    Xb = workloads.f32_to_bf16_bits(X)
    D = oracle.w4_gemm(Xb, Wq, scales, N, "bf16")
    for m, k in enumerate(ks):
        hi = (Wq[k] >> 4).astype(np.int64)
        lo = (Wq[k] & 0xF).astype(np.int64)
        codes = np.empty(N, np.int64)
        codes[0::2], codes[1::2] = hi, lo
        assert np.array_equal(D[m], (codes - 8) * 2.0 ** -6)


# --------------------------------------------------------------------------
# add + RMSNorm
# --------------------------------------------------------------------------

def test_add_rmsnorm_constant_rows():
    # a + x = 2 on every element of a row: rms = 2, so with eps = 0 the output is w exactly
    M, N = 3, 10
    a = np.full((M, N), 1.5, np.float32)
    x = np.full((M, N), 0.5, np.float32)
    w = np.linspace(-1, 1, N).astype(np.float32)
    resid, out = oracle.add_rmsnorm(a, x, w, "f32", eps=0.0)
    assert np.array_equal(resid, np.full((M, N), 2.0))
    assert np.array_equal(out, np.tile(w.astype(np.float64), (M, 1)))


def test_add_rmsnorm_eps_inside_the_root():
    # Pattern 1 of "Fusion Thinking": rrms = 1 / sqrt(mean(r^2) + eps).  r = 2 everywhere and
    # eps = 12 give 1 / sqrt(4 + 12) = 1/4, so out = r / 4 * w = w / 2 exactly.  eps outside the
    # root (1/2 + 12), eps dropped (1/2) or eps added to the sum instead of the mean
    # (1 / sqrt((4 N + 12) / N)) all give another value.
    M, N = 2, 10
    a = np.full((M, N), 1.25, np.float32)
    x = np.full((M, N), 0.75, np.float32)
    w = np.linspace(-2, 2, N).astype(np.float32)
    _, out = oracle.add_rmsnorm(a, x, w, "f32", eps=12.0)
    assert np.array_equal(out, np.tile(w.astype(np.float64) / 2, (M, 1)))
    # r = 1 and eps = 3: rrms = 1 / sqrt(1 + 3) = 1/2
    one = np.full((1, N), 0.5, np.float32)
    _, out = oracle.add_rmsnorm(one, one, w, "f32", eps=3.0)
    assert np.array_equal(out[0], w.astype(np.float64) / 2)


def test_add_rmsnorm_zero_row_is_finite_with_eps():
    # a row of zeros: mean(r^2) = 0, so eps alone keeps the root nonzero: rrms = 1 / sqrt(1/4) = 2
    # and out = 0 * 2 * w = 0 (a dropped eps would give 0 * inf = nan)
    N = 16
    z = np.zeros((3, N), np.float32)
    w = np.linspace(1, 2, N).astype(np.float32)
    resid, out = oracle.add_rmsnorm(z, z, w, "f32", eps=0.25)
    assert np.array_equal(resid, np.zeros((3, N)))
    assert np.array_equal(out, np.zeros((3, N)))
    # eps = 0 on the same row has no finite answer
    _, bad = oracle.add_rmsnorm(z, z, w, "f32", eps=0.0)
    assert not np.any(np.isfinite(bad))


def test_add_rmsnorm_unit_rms_after_normalisation():
    a = workloads.normal((4, 256), 1.0, "f32", wid=96, tid=0)
    x = workloads.normal((4, 256), 1.0, "f32", wid=96, tid=1)
    w = np.ones(256, np.float32)
    resid, out = oracle.add_rmsnorm(a, x, w, "f32", eps=0.0)
    assert np.array_equal(resid, a.astype(np.float64) + x.astype(np.float64))
    assert np.allclose(np.sqrt(np.mean(out ** 2, axis=1)), 1.0, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# composition
# --------------------------------------------------------------------------

def test_whole_pipeline_against_independent_numpy_scipy_path():
    w = workloads.WORKLOADS["square_bf16"].with_shape(M=70, N=90, K=200)
    inp = workloads.make_inputs(w, seed=3)
    got = oracle.reference(inp)
    A, B = _bf16_values(inp["A"]), _bf16_values(inp["B"])
    t = A @ B + _bf16_values(inp["bias"])[None, :]
    erf = np.vectorize(math.erf)
    gelu_exact = t * 0.5 * (1 + erf(t / math.sqrt(2)))
    ref = gelu_exact + _bf16_values(inp["R"])
    assert np.max(np.abs(got - ref)) <= 5.0e-4 + 1e-12


def test_row_subset_equals_full_result_rows():
    w = workloads.WORKLOADS["skinny_decode"].with_shape(M=16, N=64, K=96)
    inp = workloads.make_inputs(w)
    full = oracle.reference(inp)
    rows = np.array([0, 5, 15])
    assert np.array_equal(oracle.reference(inp, rows=rows), full[rows])


def test_w4_reference_equals_dense_bf16_gemm_on_dequantised_weights():
    w = workloads.WORKLOADS["w4a16_m16"].with_shape(M=4, N=32, K=256)
    inp = workloads.make_inputs(w)
    got = oracle.reference(inp)
    W = oracle.w4_dequant(inp["Wq"], inp["scales"], w.N)
    ref = _bf16_values(inp["X"]) @ W + _bf16_values(inp["bias"])[None, :]
    assert np.max(np.abs(got - ref)) <= 1e-12 * (1 + np.abs(ref).max())


# ---------------------------------------------------------------------------
# 8-bit weights: unsigned integer codes with a zero point, and OCP fp8 E4M3
# ---------------------------------------------------------------------------

def test_fp8_e4m3_decoder_matches_torch_for_every_code():
    # torch's float8_e4m3fn is an independent implementation of the same format
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    W = oracle.w8_dequant(codes, np.ones((1, 256)), "fp8", group=1, s_dtype="f64")[0]
    ref = torch.from_numpy(codes.reshape(-1).copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(W), np.isnan(ref))
    assert np.array_equal(W[~np.isnan(W)], ref[~np.isnan(ref)])
    fin = ~np.isnan(W)
    assert np.array_equal(np.signbit(W[fin]), np.signbit(ref[fin]))


def test_fp8_e4m3_anchor_values():
    # format facts: largest finite 448 (0x7E), smallest normal 2^-6 (0x08), smallest
    # subnormal 2^-9 (0x01), 1.0 = 0x38, -2.0 = 0xC0, S.1111.111 is NaN, 0x80 is -0
    codes = np.array([[0x7E, 0x08, 0x01, 0x38, 0xC0, 0x7F, 0xFF, 0x80, 0x00, 0x3C]], dtype=np.uint8)
    W = oracle.w8_dequant(codes, np.ones((1, codes.shape[1])), "fp8", group=1, s_dtype="f64")[0]
    assert list(W[:5]) == [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, -2.0]
    assert np.isnan(W[5]) and np.isnan(W[6])
    assert W[7] == 0.0 and np.signbit(W[7]) and W[8] == 0.0 and not np.signbit(W[8])
    assert W[9] == 1.5
    # positive finite codes are strictly increasing in value
    pos = oracle.w8_dequant(np.arange(0x7F, dtype=np.uint8).reshape(1, -1), np.ones((1, 0x7F)), "fp8",
                            group=1, s_dtype="f64")[0]
    assert np.all(np.diff(pos) > 0)


def test_u8_dequant_hand_computed():
    codes = np.array([[0, 1, 127, 128, 129, 255]], dtype=np.uint8)
    W = oracle.w8_dequant(codes, np.full((1, 6), 0.25), "u8", group=1, zero_point=128, s_dtype="f64")[0]
    assert list(W) == [-32.0, -31.75, -0.25, 0.0, 0.25, 31.75]


@pytest.mark.parametrize("fmt,zp", [("u8", 128), ("u8", 3), ("fp8", 0)])
def test_w8_gemm_matches_numpy_on_independently_decoded_weights(fmt, zp):
    torch = pytest.importorskip("torch")
    K, N, M, group = 96, 40, 5, 32
    r = np.random.default_rng(11)
    Wq = (workloads.fp8_codes((K, N), wid=90, tid=1) if fmt == "fp8"
          else r.integers(0, 256, (K, N), dtype=np.uint8))
    s = r.uniform(0.01, 0.02, (K // group, N))
    X = r.standard_normal((M, K))
    if fmt == "fp8":
        vals = torch.from_numpy(Wq.reshape(-1).copy()).view(torch.float8_e4m3fn).float().numpy()
        vals = vals.astype(np.float64).reshape(K, N)
    else:
        vals = Wq.astype(np.float64) - zp
    W = vals * np.repeat(s, group, axis=0)
    ref = X @ W
    got = oracle.w8_gemm(X, Wq, s, fmt, "f64", group=group, zero_point=zp, s_dtype="f64")
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    # and the dequant itself is exact
    assert np.array_equal(oracle.w8_dequant(Wq, s, fmt, group=group, zero_point=zp, s_dtype="f64"), W)


# --------------------------------------------------------------------------
# rotary position embedding (page "Fusion Thinking", Pattern 4)
# --------------------------------------------------------------------------

def _b(x):
    return workloads.f32_to_bf16_bits(np.asarray(x, np.float32))


def _f(bits):
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("interleaved,expect", [(False, [-3, -4, 1, 2]), (True, [-2, 1, -4, 3])])
def test_rope_quarter_turn_hand_values(interleaved, expect):
    # D = 4, angle pi/2 for both pairs (cos 0, sin 1): each pair (a, b) becomes (-b, a).
    # rotate-half pairs (0, 2), (1, 3); interleaved pairs (0, 1), (2, 3)
    cos, sin = np.zeros((1, 2), np.float32), np.ones((1, 2), np.float32)
    got = _f(oracle.rope(_b([[1, 2, 3, 4]]), cos, sin, interleaved=interleaved))
    assert got.tolist() == [expect]


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_with_zero_angles_is_the_identity(interleaved):
    X = workloads.normal((3, 5, 64), 1.0, "bf16", wid=91, tid=0)
    cos, sin = workloads.rope_tables(5, 64, 1.0e30)  # every angle rounds to 0 beyond i = 0
    cos[:], sin[:] = 1.0, 0.0
    assert np.array_equal(oracle.rope(X, cos, sin, interleaved=interleaved), X)


def test_rope_is_multiplication_by_a_unit_complex_number():
    # independent definition: (x_a + i x_b) * exp(i p theta_k), in complex128; the stored result is
    # within half a bf16 spacing of it (one rounding to nearest)
    D, S, pos0 = 64, 9, 5
    X = workloads.normal((S, D), 1.0, "bf16", wid=92, tid=0)
    cos, sin = workloads.rope_tables(pos0 + S, D, 10000.0)
    x = _f(X)
    z = (x[:, :D // 2] + 1j * x[:, D // 2:]) * (cos[pos0:].astype(np.float64) + 1j * sin[pos0:].astype(np.float64))
    want = np.concatenate([z.real, z.imag], axis=1)
    got = _f(oracle.rope(X, cos, sin, pos0))
    half_ulp = np.ldexp(1.0, np.floor(np.log2(np.abs(want))).astype(int) - 8)
    assert np.all(np.abs(got - want) <= half_ulp * (1 + 1e-9))
    # a rotation keeps each pair's length
    n0 = x[:, :D // 2] ** 2 + x[:, D // 2:] ** 2
    n1 = got[:, :D // 2] ** 2 + got[:, D // 2:] ** 2
    assert np.allclose(n1, n0, rtol=2.0 ** -6, atol=1e-6)


def _bf16_nearest_exact(v):
    """bf16 bits of the Fraction v rounded to nearest, ties to even, by comparing exact distances
    to the two bf16 neighbours (brute force; finite normal values)."""
    from fractions import Fraction
    if v == 0:
        return 0
    t = np.array([float(v)], np.float32).view(np.uint32)[0] >> 16  # a bf16 pattern within 2 steps of v
    cands = [int(t) + d for d in range(-2, 3)]
    vals = [Fraction(float(workloads.bf16_bits_to_f32(np.array([c], np.uint16))[0])) for c in cands]
    dist = [abs(x - v) for x in vals]
    best = min(dist)
    ties = [c for c, d in zip(cands, dist) if d == best]
    return min(ties, key=lambda c: c & 1)  # even mantissa wins a tie


def _rope_exact(X, cos, sin, pos0=0):
    """Rotate-half RoPE with exact rational arithmetic, element by element (tiny inputs only)."""
    from fractions import Fraction
    x = _f(X)
    S, D = x.shape
    out = np.empty((S, D), np.uint16)
    for r in range(S):
        for i in range(D // 2):
            a, b = Fraction(float(x[r, i])), Fraction(float(x[r, i + D // 2]))
            c, s = Fraction(float(cos[pos0 + r, i])), Fraction(float(sin[pos0 + r, i]))
            out[r, i] = _bf16_nearest_exact(a * c - b * s)
            out[r, i + D // 2] = _bf16_nearest_exact(a * s + b * c)
    return out


def test_rope_equals_exact_rational_rotation_rounded_once():
    D, S, pos0 = 16, 6, 3
    X = workloads.normal((S, D), 1.0, "bf16", wid=94, tid=0)
    cos, sin = workloads.rope_tables(pos0 + S, D, 10000.0)
    assert np.array_equal(oracle.rope(X, cos, sin, pos0), _rope_exact(X, cos, sin, pos0))


def test_rope_ties_and_near_ties_round_on_the_exact_value():
    # one row, D = 8 (pairs (i, i + 4)); each pair is built so that its exact rotated value sits on
    # or next to a point halfway between two bf16 numbers:
    #   pair 0: yb = 1 * (1 + 2^-8) + 2^-40 * 2^-40: just above the midpoint of 1 and 1 + 2^-7 ->
    #           rounds up (float64 alone would round the sum onto the midpoint, then to even = 1)
    #   pair 0: ya = 1 * 2^-40 - 2^-40 * (1 + 2^-8) ... small, exact in float64
    #   pair 1: ya = 1 * (1 + 2^-8) - 2^-40 * 2^-40: just below that midpoint -> 1
    #   pair 2: ya = 1 * (1 + 2^-8) - 0: exactly the midpoint -> ties to even -> 1
    #   pair 3: ya = 1 * (1 + 3 * 2^-8) - 0: exactly a midpoint -> to even -> 1 + 2^-6
    t = 2.0 ** -40
    xa = np.array([1.0, 1.0, 1.0, 1.0], np.float32)
    xb = np.array([t, t, 0.0, 0.0], np.float32)
    cos = np.array([[t, 1 + 2 ** -8, 1 + 2 ** -8, 1 + 3 * 2 ** -8]], np.float32)
    sin = np.array([[1 + 2 ** -8, t, 0.0, 0.0]], np.float32)
    X = _b([np.concatenate([xa, xb])])
    got = _f(oracle.rope(X, cos, sin))[0]
    assert got[4] == 1 + 2 ** -7          # pair 0, yb
    assert got[1] == 1.0                  # pair 1, ya
    assert got[2] == 1.0 and got[3] == 1 + 2 ** -6
    assert np.array_equal(oracle.rope(X, cos, sin), _rope_exact(X, cos, sin))


def test_rope_interleaved_is_rotate_half_with_columns_permuted():
    D = 128
    X = workloads.normal((2, 7, D), 1.0, "bf16", wid=93, tid=0)
    cos, sin = workloads.rope_tables(10, D, 500000.0)
    perm = np.empty(D, np.int64)
    perm[0::2], perm[1::2] = np.arange(D // 2), np.arange(D // 2) + D // 2  # column 2i <- i, 2i+1 <- i + D/2
    a = oracle.rope(np.ascontiguousarray(X[..., perm]), cos, sin, 3, interleaved=True)
    b = oracle.rope(X, cos, sin, 3)[..., perm]
    assert np.array_equal(a, b)


def test_rope_scores_depend_only_on_the_relative_position():
    # <rope(q, p + t), rope(k, p' + t)> = <rope(q, p), rope(k, p')> for exact rotations; here
    # within the bf16 rounding of the rotated operands
    w = workloads.ROPE_WORKLOADS["rope_qk_prefill"].with_shape(heads=2, Sq=16, Sk=24, D=64)
    inp = workloads.make_rope_inputs(w)
    cos, sin = workloads.rope_tables(200, 64, 10000.0)
    s0 = oracle.rope_qk(inp["Q"], inp["K"], cos, sin, q_pos0=3, k_pos0=0, alpha=inp["alpha"])
    s1 = oracle.rope_qk(inp["Q"], inp["K"], cos, sin, q_pos0=3 + 150, k_pos0=150, alpha=inp["alpha"])
    assert np.max(np.abs(s1 - s0) / (1 + np.abs(s0))) < 2e-2
    # and do change when only one side moves
    s2 = oracle.rope_qk(inp["Q"], inp["K"], cos, sin, q_pos0=3 + 150, k_pos0=0, alpha=inp["alpha"])
    assert np.max(np.abs(s2 - s0)) > 0.5


def test_rope_qk_product_pass_matches_numpy():
    w = workloads.ROPE_WORKLOADS["rope_qk_prefill"].with_shape(heads=3, Sq=20, Sk=33, D=128)
    inp = workloads.make_rope_inputs(w)
    S = oracle.rope_qk(inp["Q"], inp["K"], inp["cos"], inp["sin"], alpha=0.5)
    q = _f(oracle.rope(inp["Q"], inp["cos"], inp["sin"]))
    k = _f(oracle.rope(inp["K"], inp["cos"], inp["sin"]))
    assert np.allclose(S, 0.5 * np.einsum("bmd,bnd->bmn", q, k), rtol=1e-12, atol=1e-12)
    plain = oracle.rope_qk(inp["Q"], inp["K"], inp["cos"], inp["sin"], rotate=False)
    assert np.allclose(plain, np.einsum("bmd,bnd->bmn", _f(inp["Q"]), _f(inp["K"])), rtol=1e-12, atol=1e-12)
