"""GPU parity of rotary position embedding at operand load (page "Fusion
Thinking", Pattern 4): the standalone rotation against the oracle -- bit-exact
with the exact rounding (ties, near ties, cancellation, overflow, subnormals,
signed zeros), within its stated bound with the default fp32 rounding -- the
fused scores kernel against the oracle on ragged shapes, both pairings, both
output types and shifted positions, fused == unfused chain bitwise in both
roundings, and the requests the entry points must refuse."""
import numpy as np
import pytest
import torch

import gemm_epilogue_tile_amd as ge
import oracle
import workloads
from gpu_helpers import DEV, TOL_BF16, TOL_F32, assert_close, to_dev

pytestmark = pytest.mark.gpu

RW = workloads.ROPE_WORKLOADS["rope_qk_prefill"]


def _dev(inp):
    return (to_dev(inp["Q"]), to_dev(inp["K"]), torch.from_numpy(inp["cos"]).to(DEV),
            torch.from_numpy(inp["sin"]).to(DEV))


def _bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("interleaved", [False, True])
def test_rotation_alone_is_bit_exact(D, interleaved):
    w = RW.with_shape(heads=3, Sq=77, Sk=77, D=D, interleaved=interleaved)
    inp = workloads.make_rope_inputs(w, seed=D)
    Q, _, c, s = _dev(inp)
    cos, sin = workloads.rope_tables(200, D, 500000.0)
    got = _bits(ge.rope(Q, torch.from_numpy(cos).to(DEV), torch.from_numpy(sin).to(DEV), pos0=41,
                        interleaved=interleaved, exact=True))
    assert np.array_equal(got, oracle.rope(inp["Q"], cos, sin, 41, interleaved))


def _fast_bound(X, cos, sin, pos0, interleaved):
    """Per output element, what the default fp32 rounding may differ by from the exactly rounded
    value: one bf16 unit of it, or 2^-22 (|a| + |b|) max(|cos|, |sin|) where the two products
    cancel (a, b: the pair the element belongs to)."""
    x = workloads.bf16_bits_to_f32(X).astype(np.float64)
    S, D = x.shape[-2], x.shape[-1]
    c = cos[pos0:pos0 + S].astype(np.float64)
    t = sin[pos0:pos0 + S].astype(np.float64)
    if interleaved:
        a, b = x[..., 0::2], x[..., 1::2]
    else:
        a, b = x[..., :D // 2], x[..., D // 2:]
    m = (np.abs(a) + np.abs(b)) * np.maximum(np.abs(c), np.abs(t)) * 2.0 ** -22
    out = np.empty_like(x)
    if interleaved:
        out[..., 0::2], out[..., 1::2] = m, m
    else:
        out[..., :D // 2], out[..., D // 2:] = m, m
    return out


def _assert_scores_fast(out, inp, q_pos0, k_pos0, interleaved, what):
    """Scores of the default rounding against the oracle's (exactly rounded operands): each rotated
    operand element may be off by d = max(one bf16 unit, the cancellation term of _fast_bound), so
    |S - S_ref| <= alpha (dQ |K'|^T + |Q'| dK^T + dQ dK^T), plus the fp32 product's own tolerance."""
    alpha = inp["alpha"]
    ref = oracle.rope_qk(inp["Q"], inp["K"], inp["cos"], inp["sin"], q_pos0=q_pos0, k_pos0=k_pos0, alpha=alpha,
                         interleaved=interleaved)
    g = out.float().cpu().numpy().astype(np.float64) if isinstance(out, torch.Tensor) else out
    bound = np.zeros_like(ref)
    for b in range(ref.shape[0]):
        ops = []
        for X, p0 in ((inp["Q"][b:b + 1], q_pos0), (inp["K"][b:b + 1], k_pos0)):
            xr = workloads.bf16_bits_to_f32(oracle.rope(X, inp["cos"], inp["sin"], p0, interleaved))[0].astype(np.float64)
            d = np.maximum(np.ldexp(1.0, np.frexp(np.abs(xr))[1] - 8),
                           _fast_bound(X, inp["cos"], inp["sin"], p0, interleaved)[0])
            ops.append((np.abs(xr), d))
        (aq, dq), (ak, dk) = ops
        bound[b] = abs(alpha) * (dq @ ak.T + aq @ dk.T + dq @ dk.T)
    err = np.abs(g - ref)
    ok = err <= bound + TOL_F32 * (1 + np.abs(ref))
    i = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(ok), f"{what}: err {err[i]:.3e} > bound {bound[i]:.3e} at {i}"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("interleaved", [False, True])
def test_rotation_alone_default_rounding_within_bound(D, interleaved):
    w = RW.with_shape(heads=3, Sq=77, Sk=77, D=D, interleaved=interleaved)
    inp = workloads.make_rope_inputs(w, seed=D + 1)
    Q, _, c, s = _dev(inp)
    cos, sin = workloads.rope_tables(200, D, 500000.0)
    got = _bits(ge.rope(Q, torch.from_numpy(cos).to(DEV), torch.from_numpy(sin).to(DEV), pos0=41,
                        interleaved=interleaved))
    want = oracle.rope(inp["Q"], cos, sin, 41, interleaved)
    g = workloads.bf16_bits_to_f32(got).astype(np.float64)
    e = workloads.bf16_bits_to_f32(want).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(e))[1] - 8)  # one bf16 unit at the exact value
    err = np.abs(g - e)
    assert np.all((err <= ulp) | (err <= _fast_bound(inp["Q"], cos, sin, 41, interleaved))), np.max(err)
    # and nearly every element is the exactly rounded one
    assert np.mean(got != want) < 0.01


def _tie_cases():
    """(a, b, cos, sin) quadruples whose rotated values sit on, next to or far from points halfway
    between two bf16 numbers, cancel, overflow, are subnormal or signed zeros."""
    t = 2.0 ** -40
    m = 1 + 2 ** -8  # halfway between 1 and 1 + 2^-7
    cases = [(1.0, t, t, m), (1.0, t, m, t), (1.0, 0.0, m, 0.0), (1.0, 0.0, 1 + 3 * 2 ** -8, 0.0),
             (1.0, 2.0 ** -30, m, 2.0 ** -30), (-1.0, t, m, -t), (3.0, 1.0, 1.0, 3.0), (1.5, 1.5, 0.5, 0.5),
             (3.0e38, 3.0e38, 1.0, 0.5), (3.3e38, 1.0e38, 1.0, 0.1), (2.0 ** -130, 2.0 ** -131, 0.7, 0.3),
             (2.0 ** -120, 2.0 ** -121, 0.7, 0.3), (-0.0, 0.0, 0.5, 0.5), (0.0, -0.0, 1.0, 0.0),
             (1.0, 1.0, 0.70710677, 0.70710677), (2.0, 3.0, 0.6, 0.8)]
    rng = np.random.default_rng(7)
    while len(cases) < 64:
        # products within 2^-20 of each other: heavy cancellation
        a = float(workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(np.array([rng.normal()], np.float32)))[0])
        c = float(np.float32(rng.uniform(0.1, 1)))
        b = a
        s_ = float(np.float32(c * (1 + rng.uniform(-2 ** -20, 2 ** -20))))
        cases.append((a, b, c, s_))
    return cases


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotation_of_ties_overflow_subnormals_bit_exact(interleaved):
    # 64 pairs, one per row (position), each with its own table entry: the kernel's fast fp32 path
    # must flag every element it cannot round with certainty and redo it exactly
    D = 128
    cases = _tie_cases()
    S = len(cases)
    x = np.zeros((S, D), np.float32)
    cos = np.full((S, D // 2), 0.5, np.float32)
    sin = np.full((S, D // 2), 0.25, np.float32)
    for r, (a, b, c, s_) in enumerate(cases):
        for i in range(D // 2):  # every pair of the row carries the case, in a different pair slot too
            ia, ib = (2 * i, 2 * i + 1) if interleaved else (i, i + D // 2)
            x[r, ia], x[r, ib] = (a, b) if i % 2 == 0 else (b, a)
            cos[r, i], sin[r, i] = (c, s_) if i % 3 else (s_, c)
    X = workloads.f32_to_bf16_bits(x)[None]
    Xd = to_dev(X)
    got = _bits(ge.rope(Xd, torch.from_numpy(cos).to(DEV), torch.from_numpy(sin).to(DEV), interleaved=interleaved,
                        exact=True))
    want = oracle.rope(X, cos, sin, 0, interleaved)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} mismatches, first at {tuple(b[0] for b in bad)}: gpu {got[bad][0]:#06x} oracle {want[bad][0]:#06x}"
    # the fused scores kernel rotates the same way
    ref_q = torch.from_numpy(want.view(np.int16)).to(DEV).view(torch.bfloat16)
    fused = ge.rope_qk(Xd[:, :, :], Xd, torch.from_numpy(cos).to(DEV), torch.from_numpy(sin).to(DEV), alpha=1.0,
                       interleaved=interleaved, exact=True)
    plain = ge.rope_qk(ref_q, ref_q, alpha=1.0)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(fused, posinf=1, neginf=-1).view(torch.int32),
                       torch.nan_to_num(plain, posinf=1, neginf=-1).view(torch.int32))


@pytest.mark.parametrize("H,Sq,Sk,D", [(1, 1, 1, 64), (2, 128, 128, 128), (3, 77, 200, 128), (2, 300, 131, 64),
                                       (4, 1, 517, 128), (8, 129, 140, 64), (8, 384, 257, 128)])
@pytest.mark.parametrize("interleaved", [False, True])
def test_fused_scores_match_the_oracle(H, Sq, Sk, D, interleaved):
    w = RW.with_shape(heads=H, Sq=Sq, Sk=Sk, D=D, interleaved=interleaved, k_pos0=5, q_pos0=5 + Sk - Sq if Sk >= Sq else 5)
    inp = workloads.make_rope_inputs(w, seed=H + Sq + Sk)
    Q, K, c, s = _dev(inp)
    out = ge.rope_qk(Q, K, c, s, q_pos0=w.q_pos0, k_pos0=w.k_pos0, alpha=inp["alpha"], interleaved=interleaved)
    _assert_scores_fast(out, inp, w.q_pos0, w.k_pos0, interleaved, f"rope_qk {H}x{Sq}x{Sk}x{D} inter={interleaved}")


@pytest.mark.parametrize("interleaved", [False, True])
def test_fused_scores_exact_rounding_match_the_oracle(interleaved):
    w = RW.with_shape(heads=3, Sq=77, Sk=200, D=128, interleaved=interleaved, q_pos0=9, k_pos0=5)
    inp = workloads.make_rope_inputs(w, seed=13)
    Q, K, c, s = _dev(inp)
    out = ge.rope_qk(Q, K, c, s, q_pos0=9, k_pos0=5, alpha=inp["alpha"], interleaved=interleaved, exact=True)
    ref = oracle.rope_qk(inp["Q"], inp["K"], inp["cos"], inp["sin"], q_pos0=9, k_pos0=5, alpha=inp["alpha"],
                         interleaved=interleaved)
    assert_close(out, ref, TOL_F32, f"rope_qk exact inter={interleaved}")


def test_fused_scores_bf16_output():
    w = RW.with_shape(heads=2, Sq=200, Sk=264, D=128)
    inp = workloads.make_rope_inputs(w, seed=3)
    Q, K, c, s = _dev(inp)
    out = ge.rope_qk(Q, K, c, s, alpha=inp["alpha"], out_dtype=torch.bfloat16)
    ref = oracle.rope_qk(inp["Q"], inp["K"], inp["cos"], inp["sin"], alpha=inp["alpha"])
    assert_close(out, ref, TOL_BF16, "rope_qk bf16 out")


def test_plain_product_without_tables():
    w = RW.with_shape(heads=2, Sq=130, Sk=70, D=64)
    inp = workloads.make_rope_inputs(w, seed=4)
    Q, K, _, _ = _dev(inp)
    out = ge.rope_qk(Q, K, alpha=0.25)
    ref = oracle.rope_qk(inp["Q"], inp["K"], inp["cos"], inp["sin"], alpha=0.25, rotate=False)
    assert_close(out, ref, TOL_F32, "plain product")


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("exact", [False, True])
def test_fused_equals_the_unfused_chain_bitwise(interleaved, exact):
    # rope(Q) and rope(K) written to memory, then the plain product: the same bf16 operands reach
    # the same product code, so the scores agree bit for bit (in either rounding)
    w = RW.with_shape(heads=4, Sq=256, Sk=384, D=128, interleaved=interleaved, q_pos0=128)
    inp = workloads.make_rope_inputs(w, seed=9)
    Q, K, c, s = _dev(inp)
    fused = ge.rope_qk(Q, K, c, s, q_pos0=128, alpha=inp["alpha"], interleaved=interleaved, exact=exact)
    q2 = ge.rope(Q, c, s, pos0=128, interleaved=interleaved, exact=exact)
    k2 = ge.rope(K, c, s, pos0=0, interleaved=interleaved, exact=exact)
    unfused = ge.rope_qk(q2, k2, alpha=inp["alpha"])
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int32), unfused.view(torch.int32))


def test_full_size_prefill_sampled_heads():
    w = RW
    inp = workloads.make_rope_inputs(w)
    Q, K, c, s = _dev(inp)
    out = ge.rope_qk(Q, K, c, s, alpha=inp["alpha"]).cpu().numpy().astype(np.float64)
    heads = [0, 17, w.heads - 1]
    sub = dict(inp, Q=inp["Q"][heads], K=inp["K"][heads])
    _assert_scores_fast(out[heads], sub, w.q_pos0, w.k_pos0, w.interleaved, "rope_qk full size")
    assert np.all(np.isfinite(out))


def test_refusals():
    Q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device=DEV)
    cos = torch.zeros((8, 64), dtype=torch.float32, device=DEV)
    with pytest.raises(ge.GemmEpiError) as e:
        ge.rope_qk(Q, Q, cos, cos, q_pos0=1)  # position 8 is past the tables
    assert e.value.status == ge.ERR_INVALID_ARG
    Q96 = torch.zeros((1, 8, 96), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ge.GemmEpiError) as e:
        ge.rope_qk(Q96, Q96)
    assert e.value.status == ge.ERR_UNSUPPORTED
    with pytest.raises(ge.GemmEpiError):
        ge.rope(Q, cos, cos, out=Q)  # Y overlaps X
    out = torch.empty((1, 8, 8), dtype=torch.float32, device=DEV)
    st = ge.lib().ge_rope_qk_run(1, 8, 8, 128, ge._ptr(Q), ge._ptr(Q), ge._ptr(cos), ge._ptr(cos), 8, 0, 0, 4, 1.0,
                                 ge.F32, ge._ptr(out), None)
    assert st == ge.ERR_INVALID_ARG  # unknown flag bit
