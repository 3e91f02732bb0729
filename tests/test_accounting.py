"""Byte / FLOP accounting against the figures the pages state and closed forms."""
import pytest

import workloads
from gemm_epilogue_tile_amd import accounting


def test_swiglu_waste_per_token_llama3_8b():
    # page "Fusion Thinking", Pattern 2: about 57 KB per token at d_intermediate 14336
    assert accounting.swiglu_intermediate_bytes_per_token(14336) == 57344


def test_int4_weight_cost():
    # 4-bit codes + one bf16 scale per 128 weights
    assert accounting.w4_bits_per_weight(128) == 4.125
    # page "Fusion Thinking", Pattern 3: a 70B model drops from ~140 GB (bf16) to ~35 GB (int4)
    params = 70e9
    assert params * 2 / 1e9 == pytest.approx(140)
    assert params * 4 / 8 / 1e9 == pytest.approx(35)


def test_elementwise_add_intensity():
    # y = x + residual on bf16: 1 FLOP per element over 2 reads + 1 write of 2 bytes
    assert 1 / (3 * 2) < accounting.RIDGE / 1000


def test_square_workload_numbers():
    a = accounting.work(workloads.WORKLOADS["square_bf16"])
    assert a["flops"] == 2 * 4096 ** 3
    assert a["bytes"] == 4 * 4096 * 4096 * 2 + 4096 * 2          # A, B, R, D + bias
    assert a["unfused_bytes"] == (3 * 4096 * 4096 * 2              # GEMM: A, B, T0
                                  + 2 * 4096 * 4096 * 2 + 4096 * 2  # bias
                                  + 2 * 4096 * 4096 * 2            # GELU
                                  + 3 * 4096 * 4096 * 2)           # residual
    assert a["bound"] == "mfma"


def test_fusion_changes_bytes_not_flops():
    for name, w in workloads.WORKLOADS.items():
        a = accounting.work(w)
        assert a["unfused_bytes"] > a["bytes"], name


@pytest.mark.parametrize("name,bound", [("square_bf16", "mfma"), ("swiglu_8b", "mfma"),
                                        ("skinny_decode", "hbm"), ("w4a16_m16", "hbm"),
                                        ("w4a16_m512", "mfma")])
def test_bounds(name, bound):
    assert accounting.work(workloads.WORKLOADS[name])["bound"] == bound


def test_w4_m16_bytes():
    a = accounting.work(workloads.WORKLOADS["w4a16_m16"])
    assert a["bytes"] == 16 * 8192 * 2 + 8192 * 4096 + 64 * 8192 * 2 + 8192 * 2 + 16 * 8192 * 2
