"""The race-guard build against the normal one (an extra ordering check: the
debug library adds waits, barriers and fences, which can only remove races):
every case of race_cases.py is run with
libgemm_epi.so here and with libgemm_epi_debug.so in a child process, and the
outputs must agree bit for bit."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import gemm_epilogue_tile_amd as ge
import race_cases

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DEBUG_LIB = os.path.join(ROOT, "gemm_epilogue_tile_amd", "libgemm_epi_debug.so")

CHILD = """
import sys, numpy as np, torch
sys.path[:0] = [{root!r}, {tests!r}]
import gemm_epilogue_tile_amd as ge
ge.lib_path = {lib!r}
import race_cases
np.savez({out!r}, **race_cases.run_cases(ge, torch))
"""


def test_debug_sync_build_reproduces_every_case_bitwise(tmp_path):
    if not os.path.exists(DEBUG_LIB):
        pytest.fail(f"{DEBUG_LIB} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    mine = race_cases.run_cases(ge, torch)
    out = str(tmp_path / "debug.npz")
    code = CHILD.format(root=ROOT, tests=HERE, lib=DEBUG_LIB, out=out)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    theirs = np.load(out)
    assert sorted(theirs.files) == sorted(mine)
    for name, a in mine.items():
        b = theirs[name]
        assert a.shape == b.shape, name
        bad = np.count_nonzero(a != b)
        assert bad == 0, f"{name}: {bad} of {a.size} outputs differ from the race-guard build"


def test_ge_log_prints_plan_decisions():
    # GE_LOG=1: each plan prints its kernel choice on stderr
    code = (f"import os, sys; sys.path[:0] = [{ROOT!r}]\n"
            "os.environ['GE_LOG'] = '1'\n"
            "import torch\n"
            "import gemm_epilogue_tile_amd as ge\n"
            "ge.plan(ge.KIND_GENERIC, 16, 4096, 8192, bias=True, R=True)\n"
            "ge.plan(ge.KIND_W4, 512, 8192, 8192, b_type=ge.U4X2, bias=True, prepacked=True)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if l.startswith("ge: plan")]
    assert len(lines) == 2, r.stderr[-2000:]
    assert "kind=generic M=16 N=4096 K=8192" in lines[0] and "kernel=skinny_bf16_m16_128col_streamk" in lines[0]
    assert "kind=w4 M=512 N=8192 K=8192" in lines[1] and "kernel=tile_w4_bf16_64x256x32" in lines[1]
