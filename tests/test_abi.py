"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function ``include/gemm_epi.h``
declares, agree with the Python mirror of ``ge_desc`` on layout, validate
descriptors before touching a device, and report GE_ERR_NO_DEVICE (not
crash) when no GPU is visible.  No compute call is made here.
"""
import ctypes
import os
import re
import subprocess

import pytest

import gemm_epilogue_tile_amd as ge
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "gemm_epi.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^GE_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M)))


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # noqa: BLE001
        return False


def test_header_declares_the_boundary():
    names = _declared_functions()
    for must in ["gemm_epi_plan", "gemm_epi_run", "gemm_swiglu_run", "gemm_w4_run",
                 "gemm_epi_run_unfused", "gemm_epi_unfused_workspace_bytes", "gemm_epi_plan_destroy",
                 "ge_status_string", "ge_last_error"]:
        assert must in names
    assert sorted(ge.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    L = ge.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ge.lib_path], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(_declared_functions()) <= exported
    # internal kernels and helpers stay hidden
    assert all(n.startswith(("ge_", "gemm_")) for n in exported), sorted(exported)


def test_desc_layout_matches_c(tmp_path):
    fields = [f[0] for f in ge.Desc._fields_]
    prog = tmp_path / "layout.c"
    body = "\n".join(f'printf("{f} %zu\\n", offsetof(ge_desc, {f}));' for f in fields)
    prog.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "gemm_epi.h"\n'
                    'int main(void){' + body + 'printf("size %zu\\n", sizeof(ge_desc)); return 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", f"-I{os.path.dirname(HEADER)}", str(prog),
                    "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                  check=True).stdout.splitlines())
    for f in fields:
        assert int(got[f]) == getattr(ge.Desc, f).offset, f
    assert int(got["size"]) == ctypes.sizeof(ge.Desc)


def test_status_strings_and_version():
    L = ge.lib()
    assert L.ge_status_string(0) == b"GE_OK"
    assert L.ge_status_string(3) == b"GE_ERR_NO_DEVICE"
    assert L.ge_status_string(99) == b"GE_ERR_UNKNOWN"
    assert re.fullmatch(rb"\d+\.\d+\.\d+", L.ge_version())


def test_desc_init_defaults():
    d = ge.Desc()
    ge.lib().ge_desc_init(ctypes.byref(d))
    assert d.alpha == 1.0 and d.beta == 0.0 and d.group_size == 128 and d.zero_point == 8
    assert d.b_layout == ge.LAYOUT_KN and d.flags == 0 and d.act == 0


def _plan_status(kind=ge.KIND_GENERIC, **kw):
    L = ge.lib()
    d = ge.Desc()
    L.ge_desc_init(ctypes.byref(d))
    d.M, d.N, d.K = 64, 64, 128
    for k, v in kw.items():
        setattr(d, k, v)
    h = ctypes.c_void_p()
    s = L.gemm_epi_plan(ctypes.byref(d), kind, ctypes.byref(h))
    if s == 0:
        L.gemm_epi_plan_destroy(h)
    return s


@pytest.mark.parametrize("kw,kind,want", [
    (dict(M=0), ge.KIND_GENERIC, ge.ERR_INVALID_ARG),
    (dict(K=-1), ge.KIND_GENERIC, ge.ERR_INVALID_ARG),
    (dict(act=7), ge.KIND_GENERIC, ge.ERR_INVALID_ARG),
    (dict(flags=128), ge.KIND_GENERIC, ge.ERR_INVALID_ARG),
    (dict(b_layout=3), ge.KIND_GENERIC, ge.ERR_INVALID_ARG),
    (dict(lda=10), ge.KIND_GENERIC, ge.ERR_INVALID_ARG),
    (dict(ldd=5), ge.KIND_GENERIC, ge.ERR_INVALID_ARG),
    (dict(d_type=2), ge.KIND_GENERIC, ge.ERR_INVALID_ARG),
    (dict(a_type=0, b_type=1), ge.KIND_GENERIC, ge.ERR_UNSUPPORTED),
    (dict(flags=8), ge.KIND_GENERIC, ge.ERR_INVALID_ARG),
    (dict(M=1 << 16, N=1 << 16), ge.KIND_GENERIC, ge.ERR_UNSUPPORTED),
    (dict(act=2), ge.KIND_SWIGLU, ge.ERR_UNSUPPORTED),
    (dict(b_layout=1), ge.KIND_SWIGLU, ge.ERR_UNSUPPORTED),
    (dict(b_type=1), ge.KIND_W4, ge.ERR_UNSUPPORTED),
    (dict(b_type=2, N=63), ge.KIND_W4, ge.ERR_INVALID_ARG),
    (dict(b_type=2, K=100), ge.KIND_W4, ge.ERR_INVALID_ARG),
    (dict(b_type=2, group_size=48), ge.KIND_W4, ge.ERR_UNSUPPORTED),
    (dict(b_type=2, zero_point=16), ge.KIND_W4, ge.ERR_INVALID_ARG),
    (dict(b_type=3, zero_point=256), ge.KIND_W4, ge.ERR_INVALID_ARG),
    (dict(b_type=3, zero_point=-1), ge.KIND_W4, ge.ERR_INVALID_ARG),
    (dict(b_type=4), ge.KIND_W4, ge.ERR_INVALID_ARG),  # fp8 codes take no zero point (default is 8)
    (dict(b_type=3, flags=8), ge.KIND_W4, ge.ERR_INVALID_ARG),
    # prepacked 8-bit codes need M <= 16 and N % 128 == 0 (here M = 64, N = 64)
    (dict(b_type=4, zero_point=0, flags=16), ge.KIND_W4, ge.ERR_UNSUPPORTED),
    (dict(b_type=4, zero_point=0, flags=8), ge.KIND_W4, ge.ERR_INVALID_ARG),
    (dict(flags=32, M=33, N=128), ge.KIND_GENERIC, ge.ERR_UNSUPPORTED),
    (dict(b_type=2, flags=32), ge.KIND_W4, ge.ERR_INVALID_ARG),
    (dict(b_type=3, b_layout=1), ge.KIND_W4, ge.ERR_UNSUPPORTED),
    (dict(b_type=3, group_size=48), ge.KIND_W4, ge.ERR_UNSUPPORTED),
    (dict(b_type=4, zero_point=0, K=96, group_size=64), ge.KIND_W4, ge.ERR_INVALID_ARG),
    (dict(b_type=3, ldb=63), ge.KIND_W4, ge.ERR_INVALID_ARG),
    (dict(b_type=3, a_type=0), ge.KIND_W4, ge.ERR_UNSUPPORTED),
    (dict(b_type=3), ge.KIND_GENERIC, ge.ERR_UNSUPPORTED),
    (dict(b_type=4), ge.KIND_SWIGLU, ge.ERR_UNSUPPORTED),
    (dict(), 9, ge.ERR_INVALID_ARG),
])
def test_plan_rejects_bad_descriptors_before_any_device_call(kw, kind, want):
    assert _plan_status(kind, **kw) == want


@pytest.mark.skipif(_has_gpu(), reason="checks the no-device path")
@pytest.mark.parametrize("kind,kw", [(ge.KIND_GENERIC, {}), (ge.KIND_SWIGLU, {}),
                                     (ge.KIND_W4, dict(b_type=2)), (ge.KIND_W4, dict(b_type=3, ldb=64)),
                                     (ge.KIND_W4, dict(b_type=4, zero_point=0, group_size=32))])
def test_valid_plan_without_gpu_reports_no_device(kind, kw):
    assert _plan_status(kind, **kw) == ge.ERR_NO_DEVICE
    assert b"device" in ge.lib().ge_last_error()


def test_run_calls_reject_null_plan():
    L = ge.lib()
    p = ctypes.c_void_p(0)
    assert L.gemm_epi_run(p, None, None, None, None, None, None, None) == ge.ERR_INVALID_ARG
    assert L.gemm_epi_run_noalloc(p, None, None, None, None, None, None, None) == ge.ERR_INVALID_ARG
    assert L.gemm_swiglu_run(p, None, None, None, None, None) == ge.ERR_INVALID_ARG
    assert L.gemm_w4_run(p, None, None, None, None, None, None, None, None) == ge.ERR_INVALID_ARG
    assert L.gemm_epi_run_unfused(p, *([None] * 8)) == ge.ERR_INVALID_ARG
    assert L.gemm_swiglu_run_unfused(p, *([None] * 6)) == ge.ERR_INVALID_ARG
    assert L.gemm_w4_run_unfused(p, *([None] * 9)) == ge.ERR_INVALID_ARG
    assert L.gemm_w4_dequant_run(p, None, None, None, None) == ge.ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert L.gemm_epi_unfused_workspace_bytes(p, ctypes.byref(n)) == ge.ERR_INVALID_ARG
    assert L.gemm_epi_plan_destroy(p) == 0  # NULL is accepted


@pytest.mark.parametrize("fn", ["ge_add_rmsnorm_run", "ge_add_rmsnorm_run_unfused"])
def test_add_rmsnorm_argument_checks(fn):
    run = getattr(ge.lib(), fn)
    f = ctypes.c_float(1e-6)
    a = ctypes.c_void_p(4096)
    assert run(0, 16, a, a, a, f, ctypes.c_void_p(8192), ctypes.c_void_p(1 << 20), None) == ge.ERR_INVALID_ARG
    assert run(1, 1 << 15, a, a, a, f, ctypes.c_void_p(8192), ctypes.c_void_p(1 << 20), None) == ge.ERR_UNSUPPORTED
    assert run(2, 16, a, None, a, f, a, ctypes.c_void_p(1 << 20), None) == ge.ERR_INVALID_ARG
    # out overlapping the input
    assert run(2, 16, a, a, a, f, a, a, None) == ge.ERR_INVALID_ARG
    # negative eps
    assert run(2, 16, a, a, a, ctypes.c_float(-1.0), ctypes.c_void_p(8192), ctypes.c_void_p(1 << 20), None) \
        == ge.ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ge, "lib_path", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ge, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        ge.lib()


@pytest.mark.skipif(_has_gpu(), reason="without a GPU every host-valid descriptor must stop at NO_DEVICE")
def test_random_descriptors_get_a_documented_status_and_a_message():
    # hypothesis-generated descriptors, garbage included: the planner never crashes, returns one of
    # the documented statuses (no plan can be made without a GPU) and always leaves a message
    hyp = pytest.importorskip("hypothesis")
    st = hyp.strategies

    @hyp.settings(max_examples=400, deadline=None, database=None)
    @hyp.given(kind=st.integers(-1, 4), M=st.integers(-2, 70000), N=st.integers(-2, 70000), K=st.integers(-2, 70000),
               a_type=st.integers(-1, 5), b_type=st.integers(-1, 5), c_type=st.integers(-1, 5),
               d_type=st.integers(-1, 5), bias_type=st.integers(-1, 5), r_type=st.integers(-1, 5),
               b_layout=st.integers(-1, 2), act=st.integers(-1, 5), flags=st.integers(0, 127),
               group=st.sampled_from([0, 16, 32, 64, 100, 128, 256, 512]), zero_point=st.integers(-2, 300),
               lda=st.sampled_from([0, 1, 7, 64, 4096, 100000]), ldb=st.sampled_from([0, 1, 7, 64, 4096, 100000]),
               beta=st.sampled_from([0.0, 0.5]))
    def check(kind, M, N, K, a_type, b_type, c_type, d_type, bias_type, r_type, b_layout, act, flags, group,
              zero_point, lda, ldb, beta):
        s = _plan_status(kind, M=M, N=N, K=K, a_type=a_type, b_type=b_type, c_type=c_type, d_type=d_type,
                         bias_type=bias_type, r_type=r_type, b_layout=b_layout, act=act, flags=flags,
                         group_size=group, zero_point=zero_point, lda=lda, ldb=ldb, beta=beta)
        assert s in (ge.ERR_INVALID_ARG, ge.ERR_UNSUPPORTED, ge.ERR_NO_DEVICE, ge.ERR_ALIGN)
        assert ge.lib().ge_last_error()

    check()
