"""The C-ABI library loads, exports every entry point declared in include/mx.h,
and rejects invalid arguments on the host with a status and a message (no GPU
work is launched for any of these calls)."""
import ctypes
import os
import re

import pytest

import mxfp4_microscaling_quantization_mx_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "mx.h")).read()
    return sorted(set(re.findall(r"^\s*(?:mx_status|size_t|const char\*)\s+(mx_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mx.LIB_PATH):
        pytest.skip("libmxfp4.so not built")
    return mx.load_library()


def test_header_declares_expected_entry_points():
    assert _declared() == sorted(mx.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_version(lib):
    assert b"libmxfp4" in lib.mx_version()


def _tensor(rows, K, block=0, codes=16, scales=16, ldc=None, lds=None):
    return mx.MxTensorC(codes, scales, rows, K, ldc if ldc is not None else K // 2,
                        lds if lds is not None else K // 32, block, 0)


def test_quantize_rejects_bad_arguments(lib):
    cfg = mx.QuantCfgC(0, 0, 0, 0, 0, 0, 0, 0)
    out = _tensor(32, 48)
    st = lib.mx_quantize(ctypes.c_void_p(16), 1, 32, 48, 48, ctypes.byref(cfg), ctypes.byref(out), None)
    assert st == mx.MX_ERR_INVALID_ARG
    assert b"multiple of 32" in lib.mx_last_error()
    for bad_rounding in (3, 7, -1):
        bad_cfg = mx.QuantCfgC(0, 0, bad_rounding, 0, 0, 0, 0, 0)
        out = _tensor(32, 64)
        st = lib.mx_quantize(ctypes.c_void_p(16), 1, 32, 64, 64, ctypes.byref(bad_cfg), ctypes.byref(out), None)
        assert st == mx.MX_ERR_INVALID_ARG and b"rounding" in lib.mx_last_error()
    bad_cfg = mx.QuantCfgC(0, 0, 7, 0, 0, 0, 0, 0)
    out = _tensor(32, 64)
    st = lib.mx_quantize(ctypes.c_void_p(16), 1, 32, 64, 64, ctypes.byref(bad_cfg), ctypes.byref(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"rounding" in lib.mx_last_error()
    bad_cfg = mx.QuantCfgC(0, 0, 0, 0, 0, 3, 0, 0)
    st = lib.mx_quantize(ctypes.c_void_p(16), 1, 32, 64, 64, ctypes.byref(bad_cfg), ctypes.byref(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"scale_mode" in lib.mx_last_error()
    # output shape must match the axis
    cfg = mx.QuantCfgC(1, 0, 0, 0, 0, 0, 0, 0)
    out = _tensor(32, 64)
    st = lib.mx_quantize(ctypes.c_void_p(16), 1, 32, 64, 64, ctypes.byref(cfg), ctypes.byref(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"expected" in lib.mx_last_error()
    # misaligned source
    cfg = mx.QuantCfgC(0, 0, 0, 0, 0, 0, 0, 0)
    out = _tensor(32, 64)
    st = lib.mx_quantize(ctypes.c_void_p(18), 1, 32, 64, 64, ctypes.byref(cfg), ctypes.byref(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"aligned" in lib.mx_last_error()
    # along dim 0 any element-aligned source will do, but not a split element
    cfg = mx.QuantCfgC(1, 0, 0, 0, 0, 0, 0, 0)
    out = _tensor(64, 32)
    st = lib.mx_quantize(ctypes.c_void_p(17), 1, 32, 64, 64, ctypes.byref(cfg), ctypes.byref(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"element size" in lib.mx_last_error()
    st = lib.mx_quantize(ctypes.c_void_p(18), 0, 32, 64, 64, ctypes.byref(cfg), ctypes.byref(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"element size" in lib.mx_last_error()
    # 2-D blocks need rows % 32 == 0
    cfg = mx.QuantCfgC(0, 1, 0, 0, 0, 0, 0, 0)
    out = _tensor(48, 64, block=1)
    st = lib.mx_quantize(ctypes.c_void_p(16), 1, 48, 64, 64, ctypes.byref(cfg), ctypes.byref(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"2-D" in lib.mx_last_error()
    # empty input is a no-op
    out = _tensor(0, 64)
    cfg = mx.QuantCfgC(0, 0, 0, 0, 0, 0, 0, 0)
    assert lib.mx_quantize(None, 1, 0, 64, 64, ctypes.byref(cfg), ctypes.byref(out), None) == mx.MX_OK


def test_quantize_gather_rejects_bad_arguments(lib):
    cfg = mx.QuantCfgC(0, 0, 0, 0, 0, 0, 0, 0)
    out = _tensor(8, 64)
    src, rows = ctypes.c_void_p(16), ctypes.c_void_p(16)
    # only 1-D blocks along the last dim
    for bad in (mx.QuantCfgC(1, 0, 0, 0, 0, 0, 0, 0), mx.QuantCfgC(0, 1, 0, 0, 0, 0, 0, 0)):
        st = lib.mx_quantize_gather(src, 1, 32, 64, 64, rows, 8, ctypes.byref(bad), ctypes.byref(out), None)
        assert st == mx.MX_ERR_UNSUPPORTED and b"1-D" in lib.mx_last_error()
    bad = mx.QuantCfgC(0, 0, 0, 0, 0, 9, 0, 0)
    st = lib.mx_quantize_gather(src, 1, 32, 64, 64, rows, 8, ctypes.byref(bad), ctypes.byref(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"scale_mode" in lib.mx_last_error()
    st = lib.mx_quantize_gather(src, 1, 32, 48, 48, rows, 8, ctypes.byref(cfg), ctypes.byref(_tensor(8, 48)), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"multiple of 32" in lib.mx_last_error()
    st = lib.mx_quantize_gather(src, 1, 32, 64, 64, rows, 9, ctypes.byref(cfg), ctypes.byref(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"expected" in lib.mx_last_error()
    st = lib.mx_quantize_gather(src, 1, 32, 64, 64, None, 8, ctypes.byref(cfg), ctypes.byref(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"rows" in lib.mx_last_error()
    st = lib.mx_quantize_gather(ctypes.c_void_p(18), 1, 32, 64, 64, rows, 8, ctypes.byref(cfg), ctypes.byref(out),
                                None)
    assert st == mx.MX_ERR_INVALID_ARG and b"aligned" in lib.mx_last_error()
    # no output rows is a no-op
    assert lib.mx_quantize_gather(None, 1, 32, 64, 64, None, 0, ctypes.byref(cfg), ctypes.byref(_tensor(0, 64)),
                                  None) == mx.MX_OK


def test_transpose_rejects_bad_arguments(lib):
    a = _tensor(64, 96, block=1)
    out = _tensor(96, 64, block=1)
    for bad_in, bad_out in ((_tensor(64, 96), out), (a, _tensor(96, 64))):
        st = lib.mx_transpose(ctypes.byref(bad_in), ctypes.byref(bad_out), None)
        assert st == mx.MX_ERR_UNSUPPORTED and b"2-D" in lib.mx_last_error()
    st = lib.mx_transpose(ctypes.byref(a), ctypes.byref(_tensor(64, 96, block=1)), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"expected" in lib.mx_last_error()
    st = lib.mx_transpose(ctypes.byref(a), ctypes.byref(_tensor(96, 64, codes=8, block=1)), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"aligned" in lib.mx_last_error()
    assert lib.mx_transpose(ctypes.byref(_tensor(0, 64, block=1)), ctypes.byref(_tensor(64, 0, block=1)),
                            None) == mx.MX_OK


def test_element_types_are_validated(lib):
    """mx_tensor.elem: unknown values are refused everywhere; MXFP8/MXFP6 rows
    need K*bits/8 bytes and 2-D blocks whole 32-row groups; the gather is
    MXFP4-only; the transpose keeps the element type; the grouped GEMM checks
    K for any type."""
    cfg = mx.QuantCfgC(0, 0, 0, 0, 0, 0, 0, 0)
    bad = _tensor(32, 64)
    bad.elem = 9
    st = lib.mx_quantize(ctypes.c_void_p(16), 1, 32, 64, 64, ctypes.byref(cfg), ctypes.byref(bad), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"element type" in lib.mx_last_error()
    fp8 = _tensor(32, 64, ldc=48)          # needs 64 bytes per row
    fp8.elem = 1
    st = lib.mx_quantize(ctypes.c_void_p(16), 1, 32, 64, 64, ctypes.byref(cfg), ctypes.byref(fp8), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"strides" in lib.mx_last_error()
    fp6_2d = _tensor(48, 64, ldc=48, block=1)
    fp6_2d.elem = 3
    cfg2 = mx.QuantCfgC(0, 1, 0, 0, 0, 0, 0, 0)
    st = lib.mx_quantize(ctypes.c_void_p(16), 1, 48, 64, 64, ctypes.byref(cfg2), ctypes.byref(fp6_2d), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"2-D" in lib.mx_last_error()
    fp6 = _tensor(8, 64, ldc=48)
    fp6.elem = 3
    st = lib.mx_quantize_gather(ctypes.c_void_p(16), 1, 32, 64, 64, ctypes.c_void_p(16), 8, ctypes.byref(cfg),
                                ctypes.byref(fp6), None)
    assert st == mx.MX_ERR_UNSUPPORTED and b"MXFP4" in lib.mx_last_error()
    t_in = _tensor(64, 96, ldc=96, block=1)
    t_in.elem = 1
    st = lib.mx_transpose(ctypes.byref(t_in), ctypes.byref(_tensor(96, 64, block=1)), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"element types differ" in lib.mx_last_error()
    a = _tensor(64, 64, ldc=64)
    a.elem = 2
    b = _tensor(64, 96, block=1)
    st = lib.mx_grouped_gemm(ctypes.byref(a), ctypes.c_void_p(16), 2, ctypes.byref(b), 0, 0, ctypes.c_void_p(16), 0, 64,
                             None)
    assert st == mx.MX_ERR_INVALID_ARG and b"A.K" in lib.mx_last_error()


def test_gemm_rejects_bad_arguments(lib):
    a = _tensor(32, 64)
    b = _tensor(32, 96)
    st = lib.mx_gemm(ctypes.byref(a), ctypes.byref(b), ctypes.c_void_p(16), 0, 32, None, 0, None)
    assert st == mx.MX_ERR_INVALID_ARG and b"A.K" in lib.mx_last_error()
    b = _tensor(32, 64)
    st = lib.mx_gemm(ctypes.byref(a), ctypes.byref(b), ctypes.c_void_p(16), 0, 16, None, 0, None)
    assert st == mx.MX_ERR_INVALID_ARG and b"ldc" in lib.mx_last_error()
    st = lib.mx_gemm(ctypes.byref(a), ctypes.byref(b), None, 0, 32, None, 0, None)
    assert st == mx.MX_ERR_INVALID_ARG and b"null C" in lib.mx_last_error()
    a_mis = _tensor(32, 64, codes=8)
    st = lib.mx_gemm(ctypes.byref(a_mis), ctypes.byref(b), ctypes.c_void_p(16), 0, 32, None, 0, None)
    assert st == mx.MX_ERR_INVALID_ARG and b"aligned" in lib.mx_last_error()
    st = lib.mx_gemm(ctypes.byref(a), ctypes.byref(b), ctypes.c_void_p(16), 5, 32, None, 0, None)
    assert st == mx.MX_ERR_INVALID_ARG and b"dtype" in lib.mx_last_error()


def test_gemm_workspace_contract(lib):
    """Shapes split along K report their workspace size; mx_gemm then refuses
    a missing, short or misaligned workspace before launching anything."""
    assert lib.mx_gemm_workspace_size(2880, 2880, 16384) > 0          # weight gradient: 144 tiles
    assert lib.mx_gemm_workspace_size(16384, 5760, 2880) == 0         # fprop: whole tiles
    assert lib.mx_gemm_workspace_size(2880, 2880, 0) == 0
    assert lib.mx_gemm_workspace_size(0, 2880, 16384) == 0
    need = lib.mx_gemm_workspace_size(2880, 2880, 16384)
    a = _tensor(2880, 16384, codes=1 << 20, scales=1 << 21, ldc=8192, lds=512)
    b = _tensor(2880, 16384, codes=1 << 22, scales=1 << 23, ldc=8192, lds=512)
    C = ctypes.c_void_p(1 << 24)
    for ws, nbytes in [(None, 0), (ctypes.c_void_p(1 << 26), need - 1), (ctypes.c_void_p((1 << 26) + 16), need)]:
        st = lib.mx_gemm(ctypes.byref(a), ctypes.byref(b), C, 0, 2880, ws, nbytes, None)
        assert st == mx.MX_ERR_INVALID_ARG and b"workspace" in lib.mx_last_error()


def test_quantize_scatter_rejects_bad_arguments(lib):
    """Every rejection happens on the host, before any launch."""
    B = ctypes.byref
    cfg = mx.QuantCfgC(0, 0, 0, 0, 0, 0, 0, 0)
    sr = mx.QuantCfgC(0, 0, 1, 0, 0, 0, 0, 0)
    out = _tensor(64, 64)
    P = ctypes.c_void_p
    st = lib.mx_quantize_scatter(P(16), 1, 16, 64, 64, P(16), 4, B(sr), B(out), None)
    assert st == mx.MX_ERR_UNSUPPORTED and b"RNE" in lib.mx_last_error()
    sr8 = mx.QuantCfgC(0, 0, 2, 0, 0, 0, 0, 0)
    st = lib.mx_quantize_scatter(P(16), 1, 16, 64, 64, P(16), 4, B(sr8), B(out), None)
    assert st == mx.MX_ERR_UNSUPPORTED and b"RNE" in lib.mx_last_error()
    st = lib.mx_quantize_scatter(P(16), 1, 16, 64, 64, P(16), 4, B(mx.QuantCfgC(1, 0, 0, 0, 0, 0, 0, 0)), B(out),
                                 None)
    assert st == mx.MX_ERR_UNSUPPORTED
    st = lib.mx_quantize_scatter(P(16), 1, 16, 96, 96, P(16), 4, B(cfg), B(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"out.K" in lib.mx_last_error()
    st = lib.mx_quantize_scatter(P(16), 1, 16, 64, 64, None, 4, B(cfg), B(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"dest" in lib.mx_last_error()
    st = lib.mx_quantize_scatter(P(16), 1, 16, 64, 60, P(16), 4, B(cfg), B(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"ld_src" in lib.mx_last_error()
    st = lib.mx_quantize_scatter(P(16), 1, 16, 64, 64, P(16), -1, B(cfg), B(out), None)
    assert st == mx.MX_ERR_INVALID_ARG
    assert lib.mx_quantize_scatter(P(16), 1, 16, 64, 64, P(16), 0, B(cfg), B(out), None) == mx.MX_OK


def test_gemm_quantize_rejects_bad_arguments(lib):
    """Every rejection happens on the host, before any launch."""
    B = ctypes.byref
    a, b, out = _tensor(256, 64), _tensor(288, 64), _tensor(256, 288)
    st = lib.mx_gemm_quantize(B(a), B(_tensor(288, 96)), 0, B(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"A.K" in lib.mx_last_error()
    st = lib.mx_gemm_quantize(B(a), B(b), 7, B(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"scale mode" in lib.mx_last_error()
    st = lib.mx_gemm_quantize(B(a), B(b), 0, B(_tensor(256, 320)), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"out is" in lib.mx_last_error()
    st = lib.mx_gemm_quantize(B(a), B(b), 0, B(_tensor(256, 288, block=1)), None)
    assert st == mx.MX_ERR_UNSUPPORTED and b"1-D" in lib.mx_last_error()
    a8 = _tensor(256, 64, ldc=64)
    a8.elem = 1
    st = lib.mx_gemm_quantize(B(a8), B(b), 0, B(out), None)
    assert st == mx.MX_ERR_UNSUPPORTED and b"MXFP4" in lib.mx_last_error()
    # dense scale strides (not a multiple of 16) are not taken by the 256x256 pipeline
    st = lib.mx_gemm_quantize(B(a), B(b), 0, B(out), None)
    assert st == mx.MX_ERR_UNSUPPORTED and b"M, N >= 256" in lib.mx_last_error()
    st = lib.mx_gemm_quantize(B(_tensor(128, 64, lds=16)), B(_tensor(288, 64, lds=16)), 0,
                              B(_tensor(128, 288)), None)
    assert st == mx.MX_ERR_UNSUPPORTED
    assert lib.mx_gemm_quantize(B(_tensor(0, 64)), B(b), 0, B(_tensor(0, 288)), None) == mx.MX_OK


def test_grouped_gemm_quantize_rejects_bad_arguments(lib):
    """Every rejection happens on the host, before any launch."""
    B = ctypes.byref
    P = ctypes.c_void_p
    a, b, out = _tensor(300, 64), _tensor(288, 64, block=1), _tensor(300, 288)
    st = lib.mx_grouped_gemm_quantize(B(a), None, 2, B(b), 1024, 64, 0, B(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"offsets" in lib.mx_last_error()
    st = lib.mx_grouped_gemm_quantize(B(a), P(16), 0, B(b), 1024, 64, 0, B(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"E=0" in lib.mx_last_error()
    st = lib.mx_grouped_gemm_quantize(B(a), P(16), 2, B(b), 1024, 64, 9, B(out), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"scale mode" in lib.mx_last_error()
    st = lib.mx_grouped_gemm_quantize(B(a), P(16), 2, B(b), 1024, 64, 0, B(_tensor(300, 320)), None)
    assert st == mx.MX_ERR_INVALID_ARG and b"out is" in lib.mx_last_error()
    st = lib.mx_grouped_gemm_quantize(B(_tensor(320, 64, block=1)), P(16), 2, B(b), 1024, 64, 0,
                                      B(_tensor(320, 288)), None)
    assert st == mx.MX_ERR_UNSUPPORTED and b"1-D" in lib.mx_last_error()
    st = lib.mx_grouped_gemm_quantize(B(a), P(16), 2, B(b), 1024, 64, 0, B(out), None)
    assert st == mx.MX_ERR_UNSUPPORTED and b"N >= 256" in lib.mx_last_error()   # dense scale strides
    assert lib.mx_grouped_gemm_quantize(B(_tensor(0, 64)), P(16), 2, B(b), 1024, 64, 0, B(_tensor(0, 288)),
                                        None) == mx.MX_OK


def test_grouped_gemm_rejects_bad_arguments(lib):
    a = _tensor(64, 64)
    b = _tensor(32, 64, block=1)
    st = lib.mx_grouped_gemm(ctypes.byref(a), None, 2, ctypes.byref(b), 1024, 64,
                             ctypes.c_void_p(16), 1, 32, None)
    assert st == mx.MX_ERR_INVALID_ARG and b"offsets" in lib.mx_last_error()
    st = lib.mx_grouped_gemm(ctypes.byref(a), ctypes.c_void_p(16), 0, ctypes.byref(b), 1024, 64,
                             ctypes.c_void_p(16), 1, 32, None)
    assert st == mx.MX_ERR_INVALID_ARG and b"E=0" in lib.mx_last_error()
    a2 = _tensor(64, 64, block=1)
    st = lib.mx_grouped_gemm(ctypes.byref(a2), ctypes.c_void_p(16), 2, ctypes.byref(b), 1024, 64,
                             ctypes.c_void_p(16), 1, 32, None)
    assert st == mx.MX_ERR_UNSUPPORTED


def test_dequantize_rejects_bad_arguments(lib):
    t = _tensor(32, 64)
    st = lib.mx_dequantize(ctypes.byref(t), 0, 0, ctypes.c_void_p(16), 0, 32, None)
    assert st == mx.MX_ERR_INVALID_ARG and b"ld_dst" in lib.mx_last_error()
    st = lib.mx_dequantize(ctypes.byref(t), 2, 0, ctypes.c_void_p(16), 0, 64, None)
    assert st == mx.MX_ERR_INVALID_ARG
    assert lib.mx_gemm_workspace_size(16384, 5760, 2880) >= 0


def test_last_error_cleared_on_success(lib):
    out = _tensor(0, 64)
    cfg = mx.QuantCfgC(0, 0, 0, 0, 0, 0, 0, 0)
    bad = mx.QuantCfgC(0, 0, 9, 0, 0, 0, 0, 0)
    lib.mx_quantize(None, 1, 0, 64, 64, ctypes.byref(bad), ctypes.byref(out), None)
    assert lib.mx_last_error() != b""
    lib.mx_quantize(None, 1, 0, 64, 64, ctypes.byref(cfg), ctypes.byref(out), None)
    assert lib.mx_last_error() == b""


def test_gemm_fused_quant_a_rejects_bad_arguments(lib):
    """Host-side checks of mx_gemm_fused_quant_a, before any launch."""
    B = ctypes.byref
    P = ctypes.c_void_p
    f = lib.mx_gemm_fused_quant_a
    cfg = mx.QuantCfgC(0, 0, 0, 0, 0, 0, 0, 0)
    b = _tensor(64, 96)
    ok = (P(16), mx.MX_DT_BF16, 256, 96, 96, B(cfg), B(b), P(16), 0, 64, None)

    def call(**kw):
        args = list(ok)
        names = ["a", "a_dtype", "M", "K", "lda", "cfg", "b", "c", "c_dtype", "ldc", "stream"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(a_dtype=0) == mx.MX_ERR_UNSUPPORTED and b"bf16" in lib.mx_last_error()
    assert call(a_dtype=5) == mx.MX_ERR_INVALID_ARG
    for bad in (mx.QuantCfgC(1, 0, 0, 0, 0, 0, 0, 0), mx.QuantCfgC(0, 1, 0, 0, 0, 0, 0, 0),
                mx.QuantCfgC(0, 0, 1, 0, 0, 0, 0, 0), mx.QuantCfgC(0, 0, 2, 0, 0, 0, 0, 0)):
        assert call(cfg=B(bad)) == mx.MX_ERR_UNSUPPORTED and b"RNE" in lib.mx_last_error()
    assert call(cfg=B(mx.QuantCfgC(0, 0, 0, 0, 0, 3, 0, 0))) == mx.MX_ERR_INVALID_ARG
    assert call(cfg=None) == mx.MX_ERR_INVALID_ARG
    assert call(K=80, lda=80) == mx.MX_ERR_INVALID_ARG and b"multiple of 32" in lib.mx_last_error()
    assert call(K=128, lda=128) == mx.MX_ERR_INVALID_ARG and b"B.K" in lib.mx_last_error()
    assert call(lda=64) == mx.MX_ERR_INVALID_ARG and b"lda" in lib.mx_last_error()
    assert call(lda=100) == mx.MX_ERR_INVALID_ARG and b"aligned" in lib.mx_last_error()
    assert call(a=P(18)) == mx.MX_ERR_INVALID_ARG and b"aligned" in lib.mx_last_error()
    assert call(a=None) == mx.MX_ERR_INVALID_ARG
    assert call(c=None) == mx.MX_ERR_INVALID_ARG
    assert call(ldc=32) == mx.MX_ERR_INVALID_ARG and b"ldc" in lib.mx_last_error()
    assert call(c_dtype=7) == mx.MX_ERR_INVALID_ARG
    fp8 = mx.MxTensorC(16, 16, 64, 96, 96, 3, 0, 1)
    assert call(b=B(fp8)) == mx.MX_ERR_UNSUPPORTED and b"MXFP4" in lib.mx_last_error()
    assert call(M=-1) == mx.MX_ERR_INVALID_ARG
    assert call(M=0, a=None, c=None) == mx.MX_OK          # empty: nothing launched


def test_clip_count_rejects_bad_arguments(lib):
    """Host-side checks of mx_clip_count, before any launch."""
    B = ctypes.byref
    P = ctypes.c_void_p
    f = lib.mx_clip_count
    cfg = mx.QuantCfgC(0, 0, 0, 0, 0, 0, 0, 0)
    ok = (P(16), mx.MX_DT_BF16, 64, 96, 96, B(cfg), 0, P(64), None)

    def call(**kw):
        args = list(ok)
        names = ["src", "dtype", "R", "C", "ld", "cfg", "elem", "count", "stream"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(cfg=None) == mx.MX_ERR_INVALID_ARG
    assert call(dtype=5) == mx.MX_ERR_INVALID_ARG and b"dtype" in lib.mx_last_error()
    assert call(cfg=B(mx.QuantCfgC(2, 0, 0, 0, 0, 0, 0, 0))) == mx.MX_ERR_INVALID_ARG
    assert call(cfg=B(mx.QuantCfgC(0, 2, 0, 0, 0, 0, 0, 0))) == mx.MX_ERR_INVALID_ARG
    assert call(cfg=B(mx.QuantCfgC(0, 0, 0, 2, 0, 0, 0, 0))) == mx.MX_ERR_INVALID_ARG
    assert call(cfg=B(mx.QuantCfgC(0, 0, 0, 0, 0, 3, 0, 0))) == mx.MX_ERR_INVALID_ARG
    for e in (-1, 5):
        assert call(elem=e) == mx.MX_ERR_INVALID_ARG and b"element" in lib.mx_last_error()
    assert call(C=80, ld=80) == mx.MX_ERR_INVALID_ARG and b"multiple of 32" in lib.mx_last_error()
    assert call(cfg=B(mx.QuantCfgC(0, 1, 0, 0, 0, 0, 0, 0)), R=48) == mx.MX_ERR_INVALID_ARG
    assert b"2-D" in lib.mx_last_error()
    assert call(cfg=B(mx.QuantCfgC(1, 1, 0, 0, 0, 0, 0, 0)), R=64, C=48, ld=48) == mx.MX_ERR_INVALID_ARG
    assert call(count=None) == mx.MX_ERR_INVALID_ARG and b"count" in lib.mx_last_error()
    assert call(count=P(68)) == mx.MX_ERR_INVALID_ARG and b"aligned" in lib.mx_last_error()
    assert call(src=P(18)) == mx.MX_ERR_INVALID_ARG and b"aligned" in lib.mx_last_error()
    assert call(ld=100) == mx.MX_ERR_INVALID_ARG and b"aligned" in lib.mx_last_error()
    assert call(ld=64) == mx.MX_ERR_INVALID_ARG and b"ld_src" in lib.mx_last_error()
    assert call(src=None) == mx.MX_ERR_INVALID_ARG
    assert call(R=-1) == mx.MX_ERR_INVALID_ARG
    assert call(R=0, src=None) == mx.MX_OK               # empty: nothing launched
