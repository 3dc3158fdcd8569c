"""C-ABI tests that need no GPU: the library loads, exports every function that
include/pql.h declares, answers size queries, and rejects bad arguments before
touching a device.  No compute is launched here."""
import ctypes
import os
import re

import pytest
import torch

import precision_quantized_linear_amd as pql

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pql.h")

S = pql.SCHEMES
A, W = pql.ROLES["activation"], pql.ROLES["weight"]


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pql_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = pql.lib()
    names = header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), f"{n} declared in pql.h but not exported"
    assert L.pql_version() == 2


def _sizes(scheme, role, rows, cols):
    return pql.quantized_sizes(scheme, role, rows, cols)


def test_quantized_sizes():
    assert _sizes("fp8_tensor", "activation", 256, 512) == (256 * 512, 4, 0)
    assert _sizes("fp8_row", "weight", 12288, 3072) == (12288 * 3072, 4 * 12288, 0)
    assert _sizes("fp8_block128", "activation", 8192, 5120) == (8192 * 5120, 4 * 8192 * 40, 0)
    assert _sizes("fp8_block128", "weight", 13824, 5120) == (13824 * 5120, 4 * 108 * 40, 0)
    assert _sizes("mxfp8", "activation", 20280, 5120) == (20280 * 5120, 20280 * 160, 0)
    assert _sizes("mxfp4", "weight", 5120, 5120) == (5120 * 2560, 5120 * 160, 0)
    # packed exponents round each row up to whole chunks (4 bytes MXFP8, 8 bytes MXFP4)
    assert _sizes("mxfp8", "activation", 3, 96) == (3 * 96, 3 * 4, 0)
    assert _sizes("mxfp4", "activation", 3, 384) == (3 * 192, 3 * 16, 0)
    assert _sizes("w4a16_asym", "weight", 12288, 3072) == (12288 * 1536, 2 * 12288 * 24, 12288 * 24)
    assert _sizes("int8_row", "activation", 4096, 3072) == (4096 * 3072, 4 * 4096, 0)
    assert _sizes("int8_row", "weight", 12288, 3072) == (12288 * 3072, 4 * 12288, 0)
    # dual-scale MXFP4: fine exponents, then (256-byte aligned) the coarse fp32 scales
    assert _sizes("mxfp4_dual", "activation", 20280, 5120) == (20280 * 2560, 20280 * 160 + 4 * 20280 * 10, 0)
    assert _sizes("mxfp4_dual", "weight", 3, 512) == (3 * 256, 256 + 4 * 3, 0)


@pytest.mark.parametrize("scheme,role,rows,cols", [
    ("fp8_row", "activation", 4, 48),         # K not a multiple of 32
    ("mxfp8", "activation", 4, 16),
    ("fp8_block128", "activation", 4, 96),    # K not a multiple of 128
    ("fp8_block128", "weight", 64, 128),      # weight rows not a multiple of 128
    ("w4a16_asym", "weight", 4, 64),
    ("fp8_row", "activation", -1, 64),
    ("mxfp4_dual", "activation", 4, 256),     # K not a multiple of 512
    ("fp8_row", "activation", 4, 0),
    ("fp8_block128", "weight", (1 << 31) - 128, 1 << 20),   # 2^51 elements
])
def test_invalid_shapes_rejected(scheme, role, rows, cols):
    with pytest.raises(ValueError):
        _sizes(scheme, role, rows, cols)


def test_unsupported_combinations():
    with pytest.raises(NotImplementedError):
        _sizes("w4a16_asym", "activation", 4, 128)
    with pytest.raises(NotImplementedError):
        _sizes(9, "activation", 4, 128)
    with pytest.raises(NotImplementedError):
        _sizes("fp8_row", 2, 4, 128)


def test_workspace_sizes():
    assert pql.workspace_size("quantize", "fp8_tensor") == 4096
    assert pql.workspace_size("quantize", "mxfp8") == 0
    ws = pql.workspace_size("qlinear", "mxfp8", "activation", 20280, 5120, 5120)
    assert ws == 20280 * 5120 + ((20280 * 160 + 255) // 256) * 256
    assert pql.workspace_size("qlinear", "w4a16_asym", "activation", 16, 12288, 3072) == 0
    # a few tokens under the FP8 / int8 schemes: the fused kernel needs no workspace
    for s in ("fp8_tensor", "fp8_row", "fp8_block128", "int8_row"):
        assert pql.workspace_size("qlinear", s, "activation", 16, 12288, 3072) == 0
        assert pql.workspace_size("qlinear", s, "activation", 17, 12288, 3072) >= 17 * 3072
    assert pql.workspace_size("qlinear", "mxfp8", "activation", 1, 12288, 3072) > 3072


def test_small_m_qlinear_runs_the_fused_kernel():
    for s in ("fp8_tensor", "fp8_row", "fp8_block128", "int8_row"):
        for M in (1, 4, 5, 16):
            assert pql.kernel_name("qlinear", s, "activation", M, 3072, 3072) == f"k_qlinear_few<{s}>"
            assert not pql.kernel_name("qgemm", s, "activation", M, 3072, 3072).startswith("k_qlinear")
        # the staged activation: K <= 4096 (8192 for one token); longer K casts in the main loop
        assert pql.kernel_name("qlinear", s, "activation", 1, 3072, 8192) == f"k_qlinear_few<{s}>"
        assert pql.kernel_name("qlinear", s, "activation", 1, 3072, 8320) == f"k_qlinear_small<{s}>"
        assert pql.kernel_name("qlinear", s, "activation", 16, 3072, 4096) == f"k_qlinear_few<{s}>"
        assert pql.kernel_name("qlinear", s, "activation", 16, 3072, 4224) == f"k_qlinear_small<{s}>"
        assert not pql.kernel_name("qlinear", s, "activation", 17, 3072, 3072).startswith("k_qlinear")
    for s in ("mxfp8", "mxfp4", "mxfp4_dual", "w4a16_asym"):
        assert not pql.kernel_name("qlinear", s, "activation", 1, 3072, 3072).startswith("k_qlinear")
    with pytest.raises(ValueError):
        pql.workspace_size("qlinear", "fp8_row", "activation", 16, 128, 100)


def test_kernel_names_distinct_per_scheme():
    names = {s: pql.kernel_name("qgemm", s, "activation", 4096, 4096, 4096) for s in S}
    assert all(names.values())
    fp = [names[s] for s in ("fp8_row", "fp8_block128", "mxfp8", "mxfp4", "int8_row")]
    assert len(set(fp)) == 5
    assert pql.kernel_name("quantize", "int8_row", "activation") == "k_fp8_row<int8>"
    assert pql.kernel_name("quantize", "w4a16_asym", "activation") == ""
    assert pql.kernel_name("qgemm", "w4a16_asym", "activation", 1, 12288, 3072).startswith("k_w4a16_gemv")
    assert pql.kernel_name("qgemm", "w4a16_asym", "activation", 16, 12288, 3072).startswith("k_w4a16_gemv")
    assert pql.kernel_name("qgemm", "w4a16_asym", "activation", 32, 12288, 3072).startswith("k_w4a16_small")
    assert pql.kernel_name("qgemm", "w4a16_asym", "activation", 4096, 12288, 3072).startswith("k_w4a16_mm")
    assert pql.kernel_name("qgemm", "w4a16_asym", "activation", 256, 12288, 3072).startswith("k_w4a16_mm")
    # N not a multiple of 4 (dword scale loads of a tile's rows) keeps the older tile kernel
    assert pql.kernel_name("qgemm", "w4a16_asym", "activation", 256, 12290, 3072).startswith("k_w4a16_tile")


# ----------------------------------------------------------------- validation before launch
# Host buffers stand in for device pointers: every call below must fail in
# validation, before any device is touched.
_buf = (ctypes.c_uint8 * 4096 * 64)()
_base = (ctypes.addressof(_buf) + 255) & ~255


def _p(off=0):
    return _base + off


def _quantize(scheme=S["fp8_row"], role=A, x=None, rows=16, cols=128, ldx=128, codes=None, scales=None,
              zeros=None, ws=None, wsb=0):
    L = pql.lib()
    return L.pql_quantize(scheme, role, _p() if x is None else x, rows, cols, ldx,
                          _p(4096) if codes is None else codes, _p(8192) if scales is None else scales,
                          zeros, ws, wsb, None)


def test_quantize_validation():
    assert _quantize(x=0) == pql.PQL_ERR_INVALID_ARGUMENT                  # NULL x
    assert _quantize(ldx=120) == pql.PQL_ERR_INVALID_ARGUMENT              # ldx < cols
    assert _quantize(ldx=132) == pql.PQL_ERR_INVALID_ARGUMENT              # ldx not a multiple of 8
    assert _quantize(x=_p(4)) == pql.PQL_ERR_INVALID_ARGUMENT              # misaligned
    assert _quantize(cols=100) == pql.PQL_ERR_INVALID_ARGUMENT
    assert _quantize(scheme=S["w4a16_asym"], role=A) == pql.PQL_ERR_UNSUPPORTED
    assert _quantize(scheme=S["w4a16_asym"], role=W, zeros=None) == pql.PQL_ERR_INVALID_ARGUMENT
    assert _quantize(scheme=S["fp8_tensor"], ws=None) == pql.PQL_ERR_WORKSPACE
    assert _quantize(scheme=S["fp8_tensor"], ws=_p(16384), wsb=64) == pql.PQL_ERR_WORKSPACE
    assert _quantize(scheme=9) == pql.PQL_ERR_UNSUPPORTED
    assert _quantize(rows=0) == pql.PQL_OK                                 # empty: no-op
    assert _quantize(ldx=(1 << 63) - 8) == pql.PQL_ERR_INVALID_ARGUMENT    # row offsets would overflow
    assert _quantize(rows=1 << 20, ldx=1 << 21) == pql.PQL_ERR_INVALID_ARGUMENT   # span over 2^40 elements
    assert "ldx" in _last_error_after(lambda: _quantize(ldx=120))


def _last_error_after(fn):
    fn()
    return pql.lib().pql_last_error().decode()


def test_qgemm_validation():
    L = pql.lib()
    g = lambda scheme=S["fp8_row"], a=_p(), sa=_p(1024), wc=_p(2048), ws=_p(3072), wz=None, M=16, N=256, K=256, \
        c=_p(8192), ldc=256: L.pql_qgemm(scheme, a, sa, wc, ws, wz, M, N, K, c, ldc, None)
    assert g(K=200) == pql.PQL_ERR_INVALID_ARGUMENT
    assert g(N=0) == pql.PQL_ERR_INVALID_ARGUMENT
    assert g(ldc=100) == pql.PQL_ERR_INVALID_ARGUMENT
    assert g(sa=None) == pql.PQL_ERR_INVALID_ARGUMENT
    assert g(scheme=S["w4a16_asym"], wz=None) == pql.PQL_ERR_INVALID_ARGUMENT
    assert g(scheme=S["fp8_block128"], N=200, ldc=200) == pql.PQL_ERR_INVALID_ARGUMENT
    assert g(a=_p(8)) == pql.PQL_ERR_INVALID_ARGUMENT
    assert g(scheme=11) == pql.PQL_ERR_UNSUPPORTED
    assert g(scheme=S["w4a16_asym"], wz=_p(4100)) == pql.PQL_ERR_INVALID_ARGUMENT   # misaligned zero-points
    assert g(M=1 << 30, N=1 << 30, ldc=1 << 30) == pql.PQL_ERR_INVALID_ARGUMENT      # 2^48 output tiles
    assert g(M=0) == pql.PQL_OK
    assert g(ldc=(1 << 63) - 1) == pql.PQL_ERR_INVALID_ARGUMENT               # row offsets would overflow


def test_qlinear_validation():
    L = pql.lib()
    q = lambda scheme=S["mxfp8"], M=16, K=256, lda=256, N=256, ws=_p(16384), wsb=64: L.pql_qlinear(
        scheme, _p(), M, K, lda, _p(2048), _p(3072), None, N, _p(8192), N, ws, wsb, None)
    assert q(wsb=64) == pql.PQL_ERR_WORKSPACE
    assert q(ws=None, wsb=0) == pql.PQL_ERR_WORKSPACE
    assert q(lda=250) == pql.PQL_ERR_INVALID_ARGUMENT
    assert q(K=96, lda=96) == pql.PQL_ERR_INVALID_ARGUMENT
    # 1-16 tokens under FP8 / int8 run the fused kernel: no workspace, so a NULL one passes the checks
    for scheme in ("fp8_tensor", "fp8_row", "fp8_block128", "int8_row"):
        assert q(scheme=S[scheme], ws=None, wsb=0) != pql.PQL_ERR_WORKSPACE
    assert q(scheme=S["fp8_row"], M=17, ws=None, wsb=0) == pql.PQL_ERR_WORKSPACE


def test_dequantize_validation():
    L = pql.lib()
    d = lambda scheme=S["mxfp4"], role=A, codes=_p(), rows=16, cols=128, ldy=128: L.pql_dequantize(
        scheme, role, codes, _p(4096), None, rows, cols, _p(8192), ldy, None)
    assert d(codes=None) == pql.PQL_ERR_INVALID_ARGUMENT
    assert d(ldy=64) == pql.PQL_ERR_INVALID_ARGUMENT
    assert d(scheme=S["w4a16_sym"], role=W) == pql.PQL_ERR_INVALID_ARGUMENT     # zeros NULL
    assert d(scheme=S["w4a16_sym"], role=A) == pql.PQL_ERR_UNSUPPORTED


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-device path")
def test_valid_call_without_device_reports_hip_error():
    assert _quantize() == pql.PQL_ERR_HIP
    assert "HIP" in pql.lib().pql_last_error().decode() or "device" in pql.lib().pql_last_error().decode()


def test_python_api_errors_map_to_exceptions():
    with pytest.raises(ValueError):
        pql.quantize(torch.zeros(4, 128, dtype=torch.float32), "mxfp8")
    with pytest.raises(ValueError):
        pql.quantize(torch.zeros(4, 128, dtype=torch.bfloat16), "nvfp4")


def test_quantize_static_validation():
    L = pql.lib()
    q = lambda scheme=S["fp8_tensor"], role=A, x=_p(), rows=16, cols=128, ldx=128, scales=_p(4096), codes=_p(8192): \
        L.pql_quantize_static(scheme, role, x, rows, cols, ldx, scales, codes, None)
    assert q(scheme=S["fp8_row"]) == pql.PQL_ERR_UNSUPPORTED          # no static per-row scheme
    assert q(scheme=S["int8_row"]) == pql.PQL_ERR_UNSUPPORTED         # int8 is dynamic only
    assert q(scheme=S["mxfp8"]) == pql.PQL_ERR_UNSUPPORTED
    assert q(scales=None) == pql.PQL_ERR_INVALID_ARGUMENT
    assert q(scales=_p(4100)) == pql.PQL_ERR_INVALID_ARGUMENT         # misaligned
    assert q(scheme=S["fp8_block128"], cols=96, ldx=96) == pql.PQL_ERR_INVALID_ARGUMENT
    assert q(scheme=S["fp8_block128"], role=W, rows=64) == pql.PQL_ERR_INVALID_ARGUMENT
    assert q(rows=0) == pql.PQL_OK
    with pytest.raises(NotImplementedError):
        pql.quantize_static(torch.zeros(4, 128, dtype=torch.bfloat16), "fp8_row", "activation",
                            torch.ones(4, dtype=torch.float32))


def test_qgemm_ex_validation():
    L = pql.lib()
    g = lambda scheme=S["fp8_row"], alpha=1.0, bias=None, N=256, M=16: L.pql_qgemm_ex(
        scheme, _p(), _p(1024), _p(2048), _p(3072), None, M, N, 256, alpha, bias, _p(8192), N, None)
    assert g(scheme=S["mxfp8"], alpha=2.0) == pql.PQL_ERR_UNSUPPORTED     # no epilogue on MX
    assert g(scheme=S["mxfp4"], bias=_p(4096)) == pql.PQL_ERR_UNSUPPORTED
    assert g(alpha=float("nan")) == pql.PQL_ERR_INVALID_ARGUMENT
    assert g(alpha=float("inf")) == pql.PQL_ERR_INVALID_ARGUMENT
    assert g(bias=_p(4100)) == pql.PQL_ERR_INVALID_ARGUMENT               # misaligned bias
    assert g(bias=_p(4096), N=255) == pql.PQL_ERR_INVALID_ARGUMENT        # odd N with a bias
    assert g(scheme=S["mxfp8"], M=0) == pql.PQL_OK                        # alpha 1, no bias: any scheme
    assert g(scheme=S["int8_row"], alpha=0.5, bias=_p(4096), M=0) == pql.PQL_OK
    q = lambda scheme=S["fp8_tensor"], st=_p(512), alpha=1.0: L.pql_qlinear_ex(
        scheme, _p(), 16, 256, 256, st, _p(2048), _p(3072), None, 256, alpha, None, _p(8192), 256,
        _p(16384), 1 << 20, None)
    assert q(scheme=S["fp8_row"]) == pql.PQL_ERR_UNSUPPORTED             # static scales: tensor / block only
    assert q(scheme=S["int8_row"]) == pql.PQL_ERR_UNSUPPORTED
    assert q(st=_p(516)) == pql.PQL_ERR_INVALID_ARGUMENT
    assert q(scheme=S["w4a16_asym"], st=None, alpha=3.0) == pql.PQL_ERR_UNSUPPORTED


def test_qlinear_noalloc_limit_is_checked_before_any_device_call():
    """An activation whose codes and scales exceed the static buffer is refused by
    argument checks alone (no device is touched; the pointers are never read)."""
    L = pql.lib()
    cap = L.pql_noalloc_scratch_bytes()
    assert cap == 64 << 20
    K, N = 4096, 128
    M = cap // K + 1
    fake = 1 << 20                           # 16-byte aligned, never dereferenced on this path
    st = L.pql_qlinear_noalloc(S["fp8_row"], fake, M, K, K, None, fake, fake, None, N, ctypes.c_float(1.0), None,
                               fake, N, None)
    assert st == pql.PQL_ERR_WORKSPACE
    assert b"static scratch" in L.pql_last_error()


def test_layout_sizes():
    L = pql.lib()
    c, sc, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    for scheme, rows, cols, canon, packed in (("mxfp8", 3, 96, 3 * 3, 3 * 4), ("mxfp4", 5, 384, 5 * 12, 5 * 16),
                                              ("w4a16_asym", 4, 256, 2 * 4 * 2, 2 * 4 * 2),
                                              ("fp8_row", 7, 64, 7 * 4, 7 * 4)):
        for layout, want in ((0, canon), (1, packed)):
            assert L.pql_layout_sizes(S[scheme], W, layout, rows, cols, ctypes.byref(c), ctypes.byref(sc),
                                      ctypes.byref(z)) == pql.PQL_OK
            assert sc.value == want, (scheme, layout)
    assert L.pql_layout_sizes(S["mxfp8"], W, 2, 4, 64, None, None, None) == pql.PQL_ERR_INVALID_ARGUMENT


def test_repack_validation():
    L = pql.lib()
    fake = 1 << 20
    # unknown layout, NULL buffers, a transposing repack in place: refused before any device call
    assert L.pql_repack(S["mxfp8"], W, 0, 3, fake, None, fake + 4096, None, 4, 64, None) == pql.PQL_ERR_INVALID_ARGUMENT
    assert L.pql_repack(S["mxfp8"], W, 0, 1, None, None, fake, None, 4, 64, None) == pql.PQL_ERR_INVALID_ARGUMENT
    assert L.pql_repack(S["mxfp4"], W, 0, 1, fake, None, fake, None, 4, 64, None) == pql.PQL_ERR_INVALID_ARGUMENT
    assert L.pql_repack(S["w4a16_asym"], W, 1, 0, fake, None, fake + 4096, fake + 8192, 4, 128, None) \
        == pql.PQL_ERR_INVALID_ARGUMENT
    assert L.pql_repack(S["w4a16_asym"], A, 1, 0, fake, fake, fake, fake, 4, 128, None) == pql.PQL_ERR_UNSUPPORTED
    assert L.pql_repack(S["mxfp8"], W, 0, 1, fake, None, fake + 4096, None, 4, 48, None) == pql.PQL_ERR_INVALID_ARGUMENT


def _run_logged(code, env_value):
    """Run `code` in a fresh interpreter (PQL_LOG is read once per process) and return its stderr."""
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("PQL_LOG", None)
    if env_value is not None:
        env["PQL_LOG"] = env_value
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return r.stderr


LOG_CODE = """
import ctypes, precision_quantized_linear_amd as pql
L = pql.lib()
c_i64 = ctypes.c_int64
buf = ctypes.c_void_p(256)
S = pql.SCHEMES
# an empty GEMM (enqueues nothing), an unknown scheme, and a bad leading dimension
assert L.pql_qgemm(S["fp8_row"], buf, buf, buf, buf, None, c_i64(0), c_i64(256), c_i64(512), buf, c_i64(256), None) == 0
assert L.pql_qgemm(99, buf, buf, buf, buf, None, c_i64(8), c_i64(256), c_i64(512), buf, c_i64(256), None) != 0
assert L.pql_quantize(S["fp8_block128"], 0, buf, c_i64(4), c_i64(256), c_i64(100), buf, buf, None, None,
                      ctypes.c_size_t(0), None) != 0
"""


def test_pql_log_lines():
    """PQL_LOG=1 logs every entry-point call with its shape and outcome; unset, the library prints nothing."""
    err = _run_logged(LOG_CODE, "1")
    lines = [l for l in err.splitlines() if l.startswith("[pql] ")]
    assert len(lines) == 3, err
    assert lines[0] == "[pql] qgemm FP8_ROW M=0 N=256 K=512: nothing to do"
    assert lines[1].startswith("[pql] qgemm ") and "rejected (status" in lines[1] and "unknown scheme 99" in lines[1]
    assert lines[2].startswith("[pql] quantize FP8_BLOCK128 activation M=4 N=0 K=256: rejected (status 1)")
    assert "ldx" in lines[2]
    assert "[pql]" not in _run_logged(LOG_CODE, None)
    assert "[pql]" not in _run_logged(LOG_CODE, "0")
