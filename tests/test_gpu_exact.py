"""GPU GEMMs checked bit for bit on every output element.

The operands come from tests/gemm_check.py's ``exact_operand``: codes on a
coarse grid and power-of-two scales that differ between neighbouring rows,
K-groups and blocks, chosen so that every partial sum the kernel can form is
exact in fp32.  The oracle's float64 product is then exact too, the only
rounding left is the final one to bf16, and every element of C must equal
bf16_RNE(C64).  A stale tile, a dropped or misplaced store, or a scale taken
from the wrong row / group / block changes the bits, wherever it happens.

The cases reach every GEMM kernel (the persistent FP8 / MX / int8 kernel, the
MXFP4 kernel for K % 256 != 0, both block-128 kernels, and the W4A16 GEMV,
small-M, 256 x 64, 256 x 128 and N % 4 != 0 kernels) on ragged multi-tile
shapes.  Outputs are also written into the middle of larger sentinel-filled
buffers with a wider row stride (16-byte aligned rows and not), and every
sentinel must survive; dequantize is checked the same way.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_quantized_linear_amd as pql
from gemm_check import check_gemm_exact, exact_activation_bf16, exact_operand, exact_precondition

pytestmark = pytest.mark.gpu

DEV = "cuda"
SENTINEL = 0x7FA5          # a bf16 NaN pattern no kernel writes


def up(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def down_bf16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _operands(scheme, M, N, K, seed):
    w = exact_operand(scheme, "weight", N, K, seed + 1)
    if scheme.startswith("w4a16"):
        a = exact_activation_bf16(M, K, seed)
        return a, w, up(a), pql.from_numpy(w, DEV)
    a = exact_operand(scheme, "activation", M, K, seed)
    return a, w, pql.from_numpy(a, DEV), pql.from_numpy(w, DEV)


CASES = [
    # scheme, M, N, K, kernel
    ("fp8_tensor", 300, 520, 384, "k_gemm32_fp8"),
    ("fp8_row", 1, 256, 128, "k_gemm32_fp8"),
    ("fp8_row", 4300, 4200, 512, "k_gemm32_fp8"),
    ("int8_row", 513, 392, 640, "k_gemm32<int8>"),
    ("int8_row", 4300, 4200, 256, "k_gemm32<int8>"),
    ("mxfp8", 77, 264, 1152, "k_gemm32<mxfp8>"),
    ("mxfp8", 4300, 4200, 512, "k_gemm32<mxfp8>"),
    ("mxfp4", 300, 520, 1024, "k_gemm32<mxfp4>"),
    ("mxfp4", 4300, 4200, 512, "k_gemm32<mxfp4>"),
    ("mxfp4", 300, 520, 384, "k_gemm<mxfp4>_256x256x256"),
    ("fp8_block128", 77, 384, 640, "k_gemm_block"),
    ("fp8_block128", 4300, 2048, 640, "k_gemm_block"),
    ("fp8_block128", 4300, 4224, 384, "k_gemm_block256"),
    ("w4a16_asym", 1, 388, 1152, "k_w4a16_gemv<16 cols>"),
    ("w4a16_asym", 16, 4100, 1152, "k_w4a16_gemv<48 cols>"),
    ("w4a16_asym", 1, 388, 1024, "k_w4a16_gemv<16 cols>"),
    ("w4a16_sym", 3, 130, 2048, "k_w4a16_gemv<16 cols>"),
    ("w4a16_asym", 16, 4100, 1536, "k_w4a16_gemv<48 cols>"),
    ("w4a16_asym", 7, 100, 512, "k_w4a16_gemv<48 cols>"),
    # the 48-column GEMV's 12 waves with full 3-group batches and a partial last one (K / 128 = 48, 34, 25),
    # and the 16-column GEMV looping over several 4-group batches (64, 100 groups)
    ("w4a16_asym", 8, 4100, 6144, "k_w4a16_gemv<48 cols>"),
    ("w4a16_asym", 12, 520, 4352, "k_w4a16_gemv<48 cols>"),
    ("w4a16_sym", 5, 388, 3200, "k_w4a16_gemv<48 cols>"),
    ("w4a16_asym", 1, 260, 8192, "k_w4a16_gemv<16 cols>"),
    ("w4a16_asym", 2, 130, 12800, "k_w4a16_gemv<16 cols>"),
    ("w4a16_sym", 33, 388, 1152, "k_w4a16_small"),
    ("w4a16_asym", 300, 388, 1152, "k_w4a16_mm_256x64x64"),
    ("w4a16_asym", 2304, 4100, 512, "k_w4a16_mm_256x128x64"),
    ("w4a16_asym", 300, 390, 640, "k_w4a16_tile"),
]


@pytest.mark.parametrize("scheme,M,N,K,kernel", CASES)
def test_exact_every_element(scheme, M, N, K, kernel):
    name = pql.kernel_name("qgemm", scheme, "activation", M, N, K)
    assert name == kernel or (name.startswith(kernel) and not kernel.endswith(">")), \
        f"{scheme} {M}x{N}x{K} runs {name}, expected {kernel}"
    a, w, a_t, w_t = _operands(scheme, M, N, K, 100 + M)
    exact_precondition(a, w)
    c = pql.qgemm(a_t, w_t)
    check_gemm_exact(down_bf16(c), oracle.gemm_ref(a, w), f"{scheme} {M}x{N}x{K} ({name})")


@pytest.mark.parametrize("scheme,M,N,K", [("fp8_tensor", 300, 520, 384), ("fp8_row", 4300, 4200, 512),
                                          ("int8_row", 513, 392, 640), ("fp8_block128", 77, 384, 640),
                                          ("fp8_block128", 4300, 4224, 384)])
def test_exact_epilogue(scheme, M, N, K):
    a, w, a_t, w_t = _operands(scheme, M, N, K, 200 + M)
    rng = np.random.default_rng(M)
    bias = oracle.f32_to_bf16_rne(rng.integers(-64, 65, N).astype(np.float32) * np.float32(0.125))
    alpha = np.float32(0.5)
    exact_precondition(a, w, alpha=alpha, bias=bias)
    c = pql.qgemm(a_t, w_t, alpha=float(alpha), bias=up(bias))
    check_gemm_exact(down_bf16(c), oracle.gemm_ref(a, w, alpha=alpha, bias=bias), f"{scheme} alpha/bias")


def _sentinel_buffer(rows, cols, row0, col0, ld):
    buf = torch.full((rows + row0 + 3, ld), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    return buf, buf[row0:row0 + rows, col0:col0 + cols]


def _check_sentinels(buf, rows, cols, row0, col0, what):
    b = down_bf16(buf)
    mask = np.ones(b.shape, bool)
    mask[row0:row0 + rows, col0:col0 + cols] = False
    bad = mask & (b != SENTINEL)
    assert not bad.any(), f"{what}: {int(bad.sum())} bytes outside the output were written, first at " \
                          f"{tuple(np.argwhere(bad)[0])}"


STRIDED = [("fp8_row", 300, 520, 384), ("fp8_tensor", 4300, 4200, 256), ("int8_row", 77, 264, 256),
           ("mxfp8", 300, 520, 640), ("mxfp4", 300, 520, 512), ("mxfp4", 77, 264, 384),
           ("fp8_block128", 300, 512, 384), ("fp8_block128", 4300, 4224, 256),
           ("w4a16_asym", 5, 388, 384), ("w4a16_asym", 5, 388, 512), ("w4a16_asym", 40, 388, 384),
           ("w4a16_asym", 300, 388, 384),
           ("w4a16_asym", 300, 390, 384)]


@pytest.mark.parametrize("aligned", [True, False])
@pytest.mark.parametrize("scheme,M,N,K", STRIDED)
def test_exact_strided_output_keeps_sentinels(scheme, M, N, K, aligned):
    """C written into [2 + M + 3, ldc] with ldc > N: 16-byte aligned rows (column
    offset 8, ldc a multiple of 8) or not (column offset 3, odd ldc)."""
    a, w, a_t, w_t = _operands(scheme, M, N, K, 300 + M)
    col0, ld = (8, N + 40) if aligned else (3, N + 37)
    buf, out = _sentinel_buffer(M, N, 2, col0, ld)
    pql.qgemm(a_t, w_t, out=out)
    what = f"{scheme} {M}x{N}x{K} ldc={ld}"
    _check_sentinels(buf, M, N, 2, col0, what)
    check_gemm_exact(down_bf16(out), oracle.gemm_ref(a, w), what)


@pytest.mark.parametrize("scheme,M,N,K", [("fp8_row", 300, 520, 384), ("fp8_block128", 300, 512, 384),
                                          ("w4a16_asym", 300, 388, 384)])
def test_qlinear_strided_output_keeps_sentinels(scheme, M, N, K):
    rng = np.random.default_rng(7)
    a_bits = oracle.f32_to_bf16_rne(rng.standard_normal((M, K)).astype(np.float32))
    w_bits = oracle.f32_to_bf16_rne((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    wq = pql.quantize(up(w_bits), scheme, "weight")
    ref = pql.qlinear(up(a_bits), wq)
    buf, out = _sentinel_buffer(M, N, 1, 8, N + 24)
    y = pql.qlinear(up(a_bits), wq, out=out)
    _check_sentinels(buf, M, N, 1, 8, scheme)
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("scheme,role", [("fp8_tensor", "activation"), ("fp8_row", "weight"),
                                         ("fp8_block128", "activation"), ("fp8_block128", "weight"),
                                         ("mxfp8", "activation"), ("mxfp4", "weight"), ("int8_row", "activation"),
                                         ("w4a16_asym", "weight")])
def test_dequantize_strided_output_keeps_sentinels(scheme, role):
    rows, cols = 256, 640
    q = exact_operand(scheme, role, rows, cols, 9)
    buf, out = _sentinel_buffer(rows, cols, 2, 16, cols + 48)
    pql.dequantize(pql.from_numpy(q, DEV), out=out)
    _check_sentinels(buf, rows, cols, 2, 16, f"{scheme}/{role}")
    assert np.array_equal(down_bf16(out), oracle.dequantize(q))
