"""GPU parity at the size limits the C ABI accepts and at the degenerate sizes:

* quantizers on rows of 2^20 elements (the largest K; per-row FP8 / int8 take
  their two-pass path, every other scheme its chunk-parallel one), bit-exact;
* GEMMs with K = 2^17 (1024 to 4096 K steps, 2^25-byte buffer ranges per tile),
  against the oracle within the 1e-2 relative Frobenius gate;
* M = 0 calls, which enqueue nothing and return an empty result.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_quantized_linear_amd as pql
import workloads as wl
from gemm_check import assert_gemm
from oracle import formats as F

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 1e-2


def up(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def down_bf16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("scheme", ["fp8_tensor", "fp8_row", "fp8_block128", "mxfp8", "mxfp4", "int8_row"])
def test_quantize_longest_rows(scheme):
    rows, cols = 3, 1 << 20
    x = wl.small_case(77, rows, cols, 1.0)
    ref = oracle.quantize(x, scheme, "activation")
    got = pql.to_numpy(pql.quantize(up(x), scheme, "activation"))
    assert np.array_equal(np.asarray(got["codes"]).view(np.uint8), np.asarray(ref["codes"]).view(np.uint8))
    gs, rs = np.asarray(got["scales"]), np.asarray(ref["scales"])
    if rs.dtype == np.float32:
        gs, rs = gs.view(np.uint32), rs.view(np.uint32)
    assert np.array_equal(gs.reshape(rs.shape), rs)


def random_q(scheme, role, rows, cols, seed):
    """Seeded random codes and scales on the format's grid (an already-quantized
    operand, so the long-K GEMMs need no quantizer pass over 10^8 elements)."""
    rng = np.random.default_rng(seed)
    q = {"scheme": scheme, "role": role, "rows": rows, "cols": cols, "zeros": None}
    if scheme in ("fp8_row", "fp8_block128", "mxfp8"):
        codes = rng.integers(0, 0x7F, size=(rows, cols)).astype(np.uint8) | \
            (rng.integers(0, 2, size=(rows, cols)).astype(np.uint8) << 7)
        q["codes"] = codes
    elif scheme == "mxfp4":
        q["codes"] = rng.integers(0, 256, size=(rows, cols // 2)).astype(np.uint8)
    elif scheme == "int8_row":
        q["codes"] = rng.integers(-128, 128, size=(rows, cols)).astype(np.int8)
    else:   # w4a16_asym
        q["codes"] = F.pack_int4(rng.integers(0, 16, size=(rows, cols)).astype(np.uint8))
        q["scales"] = wl.f32_to_bf16_bits(rng.uniform(0.5, 1.5, size=(rows, cols // 128)).astype(np.float32) * 1e-3)
        q["zeros"] = rng.integers(0, 16, size=(rows, cols // 128)).astype(np.uint8)
        return q
    if scheme == "fp8_row" or scheme == "int8_row":
        q["scales"] = rng.uniform(0.5, 2.0, size=rows).astype(np.float32) * np.float32(1e-3)
    elif scheme == "fp8_block128":
        shape = (rows, cols // 128) if role == "activation" else (rows // 128, cols // 128)
        q["scales"] = rng.uniform(0.5, 2.0, size=shape).astype(np.float32) * np.float32(1e-3)
    else:   # e8m0 exponents around 2^-10
        q["scales"] = rng.integers(112, 122, size=(rows, cols // 32)).astype(np.uint8)
    return q


@pytest.mark.parametrize("scheme", ["fp8_row", "fp8_block128", "mxfp8", "mxfp4", "int8_row", "w4a16_asym"])
def test_qgemm_long_k(scheme):
    M, N, K = 37, 128, 1 << 17
    wq = random_q(scheme, "weight", N, K, 79)
    if scheme == "w4a16_asym":
        a = wl.small_case(78, M, K, 1.0)
        c = pql.qgemm(up(a), pql.from_numpy(wq, DEV))
    else:
        a = random_q(scheme, "activation", M, K, 78)
        c = pql.qgemm(pql.from_numpy(a, DEV), pql.from_numpy(wq, DEV))
    assert_gemm(down_bf16(c), a, wq, f"{scheme} K=2^17")


@pytest.mark.parametrize("scheme", ["fp8_tensor", "fp8_row", "mxfp4", "int8_row", "w4a16_asym"])
def test_empty_activation(scheme):
    K, N = 256, 128
    wq = pql.quantize(up(wl.small_case(80, N, K, 0.02)), scheme, "weight")
    x = torch.empty((0, K), dtype=torch.bfloat16, device=DEV)
    y = pql.qlinear(x, wq)
    assert tuple(y.shape) == (0, N)
    y3 = pql.qlinear(torch.empty((2, 0, K), dtype=torch.bfloat16, device=DEV), wq)
    assert tuple(y3.shape) == (2, 0, N)
    if scheme != "w4a16_asym":
        q = pql.quantize(x, scheme, "activation")
        assert q.rows == 0
