"""GPU parity of the widened rows through the C ABI, against the CPU oracle:

* static FP8 scales (per tensor, per 128-block): codes bit-exact, including
  quotients beyond 448 that saturate and scales small enough to take the
  full-precision division;
* int8 W8A8 per row (dynamic): codes and scales bit-exact, dequantize
  bit-exact, GEMM within the 1e-2 relative Frobenius gate and the
  per-element bound of tests/gemm_check.py;
* the fused epilogue alpha * (A W^T) + bias on the FP8 and int8 GEMMs, and
  qlinear with static activation scales.
Small cases span several tiles with ragged tails; the full-size cases use the
benchmark's C2 / C3 shapes and check sampled rows and columns that cover
every 256 x 256 output tile.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_quantized_linear_amd as pql
import workloads as wl
from gemm_check import assert_gemm, check_gemm, tile_sample
from oracle import formats as F

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 1e-2
EPI_SCHEMES = ("fp8_tensor", "fp8_row", "fp8_block128", "int8_row")


def up(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def down_bf16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32_up(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def codes_u8(c) -> np.ndarray:
    return np.asarray(c).view(np.uint8)


def assert_same(got_codes, ref_codes, what):
    g, r = codes_u8(got_codes), codes_u8(ref_codes)
    bad = np.argwhere(g != r)
    assert len(bad) == 0, f"{what}: {len(bad)} codes differ, first at {tuple(bad[0])}: gpu {g[tuple(bad[0])]:#x} " \
                          f"oracle {r[tuple(bad[0])]:#x}"


def mixed_input(seed, rows, cols, std=1.0):
    """Normal data with zero rows, -0, ties after exact scales, tiny values and outliers."""
    x = wl.bf16_bits_to_f32(wl.small_case(seed, rows, cols, std)).copy()
    rng = np.random.default_rng(seed + 3)
    if rows > 2:
        x[1, :] = 0.0
    x[0, :8] = np.array([127, -16.5, 1.5, 2.5, -127, 0.5, 3.5, -2.5], np.float32) * np.float32(std / 16)
    if rows > 3:
        x[2, 16:48] = np.float32(1e-39)
    idx = rng.integers(0, rows * cols, 40)
    x.reshape(-1)[idx] *= np.float32(9.0)
    bits = wl.f32_to_bf16_bits(x)
    bits.reshape(-1)[rng.integers(0, rows * cols, 16)] = 0x8000
    return bits


def static_scales(x_bits, scheme, role, seed, lo=0.125, hi=4.0):
    """Positive fp32 scales around the dynamic ones: amax / 448 times a factor in
    [lo, hi] per block, so some blocks saturate and some use a small fraction of the
    range; one tensor scale is half the dynamic one, so it always saturates."""
    rng = np.random.default_rng(seed)
    d = np.asarray(oracle.quantize(x_bits, scheme, role)["scales"], np.float32)
    f = np.full(d.shape, 0.5) if scheme == "fp8_tensor" else rng.uniform(lo, hi, size=d.shape)
    f.reshape(-1)[0] = 0.5       # the first block saturates in every case
    return (d * f).astype(np.float32)


# ----------------------------------------------------------------- static FP8 scales
STATIC_CASES = []
for scheme in ("fp8_tensor", "fp8_block128"):
    for role in ("activation", "weight"):
        for rows, cols in ((1, 128), (37, 384), (384, 640), (300, 1152)):
            if scheme == "fp8_block128" and role == "weight" and rows % 128:
                continue
            STATIC_CASES.append((scheme, role, rows, cols))


@pytest.mark.parametrize("scheme,role,rows,cols", STATIC_CASES)
def test_static_quantize_bit_exact(scheme, role, rows, cols):
    x = mixed_input(rows * 3 + cols, rows, cols, 0.02 if role == "weight" else 1.0)
    s = static_scales(x, scheme, role, rows + cols)
    ref = oracle.quantize_static(x, scheme, role, s)
    q = pql.quantize_static(up(x), scheme, role, f32_up(s))
    assert_same(q.codes.cpu().numpy(), ref["codes"], f"{scheme}/{role} {rows}x{cols}")
    assert np.any(codes_u8(ref["codes"]) & 0x7F == 0x7E)      # saturation is exercised


@pytest.mark.parametrize("s", [2.0 ** -100, 2.0 ** -80, 3.0e-30, 0.25, 1.0e30])
def test_static_quantize_extreme_scales(s):
    """Scales below 2^-80 take the full-precision division; huge scales flush to 0;
    inputs near the bf16 maximum overflow the fp32 quotient and must still saturate
    with their own sign."""
    x = mixed_input(4, 64, 256)
    x[3, :6] = wl.f32_to_bf16_bits(np.array([3.0e38, -3.0e38, 1.0e38, -2.0e37, 448.0, -449.0], np.float32))
    sc = np.array([s], np.float32)
    ref = oracle.quantize_static(x, "fp8_tensor", "activation", sc)
    q = pql.quantize_static(up(x), "fp8_tensor", "activation", f32_up(sc))
    assert_same(q.codes.cpu().numpy(), ref["codes"], f"s={s}")


@pytest.mark.parametrize("scheme", ["fp8_tensor", "fp8_block128"])
def test_qlinear_static_activation_scales(scheme):
    M, N, K = 300, 384, 640
    a, w = mixed_input(21, M, K), wl.small_case(22, N, K, 0.02)
    sa = static_scales(a, scheme, "activation", 23)
    wq_ref = oracle.quantize(w, scheme, "weight")
    wq = pql.from_numpy(wq_ref, DEV)
    y = pql.qlinear(up(a), wq, act_scales=f32_up(sa))
    aq_ref = oracle.quantize_static(a, scheme, "activation", sa)
    assert_gemm(down_bf16(y), aq_ref, wq_ref, scheme)
    # the same as quantize_static followed by qgemm, bit for bit
    aq = pql.quantize_static(up(a), scheme, "activation", f32_up(sa))
    assert torch.equal(y.view(torch.int16), pql.qgemm(aq, wq).view(torch.int16))


# ----------------------------------------------------------------- int8 per row
INT8_CASES = [(role, r, c) for role in ("activation", "weight")
              for r, c in ((1, 128), (37, 384), (300, 1152), (384, 640), (9, 12288))]


@pytest.mark.parametrize("role,rows,cols", INT8_CASES)
def test_int8_quantize_bit_exact(role, rows, cols):
    x = mixed_input(rows * 5 + cols, rows, cols, 0.02 if role == "weight" else 1.0)
    ref = oracle.quantize(x, "int8_row", role)
    got = pql.to_numpy(pql.quantize(up(x), "int8_row", role))
    assert_same(got["codes"], ref["codes"], f"int8/{role} {rows}x{cols}")
    assert np.array_equal(np.asarray(got["scales"]).view(np.uint32), ref["scales"].view(np.uint32))


def test_int8_quantize_all_zero_and_dequantize():
    z = np.zeros((64, 256), np.uint16)
    got = pql.to_numpy(pql.quantize(up(z), "int8_row", "weight"))
    assert not codes_u8(got["codes"]).any() and np.all(got["scales"] == 1.0)
    x = mixed_input(31, 256, 640)
    ref_q = oracle.quantize(x, "int8_row", "activation")
    y = pql.dequantize(pql.from_numpy(ref_q, DEV))
    assert np.array_equal(down_bf16(y), oracle.dequantize(ref_q))


GEMM_SHAPES = [(1, 256, 128), (77, 384, 256), (256, 256, 640), (300, 640, 1152), (513, 128, 384),
               (4300, 4200, 512)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_int8_qgemm_matches_oracle(M, N, K):
    a = wl.pow2_blocks(wl.small_case(1000 + M, M, K, 1.0), M, 1, 32)
    w = wl.pow2_blocks(wl.small_case(2000 + N, N, K, 0.02), N, 1, 128)
    aq, wq = oracle.quantize(a, "int8_row", "activation"), oracle.quantize(w, "int8_row", "weight")
    c = pql.qgemm(pql.from_numpy(aq, DEV), pql.from_numpy(wq, DEV))
    assert_gemm(down_bf16(c), aq, wq, f"{M}x{N}x{K}")


def test_int8_extreme_codes_sum_exactly():
    """Every code at -128 / 127 (the int32 sums' largest magnitudes): K = 2048 gives
    |sum| up to 2048 * 128 * 128 = 2^25, so the conversion to fp32 is exercised too."""
    M, N, K = 64, 256, 2048
    rng = np.random.default_rng(3)
    ca = rng.choice(np.array([-128, 127], np.int8), size=(M, K))
    cw = rng.choice(np.array([-128, 127], np.int8), size=(N, K))
    ca[0, :], cw[0, :] = -128, -128
    aq = {"scheme": "int8_row", "role": "activation", "rows": M, "cols": K, "codes": ca,
          "scales": np.full(M, 2.0 ** -10, np.float32), "zeros": None}
    wq = {"scheme": "int8_row", "role": "weight", "rows": N, "cols": K, "codes": cw,
          "scales": np.full(N, 2.0 ** -12, np.float32), "zeros": None}
    cb = down_bf16(pql.qgemm(pql.from_numpy(aq, DEV), pql.from_numpy(wq, DEV)))
    ref = oracle.gemm_ref(aq, wq)
    assert F.bf16_to_f32(cb)[0, 0] == ref[0, 0] == 2048 * 128 * 128 * 2.0 ** -22
    assert_gemm(cb, aq, wq, "extreme codes")


# ----------------------------------------------------------------- fused epilogue
@pytest.mark.parametrize("scheme", EPI_SCHEMES)
@pytest.mark.parametrize("M,N,K", [(77, 384, 256), (300, 640, 1152), (4300, 4224, 512)])
def test_epilogue_alpha_bias(scheme, M, N, K):
    a = wl.pow2_blocks(wl.small_case(3000 + M, M, K, 1.0), M, 1, 32)
    w = wl.pow2_blocks(wl.small_case(4000 + N, N, K, 0.02), N, 128 if scheme == "fp8_block128" else 1, 128)
    aq, wq = oracle.quantize(a, scheme, "activation"), oracle.quantize(w, scheme, "weight")
    rng = np.random.default_rng(M + N)
    alpha = np.float32(0.37)
    bias = wl.f32_to_bf16_bits(rng.normal(0, 0.5, N).astype(np.float32))
    aq_t, wq_t = pql.from_numpy(aq, DEV), pql.from_numpy(wq, DEV)
    c = pql.qgemm(aq_t, wq_t, alpha=float(alpha), bias=up(bias))
    assert_gemm(down_bf16(c), aq, wq, f"{scheme} {M}x{N}x{K}", alpha=alpha, bias=bias)
    # alpha alone, and the default epilogue is the plain GEMM bit for bit
    c2 = pql.qgemm(aq_t, wq_t, alpha=2.0)
    assert_gemm(down_bf16(c2), aq, wq, f"{scheme} {M}x{N}x{K} alpha", alpha=np.float32(2.0))
    c1 = pql.qgemm(aq_t, wq_t, alpha=1.0, bias=None)
    c0 = pql.qgemm(aq_t, wq_t)
    assert torch.equal(c1.view(torch.int16), c0.view(torch.int16))


def test_epilogue_rejected_where_undefined():
    x = up(wl.small_case(1, 64, 256))
    wq = pql.quantize(up(wl.small_case(2, 128, 256, 0.02)), "mxfp8", "weight")
    with pytest.raises(NotImplementedError):
        pql.qlinear(x, wq, bias=torch.zeros(128, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(NotImplementedError):
        pql.qlinear(x, wq, alpha=0.5)


# ----------------------------------------------------------------- full size (C2 / C3 shapes)
def test_full_size_int8_on_c2_shape():
    w_ = wl.WORKLOADS["fp8_row_dit"]
    a_bits, w_bits = wl.activation(w_), wl.weight(w_)
    wq = pql.quantize(up(w_bits), "int8_row", "weight")
    aq = pql.quantize(up(a_bits), "int8_row", "activation")
    rng_bias = wl.f32_to_bf16_bits(np.random.default_rng(5).normal(0, 0.1, w_.N).astype(np.float32))
    y = pql.qlinear(up(a_bits), wq, alpha=0.75, bias=up(rng_bias))
    aq_np, wq_np = pql.to_numpy(aq), pql.to_numpy(wq)
    ra, rw = tile_sample(w_.M, 11, extra=range(w_.M - 40, w_.M)), tile_sample(w_.N, 12)
    ref_a = oracle.quantize(np.ascontiguousarray(a_bits[ra]), "int8_row", "activation")
    ref_w = oracle.quantize(np.ascontiguousarray(w_bits[rw]), "int8_row", "weight")
    assert_same(aq_np["codes"][ra], ref_a["codes"], "A rows")
    assert_same(wq_np["codes"][rw], ref_w["codes"], "W rows")
    assert np.array_equal(aq_np["scales"][ra].view(np.uint32), ref_a["scales"].view(np.uint32))
    assert np.array_equal(wq_np["scales"][rw].view(np.uint32), ref_w["scales"].view(np.uint32))
    ref = oracle.gemm_ref(ref_a, ref_w, alpha=np.float32(0.75), bias=rng_bias[rw])
    t = oracle.gemm_abs_ref(ref_a, ref_w, alpha=np.float32(0.75))
    check_gemm(down_bf16(y)[np.ix_(ra, rw)], ref, t, w_.K, "int8 C2 shape")


@pytest.mark.parametrize("name,scheme", [("fp8_row_dit", "fp8_row"), ("fp8_block_dit", "fp8_block128")])
def test_full_size_epilogue(name, scheme):
    w_ = wl.WORKLOADS[name]
    a_bits, w_bits = wl.activation(w_), wl.weight(w_)
    wq = pql.quantize(up(w_bits), scheme, "weight")
    aq = pql.quantize(up(a_bits), scheme, "activation")
    bias = wl.f32_to_bf16_bits(np.random.default_rng(6).normal(0, 0.1, w_.N).astype(np.float32))
    c = pql.qgemm(aq, wq, alpha=1.5, bias=up(bias))
    aq_np, wq_np = pql.to_numpy(aq), pql.to_numpy(wq)
    ra, rw = tile_sample(w_.M, 13, extra=range(w_.M - 24, w_.M)), tile_sample(w_.N, 14)
    a_rows = dict(aq_np, codes=aq_np["codes"][ra], scales=aq_np["scales"][ra], rows=len(ra))
    w_rows = dict(wq_np, codes=wq_np["codes"][rw], rows=len(rw))
    if scheme == "fp8_block128":   # per-row view of the weight's 128x128 block scales
        w_rows["scales"] = wq_np["scales"][rw // 128]
        w_rows["role"] = "activation"
    else:
        w_rows["scales"] = wq_np["scales"][rw]
    ref = oracle.gemm_ref(a_rows, w_rows, alpha=np.float32(1.5), bias=bias[rw])
    t = oracle.gemm_abs_ref(a_rows, w_rows, alpha=np.float32(1.5))
    check_gemm(down_bf16(c)[np.ix_(ra, rw)], ref, t, w_.K, name)
