"""GPU parity of the fused quantize + GEMM for a few tokens (M <= 16; "vLLM-Omni
Online Quantization complete guide", section "How online quantization works
underneath": the activation-quantize prologue fusion).

qlinear with M <= 16 runs one kernel that quantizes the bf16 activation with
the scheme's activation rule inside the GEMM (FP8 per tensor / per token /
per 1x128 group, int8 per token; static scales for the FP8 tensor and block
schemes).  Checked against the oracle (quantize the activation, then the exact
float64 GEMM): bit for bit on activations whose quantization is exact, within
the per-element bound on random, power-of-two scaled activations with
outliers, with the alpha / bias epilogue, static scales (saturating ones
included), strided outputs and tile-covering samples of the DiT-shaped
weights.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_quantized_linear_amd as pql
import workloads as wl
from gemm_check import (assert_gemm, check_gemm, check_gemm_exact, exact_operand, exact_precondition,
                        fused_exact_activation, tile_sample)
from test_gpu_parity import down_bf16, hard_input, up

pytestmark = pytest.mark.gpu

DEV = "cuda"
FUSED = ("fp8_tensor", "fp8_row", "int8_row", "fp8_block128")


def fused_kernel(scheme, M, K):
    """The fused kernel qlinear runs: the staged-activation variant quantizes the activation once per
    workgroup into LDS (K <= 4096, or 8192 for one token); longer K casts in the main loop."""
    few = K <= (8192 if M == 1 else 4096)
    return f"k_qlinear_{'few' if few else 'small'}<{scheme}>"


def _weight(scheme, N, K, seed):
    w = wl.pow2_blocks(wl.small_case(seed, N, K, 0.02), seed, 128 if scheme == "fp8_block128" else 1, 128)
    wq = oracle.quantize(w, scheme, "weight")
    return wq, pql.from_numpy(wq, DEV)


@pytest.mark.parametrize("scheme", FUSED)
@pytest.mark.parametrize("M", [1, 2, 5, 16])
def test_fused_exact(scheme, M):
    N, K = (512 if scheme == "fp8_block128" else 520), 512
    assert pql.kernel_name("qlinear", scheme, "activation", M, N, K) == fused_kernel(scheme, M, K)
    a_bits = fused_exact_activation(scheme, M, K, 10 + M)
    wq = exact_operand(scheme, "weight", N, K, 20 + M)
    aq = oracle.quantize(a_bits, scheme, "activation")
    exact_precondition(aq, wq)
    y = pql.qlinear(up(a_bits), pql.from_numpy(wq, DEV))
    check_gemm_exact(down_bf16(y), oracle.gemm_ref(aq, wq), f"{scheme} M={M}")


# the staged-activation kernel at 1, 4 and 16 staged rows, and (K past its stage) the kernel that casts
# in its main loop; N >= 8200 or so selects the staged kernel's 48-column workgroups (fewer columns per CU
# than 32-column ones), here with a ragged last workgroup (8232 = 171 x 48 + 24; block-128: 8320)
@pytest.mark.parametrize("scheme", FUSED)
@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (3, 300 * 4, 640), (16, 4100, 3072), (9, 384, 1152),
                                   (1, 256, 6144), (1, 256, 8320), (2, 384, 4224), (16, 256, 4352),
                                   (1, 8232, 640), (3, 8232, 640), (16, 8232, 1152), (1, 8232, 6144),
                                   (16, 8232, 4096)])
def test_fused_matches_oracle(scheme, M, N, K):
    if scheme == "fp8_block128":
        N = -(-N // 128) * 128
    assert pql.kernel_name("qlinear", scheme, "activation", M, N, K) == fused_kernel(scheme, M, K)
    a_bits = wl.pow2_blocks(wl.small_case(M * 31 + K, M, K), M, 1, 128).copy()
    a_bits[0, :7] = 0x8000                                   # -0 and zeros among the codes
    a_bits[M - 1, K // 2] = wl.f32_to_bf16_bits(np.array([300.0], np.float32))[0]   # an outlier
    wq, wq_t = _weight(scheme, N, K, 50 + N)
    y = pql.qlinear(up(a_bits), wq_t)
    assert_gemm(down_bf16(y), oracle.quantize(a_bits, scheme, "activation"), wq, f"{scheme} {M}x{N}x{K}")


@pytest.mark.parametrize("scheme", FUSED)
@pytest.mark.parametrize("N", [512, 8320])   # 32- and 48-column workgroups
def test_fused_epilogue_and_strided_output(scheme, N):
    from test_gpu_exact import _check_sentinels, _sentinel_buffer
    M, K = 7, 640
    a_bits = wl.small_case(61, M, K)
    wq, wq_t = _weight(scheme, N, K, 62)
    bias = wl.f32_to_bf16_bits(np.random.default_rng(3).normal(0, 0.5, N).astype(np.float32))
    buf, out = _sentinel_buffer(M, N, 2, 8, N + 40)
    pql.qlinear(up(a_bits), wq_t, out=out, alpha=0.625, bias=up(bias))
    _check_sentinels(buf, M, N, 2, 8, scheme)
    assert_gemm(down_bf16(out), oracle.quantize(a_bits, scheme, "activation"), wq, scheme,
                alpha=np.float32(0.625), bias=bias)


@pytest.mark.parametrize("scheme", ["fp8_tensor", "fp8_block128"])
@pytest.mark.parametrize("tiny", [False, True])
@pytest.mark.parametrize("N", [384, 8320])   # 32- and 48-column workgroups
def test_fused_static_scales(scheme, tiny, N):
    """Static activation scales, including ones far below amax / 448 (quotients saturate)."""
    M, K = 5, 1024
    a_bits = hard_input(71, M, K)
    rng = np.random.default_rng(72)
    shape = (1,) if scheme == "fp8_tensor" else (M, K // 128)
    sa = rng.uniform(0.002, 0.02, shape).astype(np.float32)
    if tiny:
        sa = sa * np.float32(1e-3)
    wq, wq_t = _weight(scheme, N, K, 73)
    y = pql.qlinear(up(a_bits), wq_t, act_scales=torch.from_numpy(sa.reshape(-1)).to(DEV))
    aq = oracle.quantize_static(a_bits, scheme, "activation", sa)
    assert_gemm(down_bf16(y), aq, wq, f"{scheme} static tiny={tiny}", flag=False)


def test_fused_matches_unfused_path_closely():
    """The fused kernel and quantize + qgemm see identical codes; their sums differ only in order."""
    M, N, K = 16, 1024, 3072
    a = up(wl.small_case(81, M, K))
    wq = pql.quantize(up(wl.small_case(82, N, K, 0.02)), "fp8_row", "weight")
    y = pql.qlinear(a, wq)
    ref = pql.qgemm(pql.quantize(a, "fp8_row", "activation"), wq)
    d = (y.float() - ref.float()).abs()
    assert float(d.max()) <= float(2.0 ** -7 * ref.float().abs().max())


@pytest.mark.parametrize("name,scheme", [("fp8_row_dit", "fp8_row"), ("fp8_row_dit", "int8_row"),
                                         ("fp8_block_dit", "fp8_block128")])
@pytest.mark.parametrize("M", [1, 16])
def test_fused_full_size_weights(name, scheme, M):
    w_ = wl.WORKLOADS[name]
    a_bits = wl.activation(w_, M)
    w_bits = wl.weight(w_)
    wq_t = pql.quantize(up(w_bits), scheme, "weight")
    y = pql.qlinear(up(a_bits), wq_t)
    assert pql.kernel_name("qlinear", scheme, "activation", M, w_.N, w_.K) == fused_kernel(scheme, M, w_.K)
    rw = tile_sample(w_.N, 5, tile=128, per_tile=1)
    wq_np = pql.to_numpy(wq_t)
    w_rows = dict(wq_np, codes=wq_np["codes"][rw], rows=len(rw))
    if scheme == "fp8_block128":
        w_rows["scales"] = np.asarray(wq_np["scales"], np.float32)[rw // 128]
        w_rows["role"] = "activation"
    else:
        w_rows["scales"] = wq_np["scales"][rw]
    aq = oracle.quantize(a_bits, scheme, "activation")
    check_gemm(down_bf16(y)[:, rw], oracle.gemm_ref(aq, w_rows), oracle.gemm_abs_ref(aq, w_rows), w_.K,
               f"{name} {scheme} M={M}")
