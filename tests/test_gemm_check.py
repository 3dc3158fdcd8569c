"""The per-element GEMM checks of tests/gemm_check.py, exercised on the CPU.

A check is only useful if a correct result passes it and a plausible kernel
mistake fails it.  The "correct" results here are the oracle's own product
rounded once to bf16 (what an exact kernel would store); the mistakes are
planted in copies of that result or computed by the oracle from deliberately
mis-indexed operands: a dropped store, a stale element, a product taken with
the neighbouring row's or K-group's scale, and a one-ulp change."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gemm_check import (bf16_f64, check_gemm, check_gemm_exact, exact_operand, exact_precondition,
                        tile_sample, w4a16_terms)
from oracle import formats as F


def _round_bf16(c64):
    return F.f32_to_bf16_rne(np.asarray(c64, np.float64).astype(np.float32))


def _random_case(scheme, M=128, N=256, K=512):
    a = wl.pow2_blocks(wl.small_case(21, M, K), 21, 1, 32)
    w = wl.pow2_blocks(wl.small_case(22, N, K, 0.02), 22, 128, 128)
    aq, wq = oracle.quantize(a, scheme, "activation"), oracle.quantize(w, scheme, "weight")
    return aq, wq, oracle.gemm_ref(aq, wq), oracle.gemm_abs_ref(aq, wq), K


@pytest.mark.parametrize("scheme", ["fp8_row", "fp8_block128", "mxfp8", "mxfp4"])
def test_correct_result_passes(scheme):
    aq, wq, c64, t, K = _random_case(scheme)
    check_gemm(_round_bf16(c64), c64, t, K, scheme)


@pytest.mark.parametrize("scheme", ["fp8_row", "fp8_block128", "mxfp8", "mxfp4"])
def test_dropped_or_stale_element_fails(scheme):
    aq, wq, c64, t, K = _random_case(scheme)
    good = _round_bf16(c64)
    # a typical element (|C| near the median): one wrong value there stays inside the
    # 1e-2 Frobenius gate on this 128 x 256 output, so only the per-element bound sees it
    mag = np.abs(c64)
    i, j = np.unravel_index(np.argmin(np.abs(mag - np.median(mag))), c64.shape)
    for planted in (0, good[i, (j + 1) % c64.shape[1]], good[(i + 1) % c64.shape[0], j]):
        bad = good.copy()
        bad[i, j] = planted
        with pytest.raises(AssertionError, match="per-element bound"):
            check_gemm(bad, c64, t, K, scheme, flag=False)


def test_neighbouring_row_scale_fails():
    aq, wq, c64, t, K = _random_case("fp8_row")
    wrong = dict(wq, scales=np.roll(wq["scales"], 1))       # row n takes row n-1's scale
    c_bad = _round_bf16(oracle.gemm_ref(aq, wrong))
    with pytest.raises(AssertionError):
        check_gemm(c_bad, c64, t, K, flag=False)


def test_neighbouring_k_group_scale_fails():
    aq, wq, c64, t, K = _random_case("fp8_block128")
    wrong = dict(aq, scales=np.roll(aq["scales"], 1, axis=1))    # group g takes group g-1's scale
    c_bad = _round_bf16(oracle.gemm_ref(wrong, wq))
    with pytest.raises(AssertionError):
        check_gemm(c_bad, c64, t, K, flag=False)


@pytest.mark.parametrize("scheme", ["fp8_tensor", "fp8_row", "fp8_block128", "mxfp8", "mxfp4", "int8_row"])
def test_exact_case_passes_and_catches_one_ulp(scheme):
    a = exact_operand(scheme, "activation", 40, 640, 1)
    w = exact_operand(scheme, "weight", 128, 640, 2)
    exact_precondition(a, w)
    c64 = oracle.gemm_ref(a, w)
    good = _round_bf16(c64)
    check_gemm_exact(good, c64, scheme)
    bad = good.copy()
    bad[7, 9] ^= np.uint16(1)
    with pytest.raises(AssertionError, match="1 of"):
        check_gemm_exact(bad, c64, scheme)


def test_exact_case_neighbour_scale_changes_bits():
    a = exact_operand("mxfp8", "activation", 40, 640, 1)
    w = exact_operand("mxfp8", "weight", 128, 640, 2)
    c64 = oracle.gemm_ref(a, w)
    wrong = dict(w, scales=np.roll(w["scales"], 1, axis=1))
    with pytest.raises(AssertionError):
        check_gemm_exact(_round_bf16(oracle.gemm_ref(a, wrong)), c64)


def test_exact_w4a16_case():
    from gemm_check import exact_activation_bf16
    a = exact_activation_bf16(33, 1152, 3)
    for scheme in ("w4a16_asym", "w4a16_sym"):
        w = exact_operand(scheme, "weight", 64, 1152, 4)
        exact_precondition(a, w)
        c64 = oracle.gemm_ref(a, w)
        check_gemm_exact(_round_bf16(c64), c64, scheme)


def test_w4a16_bound_terms_cover_weight_rounding():
    """A kernel that rounds each dequantized weight to bf16 stays inside the W4A16 bound."""
    a = wl.small_case(31, 16, 384)
    w = oracle.quantize(wl.small_case(32, 96, 384, 0.02), "w4a16_asym", "weight")
    c64 = oracle.gemm_ref(a, w)
    w_bf16 = bf16_f64(oracle.dequantize(w))              # bf16((q - z) s)
    c_rounded = bf16_f64(a) @ w_bf16.T
    wr, t_off = w4a16_terms(a, w)
    check_gemm(_round_bf16(c_rounded), c64, oracle.gemm_abs_ref(a, w), 384, weight_round=wr, t_acc=t_off)


def test_tile_sample_covers_every_tile():
    idx = tile_sample(8192 + 77, 5)
    tiles = set((idx // 256).tolist())
    assert tiles == set(range((8192 + 77 + 255) // 256))
    assert idx[0] == 0 and idx[-1] == 8192 + 76
