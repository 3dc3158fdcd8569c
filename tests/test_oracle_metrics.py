"""Pins for the oracle's similarity metrics and the per-element GEMM magnitude
sum (CPU only).

* The metric set of the online-quantization guide's similarity report, worked
  by hand in tests/golden/similarity_worked_example.txt.
* Identities every definition must satisfy: a candidate equal to its
  reference, a scaled copy (cosine 1, relative L2 = |k - 1|), the negation.
* gemm_abs_ref (sum over k of |a_hat_k w_hat_k|) against exact rationals on
  tiny operands, and against the GEMM itself when every operand is
  non-negative.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from golden_io import keyed, parse_floats
from oracle import formats as F
from oracle import metrics as MET
from workloads import small_case


@pytest.mark.parametrize("case", ["1", "2"])
def test_similarity_worked_examples(case):
    d = keyed("similarity_worked_example.txt")
    ref = parse_floats(d["ref" + case][0])
    cand = parse_floats(d["cand" + case][0])
    got = MET.similarity(cand, ref)
    want = {row[0]: float(row[1]) for row in d["want" + case]}
    assert set(want) == set(got)
    for k, v in want.items():
        assert got[k] == pytest.approx(v, rel=1e-12, abs=1e-15), k


def test_similarity_identical():
    r = np.array([[0.5, -2.0], [3.0, 1.0]])
    m = MET.similarity(r, r)
    assert m["cosine_similarity"] == pytest.approx(1.0, abs=1e-15)
    assert m["mae"] == m["mse"] == m["rmse"] == m["max_abs"] == m["l2"] == m["relative_l2"] == 0.0
    assert m["psnr_db"] == math.inf
    assert MET.meets_starting_thresholds(m)


def test_similarity_scaled_copy():
    r = np.arange(1.0, 9.0)
    m = MET.similarity(1.25 * r, r)
    assert m["cosine_similarity"] == pytest.approx(1.0, abs=1e-15)
    assert m["relative_l2"] == pytest.approx(0.25, rel=1e-15)
    assert m["max_abs"] == pytest.approx(0.25 * 8)


def test_similarity_thresholds():
    r = np.linspace(-1.0, 1.0, 101)
    # noise of rms 0.2 on a range of 2: psnr = 10 log10(4 / 0.04) = 20 dB exactly at the edge
    noisy = r + np.where(np.arange(101) % 2 == 0, 0.2, -0.2)
    m = MET.similarity(noisy, r)
    assert m["psnr_db"] == pytest.approx(20.0, abs=1e-9)
    assert not MET.meets_starting_thresholds(MET.similarity(-r, r))


def test_similarity_rejects_bad_shapes():
    with pytest.raises(ValueError):
        MET.similarity(np.zeros(3), np.zeros(4))
    with pytest.raises(ValueError):
        MET.similarity(np.zeros(0), np.zeros(0))


def _fp8_row(codes, scales):
    rows, cols = codes.shape
    return {"scheme": "fp8_row", "role": "activation", "rows": rows, "cols": cols,
            "codes": codes.astype(np.uint8), "scales": np.asarray(scales, np.float32), "zeros": None}


def test_gemm_abs_ref_exact_rationals():
    rng = np.random.default_rng(3)
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    for M, N, K in ((1, 1, 32), (2, 3, 64), (3, 2, 96)):
        ca = rng.choice(finite, (M, K)).astype(np.uint8)
        cw = rng.choice(finite, (N, K)).astype(np.uint8)
        sa = rng.uniform(0.01, 2, M).astype(np.float32)
        sw = rng.uniform(0.01, 2, N).astype(np.float32)
        a, w = _fp8_row(ca, sa), dict(_fp8_row(cw, sw), role="weight")
        got = oracle.gemm_abs_ref(a, w)
        va, vw = F.e4m3_decode(ca), F.e4m3_decode(cw)
        for m in range(M):
            for n in range(N):
                exact = sum(abs(Fraction(float(va[m, k])) * Fraction(float(sa[m]))
                                * Fraction(float(vw[n, k])) * Fraction(float(sw[n]))) for k in range(K))
                assert abs(Fraction(float(got[m, n])) - exact) <= K * Fraction(2) ** -53 * exact


def test_gemm_abs_ref_equals_gemm_for_non_negative_operands():
    a_bits = small_case(11, 5, 256) & np.uint16(0x7FFF)     # clear the sign bit: a >= 0
    w_bits = small_case(12, 7, 256, 0.02) & np.uint16(0x7FFF)
    aq, wq = oracle.quantize(a_bits, "mxfp8", "activation"), oracle.quantize(w_bits, "mxfp8", "weight")
    assert np.array_equal(oracle.gemm_abs_ref(aq, wq), oracle.gemm_ref(aq, wq))
    # and a sign flip of any operand leaves it unchanged
    neg = dict(aq, codes=(aq["codes"] ^ np.uint8(0x80)))
    assert np.array_equal(oracle.gemm_abs_ref(neg, wq), oracle.gemm_abs_ref(aq, wq))
    assert np.allclose(oracle.gemm_ref(neg, wq), -oracle.gemm_ref(aq, wq), rtol=0, atol=0)


def test_gemm_abs_ref_alpha_scales_magnitude():
    a = small_case(13, 4, 128)
    wq = oracle.quantize(small_case(14, 3, 128, 0.02), "fp8_row", "weight")
    aq = oracle.quantize(a, "fp8_row", "activation")
    t = oracle.gemm_abs_ref(aq, wq)
    assert np.array_equal(oracle.gemm_abs_ref(aq, wq, alpha=-0.5), 0.5 * t)
