"""Pins for the oracle's reference GEMM (CPU only).

* Hand-checked tiny products whose value a reader can verify by eye.
* Random tiny shapes computed exactly with ``fractions.Fraction`` from the
  codes and scales, which the float64 path must match within the float64
  summation bound K * 2^-53 * sum|terms|.
* Operand orientation: A[M, K] times W[N, K]^T on non-square shapes with
  distinct rows, so a transposed or swapped operand fails.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import formats as F
from workloads import f32_to_bf16_bits, small_case


def _mx_from_codes(nibbles_or_codes, scale_codes, fmt):
    rows, cols = nibbles_or_codes.shape
    codes = nibbles_or_codes if fmt == "mxfp8" else F.pack_fp4(nibbles_or_codes)
    return {"scheme": fmt, "role": "activation", "rows": rows, "cols": cols,
            "codes": codes.astype(np.uint8), "scales": np.asarray(scale_codes, np.uint8), "zeros": None}


def test_mxfp4_all_ones_is_k():
    """1x32 . 32x1, every code 1.0 (0x2), scales 2^0 (code 127): C = 32."""
    a = _mx_from_codes(np.full((1, 32), 0x2, np.uint8), [[127]], "mxfp4")
    w = dict(a, role="weight")
    assert oracle.gemm_ref(a, w).tolist() == [[32.0]]


def test_mxfp4_sign_alternating_cancels():
    """Codes alternate +1 / -1 (0x2 / 0xA) against all +1: C = 0."""
    alt = np.tile(np.array([0x2, 0xA], np.uint8), 16)[None, :]
    a = _mx_from_codes(alt, [[127]], "mxfp4")
    w = _mx_from_codes(np.full((1, 32), 0x2, np.uint8), [[127]], "mxfp4")
    assert oracle.gemm_ref(a, w).tolist() == [[0.0]]


def test_mxfp8_single_nonzero_product():
    """One non-zero per operand at the same k: 448 * 2^-3 times -1.5 * 2^4 = -1344."""
    ca = np.zeros((1, 64), np.uint8)
    cw = np.zeros((1, 64), np.uint8)
    ca[0, 40] = 0x7E        # 448, in block 1
    cw[0, 40] = 0xBC        # -1.5
    a = _mx_from_codes(ca, [[127, 124]], "mxfp8")
    w = _mx_from_codes(cw, [[127, 131]], "mxfp8")
    assert oracle.gemm_ref(a, w).tolist() == [[448 * 2.0 ** -3 * -1.5 * 2.0 ** 4]]


def test_block128_two_groups_scale_separately():
    """K = 256: group 0 all codes 1.0 with s_a = 2, s_w = 3; group 1 all codes 2.0 with
    s_a = 0.5, s_w = 0.25 (weight block row 0).  C = 2*3*128*1 + 0.5*0.25*128*4 = 832."""
    ca = np.concatenate([np.full(128, 0x38), np.full(128, 0x40)]).astype(np.uint8)[None, :]
    cw = np.tile(ca, (128, 1))
    a = {"scheme": "fp8_block128", "role": "activation", "rows": 1, "cols": 256,
         "codes": ca, "scales": np.array([[2.0, 0.5]], np.float32), "zeros": None}
    w = {"scheme": "fp8_block128", "role": "weight", "rows": 128, "cols": 256,
         "codes": cw, "scales": np.array([[3.0, 0.25]], np.float32), "zeros": None}
    c = oracle.gemm_ref(a, w)
    assert c.shape == (1, 128) and np.all(c == 832.0)


def test_w4a16_hand_checked():
    """A = [1, 2, 0...], one group, codes q = [3, 15, ...], z = 5, s = 0.5:
    C = 1*(3-5)*0.5 + 2*(15-5)*0.5 = 9."""
    a = np.zeros((1, 128), np.float32)
    a[0, 0], a[0, 1] = 1.0, 2.0
    q = np.full((1, 128), 5, np.uint8)
    q[0, 0], q[0, 1] = 3, 15
    w = {"scheme": "w4a16_asym", "role": "weight", "rows": 1, "cols": 128,
         "codes": F.pack_int4(q), "scales": f32_to_bf16_bits(np.array([[0.5]], np.float32)),
         "zeros": np.array([[5]], np.uint8)}
    assert oracle.gemm_ref(f32_to_bf16_bits(a), w).tolist() == [[9.0]]


def _frac_dequant(q):
    """Exact rationals decode(code) * scale, straight from the code/scale arrays."""
    scheme, rows, cols = q["scheme"], q["rows"], q["cols"]
    out = [[None] * cols for _ in range(rows)]
    for r in range(rows):
        for k in range(cols):
            if scheme in ("fp8_tensor", "fp8_row", "fp8_block128"):
                v = Fraction(float(F.e4m3_decode(np.array([q["codes"][r, k]], np.uint8))[0]))
                if scheme == "fp8_tensor":
                    s = q["scales"].reshape(-1)[0]
                elif scheme == "fp8_row":
                    s = q["scales"][r]
                elif q["role"] == "activation":
                    s = q["scales"][r, k // 128]
                else:
                    s = q["scales"][r // 128, k // 128]
                out[r][k] = v * Fraction(float(s))
            elif scheme == "int8_row":
                byte = int(np.asarray(q["codes"]).view(np.uint8)[r, k])
                v = Fraction(byte - 256 if byte > 127 else byte)       # two's complement by hand
                out[r][k] = v * Fraction(float(q["scales"][r]))
            elif scheme in ("mxfp8", "mxfp4", "mxfp4_dual"):
                if scheme == "mxfp8":
                    c = q["codes"][r, k]
                    v = Fraction(float(F.e4m3_decode(np.array([c], np.uint8))[0]))
                else:
                    byte = int(q["codes"][r, k // 2])
                    nib = (byte >> 4) if k % 2 else (byte & 0xF)
                    v = Fraction(float(F.e2m1_decode(np.array([nib]))[0]))
                X = int(q["scales"][r, k // 32]) - 127
                out[r][k] = v * (Fraction(2) ** X)
                if scheme == "mxfp4_dual":     # times the coarse fp32 scale of the 512-block
                    out[r][k] *= Fraction(float(np.float32(q["coarse"][r, k // 512])))
            else:
                word = int(q["codes"][r, k // 8])
                code = (word >> (4 * (k % 8))) & 0xF
                z = int(q["zeros"][r, k // 128])
                s = Fraction(float(F.bf16_to_f32(np.array([q["scales"][r, k // 128]], np.uint16))[0]))
                out[r][k] = (code - z) * s
    return out


@pytest.mark.parametrize("scheme", ["fp8_tensor", "fp8_row", "fp8_block128", "mxfp8", "mxfp4",
                                    "w4a16_asym", "int8_row", "mxfp4_dual"])
def test_random_tiny_gemm_against_exact_rationals(scheme):
    rng = np.random.default_rng(7 + len(scheme) * 31 + ord(scheme[-1]))
    for trial in range(3):
        M, N = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        K = int(rng.choice([128, 256])) if scheme in ("fp8_block128", "w4a16_asym") else int(rng.choice([32, 64, 128, 256]))
        if scheme == "mxfp4_dual":
            K = int(rng.choice([512, 1024]))
        Nw = 128 if scheme == "fp8_block128" else N
        a_bits = small_case(1000 + trial, M, K, 1.0)
        w_bits = small_case(2000 + trial, Nw, K, 0.02)
        w_q = oracle.quantize(w_bits, scheme, "weight")
        if scheme == "w4a16_asym":
            a_in = a_bits
            A = [[Fraction(float(v)) for v in row] for row in F.bf16_to_f32(a_bits)]
        else:
            a_in = oracle.quantize(a_bits, scheme, "activation")
            A = _frac_dequant(a_in)
        W = _frac_dequant(w_q)
        c = oracle.gemm_ref(a_in, w_q)
        assert c.shape == (M, Nw)
        for m in range(M):
            for n in range(min(Nw, 3)):
                terms = [A[m][k] * W[n][k] for k in range(K)]
                exact = sum(terms, Fraction(0))
                bound = K * 2.0 ** -53 * float(sum(abs(t) for t in terms))
                assert abs(c[m, n] - float(exact)) <= bound + 1e-300, (m, n)


def test_orientation_a_times_w_transposed():
    """A[2, 128] with distinct rows times W[3, 128]: C[m, n] = <A[m], W[n]>."""
    a = np.zeros((2, 128), np.float32)
    a[0, 0] = 1.0
    a[1, 1] = 1.0
    q = np.full((3, 128), 8, np.uint8)
    q[:, 0] = [9, 10, 11]       # (q - z) = 1, 2, 3 at k = 0
    q[:, 1] = [12, 13, 14]      # 4, 5, 6 at k = 1
    w = {"scheme": "w4a16_sym", "role": "weight", "rows": 3, "cols": 128,
         "codes": F.pack_int4(q), "scales": f32_to_bf16_bits(np.ones((3, 1), np.float32)),
         "zeros": np.full((3, 1), 8, np.uint8)}
    assert oracle.gemm_ref(f32_to_bf16_bits(a), w).tolist() == [[1, 2, 3], [4, 5, 6]]


def test_rel_fro_error():
    ref = np.array([[3.0, 4.0]])
    assert oracle.rel_fro_error(ref, ref) == 0.0
    assert abs(oracle.rel_fro_error(np.array([[3.0, 4.05]]), ref) - 0.01) < 1e-12


def test_epilogue_alpha_bias_hand_checked():
    """FP8 per tensor, K = 32: A codes all 1.0 (0x38) with s_a = 2; W row 0 all 0.5
    (0x30), row 1 all 2.0 (0x40), s_w = 1.  Products 2*32*0.5 = 32 and 2*32*2 = 128;
    alpha = 0.5, bias = [1, -3]: C = [17, 61]."""
    a = {"scheme": "fp8_tensor", "role": "activation", "rows": 1, "cols": 32,
         "codes": np.full((1, 32), 0x38, np.uint8), "scales": np.array([2.0], np.float32), "zeros": None}
    w = {"scheme": "fp8_tensor", "role": "weight", "rows": 2, "cols": 32,
         "codes": np.stack([np.full(32, 0x30), np.full(32, 0x40)]).astype(np.uint8),
         "scales": np.array([1.0], np.float32), "zeros": None}
    bias = f32_to_bf16_bits(np.array([1.0, -3.0], np.float32))
    assert oracle.gemm_ref(a, w).tolist() == [[32.0, 128.0]]
    assert oracle.gemm_ref(a, w, alpha=0.5, bias=bias).tolist() == [[17.0, 61.0]]
    assert oracle.gemm_ref_entries(a, w, [0], [1], alpha=0.5, bias=bias).tolist() == [[61.0]]


def test_int8_hand_checked():
    """int8 per row, K = 4: A = [127, -128, 1, 0] with s_a = 0.5, W = [1, 1, 2, 5] with
    s_w = 4: sum = 127 - 128 + 2 = 1, C = 1 * 0.5 * 4 = 2."""
    a = {"scheme": "int8_row", "role": "activation", "rows": 1, "cols": 4,
         "codes": np.array([[127, -128, 1, 0]], np.int8), "scales": np.array([0.5], np.float32), "zeros": None}
    w = {"scheme": "int8_row", "role": "weight", "rows": 1, "cols": 4,
         "codes": np.array([[1, 1, 2, 5]], np.int8), "scales": np.array([4.0], np.float32), "zeros": None}
    assert oracle.gemm_ref(a, w).tolist() == [[2.0]]


@pytest.mark.parametrize("scheme", ["fp8_tensor", "fp8_row", "fp8_block128", "int8_row"])
def test_random_tiny_epilogue_against_exact_rationals(scheme):
    """alpha * sum + bias against Fractions: a dropped alpha, a bias on the wrong axis
    (rows instead of columns) or a bias scaled by alpha fails."""
    rng = np.random.default_rng(17 + len(scheme))
    M, N, K = 3, 128 if scheme == "fp8_block128" else 5, 256
    a_q = oracle.quantize(small_case(300, M, K, 1.0), scheme, "activation")
    w_q = oracle.quantize(small_case(301, N, K, 0.02), scheme, "weight")
    alpha = np.float32(rng.uniform(0.25, 3.0))
    bias = f32_to_bf16_bits(rng.normal(0, 1, N).astype(np.float32))
    bias_f = [Fraction(float(v)) for v in F.bf16_to_f32(bias)]
    A, W = _frac_dequant(a_q), _frac_dequant(w_q)
    c = oracle.gemm_ref(a_q, w_q, alpha=alpha, bias=bias)
    for m in range(M):
        for n in range(min(N, 6)):
            terms = [A[m][k] * W[n][k] for k in range(K)]
            exact = Fraction(float(alpha)) * sum(terms, Fraction(0)) + bias_f[n]
            bound = 4 * K * 2.0 ** -53 * (float(alpha) * float(sum(abs(t) for t in terms)) + abs(float(bias_f[n])))
            assert abs(c[m, n] - float(exact)) <= bound + 1e-300, (m, n)


def test_mxfp4_dual_two_coarse_blocks_scale_separately():
    """K = 1024: coarse block 0 all codes 1.0 (0x2) with s_c 2 (A) and 3 (W); block 1 all
    codes 2.0 (0x4) with s_c 0.5 and 0.25; fine exponents 0.  C = 2*3*512*1 + 0.5*0.25*512*4 = 3328."""
    nib = np.concatenate([np.full(512, 0x2), np.full(512, 0x4)]).astype(np.uint8)[None, :]
    fine = np.full((1, 32), 127, np.uint8)
    a = {"scheme": "mxfp4_dual", "role": "activation", "rows": 1, "cols": 1024, "codes": F.pack_fp4(nib),
         "scales": fine, "coarse": np.array([[2.0, 0.5]], np.float32), "zeros": None}
    w = dict(a, role="weight", coarse=np.array([[3.0, 0.25]], np.float32))
    assert oracle.gemm_ref(a, w).tolist() == [[3328.0]]
