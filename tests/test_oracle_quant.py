"""Pins for the oracle's quantizers and dequantizers (CPU only).

What pins them, besides the codecs' own pins:
* hand-worked examples under tests/golden/ (FP8 per-tensor, MX, int4);
* the e8m0 exponent rule at powers of two and their predecessors;
* exact reproduction: tensors built from chosen codes and power-of-two scales
  (with one element at the format maximum) must come back unchanged, per row,
  per block and per group -- a transposed or mis-indexed scale fails here;
* the per-element error bound of half a grid step times the scale;
* the double rounding of the fp32 quotient, on inputs found by an exact
  rational search;
* torch's own e4m3fn cast for the special case s = 1.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from golden_io import keyed, parse_floats, parse_hex
from workloads import f32_to_bf16_bits, small_case
import workloads as wl


def bf16(vals):
    v = np.asarray(vals, dtype=np.float32)
    b = f32_to_bf16_bits(v)
    assert np.array_equal(F.bf16_to_f32(b), v), "fixture value not bf16-exact"
    return b


# ---------------------------------------------------------------- golden examples
def test_golden_fp8_tensor():
    g = keyed("fp8_tensor_worked_example.txt")
    x = bf16(np.stack([parse_floats(r) for r in g["input"]]))
    q = oracle.quantize(x, "fp8_tensor")
    assert q["scales"].dtype == np.float32 and q["scales"].tolist() == [float(g["scale"][0][0])]
    expect = np.stack([parse_hex(r) for r in g["codes"]]).astype(np.uint8)
    assert np.array_equal(q["codes"], expect)


@pytest.mark.parametrize("role", ["activation", "weight"])
def test_golden_mx(role):
    g = keyed("mx_worked_example.txt")
    row = np.concatenate([parse_floats(g[f"input_block{i}"][0]) for i in range(3)])
    x = bf16(row[None, :])
    q8 = oracle.quantize(x, "mxfp8", role)
    assert q8["scales"].tolist() == [parse_hex(g["mxfp8_scales"][0]).tolist()]
    c0 = parse_hex(g["mxfp8_codes_block0"][0])
    c2 = parse_hex(g["mxfp8_codes_block2"][0])
    exp8 = np.zeros(96, np.uint8)
    exp8[:len(c0)] = c0
    exp8[64:64 + len(c2)] = c2
    assert np.array_equal(q8["codes"][0], exp8)
    q4 = oracle.quantize(x, "mxfp4", role)
    assert q4["scales"].tolist() == [parse_hex(g["mxfp4_scales"][0]).tolist()]
    b0 = parse_hex(g["mxfp4_bytes_block0"][0])
    b2 = parse_hex(g["mxfp4_bytes_block2"][0])
    exp4 = np.zeros(48, np.uint8)
    exp4[:len(b0)] = b0
    exp4[32:32 + len(b2)] = b2
    assert np.array_equal(q4["codes"][0], exp4)


@pytest.mark.parametrize("sym", [False, True])
def test_golden_int4(sym):
    g = keyed("int4_worked_example.txt")
    x = np.zeros(128, np.float64)
    first = parse_floats(g["input"][0])
    x[:len(first)] = first
    q = oracle.quantize(bf16(x[None, :]), "w4a16_sym" if sym else "w4a16_asym", "weight")
    key = "sym" if sym else "asym"
    assert q["scales"].tolist() == [[int(g[f"{key}_scale_bits"][0][0], 16)]]
    assert q["zeros"].tolist() == [[int(g[f"{key}_zero"][0][0])]]
    words = [int(g[f"{key}_word0"][0][0], 16)] + [int(g[f"{key}_rest"][0][0], 16)] * 15
    assert q["codes"].tolist() == [words]


# ---------------------------------------------------------------- e8m0 exponent rule
@pytest.mark.parametrize("emax", [8, 2])
def test_e8m0_rule_powers_of_two(emax):
    for k in range(-133, 128):
        a = np.float32(2.0 ** k)
        if a == 0:
            continue
        assert oracle.mx_exponent(np.array([a]), emax)[0] == np.clip(k - emax, -127, 127)
        below = np.nextafter(a, np.float32(0), dtype=np.float32)
        if below > 0:
            assert oracle.mx_exponent(np.array([below]), emax)[0] == np.clip(k - 1 - emax, -127, 127)
    assert oracle.mx_exponent(np.array([0.0]), emax)[0] == -127
    assert oracle.mx_exponent(np.array([np.float32(3.3e38)]), emax)[0] == 127 - emax


def test_mx_block_at_format_max_has_unit_scale():
    x = np.zeros((1, 64), np.float32)
    x[0, 0] = 448.0
    x[0, 33] = -6.0
    q8 = oracle.quantize(bf16(x), "mxfp8")
    q4 = oracle.quantize(bf16(x), "mxfp4")
    assert q8["scales"][0, 0] == 127 and q8["codes"][0, 0] == 0x7E
    assert q4["scales"][0, 1] == 127 and (q4["codes"][0, 16] >> 4) == 0xF


# ---------------------------------------------------------------- exact reproduction
def _rng(seed):
    return np.random.default_rng(seed)


def test_fp8_exact_reproduction_tensor_row_block():
    rng = _rng(21)
    fin = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    R, K = 256, 384
    codes = rng.choice(fin, (R, K)).astype(np.uint8)
    # per-row scales 2^j: every row has one element at +-448
    j_row = rng.integers(-20, 10, R)
    codes_r = codes.copy()
    codes_r[np.arange(R), rng.integers(0, K, R)] = rng.choice([0x7E, 0xFE], R)
    x = F.e4m3_decode(codes_r) * np.ldexp(1.0, j_row)[:, None]
    q = oracle.quantize(bf16(x), "fp8_row", "weight")
    assert np.array_equal(q["codes"], codes_r)
    assert np.array_equal(q["scales"], np.ldexp(1.0, j_row).astype(np.float32))
    # per-tensor
    xt = F.e4m3_decode(codes_r) * 2.0 ** -3
    q = oracle.quantize(bf16(xt), "fp8_tensor")
    assert np.array_equal(q["codes"], codes_r) and q["scales"].tolist() == [2.0 ** -3]
    # activation 1x128 groups
    j_g = rng.integers(-15, 15, (R, K // 128))
    cg = codes.copy().reshape(R, K // 128, 128)
    for r in range(R):
        for g in range(K // 128):
            cg[r, g, rng.integers(0, 128)] = 0x7E
    cg = cg.reshape(R, K)
    x = F.e4m3_decode(cg) * np.repeat(np.ldexp(1.0, j_g), 128, axis=1)
    q = oracle.quantize(bf16(x), "fp8_block128", "activation")
    assert np.array_equal(q["codes"], cg)
    assert np.array_equal(q["scales"], np.ldexp(1.0, j_g).astype(np.float32))
    # weight 128x128 blocks
    j_b = rng.integers(-15, 15, (R // 128, K // 128))
    cb = codes.copy()
    for rb in range(R // 128):
        for g in range(K // 128):
            cb[rb * 128 + rng.integers(0, 128), g * 128 + rng.integers(0, 128)] = 0xFE
    sc = np.repeat(np.repeat(np.ldexp(1.0, j_b), 128, axis=0), 128, axis=1)
    q = oracle.quantize(bf16(F.e4m3_decode(cb) * sc), "fp8_block128", "weight")
    assert np.array_equal(q["codes"], cb)
    assert np.array_equal(q["scales"], np.ldexp(1.0, j_b).astype(np.float32))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_exact_reproduction(fmt):
    rng = _rng(22)
    R, K = 64, 256
    if fmt == "mxfp8":
        fin = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
        codes = rng.choice(fin, (R, K)).astype(np.uint8)
        top = np.array([0x7E, 0xFE])
        dec = F.e4m3_decode
    else:
        codes = rng.integers(0, 16, (R, K)).astype(np.uint8)
        top = np.array([0x7, 0xF])
        dec = F.e2m1_decode
    cb = codes.reshape(R, K // 32, 32)
    for r in range(R):
        for b in range(K // 32):
            cb[r, b, rng.integers(0, 32)] = rng.choice(top)
    codes = cb.reshape(R, K)
    X = rng.integers(-100, 100, (R, K // 32))
    x = dec(codes) * np.repeat(np.ldexp(1.0, X), 32, axis=1)
    q = oracle.quantize(bf16(x), fmt)
    assert np.array_equal(q["scales"], (X + 127).astype(np.uint8))
    want = codes if fmt == "mxfp8" else F.pack_fp4(codes)
    # -0 elements may appear as +0 only where the code itself is a zero: codes keep sign
    assert np.array_equal(q["codes"], want)


@pytest.mark.parametrize("sym", [False, True])
def test_int4_exact_reproduction(sym):
    rng = _rng(23)
    R, K = 32, 512
    G = K // 128
    j = rng.integers(-12, 0, (R, G))
    if sym:
        z = np.full((R, G), 8)
        q = rng.integers(1, 16, (R, K)).reshape(R, G, 128)   # q - 8 in [-7, 7]
        q[:, :, 0] = 15                                      # amax = 7 * 2^j
    else:
        z = rng.integers(0, 16, (R, G))
        q = rng.integers(0, 16, (R, K)).reshape(R, G, 128)
        q[:, :, 0] = 0
        q[:, :, 1] = 15
    x = (q - z[:, :, None]) * np.ldexp(1.0, j)[:, :, None]
    out = oracle.quantize(bf16(x.reshape(R, K)), "w4a16_sym" if sym else "w4a16_asym", "weight")
    assert np.array_equal(F.unpack_int4(out["codes"]), q.reshape(R, K).astype(np.uint8))
    assert np.array_equal(out["zeros"], z.astype(np.uint8))
    assert np.array_equal(F.bf16_to_f32(out["scales"]), np.ldexp(1.0, j).astype(np.float32))


# ---------------------------------------------------------------- error bounds
def _grid_half_step(v, fmt):
    a = np.abs(v)
    emin, mb = (-6, 3) if fmt == "e4m3" else (0, 1)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), emin)
    return np.ldexp(0.5, (e - mb).astype(int))


@pytest.mark.parametrize("scheme,role", [("fp8_tensor", "activation"), ("fp8_row", "activation"),
                                         ("fp8_row", "weight"), ("fp8_block128", "activation"),
                                         ("fp8_block128", "weight")])
def test_fp8_error_bound(scheme, role):
    x = small_case(31, 256, 512, 1.0)
    xf = F.bf16_to_f32(x).astype(np.float64)
    q = oracle.quantize(x, scheme, role)
    dq = oracle.dequant_exact(q)
    s = oracle.quant._expand_scale_f32(q).astype(np.float64)
    bound = _grid_half_step(xf / s, "e4m3") * s + np.abs(xf) * 2.0 ** -24
    assert np.all(np.abs(xf - dq) <= bound)
    # every unit's largest element maps to +-448 * s (within the fp32 quotient rounding)
    assert np.max(np.abs(dq)) <= 448 * np.max(s)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_error_bound(fmt):
    x = small_case(32, 128, 512, 1.0)
    xf = F.bf16_to_f32(x).astype(np.float64)
    q = oracle.quantize(x, fmt)
    dq = oracle.dequant_exact(q)
    sc = np.repeat(F.e8m0_decode(q["scales"]), 32, axis=1)
    v = xf / sc
    vmax = 448.0 if fmt == "mxfp8" else 6.0
    sat = np.abs(v) > vmax
    half = _grid_half_step(v, "e4m3" if fmt == "mxfp8" else "e2m1") * sc
    assert np.all(np.abs(xf - dq)[~sat] <= half[~sat])
    assert np.all(np.abs(dq[sat]) == vmax * sc[sat])


@pytest.mark.parametrize("sym", [False, True])
def test_int4_error_bound(sym):
    x = small_case(33, 64, 1024, 0.02)
    xf = F.bf16_to_f32(x).astype(np.float64).reshape(64, 8, 128)
    q = oracle.quantize(x, "w4a16_sym" if sym else "w4a16_asym", "weight")
    dq = oracle.dequant_exact(q).reshape(64, 8, 128)
    s = F.bf16_to_f32(q["scales"]).astype(np.float64)
    if sym:
        s32 = (np.max(np.abs(xf), axis=2).astype(np.float32) / np.float32(7)).astype(np.float64)
        span = 7.0
    else:
        d = (np.maximum(xf.max(2), 0) - np.minimum(xf.min(2), 0)).astype(np.float32)
        s32 = (d / np.float32(15)).astype(np.float64)
        span = 15.0
    bound = 0.5 * s + span * np.abs(s32 - s) + 1e-12
    assert np.all(np.abs(xf - dq) <= bound[:, :, None] * 1.0000001)


# ---------------------------------------------------------------- double rounding
def _e4m3_exact_rational(qf: Fraction) -> int:
    """e4m3 code of the exact rational (no fp32 step), by search over the table."""
    vals = [(c, Fraction(float(F.e4m3_decode(np.array([c], np.uint8))[0]))) for c in range(0x7F)]
    a = min(abs(qf), Fraction(448))
    best = min(vals, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))
    return best[0] | (0x80 if qf < 0 else 0)


def test_fp32_quotient_is_formed_before_the_e4m3_rounding():
    """Find bf16 (amax, x) where the exact x/s lies just off an e4m3 midpoint while
    the fp32 quotient lands on it (e.g. amax 1.34375, x 1.0078125: fp32 x/s = 336,
    the midpoint of 320 and 352).  The scheme rounds the fp32 quotient, ties to
    even (0x7A); rounding the exact rational would give 0x7B."""
    found = 0
    for ab in range(0x3FAC, 0x3FD8):
        amax = F.bf16_to_f32(np.array([ab], np.uint16))[0]
        s = np.float32(amax / np.float32(448))
        xs = F.bf16_to_f32(np.arange(0x3F80, ab + 1, dtype=np.uint16))
        q32 = (xs / s).astype(np.float32)
        for xv, qv in zip(xs, q32):
            exact = Fraction(float(xv)) / Fraction(float(s))
            if Fraction(float(qv)) == exact:
                continue
            c_exact = _e4m3_exact_rational(exact)
            c_fp32 = _e4m3_exact_rational(Fraction(float(qv)))
            if c_exact == c_fp32:
                continue
            x = np.zeros((1, 2), np.float32)
            x[0, 0] = amax
            x[0, 1] = xv
            q = oracle.quantize(f32_to_bf16_bits(x), "fp8_tensor")
            assert q["scales"][0] == s
            assert q["codes"][0, 1] == c_fp32
            found += 1
        if found >= 3:
            break
    assert found >= 3


# ---------------------------------------------------------------- special cases
def test_fp8_unit_scale_matches_torch_cast():
    x = small_case(41, 64, 256, 30.0)
    xf = F.bf16_to_f32(x)
    xf = np.clip(xf, -447, 447)
    xf[0, 0] = 448.0
    xb = f32_to_bf16_bits(xf)
    q = oracle.quantize(xb, "fp8_tensor")
    assert q["scales"].tolist() == [1.0]
    ref = torch.from_numpy(F.bf16_to_f32(xb)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q["codes"], ref)


def test_zero_inputs():
    z = np.zeros((128, 256), np.uint16)
    for scheme in ("fp8_tensor", "fp8_row", "fp8_block128"):
        q = oracle.quantize(z, scheme, "weight")
        assert np.all(q["codes"] == 0) and np.all(q["scales"] == 1.0)
    for scheme in ("mxfp8", "mxfp4"):
        q = oracle.quantize(z, scheme)
        assert np.all(q["codes"] == 0) and np.all(q["scales"] == 0)
    q = oracle.quantize(z, "w4a16_asym", "weight")
    assert np.all(q["zeros"] == 0) and np.all(F.bf16_to_f32(q["scales"]) == 1.0)
    assert np.all(q["codes"] == 0)
    q = oracle.quantize(z, "w4a16_sym", "weight")
    assert np.all(q["zeros"] == 8) and np.all(q["codes"] == 0x88888888)


def test_negative_zero_and_tiny_keep_sign():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    x[0, 1] = -1e-6
    xb = f32_to_bf16_bits(x)
    xb[0, 2] = 0x8000
    q8 = oracle.quantize(xb, "mxfp8")
    assert q8["codes"][0, 1] == 0x80 and q8["codes"][0, 2] == 0x80
    q = oracle.quantize(xb, "fp8_row")
    assert q["codes"][0, 1] == 0x80 and q["codes"][0, 2] == 0x80


def test_subnormal_amax():
    # amax = 2^-133 (smallest bf16 subnormal): s = fp32(2^-133 / 448) is the fp32
    # subnormal 146 * 2^-149 (bits 0x92); x / s = 65536 / 146 = 448.9 saturates to 0x7E.
    x = np.zeros((1, 128), np.uint16)
    x[0, 5] = 0x0001
    q = oracle.quantize(x, "fp8_row")
    assert q["scales"].view(np.uint32).tolist() == [0x92]
    assert q["codes"][0, 5] == 0x7E and np.count_nonzero(q["codes"]) == 1
    # MX: X = floor(log2 2^-133) - 8 = -141, clamped to -127 (code 0); 2^-133 * 2^127 = 2^-6
    q = oracle.quantize(x, "mxfp8")
    assert q["scales"][0, 0] == 0 and q["codes"][0, 5] == 0x08


def test_dequantize_rounds_once_to_bf16():
    rng = _rng(51)
    x = small_case(52, 64, 256, 1.0)
    for scheme, role in (("fp8_row", "activation"), ("fp8_block128", "weight"),
                         ("mxfp8", "activation"), ("mxfp4", "weight"), ("w4a16_asym", "weight")):
        q = oracle.quantize(x if scheme != "fp8_block128" else small_case(53, 128, 256), scheme, role)
        y = oracle.dequantize(q)
        exact = oracle.dequant_exact(q)
        # bf16 of the exact product (products are exact in fp32 here) == torch's cast
        ref = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
        assert np.array_equal(y, ref.view(np.uint16)), scheme


def test_scheme_validation():
    x = np.zeros((2, 96), np.uint16)
    with pytest.raises(ValueError):
        oracle.quantize(x, "fp8_block128")
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 48), np.uint16), "mxfp8")
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 128), np.uint16), "w4a16_asym", "activation")
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((64, 128), np.uint16), "fp8_block128", "weight")
    with pytest.raises(ValueError):
        oracle.quantize(x, "nvfp4")


# ---------------------------------------------------------------- static FP8 scales
def test_golden_fp8_static_tensor():
    g = keyed("fp8_static_tensor_worked_example.txt")
    x = bf16(np.stack([parse_floats(r) for r in g["input"]]))
    s = np.array([float(g["scale"][0][0])], np.float32)
    q = oracle.quantize_static(x, "fp8_tensor", "activation", s)
    expect = np.stack([parse_hex(r) for r in g["codes"]]).astype(np.uint8)
    assert np.array_equal(q["codes"], expect)
    assert q["scales"].tolist() == [0.03125]


@pytest.mark.parametrize("role", ["activation", "weight"])
def test_fp8_static_block_exact_reproduction_and_placement(role):
    """Static 128-block scales: x built as codes times a distinct power-of-two scale per
    block comes back unchanged only if each block is divided by its own scale (a
    transposed or mis-indexed scale array fails)."""
    rng = np.random.default_rng(5)
    rows, cols = 256, 384
    vals = F.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8))
    codes = rng.choice(np.arange(0x00, 0x7F), size=(rows, cols)).astype(np.uint8)
    signs = rng.choice([0, 0x80], size=(rows, cols)).astype(np.uint8)
    codes = codes | signs
    codes[codes == 0x80] = 0x00
    if role == "activation":
        sh = (rows, cols // 128)
        s = np.ldexp(1.0, rng.integers(-12, 4, size=sh)).astype(np.float32)
        per = np.repeat(s, 128, axis=1)
    else:
        sh = (rows // 128, cols // 128)
        s = np.ldexp(1.0, rng.integers(-12, 4, size=sh)).astype(np.float32)
        per = np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)
    x = F.e4m3_decode(codes) * per
    xb = bf16(x.astype(np.float32))
    q = oracle.quantize_static(xb, "fp8_block128", role, s)
    assert np.array_equal(q["codes"], codes)
    assert vals.max() == 448.0


def test_fp8_static_saturates_beyond_448_s():
    """A static scale below amax / 448 saturates: |x| / s above 448 gives +-448."""
    x = bf16([[1.0, -1.0, 0.5, 2.0 ** -20, -2.0 ** 10, 448.0 / 64]])
    q = oracle.quantize_static(x, "fp8_tensor", "activation", np.array([2.0 ** -6], np.float32))
    # 64, -64, 32, 2^-14 (below the smallest subnormal 2^-9, rounds to 0), -65536 -> -448, 448
    assert q["codes"].tolist() == [[0x68, 0xE8, 0x60, 0x00, 0xFE, 0x7E]]
    # quotients that overflow fp32 (2^127 / 2^-2 = 2^129) are infinite and saturate with their sign
    x = bf16([[2.0 ** 127, -(2.0 ** 127), -0.0, 1.0]])
    q = oracle.quantize_static(x, "fp8_tensor", "activation", np.array([0.25], np.float32))
    assert q["codes"].tolist() == [[0x7E, 0xFE, 0x80, 0x48]]


def test_fp8_static_with_the_dynamic_scale_equals_dynamic():
    x = small_case(11, 6, 256, 1.0)
    for scheme, role in (("fp8_tensor", "activation"), ("fp8_block128", "activation")):
        d = oracle.quantize(x, scheme, role)
        s = oracle.quantize_static(x, scheme, role, d["scales"])
        assert np.array_equal(d["codes"], s["codes"])


def test_static_scheme_validation():
    x = small_case(1, 2, 128, 1.0)
    with pytest.raises(ValueError):
        oracle.quantize_static(x, "fp8_row", "activation", np.ones(2, np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_static(x, "int8_row", "activation", np.ones(2, np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_static(x, "fp8_tensor", "activation", np.array([0.0], np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_static(x, "fp8_tensor", "activation", np.array([np.inf], np.float32))


# ---------------------------------------------------------------- int8 per row
def test_golden_int8_row():
    g = keyed("int8_row_worked_example.txt")
    x = bf16(np.stack([parse_floats(r) for r in g["input"]]))
    for role in ("activation", "weight"):
        q = oracle.quantize(x, "int8_row", role)
        assert q["scales"].tolist() == [float(v) for v in g["scale"][0]]
        expect = np.stack([parse_hex(r) for r in g["codes"]]).astype(np.uint8)
        assert np.array_equal(q["codes"].view(np.uint8), expect)


def test_int8_exact_reproduction():
    """Rows k * 2^e with integer k in [-127, 127] and k = 127 present: s = 2^e and the
    codes are k, row by row with distinct e (a mis-indexed scale fails)."""
    rng = np.random.default_rng(9)
    rows, cols = 8, 96
    k = rng.integers(-127, 128, size=(rows, cols))
    k[:, 5] = 127
    e = np.arange(-6, -6 + rows)
    x = bf16((k * np.ldexp(1.0, e)[:, None]).astype(np.float32))
    q = oracle.quantize(x, "int8_row", "activation")
    assert np.array_equal(q["codes"].astype(np.int64), k)
    assert np.array_equal(q["scales"], np.ldexp(1.0, e).astype(np.float32))


def test_int8_error_bound_and_range():
    x = small_case(3, 16, 512, 1.0)
    q = oracle.quantize(x, "int8_row", "weight")
    xf = F.bf16_to_f32(x).astype(np.float64)
    s = q["scales"].astype(np.float64)[:, None]
    assert q["codes"].min() >= -127 and q["codes"].max() <= 127
    # half a step, plus the fp32 rounding of the quotient (at most 127 * 2^-24 steps)
    assert np.all(np.abs(q["codes"] * s - xf) <= s * (0.5 + 2.0 ** -16))
    assert np.all(np.abs(q["codes"]).max(axis=1) == 127)


def test_int8_dequantize_rounds_once():
    x = small_case(4, 3, 64, 1.0)
    q = oracle.quantize(x, "int8_row", "activation")
    y = F.bf16_to_f32(oracle.dequantize(q))
    prod = (q["codes"].astype(np.float32) * q["scales"][:, None]).astype(np.float32)
    assert np.array_equal(y, F.bf16_to_f32(F.f32_to_bf16_rne(prod)))


# ----------------------------------------------------------------- dual-scale MXFP4
def test_mxfp4_dual_worked_example():
    """tests/golden/mxfp4_dual_worked_example.txt: coarse fp32 scale, fine exponents and
    codes worked by hand (every element not listed is 0 with code 0; unlisted blocks
    are all-zero, fine code 0)."""
    from golden_io import keyed
    d = keyed("mxfp4_dual_worked_example.txt")
    x = np.zeros((2, 512), np.float32)
    for r, k, v in d["x"]:
        x[int(r), int(k)] = np.float32(float(v))
    q = oracle.quantize(wl.f32_to_bf16_bits(x), "mxfp4_dual", "activation")
    coarse = np.asarray(q["coarse"], np.float32).view(np.uint32)
    for r, h in d["coarse"]:
        assert coarse[int(r), 0] == int(h, 16)
    fine = np.zeros((2, 16), np.uint8)
    for r, b, c in d["fine"]:
        fine[int(r), int(b)] = int(c)
    assert np.array_equal(q["scales"], fine)
    codes = np.zeros((2, 512), np.uint8)
    for r, k, c in d["code"]:
        codes[int(r), int(k)] = int(c, 16)
    assert np.array_equal(F.unpack_fp4(q["codes"]), codes)


@pytest.mark.parametrize("coarse_mant", [1.0, 1.5])
def test_mxfp4_dual_exact_reproduction(coarse_mant):
    """Values e2m1 * 2^X * s_c with s_c = m 2^j (m = 1 or 1.5, exact in bf16 together with
    any e2m1 value) and one element of each 512-block at 6 * s_c: the coarse scale, fine
    exponents and codes come back exactly, including a non-power-of-two coarse scale."""
    rng = np.random.default_rng(int(coarse_mant * 10))
    rows, cols = 6, 1024
    nib = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    X = rng.integers(-6, 1, (rows, cols // 32))
    X[:, ::16] = 0                                     # the block holding the 6 keeps X = 0
    nib[:, ::512] = 0x7                                # +6 in every 512-block's first element
    j = rng.integers(-4, 5, (rows, cols // 512))
    s_c = (coarse_mant * np.ldexp(1.0, j)).astype(np.float32)
    # every 32-block needs a magnitude-6 element for its X to be recovered exactly
    nib[:, 5::32] = 0xF
    vals = F.e2m1_decode(nib) * np.repeat(np.ldexp(1.0, X), 32, axis=1) * np.repeat(s_c, 512, axis=1)
    bits = wl.f32_to_bf16_bits(vals.astype(np.float32))
    assert np.array_equal(F.bf16_to_f32(bits).astype(np.float64), vals)       # representable
    q = oracle.quantize(bits, "mxfp4_dual", "weight")
    assert np.array_equal(np.asarray(q["coarse"], np.float32), s_c)
    assert np.array_equal(q["scales"].astype(np.int64) - 127, X)
    # the sign of zero is kept, so compare values (and codes away from zero)
    got = F.unpack_fp4(q["codes"])
    assert np.array_equal(F.e2m1_decode(got), F.e2m1_decode(nib))
    assert np.array_equal(oracle.dequant_exact(q), vals)


def test_mxfp4_dual_error_bound_and_zero_blocks():
    x = wl.small_case(77, 16, 2048).copy()
    x[3, 512:1024] = 0                                   # an all-zero coarse block
    x[5, :32] = 0                                        # an all-zero fine block
    q = oracle.quantize(x, "mxfp4_dual", "activation")
    xf = F.bf16_to_f32(x).astype(np.float64)
    assert q["coarse"][3, 1] == 1.0 and np.all(F.unpack_fp4(q["codes"])[3, 512:1024] & 7 == 0)
    assert q["scales"][5, 0] == 0
    s_c = np.repeat(np.asarray(q["coarse"], np.float64), 512, axis=1)
    X = np.repeat(q["scales"].astype(np.int64) - 127, 32, axis=1)
    v = (xf / s_c).astype(np.float32).astype(np.float64) * np.ldexp(1.0, -X)     # the grid value
    dq = oracle.dequant_exact(q)
    sat = np.abs(v) > 6
    # half an e2m1 ulp at the element's binade (0.5 below 1, then 0.5, 0.5, 1, 1, 2 ...)
    e = np.maximum(np.floor(np.log2(np.maximum(np.abs(v), 1e-300))), 0)
    half_ulp = np.ldexp(0.25, e.astype(np.int64))
    bound = half_ulp * np.ldexp(1.0, X) * s_c + np.abs(xf) * 2.0 ** -23
    assert np.all(np.abs(xf - dq)[~sat] <= bound[~sat])
    assert np.all(np.abs(dq[sat]) == 6 * np.ldexp(1.0, X[sat]) * s_c[sat])


def test_mxfp4_dual_dequantize_rounds_once():
    x = wl.small_case(78, 8, 512)
    q = oracle.quantize(x, "mxfp4_dual", "activation")
    want = F.f32_to_bf16_rne(oracle.dequant_exact(q).astype(np.float32))   # exact value, one rounding
    assert np.array_equal(oracle.dequantize(q), want)


def test_mxfp4_dual_rejects_k_not_multiple_of_512():
    with pytest.raises(ValueError):
        oracle.quantize(wl.small_case(1, 2, 256), "mxfp4_dual", "activation")
