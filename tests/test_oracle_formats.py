"""Pins for the oracle's element codecs (CPU only).

Each codec is checked against something other than itself: the hand-written
code tables under tests/golden/, an exhaustive brute-force nearest-value search
over the code table, every rounding midpoint, and torch's own float8 decoders
and round-to-nearest-even casts (library routines).
"""
import numpy as np
import pytest
import torch

from oracle import formats as F
from golden_io import code_table


def _brute_nearest_even(v, codes, values):
    """Nearest representable value to v, ties to the code with an even mantissa lsb,
    saturating to the largest finite magnitude; sign of zero kept.  Pure search."""
    out = []
    finite = [(c, x) for c, x in zip(codes, values) if np.isfinite(x)]
    vmax = max(abs(x) for _, x in finite)
    for t in v:
        a = min(abs(t), vmax)
        best = None
        for c, x in finite:
            if x < 0 or (x == 0 and np.signbit(x)):
                continue
            d = abs(x - a)
            if best is None or d < best[0] or (d == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
                best = (d, c, x)
        out.append((best[1], np.signbit(t)))
    return out


# ---------------------------------------------------------------- e4m3fn
def test_e4m3_golden_spot_values():
    for code, val in code_table("e4m3fn_codes.txt"):
        got = F.e4m3_decode(np.array([code], np.uint8))[0]
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def test_e4m3_decode_strictly_monotone():
    v = F.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    assert v[-1] == 448.0 and F.E4M3_MAX == 448.0


def test_e4m3_every_midpoint_ties_to_even():
    v = F.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (v[:-1] + v[1:]) / 2
    got = F.e4m3_encode(mids)
    lo = np.arange(0, 0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, expect.astype(np.uint8))
    # the examples a reader can check by eye
    assert F.e4m3_encode(np.array([17.0, 19.0, 2.0 ** -10, 3 * 2.0 ** -10])).tolist() == [
        0x58, 0x5A, 0x00, 0x02]


def test_e4m3_matches_brute_force_search():
    rng = np.random.default_rng(11)
    table = list(range(256))
    vals = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    v = np.concatenate([
        rng.standard_normal(400) * 30,
        rng.uniform(-1, 1, 200) * 2.0 ** -7,
        rng.uniform(440, 600, 50) * rng.choice([-1, 1], 50),
        [0.0, -0.0, 1e-30, -1e-30, 464.0, 1e9, -1e9],
    ])
    brute = _brute_nearest_even(v, table, vals)
    got = F.e4m3_encode(v)
    for g, (c, neg), t in zip(got, brute, v):
        assert g == (c | (0x80 if neg else 0)), (t, hex(g), hex(c))


def test_e4m3_saturates_and_keeps_zero_sign():
    got = F.e4m3_encode(np.array([448.0, 449.0, 463.99, 464.0, 1e6, -1e6, -0.0, -1e-9, 1e-9]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00]


def test_e4m3_agrees_with_torch_rne_cast_below_464():
    # torch's fp32 -> float8_e4m3fn cast rounds to nearest even but does not
    # saturate; below 464 the two definitions coincide.
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(200_000) * rng.choice([1e-3, 0.1, 1, 10, 100], 200_000),
        rng.uniform(-463.9, 463.9, 50_000),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_nonfinite_rejected():
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([np.inf]))
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([np.nan]))


# ---------------------------------------------------------------- e2m1
def test_e2m1_golden_full_table():
    table = code_table("e2m1_codes.txt")
    assert len(table) == 16
    for code, val in table:
        got = F.e2m1_decode(np.array([code]))[0]
        assert got == val and np.signbit(got) == np.signbit(val), hex(code)
        assert F.e2m1_encode(np.array([val]))[0] == code


def test_e2m1_midpoints_and_saturation():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.99, 100.0, -5.0, -0.25, -0.0])
    assert F.e2m1_encode(v).tolist() == [0, 2, 2, 4, 4, 6, 6, 7, 7, 7, 0xE, 0x8, 0x8]


def test_e2m1_matches_brute_force_search():
    rng = np.random.default_rng(12)
    vals = F.e2m1_decode(np.arange(16))
    v = np.concatenate([rng.uniform(-8, 8, 2000), [0.0, -0.0, 6.0, -6.0, 1e-20]])
    brute = _brute_nearest_even(v, list(range(16)), vals)
    got = F.e2m1_encode(v)
    for g, (c, neg), t in zip(got, brute, v):
        assert g == (c | (0x8 if neg else 0)), (t, g, c)


# ---------------------------------------------------------------- e8m0
def test_e8m0_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = F.e8m0_decode(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


# ---------------------------------------------------------------- bf16
def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100_000) * rng.choice([1e-30, 1e-3, 1, 1e3, 1e30], 100_000)).astype(np.float32)
    # exact ties: low half-word 0x8000 with even and odd kept lsb
    ties = (np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x00008000, 0x00018000], np.uint32)
            .view(np.float32))
    x = np.concatenate([x, ties, np.array([3.4e38, -3.4e38, 1e-45], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f32_to_bf16_rne(x), ref)
    back = F.bf16_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


# ---------------------------------------------------------------- packing
def test_fp4_packing_low_nibble_first():
    n = np.array([[0x1, 0x2, 0x3, 0xF]], np.uint8)
    p = F.pack_fp4(n)
    assert p.tolist() == [[0x21, 0xF3]]
    assert np.array_equal(F.unpack_fp4(p), n)


def test_int4_packing_bit_positions():
    codes = np.arange(16, dtype=np.uint8).reshape(1, 16)
    p = F.pack_int4(codes)
    assert p.tolist() == [[0x76543210, 0xFEDCBA98]]
    assert np.array_equal(F.unpack_int4(p), codes)


# ----------------------------------------------------------------- packed MX exponents
def test_pack_mx_scales_hand_example():
    # 2 rows x 5 blocks, chunk 4: chunk 0 holds blocks 0-3 of each row, chunk 1
    # block 4 and three pad bytes of 127 (written out by hand).
    s = np.array([[10, 11, 12, 13, 14],
                  [20, 21, 22, 23, 24]], np.uint8)
    want = np.array([[[10, 11, 12, 13], [20, 21, 22, 23]],
                     [[14, 127, 127, 127], [24, 127, 127, 127]]], np.uint8)
    assert np.array_equal(F.pack_mx_scales(s, 4), want)


def test_pack_mx_scales_positions():
    # every exponent lands at [blk // c, r, blk % c], each position is used once,
    # and the pads are 127
    rng = np.random.default_rng(3)
    for rows, nblk, c in ((3, 8, 8), (5, 12, 4), (4, 36, 8), (1, 1, 4)):
        s = rng.integers(0, 255, (rows, nblk)).astype(np.uint8)
        p = F.pack_mx_scales(s, c)
        assert p.shape == (-(-nblk // c), rows, c)
        for r in range(rows):
            for blk in range(nblk):
                assert p[blk // c, r, blk % c] == s[r, blk]
        assert (p.size - rows * nblk) == int(np.sum(p == 127)) - int(np.sum(s == 127))
