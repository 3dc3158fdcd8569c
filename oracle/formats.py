"""Element formats of the quantized-linear path (oracle; test infrastructure).

The pages name the code dtypes (float8_e4m3fn codes, float8_e8m0fnu shared
exponents, float4_e2m1fn_x2 fp4 pairs: "vLLM-Omni Online Quantization complete
guide", section "How online quantization works underneath", steps 2-3) but do
not define them.  The definitions below are the textbook OCP ones:

* e4m3fn: sign, 4 exponent bits (bias 7), 3 mantissa bits.  Normal values
  (1 + m/8) * 2^(E-7), subnormals m * 2^-9, largest finite 448 (0x7E).
  0x7F / 0xFF are NaN; there is no infinity.
* e2m1: sign (bit 3), 2 exponent bits (bias 1), 1 mantissa bit.  Magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6.  No infinity or NaN.
* e8m0: an unsigned biased exponent, value 2^(c-127); 255 is NaN.

Rounding onto a grid is round-to-nearest, ties to even, saturating at the
largest finite magnitude, keeping the sign of zero.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


# ---------------------------------------------------------------- decoding
def e4m3_decode(codes) -> np.ndarray:
    """e4m3fn code (uint8) -> float64 value; NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, E - 7)
    sub = m * 2.0 ** -9
    mag = np.where(E == 0, sub, normal)
    mag = np.where((E == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def e2m1_decode(nibbles) -> np.ndarray:
    """e2m1 code (0..15) -> float64 value."""
    c = np.asarray(nibbles).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    E = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(E == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, E - 1))
    return sign * mag


def e8m0_decode(codes) -> np.ndarray:
    """e8m0 code -> 2^(c-127) as float64 (code 255 -> NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, v)


# ---------------------------------------------------------------- encoding
def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for a > 0 (exact, via frexp); 0 maps to a large negative."""
    m, e = np.frexp(a)
    return np.where(a > 0, e - 1, -10_000)


def _rne_sat(v, vmax: float, emin: int, mbits: int):
    """Round |v| to the grid of a binary format, nearest-even, saturating.

    The grid has ``mbits`` mantissa bits and smallest normal exponent ``emin``
    (values below 2^emin share the spacing 2^(emin - mbits)).  Returns
    (sign, rounded magnitude) in float64.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input is outside the quantizer's domain")
    sign = np.signbit(v)
    a = np.minimum(np.abs(v), vmax)
    e = np.maximum(_floor_log2(a), emin)
    ulp = np.ldexp(1.0, e - mbits)
    r = np.rint(a / ulp) * ulp          # np.rint rounds half to even; a/ulp is exact
    return sign, np.minimum(r, vmax)


def e4m3_encode(v) -> np.ndarray:
    """float64 -> e4m3fn code, RNE and saturating to +-448, sign of zero kept."""
    sign, r = _rne_sat(v, E4M3_MAX, -6, 3)
    E = np.maximum(_floor_log2(r), -6)
    normal = r >= 2.0 ** -6
    m_norm = np.rint(r / np.ldexp(1.0, E) * 8.0 - 8.0)
    code_norm = ((E + 7) << 3) + m_norm.astype(np.int64)
    code_sub = np.rint(r / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_norm, code_sub)
    code = code | np.where(sign, 0x80, 0)
    return code.astype(np.uint8)


def e2m1_encode(v) -> np.ndarray:
    """float64 -> e2m1 nibble (0..15), RNE and saturating to +-6, sign of zero kept."""
    sign, r = _rne_sat(v, E2M1_MAX, 0, 1)
    E = np.maximum(_floor_log2(r), 0)
    normal = r >= 1.0
    m_norm = np.rint(r / np.ldexp(1.0, E) * 2.0 - 2.0)
    code_norm = ((E + 1) << 1) + m_norm.astype(np.int64)
    code_sub = np.rint(r / 0.5).astype(np.int64)
    code = np.where(normal, code_norm, code_sub)
    code = code | np.where(sign, 0x8, 0)
    return code.astype(np.uint8)


# ---------------------------------------------------------------- bf16 / fp32
def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit pattern -> float32 (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(x) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (inf stays inf, NaN stays NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)


# ---------------------------------------------------------------- packing
def pack_fp4(nibbles: np.ndarray) -> np.ndarray:
    """[R, K] e2m1 nibbles -> [R, K/2] bytes; element 2j in the low nibble."""
    n = np.asarray(nibbles, dtype=np.uint8)
    return (n[:, 0::2] & 0xF) | ((n[:, 1::2] & 0xF) << 4)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """[R, K] int4 codes (0..15) -> uint32 [R, K/8]; element k at bits 4*(k mod 8)."""
    c = np.asarray(codes, dtype=np.uint32).reshape(codes.shape[0], -1, 8)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    return np.bitwise_or.reduce((c & 0xF) << shifts, axis=2).astype(np.uint32)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint32)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    return ((p[:, :, None] >> shifts) & 0xF).astype(np.uint8).reshape(p.shape[0], -1)


def pack_mx_scales(scales: np.ndarray, chunk: int) -> np.ndarray:
    """The library's packed MX exponent layout, written out from its definition.

    The pages fix one e8m0 exponent per 32 consecutive K-elements but not how
    they are stored; the library keeps them as [G, rows, chunk] with chunk = 4
    (MXFP8) or 8 (MXFP4) and G = ceil(nblk / chunk): entry [g, r, b] is row r's
    exponent of block chunk * g + b, and entries past the row's last block are
    127 (the code of 1.0).  Plain loops, no reshapes."""
    s = np.asarray(scales, dtype=np.uint8)
    rows, nblk = s.shape
    G = (nblk + chunk - 1) // chunk
    out = np.full((G, rows, chunk), 127, dtype=np.uint8)
    for r in range(rows):
        for blk in range(nblk):
            out[blk // chunk, r, blk % chunk] = s[r, blk]
    return out
