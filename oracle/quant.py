"""Quantizers and dequantizers (oracle; test infrastructure).

Each scheme takes a bf16 tensor x[rows, cols] (activations: rows = tokens M;
weights: rows = output channels N; cols = K, the contraction axis) and returns
codes plus scales in the canonical layouts:

=============  ============================  ===============================
scheme         codes                         scales (zeros)
=============  ============================  ===============================
fp8_tensor     u8 e4m3fn [rows, cols]        f32 [1]
fp8_row        u8 e4m3fn [rows, cols]        f32 [rows]
fp8_block128   u8 e4m3fn [rows, cols]        act f32 [rows, cols/128];
                                             wt  f32 [rows/128, cols/128]
mxfp8          u8 e4m3fn [rows, cols]        u8 e8m0 [rows, cols/32]
mxfp4          u8 two e2m1 [rows, cols/2]    u8 e8m0 [rows, cols/32]
mxfp4_dual     u8 two e2m1 [rows, cols/2]    u8 e8m0 [rows, cols/32] (fine),
                                             f32 [rows, cols/512] ("coarse")
w4a16_asym     u32 eight int4 [rows, cols/8] bf16 [rows, cols/128]
                                             (u8 zero-points [rows, cols/128])
w4a16_sym      as w4a16_asym, zero-point fixed at 8
int8_row       i8 [rows, cols]               f32 [rows]
=============  ============================  ===============================

Sources: FP8 scale granularities (tensor, token, 128x128 block, all dynamic
and symmetric) from "[vLLM] Other quantization: FP8, ModelOpt, INC, TorchAO,
Quark", section "FP8".  MX scales (one e8m0 exponent per 32 K-elements) and
fp4 packing from "vLLM-Omni Online Quantization complete guide", section "How
online quantization works underneath", steps 2-3.  Static FP8 scales (a
supplied scale per tensor or per 128-block instead of a computed one) from
the FP8 section's list of scheme keys.  int8 W8A8 online (dynamic
activation scales only; a static activation scheme is an error) from the
online-quantization guide, sections "Key parameters in detail" and "How
online quantization works underneath".  int4 group-128 from
"vLLM-Omni accelerates inference with AutoRound quantization", section
"Usage" (the auto-round command and the checkpoint's quantization_config).

Readings where the pages are silent (all listed in the design notes):
* FP8 scale s = fp32(amax / 448); the fp32 quotient fp32(x / s) is formed
  first, then rounded to e4m3fn (round-to-nearest-even, saturating).
  If s comes out 0 (amax = 0, or amax so small that amax/448 underflows),
  s = 1.
* Static FP8: the supplied fp32 scale replaces s; the quotient is rounded
  the same way and saturates at +-448 (a calibrated scale can be smaller
  than amax / 448).  Static schemes are FP8 per tensor and per 128-block.
* int8 (symmetric, per row: per token for activations, per output channel
  for weights): s = fp32(amax / 127), 1 if that is 0;
  q = clamp(rne(fp32(x / s)), -128, 127).
* MX shared exponent X = clamp(floor(log2 amax) - emax, -127, 127), emax = 8
  for e4m3 and 2 for e2m1; the element is rounded from x * 2^-X; amax = 0
  gives X = -127 (code 0).
* Dual-scale MXFP4 (two online scale levels, fine per 32 and coarse per 512
  K-elements, with the calibrated multiplier of offline checkpoints replaced
  by ones; "vLLM-Omni Online Quantization complete guide", sections "How
  online quantization works underneath" and "Key parameters in detail"): the
  page names the levels but not their formats.  Read as: a coarse fp32 scale
  per (row, 512-block) s_c = fp32(amax_512 / 6), 1 if that is 0; the
  quotient v = fp32(x / s_c) (correctly rounded, formed first, as for FP8);
  then plain MX on v: a fine e8m0 exponent per 32-block
  X = clamp(floor(log2 max|v|) - 2, -127, 127) and q = RNE_sat_e2m1(v * 2^-X).
  A unit multiplier leaves x unchanged.  K must be a multiple of 512.
  Dequantized: decode(q) * 2^X * s_c.
* int4 round-to-nearest: range [min(0, min x), max(0, max x)],
  s = bf16(fp32(fp32(xmax - xmin) / 15)), z = clamp(rne(fp32(-xmin / s)), 0, 15),
  q = clamp(rne(fp32(x / s)) + z, 0, 15).  Symmetric: z = 8,
  s = bf16(fp32(amax / 7)).  A zero s (all-zero group, or underflow) gives
  s = 1, z = 0 (asym) / 8 (sym).
"""
from __future__ import annotations

import numpy as np

from .formats import (
    E2M1_MAX, E4M3_MAX, bf16_to_f32, e2m1_decode, e2m1_encode, e4m3_decode,
    e4m3_encode, e8m0_decode, f32_to_bf16_rne, pack_fp4, pack_int4,
    unpack_fp4, unpack_int4,
)

SCHEMES = ("fp8_tensor", "fp8_row", "fp8_block128", "mxfp8", "mxfp4",
           "w4a16_asym", "w4a16_sym", "int8_row", "mxfp4_dual")
STATIC_SCHEMES = ("fp8_tensor", "fp8_block128")
ROLES = ("activation", "weight")

_F32 = np.float32


def _check(x_bits, scheme, role):
    if scheme not in SCHEMES:
        raise ValueError(f"unknown scheme {scheme!r}")
    if role not in ROLES:
        raise ValueError(f"unknown role {role!r}")
    x_bits = np.asarray(x_bits)
    if x_bits.dtype != np.uint16 or x_bits.ndim != 2:
        raise ValueError("x must be a 2-D array of bf16 bit patterns (uint16)")
    rows, cols = x_bits.shape
    if scheme.startswith("w4a16") and role != "weight":
        raise ValueError("W4A16 quantizes weights only")
    if scheme in ("mxfp8", "mxfp4") and cols % 32:
        raise ValueError("MX schemes need K % 32 == 0")
    if scheme == "mxfp4_dual" and cols % 512:
        raise ValueError("dual-scale MXFP4 needs K % 512 == 0")
    if (scheme == "fp8_block128" or scheme.startswith("w4a16")) and cols % 128:
        raise ValueError("block-128 / group-128 schemes need K % 128 == 0")
    if scheme == "fp8_block128" and role == "weight" and rows % 128:
        raise ValueError("128x128 weight blocks need rows % 128 == 0")
    return x_bits, rows, cols


# ---------------------------------------------------------------- FP8, fp32 scale
def _fp8_scale(amax_f32: np.ndarray) -> np.ndarray:
    """s = fp32(amax / 448), or 1 where that is 0."""
    s = (amax_f32.astype(_F32) / _F32(E4M3_MAX)).astype(_F32)
    return np.where(s == 0, _F32(1.0), s).astype(_F32)


def _fp8_codes(x_f32: np.ndarray, s_f32: np.ndarray) -> np.ndarray:
    """e4m3fn(RNE_sat(fp32(x / s))) elementwise; s broadcasts against x."""
    q = (x_f32 / s_f32).astype(_F32)        # IEEE binary32 division, RNE
    return e4m3_encode(q.astype(np.float64))


def _quant_fp8_tensor(x):
    amax = np.max(np.abs(x)) if x.size else _F32(0)
    s = _fp8_scale(np.asarray([amax], dtype=_F32))
    return _fp8_codes(x, s[0]), s


def _quant_fp8_row(x):
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], _F32)
    s = _fp8_scale(amax)
    return _fp8_codes(x, s[:, None]), s


def _quant_fp8_block(x, role):
    rows, cols = x.shape
    g = cols // 128
    if role == "activation":
        xb = x.reshape(rows, g, 128)
        amax = np.max(np.abs(xb), axis=2) if rows else np.zeros((0, g), _F32)
        s = _fp8_scale(amax)                                  # [rows, g]
        codes = _fp8_codes(xb, s[:, :, None]).reshape(rows, cols)
    else:
        rb = rows // 128
        xb = x.reshape(rb, 128, g, 128)
        amax = np.max(np.abs(xb), axis=(1, 3)) if rb else np.zeros((0, g), _F32)
        s = _fp8_scale(amax)                                  # [rows/128, g]
        codes = _fp8_codes(xb, s[:, None, :, None]).reshape(rows, cols)
    return codes, s


# ---------------------------------------------------------------- MX, e8m0 scale
def mx_exponent(amax_f32, emax: int) -> np.ndarray:
    """Shared exponent X = clamp(floor(log2 amax) - emax, -127, 127); amax=0 -> -127."""
    a = np.asarray(amax_f32, dtype=np.float64)
    _, e = np.frexp(a)                  # a = m * 2^e with m in [0.5, 1): floor(log2 a) = e - 1
    X = np.where(a > 0, (e - 1) - emax, -127)
    return np.clip(X, -127, 127).astype(np.int64)


def _quant_mx(x, fmt):
    rows, cols = x.shape
    xb = x.reshape(rows, cols // 32, 32).astype(np.float64)
    amax = np.max(np.abs(xb), axis=2) if rows else np.zeros((0, cols // 32))
    emax = 8 if fmt == "mxfp8" else 2
    X = mx_exponent(amax, emax)                                # [rows, cols/32]
    v = xb * np.ldexp(1.0, -X)[:, :, None]                     # exact scaling
    if fmt == "mxfp8":
        codes = e4m3_encode(v).reshape(rows, cols)
    else:
        codes = pack_fp4(e2m1_encode(v).reshape(rows, cols))
    return codes, (X + 127).astype(np.uint8)


def _quant_mx4_dual(x):
    """Two scale levels: coarse fp32 s_c per 512-block, then MX (e2m1, emax 2) on the
    quotients v = fp32(x / s_c)."""
    rows, cols = x.shape
    nb = cols // 512
    xc = x.reshape(rows, nb, 512)
    amax = np.max(np.abs(xc), axis=2) if rows else np.zeros((0, nb), _F32)
    s_c = (amax.astype(_F32) / _F32(E2M1_MAX)).astype(_F32)
    s_c = np.where(s_c == 0, _F32(1.0), s_c).astype(_F32)              # [rows, cols/512]
    v = (xc / s_c[:, :, None]).astype(_F32)                             # fp32 quotient, RNE
    vb = v.reshape(rows, cols // 32, 32).astype(np.float64)
    vmax = np.max(np.abs(vb), axis=2) if rows else np.zeros((0, cols // 32))
    X = mx_exponent(vmax, 2)                                            # fine exponents [rows, cols/32]
    codes = pack_fp4(e2m1_encode(vb * np.ldexp(1.0, -X)[:, :, None]).reshape(rows, cols))
    return codes, (X + 127).astype(np.uint8), s_c


# ---------------------------------------------------------------- int4 RTN
def _rne_int(v_f32):
    return np.rint(v_f32.astype(np.float64))                   # half to even


def _quant_int4(x, sym: bool):
    rows, cols = x.shape
    xg = x.reshape(rows, cols // 128, 128)
    if sym:
        amax = np.max(np.abs(xg), axis=2) if rows else np.zeros((0, cols // 128), _F32)
        s32 = (amax.astype(_F32) / _F32(7.0)).astype(_F32)
        s_bits = f32_to_bf16_rne(s32)
        s = bf16_to_f32(s_bits)
        zero_s = s == 0
        s = np.where(zero_s, _F32(1.0), s).astype(_F32)
        s_bits = np.where(zero_s, f32_to_bf16_rne(np.ones_like(s)), s_bits)
        z = np.full(s.shape, 8.0)
    else:
        xmin = np.minimum(np.min(xg, axis=2), _F32(0)) if rows else np.zeros((0, cols // 128), _F32)
        xmax = np.maximum(np.max(xg, axis=2), _F32(0)) if rows else np.zeros((0, cols // 128), _F32)
        d = (xmax.astype(_F32) - xmin.astype(_F32)).astype(_F32)
        s32 = (d / _F32(15.0)).astype(_F32)
        s_bits = f32_to_bf16_rne(s32)
        s = bf16_to_f32(s_bits)
        zero_s = s == 0
        s = np.where(zero_s, _F32(1.0), s).astype(_F32)
        s_bits = np.where(zero_s, f32_to_bf16_rne(np.ones_like(s)), s_bits)
        z = np.clip(_rne_int((-xmin.astype(_F32) / s).astype(_F32)), 0, 15)
        z = np.where(zero_s, 0.0, z)
    q = _rne_int((xg / s[:, :, None]).astype(_F32)) + z[:, :, None]
    q = np.clip(q, 0, 15).astype(np.uint8).reshape(rows, cols)
    return pack_int4(q), s_bits.astype(np.uint16), z.astype(np.uint8)


# ---------------------------------------------------------------- int8, fp32 scale
def _quant_int8_row(x):
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], _F32)
    s = (amax.astype(_F32) / _F32(127.0)).astype(_F32)
    s = np.where(s == 0, _F32(1.0), s).astype(_F32)
    q = _rne_int((x / s[:, None]).astype(_F32))              # fp32 quotient, then RNE
    return np.clip(q, -128, 127).astype(np.int8), s


# ---------------------------------------------------------------- public API
def quantize(x_bits, scheme: str, role: str = "activation") -> dict:
    """Quantize a bf16 tensor; returns {"codes", "scales", "zeros"} (canonical layouts)."""
    x_bits, rows, cols = _check(x_bits, scheme, role)
    x = bf16_to_f32(x_bits)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the quantizer's domain")
    zeros = None
    if scheme == "fp8_tensor":
        codes, scales = _quant_fp8_tensor(x)
    elif scheme == "fp8_row":
        codes, scales = _quant_fp8_row(x)
    elif scheme == "fp8_block128":
        codes, scales = _quant_fp8_block(x, role)
    elif scheme in ("mxfp8", "mxfp4"):
        codes, scales = _quant_mx(x, scheme)
    elif scheme == "int8_row":
        codes, scales = _quant_int8_row(x)
    elif scheme == "mxfp4_dual":
        codes, scales, coarse = _quant_mx4_dual(x)
        return {"scheme": scheme, "role": role, "rows": rows, "cols": cols,
                "codes": codes, "scales": scales, "coarse": coarse, "zeros": None}
    else:
        codes, scales, zeros = _quant_int4(x, scheme == "w4a16_sym")
    return {"scheme": scheme, "role": role, "rows": rows, "cols": cols,
            "codes": codes, "scales": scales, "zeros": zeros}


def _static_scale_shape(scheme, role, rows, cols):
    if scheme == "fp8_tensor":
        return (1,)
    return (rows, cols // 128) if role == "activation" else (rows // 128, cols // 128)


def quantize_static(x_bits, scheme: str, role: str, scales) -> dict:
    """FP8 quantization with supplied (static, calibrated) fp32 scales.

    ``scales`` has the scheme's canonical scale shape (f32[1] per tensor;
    f32[rows, cols/128] or f32[rows/128, cols/128] per 128-block) and every
    value must be finite and positive.  Codes are RNE_sat(fp32(x / s)): the
    amax pass is skipped, and values beyond 448 s saturate.
    """
    if scheme not in STATIC_SCHEMES:
        raise ValueError(f"static scales are defined for {STATIC_SCHEMES} only, not {scheme!r}")
    x_bits, rows, cols = _check(x_bits, scheme, role)
    x = bf16_to_f32(x_bits)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the quantizer's domain")
    s = np.asarray(scales, dtype=_F32).reshape(_static_scale_shape(scheme, role, rows, cols))
    if not (np.all(np.isfinite(s)) and np.all(s > 0)):
        raise ValueError("static scales must be finite and positive")
    q = {"scheme": scheme, "role": role, "rows": rows, "cols": cols, "scales": s.copy(), "zeros": None}
    with np.errstate(over="ignore"):
        quot = (x / _expand_scale_f32(q)).astype(_F32)   # may overflow to +-inf for tiny s
    # Saturation first: every |quotient| above 448 (an infinite one included)
    # encodes as 448 with its sign, exactly as RNE_sat does for finite values.
    q["codes"] = e4m3_encode(np.clip(quot, -E4M3_MAX, E4M3_MAX).astype(np.float64))
    return q


def _expand_scale_f32(q) -> np.ndarray:
    """Per-element fp32 scale [rows, cols] for the fp32-scaled FP8 schemes."""
    rows, cols, s = q["rows"], q["cols"], np.asarray(q["scales"], dtype=_F32)
    if q["scheme"] == "fp8_tensor":
        return np.full((rows, cols), s.reshape(-1)[0], dtype=_F32)
    if q["scheme"] in ("fp8_row", "int8_row"):
        return np.repeat(s.reshape(rows, 1), cols, axis=1)
    if q["role"] == "activation":
        return np.repeat(s.reshape(rows, cols // 128), 128, axis=1)
    return np.repeat(np.repeat(s.reshape(rows // 128, cols // 128), 128, axis=0), 128, axis=1)


def _decoded(q):
    """(element values, per-element scale) in float64, both exact."""
    scheme, rows, cols = q["scheme"], q["rows"], q["cols"]
    if scheme in ("fp8_tensor", "fp8_row", "fp8_block128"):
        return e4m3_decode(q["codes"]), _expand_scale_f32(q).astype(np.float64)
    if scheme == "int8_row":
        return np.asarray(q["codes"], dtype=np.int8).astype(np.float64), _expand_scale_f32(q).astype(np.float64)
    if scheme in ("mxfp8", "mxfp4", "mxfp4_dual"):
        vals = e4m3_decode(q["codes"]) if scheme == "mxfp8" else e2m1_decode(unpack_fp4(q["codes"]))
        sc = np.repeat(e8m0_decode(q["scales"]).reshape(rows, cols // 32), 32, axis=1)
        if scheme == "mxfp4_dual":   # 2^X (exact) times the coarse fp32 scale (exact in float64)
            sc = sc * np.repeat(np.asarray(q["coarse"], np.float32).astype(np.float64).reshape(rows, cols // 512),
                                512, axis=1)
        return vals, sc
    codes = unpack_int4(q["codes"]).astype(np.float64)
    z = np.repeat(np.asarray(q["zeros"], dtype=np.float64).reshape(rows, cols // 128), 128, axis=1)
    s = np.repeat(bf16_to_f32(q["scales"]).astype(np.float64).reshape(rows, cols // 128), 128, axis=1)
    return codes - z, s


def dequant_exact(q) -> np.ndarray:
    """Exact dequantized values decode(q) * scale in float64 (the GEMM operand)."""
    vals, sc = _decoded(q)
    return vals * sc


def dequantize(q) -> np.ndarray:
    """bf16 bits of bf16_RNE(fp32(decode(q) * scale)) (int4: (q - z) * s; dual-scale
    MXFP4: fp32(decode(q) * 2^X) is exact, then one rounding of its product with the
    coarse fp32 scale)."""
    if q["scheme"] == "mxfp4_dual":
        rows, cols = q["rows"], q["cols"]
        fine = (e2m1_decode(unpack_fp4(q["codes"]))
                * np.repeat(e8m0_decode(q["scales"]).reshape(rows, cols // 32), 32, axis=1)).astype(_F32)
        coarse = np.repeat(np.asarray(q["coarse"], _F32).reshape(rows, cols // 512), 512, axis=1)
        with np.errstate(over="ignore"):
            return f32_to_bf16_rne((fine * coarse).astype(_F32))
    vals, sc = _decoded(q)
    prod = (vals.astype(_F32) * sc.astype(_F32)).astype(_F32)   # one fp32 rounding
    with np.errstate(over="ignore"):
        return f32_to_bf16_rne(prod)
