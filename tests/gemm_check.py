"""Per-element GEMM checks and exactly-summable GEMM operands, shared by the GPU
parity tests (test infrastructure; no GPU needed to import).

Two kinds of check, both on every output element that a test compares:

* ``check_gemm``: random operands.  Besides the relative Frobenius gate of
  1e-2, every element must satisfy

      |C_gpu - C64| <= 2^-8 |C64| + 8 K 2^-24 T (+ the W4A16 terms below),

  with C64 the oracle's exact float64 product and T = sum_k |a_hat_k w_hat_k|
  (``oracle.gemm_abs_ref``).  2^-8 |C64| covers the final rounding to bf16
  (unit roundoff 2^-8, applied to a value within the accumulation error of
  C64); K 2^-24 T is the worst-case error of adding K exactly-formed products
  one by one in fp32.  The matrix cores do not add that way: a probe of the
  fp8 32x32x64 instruction with two cancelling +-448*448 products among 126
  tiny ones (every other operand in range) returned errors up to 3.9 K 2^-24 T,
  i.e. its dot product keeps about two bits fewer than an fp32 sum, with
  truncation.  The factor 8 covers that with a margin of two, plus the few
  extra fp32 roundings of scale products, promotion FMAs and the epilogue.
  A stale or missing output, or a product taken with a wrong scale, breaks
  the bound unless that element happens to be close to zero.
  W4A16 adds two terms.  The tile kernels round each dequantized weight
  (q - z) s to bf16 before the matrix core, so 2^-8 T more.  The small-M
  kernel keeps codes as integers and sums a (128 + q) and a (128 + z), so its
  fp32 sums run over sum_k |a_k| s_k (256 + q_k + z_k), which replaces T in
  the accumulation term.

* ``check_gemm_exact``: operands built on a coarse grid (``exact_operand``)
  so that every partial sum, in any order, is exactly representable in 21
  bits (so also by a dot product that keeps fewer bits than fp32).
  Then the only rounding left is the final one to bf16, and every element
  must equal bf16_RNE(C64) bit for bit.  Scales are powers of two chosen so
  that neighbouring rows, K-groups and blocks differ by at least 2x: a
  mis-indexed scale, a stale tile or a dropped store changes the bits.
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle import formats as F
from oracle import metrics as MET

U_FP32 = 2.0 ** -24
U_BF16 = 2.0 ** -8
ACC_FACTOR = 8.0        # see the module docstring: measured worst case 3.9
FROB_TOL = 1e-2          # the stated relative Frobenius tolerance
FROB_FLAG = 5e-3         # measured errors are ~2e-3; anything above this is a drift


def bf16_f64(bits) -> np.ndarray:
    return F.bf16_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


def _first(mask, *arrays):
    idx = tuple(np.argwhere(mask)[0])
    return idx, [a[idx] for a in arrays]


def w4a16_terms(a_bits, wq: dict):
    """(weight rounding term 2^-8 T, offset sum sum_k |a_k| s_k (256 + q_k + z_k)) for W4A16."""
    A = np.abs(bf16_f64(a_bits))
    rows, cols = wq["rows"], wq["cols"]
    q = F.unpack_int4(wq["codes"]).astype(np.float64)
    z = np.repeat(np.asarray(wq["zeros"], np.float64).reshape(rows, cols // 128), 128, axis=1)
    s = np.repeat(bf16_f64(wq["scales"]).reshape(rows, cols // 128), 128, axis=1)
    t = oracle.gemm_abs_ref(np.asarray(a_bits, np.uint16), wq)
    t_off = A @ (s * (256.0 + q + z)).T
    return U_BF16 * t, t_off


def check_gemm(c_gpu_bits, c64, t, K, what="", weight_round=None, t_acc=None, flag=True):
    """Frobenius gate plus the per-element bound (module docstring)."""
    c = bf16_f64(c_gpu_bits)
    c64 = np.asarray(c64, np.float64)
    assert c.shape == c64.shape, f"{what}: shape {c.shape} vs {c64.shape}"
    sim = MET.similarity(c, c64)
    err = sim["relative_l2"]
    assert err <= FROB_TOL, f"{what}: relative Frobenius error {err:.3e} > {FROB_TOL}; {MET.format_similarity(sim)}"
    if flag:
        assert err <= FROB_FLAG, f"{what}: relative Frobenius error {err:.3e} (expected ~2e-3); " \
                                 f"{MET.format_similarity(sim)}"
    bound = U_BF16 * np.abs(c64) + ACC_FACTOR * K * U_FP32 * np.asarray(t if t_acc is None else t_acc)
    if weight_round is not None:
        bound = bound + weight_round
    diff = np.abs(c - c64)
    bad = ~(diff <= bound)            # NaN outputs are failures too
    if bad.any():
        idx, (got, want, b) = _first(bad, c, c64, bound)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside the per-element bound; "
                             f"first at {idx}: gpu {got!r} oracle {want!r} bound {b:.3e}; "
                             f"{MET.format_similarity(sim)}")
    return sim


def check_gemm_exact(c_gpu_bits, c64, what=""):
    """Every element equals bf16_RNE(C64); C64 must be exact in fp32."""
    c64 = np.asarray(c64, np.float64)
    c32 = c64.astype(np.float32)
    assert np.array_equal(c32.astype(np.float64), c64), f"{what}: the exact case is not representable in fp32"
    want = F.f32_to_bf16_rne(c32)
    got = np.asarray(c_gpu_bits, np.uint16)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    bad = got != want
    if bad.any():
        idx, (g, w, v) = _first(bad, got, want, c64)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements differ; first at {idx}: "
                             f"gpu 0x{int(g):04x} want 0x{int(w):04x} (exact {v!r})")


# ----------------------------------------------------------------------------- sampling
def tile_sample(n: int, seed: int, tile: int = 256, per_tile: int = 2, extra=()) -> np.ndarray:
    """Indices covering every tile of ``tile`` rows (or columns): each tile's first and
    last index plus ``per_tile`` random ones, and ``extra``."""
    rng = np.random.default_rng(seed)
    idx = set(int(i) for i in extra if 0 <= i < n)
    for t0 in range(0, n, tile):
        t1 = min(n, t0 + tile)
        idx.update((t0, t1 - 1))
        idx.update(int(i) for i in rng.integers(t0, t1, per_tile))
    return np.array(sorted(idx))


# ----------------------------------------------------------------------------- exact operands
def _e4m3_grid_codes():
    """e4m3fn codes whose values are multiples of 1/4 with |v| <= 4 (signed zero included)."""
    codes = np.arange(256, dtype=np.uint8)
    v = F.e4m3_decode(codes)
    ok = np.isfinite(v) & (np.abs(v) <= 4) & (np.mod(v * 4, 1) == 0)
    return codes[ok]


def exact_operand(scheme: str, role: str, rows: int, cols: int, seed: int) -> dict:
    """A quantized operand (oracle dict, canonical layout) on a grid that keeps every
    partial sum of the GEMM exact in fp32 (see ``exact_precondition``), with
    power-of-two scales that differ between neighbouring rows / groups / blocks."""
    rng = np.random.default_rng(seed)
    r = np.arange(rows)[:, None]
    q = {"scheme": scheme, "role": role, "rows": rows, "cols": cols, "zeros": None}
    if scheme in ("fp8_tensor", "fp8_row", "fp8_block128", "mxfp8"):
        q["codes"] = rng.choice(_e4m3_grid_codes(), (rows, cols)).astype(np.uint8)
    if scheme == "fp8_tensor":
        q["scales"] = np.array([2.0 ** int(rng.integers(-1, 2))], np.float32)
    elif scheme in ("fp8_row", "int8_row"):
        q["scales"] = np.ldexp(1.0, (np.arange(rows) + seed) % 3 - 1).astype(np.float32)
    elif scheme == "fp8_block128":
        g = np.arange(cols // 128)[None, :]
        br = r if role == "activation" else np.arange(rows // 128)[:, None]
        q["scales"] = np.ldexp(1.0, (br + 2 * g + seed) % 3 - 1).astype(np.float32)
    if scheme == "int8_row":
        q["codes"] = rng.integers(-16, 17, (rows, cols)).astype(np.int8)
    if scheme in ("mxfp8", "mxfp4", "mxfp4_dual"):
        if scheme != "mxfp8":
            q["codes"] = F.pack_fp4(rng.integers(0, 16, (rows, cols)).astype(np.uint8))
        b = np.arange(cols // 32)[None, :]
        if scheme == "mxfp4_dual":   # two levels multiply: exponents -1 / 0, alternating along rows and K
            q["scales"] = ((r + b + seed) % 2 - 1 + 127).astype(np.uint8)
        else:
            q["scales"] = ((r + 2 * b + seed) % 3 - 1 + 127).astype(np.uint8)
    if scheme == "mxfp4_dual":   # coarse scales: powers of two per (row, 512-block), neighbours 2x apart
        cb = np.arange(cols // 512)[None, :]
        q["coarse"] = np.ldexp(1.0, (r + cb + seed) % 2 - 1).astype(np.float32)
    if scheme.startswith("w4a16"):
        q["codes"] = F.pack_int4(rng.integers(0, 16, (rows, cols)).astype(np.uint8))
        g = np.arange(cols // 128)[None, :]
        q["scales"] = F.f32_to_bf16_rne(np.ldexp(1.0, -((r + 2 * g + seed) % 4)).astype(np.float32))
        q["zeros"] = (rng.integers(0, 16, (rows, cols // 128)) if scheme == "w4a16_asym"
                      else np.full((rows, cols // 128), 8)).astype(np.uint8)
    return q


def exact_activation_bf16(rows: int, cols: int, seed: int) -> np.ndarray:
    """bf16 bits of integers in [-8, 8] (the W4A16 activation of an exact case)."""
    v = np.random.default_rng(seed).integers(-8, 9, (rows, cols)).astype(np.float32)
    return F.f32_to_bf16_rne(v)


def _grid_bits(X: np.ndarray) -> int:
    """Smallest p >= 0 with every value of X a multiple of 2^-p."""
    for p in range(64):
        if np.all(np.mod(X * 2.0 ** p, 1) == 0):
            return p
    raise AssertionError("values are not on a binary grid")


def exact_precondition(a, wq: dict, alpha=None, bias=None):
    """Assert that the grid of the operands keeps every partial sum exact in fp32.
    With every product a multiple of 2^-p, a partial sum is exact when its magnitude
    (at most T, plus the bias) stays below 2^(24 - p); the check asks for 2^(21 - p),
    which also holds a matrix-core dot product that keeps two or three bits fewer.  For W4A16 the integer-code
    kernel also sums a (128 + q) and a (128 + z) per K-group, which must stay below
    2^21 as integers (the activation is integer-valued here)."""
    from oracle.gemm import _a_hat   # the oracle's own dequantized operand
    A = _a_hat(a)
    W = oracle.dequant_exact(wq)
    p = _grid_bits(A) + _grid_bits(W) + (0 if alpha is None else max(0, -int(np.log2(abs(alpha)))))
    t = oracle.gemm_abs_ref(a, wq, alpha=alpha)
    if bias is not None:
        b = bf16_f64(bias)
        p = max(p, _grid_bits(b))
        t = t + np.abs(b)[None, :]
    assert float(t.max(initial=0.0)) * 2.0 ** p < 2.0 ** 21, "partial sums could exceed the exact range"
    if wq["scheme"].startswith("w4a16"):
        assert _grid_bits(A) == 0
        per_group = np.abs(A).reshape(A.shape[0], -1, 128).sum(axis=2)   # the integer sums run per K-group
        assert float(per_group.max(initial=0.0)) * 2 * 143 < 2.0 ** 21


def assert_gemm(c_bits, a, wq: dict, what="", alpha=None, bias=None, flag=True):
    """check_gemm against the oracle for a whole output: ``a`` is the quantized activation
    (dict) or, for W4A16, the bf16 activation bits."""
    K = wq["cols"]
    c64 = oracle.gemm_ref(a, wq, alpha=alpha, bias=bias)
    t = oracle.gemm_abs_ref(a, wq, alpha=alpha)
    wr = t_off = None
    if wq["scheme"].startswith("w4a16"):
        wr, t_off = w4a16_terms(a, wq)
    return check_gemm(c_bits, c64, t, K, what, weight_round=wr, t_acc=t_off, flag=flag)


def fused_exact_activation(scheme: str, M: int, K: int, seed: int) -> np.ndarray:
    """bf16 bits of an activation whose quantization is exact: values on the code grid
    times a power of two per scale unit (tensor, row, or (row, 128-group)), with one
    element per unit at the format's largest code, so that every scale comes out a power
    of two and every code reproduces its value.  The GEMM on the result is then exact
    (``exact_precondition``), which lets the fused quantize + GEMM be checked bit for bit."""
    rng = np.random.default_rng(seed)
    if scheme == "int8_row":
        vals, top, j0 = rng.integers(-16, 17, (M, K)).astype(np.float64), 127.0, -1
    else:
        # multiples of 32 up to 448 (all e4m3 codes): products then span few bits, so that
        # the matrix core's dot product (which aligns its products to the largest one in a
        # window narrower than fp32) adds them exactly
        vals = 32.0 * rng.integers(-14, 15, (M, K)).astype(np.float64)
        top, j0 = 448.0, -3
    if scheme == "fp8_tensor":
        j = np.full((M, K), float(rng.integers(-1, 1) + j0))
        vals[int(rng.integers(0, M)), int(rng.integers(0, K))] = top * (1 if rng.integers(0, 2) else -1)
    elif scheme in ("fp8_row", "int8_row"):
        j = np.repeat(((np.arange(M) + seed) % 2 - 1 + j0)[:, None].astype(np.float64), K, axis=1)
        vals[np.arange(M), rng.integers(0, K, M)] = top
    else:   # fp8_block128: a power of two and a planted maximum per (row, 128-group)
        G = K // 128
        jg = (np.arange(M)[:, None] + np.arange(G)[None, :] + seed) % 2 - 1 + j0
        j = np.repeat(jg.astype(np.float64), 128, axis=1)
        for g in range(G):
            vals[np.arange(M), 128 * g + rng.integers(0, 128, M)] = -top
    x = vals * np.ldexp(1.0, j.astype(np.int64))
    bits = F.f32_to_bf16_rne(x.astype(np.float32))
    assert np.array_equal(F.bf16_to_f32(bits).astype(np.float64), x)
    return bits
