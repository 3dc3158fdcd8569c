"""Reference scaled GEMM (oracle; test infrastructure).

C = A_hat @ W_hat^T where A_hat and W_hat are the exactly dequantized operands
(decode(code) * scale, or (q - z) * s for int4, in float64).  For W4A16 the
activation is the bf16 input itself, widened exactly.  The product is the
plain float64 matmul: exact products, float64 sums.  This is the definition
the GPU's fp32-accumulated, bf16-rounded result is measured against.

The pages give the shape of the operation only: a linear layer's forward
flattens the input to 2-D, quantizes the activation, multiplies with the
quantized weight, and restores the shape ("vLLM-Omni Online Quantization
complete guide", section "How online quantization works underneath",
step 3).  A is [M, K] (tokens x input channels), W is [N, K] (output x input
channels, the linear layer's own layout), C is [M, N].

The fused epilogue alpha * (A @ B) + bias, named for the FP8 path in the same
section, is C = alpha * (A_hat @ W_hat^T) + bias[n] with a scalar fp32 alpha
and a bf16 bias per output column, both widened exactly.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32
from .quant import dequant_exact


def _a_hat(a) -> np.ndarray:
    if isinstance(a, dict):
        return dequant_exact(a)
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise ValueError("an unquantized activation must be bf16 bits (uint16)")
    return bf16_to_f32(a).astype(np.float64)


def _epilogue(prod, alpha, bias, cols=None):
    if alpha is not None and alpha != 1.0:
        prod = float(np.float32(alpha)) * prod
    if bias is not None:
        b = np.asarray(bias)
        if b.dtype != np.uint16 or b.ndim != 1:
            raise ValueError("bias must be a 1-D array of bf16 bits (uint16)")
        b = bf16_to_f32(b).astype(np.float64)
        prod = prod + (b if cols is None else b[np.asarray(cols)])[None, :]
    return prod


def gemm_ref(a, w_q: dict, alpha=None, bias=None) -> np.ndarray:
    """float64 C[M, N] = alpha * (A_hat @ W_hat^T) + bias.

    ``a`` is a quantized activation (dict from ``quantize``) or, for W4A16,
    the bf16 activation bits.  ``w_q`` is a quantized weight.  ``alpha``
    (fp32, default 1) and ``bias`` (bf16 bits [N], default none) are the
    fused epilogue.
    """
    A = _a_hat(a)
    W = dequant_exact(w_q)
    if A.shape[1] != W.shape[1]:
        raise ValueError("K mismatch")
    if bias is not None and np.asarray(bias).shape != (W.shape[0],):
        raise ValueError("bias must have one entry per output column")
    return _epilogue(A @ W.T, alpha, bias)


def gemm_ref_entries(a, w_q: dict, rows, cols, alpha=None, bias=None) -> np.ndarray:
    """C[rows[i], cols[j]] for the given index lists, each as one dot product."""
    A = _a_hat(a)[np.asarray(rows)]
    W = dequant_exact(w_q)[np.asarray(cols)]
    return _epilogue(A @ W.T, alpha, bias, cols)


def gemm_abs_ref(a, w_q: dict, alpha=None) -> np.ndarray:
    """float64 T[M, N] = |alpha| * (|A_hat| @ |W_hat|^T): for each output, the sum of
    the magnitudes of the K products the GEMM adds up.

    Rounding-error analysis of any summation of those products is stated in
    terms of this sum (a sum of n terms carried in a format with unit roundoff
    u is off by at most about n * u * T), so it is what a per-element
    tolerance on C is measured against.
    """
    A = np.abs(_a_hat(a))
    W = np.abs(dequant_exact(w_q))
    if A.shape[1] != W.shape[1]:
        raise ValueError("K mismatch")
    t = A @ W.T
    return abs(float(np.float32(alpha))) * t if alpha is not None else t


def rel_fro_error(c_test, c_ref) -> float:
    """||c_test - c_ref||_F / ||c_ref||_F in float64."""
    c_test = np.asarray(c_test, dtype=np.float64)
    c_ref = np.asarray(c_ref, dtype=np.float64)
    den = np.linalg.norm(c_ref)
    num = np.linalg.norm(c_test - c_ref)
    return float(num / den) if den > 0 else float(num)
