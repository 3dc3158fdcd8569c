"""CPU oracle for the quantized-linear path (test infrastructure only).

This package is the plain, slow, obviously-correct definition that the HIP
kernels are checked against.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the library itself never does, and
it shares no code with the HIP path.

Inputs are bf16 bit patterns (uint16).  Scale arithmetic is IEEE binary32 with
round-to-nearest-even, done with NumPy float32 operations (correctly rounded,
no flush-to-zero).  Rounding onto a low-precision grid is done in float64,
where it is exact.  The GEMM is the exact product of the dequantized operands,
accumulated in float64.

Sources (page title, section):
* "[vLLM] Other quantization: FP8, ModelOpt, INC, TorchAO, Quark", section
  "FP8": tensor-, token- and 128x128-block-wise dynamic symmetric FP8 scales.
* "vLLM-Omni Online Quantization complete guide", section "How online
  quantization works underneath", steps 2-3: FP8 e4m3fn codes with one
  e8m0 exponent scale per 32 K-elements (MXFP8); fp4 e2m1 packed two per
  byte (MXFP4); activations quantized on every call, weights once at load.
* "vLLM-Omni accelerates inference with AutoRound quantization", section
  "Usage" (quantizing a new model): int4 weights, group size 128, zero
  tuning iterations read as round-to-nearest.
* The same FP8 section's scheme keys for static (supplied) tensor and
  128-block scales; the online-quantization guide's int8 online path
  (sections "Key parameters in detail" and "How online quantization works
  underneath") and its fused FP8 epilogue alpha * (A @ B) + bias.

Every function is pinned by the CPU tests (closed forms, exhaustive code
tables, exact reproduction, error bounds, brute-force tiny GEMMs).  No
function here is "parity unpinned".
"""
from .formats import (  # noqa: F401
    E4M3_MAX, E2M1_MAX, e4m3_decode, e4m3_encode, e2m1_decode, e2m1_encode,
    e8m0_decode, bf16_to_f32, f32_to_bf16_rne, pack_fp4, unpack_fp4,
    pack_int4, unpack_int4,
)
from .quant import (  # noqa: F401
    SCHEMES, STATIC_SCHEMES, quantize, quantize_static, dequantize, dequant_exact, mx_exponent,
)
from .gemm import gemm_abs_ref, gemm_ref, gemm_ref_entries, rel_fro_error  # noqa: F401
