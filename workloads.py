"""Seeded synthetic inputs for the quantized-linear path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It draws random numbers and stores them as bf16 bit patterns; it
holds none of the quantization or GEMM arithmetic.  Every generator is seeded,
so the oracle and the GPU see identical bits.

Workload shapes follow diffusion-transformer linears:

* ``fp8_tensor_small``  FP8 per-tensor, A[256x512], W[512x512].
* ``fp8_row_dit``       FP8 per-token x per-channel, M=4096 (a 64x64 latent
                         grid), K=3072, N=12288; 1% of A's K-channels x20.
* ``fp8_block_dit``     FP8 1x128 / 128x128 block scales, M=8192, K=5120,
                         N=13824.
* ``mx_video_dit``      MXFP8 / MXFP4, M=20280 (a 30x52x13 video latent),
                         K=5120, N=5120; 0.5% of A's K-channels x50.
* ``w4a16_dit``         int4 group-128 weights, K=3072, N=12288,
                         M in {1, 16, 256, 4096}.

Activations are N(0,1), weights N(0, 0.02^2).  Seeds: workload i draws A with
``1000*i+1``, W with ``1000*i+2``, the outlier channels with ``1000*i+3`` and
the int4 codes / zero-points / scales with ``1000*i+4 / +5 / +6``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    schemes: tuple
    M: int
    N: int
    K: int
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    m_sweep: tuple = field(default_factory=tuple)


WORKLOADS = {
    w.name: w
    for w in (
        Workload("fp8_tensor_small", 0, ("fp8_tensor",), 256, 512, 512),
        Workload("fp8_row_dit", 1, ("fp8_row",), 4096, 12288, 3072, 0.01, 20.0),
        Workload("fp8_block_dit", 2, ("fp8_block128",), 8192, 13824, 5120),
        Workload("mx_video_dit", 3, ("mxfp8", "mxfp4"), 20280, 5120, 5120, 0.005, 50.0),
        Workload("w4a16_dit", 4, ("w4a16_asym",), 4096, 12288, 3072,
                 m_sweep=(1, 16, 256, 4096)),
    )
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Store float32 samples as bf16 (round to nearest even on the bit pattern).

    Only used to turn random draws into bf16 storage; inputs are finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly (for building test data)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(seed: int, K: int, frac: float) -> np.ndarray:
    n = int(round(frac * K))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(K, n, replace=False))


def normal_bf16(seed: int, rows: int, cols: int, std: float = 1.0,
                outlier_cols: np.ndarray | None = None,
                outlier_mult: float = 1.0) -> np.ndarray:
    """bf16 bits of N(0, std^2) samples; optional K-channels scaled before rounding."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if outlier_cols is not None and len(outlier_cols):
        x[:, outlier_cols] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


def activation(w: Workload, M: int | None = None) -> np.ndarray:
    """A[M, K] as bf16 bits for workload ``w`` (rows beyond M are not drawn)."""
    M = w.M if M is None else M
    oc = outlier_channels(1000 * w.index + 3, w.K, w.outlier_frac)
    return normal_bf16(1000 * w.index + 1, M, w.K, 1.0, oc, w.outlier_mult)


def weight(w: Workload) -> np.ndarray:
    """W[N, K] as bf16 bits, N(0, 0.02^2)."""
    return normal_bf16(1000 * w.index + 2, w.N, w.K, 0.02)


def int4_weight_parts(w: Workload):
    """Unpacked int4 weight parts for the W4A16 workload.

    Returns (codes u8[N, K] in 0..15, zeros u8[N, K/128] in 0..15,
    scales bf16 bits [N, K/128] = bf16(0.003 * U[0.5, 1.5))), so that the
    dequantized weights have a spread close to the other workloads' N(0, 0.02^2).
    """
    N, K = w.N, w.K
    codes = np.random.default_rng(1000 * w.index + 4).integers(0, 16, (N, K), dtype=np.uint8)
    zeros = np.random.default_rng(1000 * w.index + 5).integers(0, 16, (N, K // 128), dtype=np.uint8)
    u = np.random.default_rng(1000 * w.index + 6).uniform(0.5, 1.5, (N, K // 128)).astype(np.float32)
    scales = f32_to_bf16_bits(u * np.float32(0.003))
    return codes, zeros, scales


def pack_int4_codes(codes: np.ndarray) -> np.ndarray:
    """Store generated int4 codes [R, K] in the canonical u32 layout [R, K/8]
    (element k at bits 4*(k mod 8)), as a checkpoint loader would hand them over."""
    c = np.asarray(codes, dtype=np.uint32).reshape(codes.shape[0], -1, 8)
    out = np.zeros(c.shape[:2], dtype=np.uint32)
    for j in range(8):
        out |= (c[:, :, j] & 0xF) << np.uint32(4 * j)
    return out


def small_case(seed: int, rows: int, cols: int, std: float = 1.0) -> np.ndarray:
    """A small seeded bf16 tensor for parity cases that span several tiles."""
    return normal_bf16(seed, rows, cols, std)


def pow2_blocks(bits: np.ndarray, seed: int, row_block: int, col_block: int) -> np.ndarray:
    """Multiply a bf16 tensor by 2^(e_i + f_j), e per block of ``row_block`` rows and f per
    block of ``col_block`` columns, each cycling through 0, 1, 2 (offset by ``seed``), so
    that neighbouring blocks differ in magnitude by 2x or 4x.  Power-of-two scaling of
    bf16 values is exact.  Parity cases use it so that a scale taken from a
    neighbouring row, K-group or block is off by at least a factor of 2."""
    b = np.asarray(bits, dtype=np.uint16)
    rows, cols = b.shape
    e = (np.arange(rows) // row_block + seed) % 3
    f = (2 * (np.arange(cols) // col_block) + seed) % 3
    x = bf16_bits_to_f32(b) * np.ldexp(np.float32(1.0), (e[:, None] + f[None, :])).astype(np.float32)
    return f32_to_bf16_bits(x)
