"""Similarity metrics between a candidate output and its reference (oracle; test
infrastructure).

The online-quantization guide ("vLLM-Omni Online Quantization complete guide",
section "Verification and caveats", item 1) checks a quantized run against its
bf16 baseline with a trajectory-similarity tool that reports cosine
similarity, mean absolute error, mean squared error and its root, the largest
absolute difference, the L2 norm of the difference and that norm relative to
the reference, and a PSNR in decibels; it suggests starting thresholds of
PSNR >= 20 dB and cosine similarity >= 0.98.  The page names the metrics but
does not define them; the textbook definitions are used, over the flattened
tensors, in float64 (d = candidate - reference):

* cosine_similarity = <c, r> / (||c|| ||r||)   (1 when both are all zero,
  0 when exactly one is)
* mae = mean |d|,  mse = mean d^2,  rmse = sqrt(mse),  max_abs = max |d|
* l2 = ||d||_2,  relative_l2 = ||d||_2 / ||r||_2   (0 when d = 0, inf when
  only r = 0)
* psnr_db = 10 log10(peak^2 / mse) with peak = max(r) - min(r), the
  reference's value range (inf when mse = 0).  The page does not say which
  peak; the reference's own range is the reading used here.
"""
from __future__ import annotations

import math

import numpy as np

STARTING_THRESHOLDS = {"psnr_db": 20.0, "cosine_similarity": 0.98}


def _flat(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).reshape(-1)


def cosine_similarity(cand, ref) -> float:
    c, r = _flat(cand), _flat(ref)
    nc, nr = float(np.linalg.norm(c)), float(np.linalg.norm(r))
    if nc == 0.0 or nr == 0.0:
        return 1.0 if nc == nr else 0.0
    return float(np.dot(c, r) / (nc * nr))


def similarity(cand, ref) -> dict:
    """Every metric of the similarity report for one pair of tensors."""
    c, r = _flat(cand), _flat(ref)
    if c.shape != r.shape:
        raise ValueError(f"shape mismatch: {c.shape} vs {r.shape}")
    if c.size == 0:
        raise ValueError("empty tensors have no similarity")
    d = c - r
    ad = np.abs(d)
    mse = float(np.mean(d * d))
    l2 = float(np.linalg.norm(d))
    nr = float(np.linalg.norm(r))
    if l2 == 0.0:
        rel = 0.0
    else:
        rel = l2 / nr if nr > 0 else math.inf
    peak = float(np.max(r) - np.min(r))
    ratio = peak * peak / mse if mse != 0.0 else math.inf
    if mse == 0.0:
        psnr = math.inf
    elif not ratio > 0.0:     # a zero range, or an infinite error: no signal above the noise
        psnr = -math.inf if ratio == 0.0 or ratio != ratio else math.nan
    else:
        psnr = 10.0 * math.log10(ratio)
    return {"cosine_similarity": cosine_similarity(c, r), "mae": float(np.mean(ad)), "mse": mse,
            "rmse": math.sqrt(mse), "max_abs": float(np.max(ad)), "l2": l2, "relative_l2": rel,
            "psnr_db": psnr}


def meets_starting_thresholds(m: dict) -> bool:
    """The guide's suggested starting point: psnr_db >= 20 and cosine >= 0.98."""
    return (m["psnr_db"] >= STARTING_THRESHOLDS["psnr_db"]
            and m["cosine_similarity"] >= STARTING_THRESHOLDS["cosine_similarity"])


def format_similarity(m: dict) -> str:
    return ", ".join(f"{k} {v:.4g}" for k, v in m.items())
