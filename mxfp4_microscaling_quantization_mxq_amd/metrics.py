"""Quality metrics of a quantized tensor or product (host, float64, untimed).

NMSE = sum (x - x_hat)^2 / sum x^2 and cosine similarity
cos = sum x * x_hat / (||x|| * ||x_hat||) over the flattened tensors, the
two figures the TransFP4 page ("Portable FP4 quantization for heterogeneous
accelerators", sec. 3.2, evaluation metrics) reports per format.  They
describe results the library produced; no step of the quantizers or products
runs here.
"""
from __future__ import annotations

import numpy as np


def nmse_cosine(x, x_hat):
    """(NMSE, cosine) of x_hat against the reference x, in float64."""
    x = np.asarray(x, dtype=np.float64).ravel()
    xh = np.asarray(x_hat, dtype=np.float64).ravel()
    if x.shape != xh.shape:
        raise ValueError(f"shapes differ: {x.shape} vs {xh.shape}")
    d = x - xh
    sxx = float(np.dot(x, x))
    shh = float(np.dot(xh, xh))
    nmse = float(np.dot(d, d)) / sxx if sxx > 0 else float("nan")
    cos = float(np.dot(x, xh)) / np.sqrt(sxx * shh) if sxx > 0 and shh > 0 else float("nan")
    return nmse, cos


def bf16_bits_to_f64(b):
    """bf16 bit patterns (uint16) -> float64 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
