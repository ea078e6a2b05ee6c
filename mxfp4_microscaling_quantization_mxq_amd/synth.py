"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no quantization arithmetic: it only draws random tensors
and rounds them to their storage type (fp32, or bf16 kept as uint16 bit
patterns).  Both the GPU path and the CPU oracle receive these arrays.

Recipe (one generator per (workload id, tensor id)):
  rng = numpy Generator(PCG64(SeedSequence([workload, tensor])))
  values are drawn in float64, row chunk by row chunk, cast to fp32 with
  round-to-nearest-even, and to bf16 from fp32 with round-to-nearest-even;
  outliers: exactly round(p * n) distinct flat positions (rng.choice without
  replacement) are MULTIPLIED by the factor.

The heavy-tailed shapes follow the synthetic-tensor experiment of the
TransFP4 page ("Portable FP4 quantization for heterogeneous accelerators",
sec. 3.1, Table 4: Laplace/Student-t bodies with a small fraction of large
outliers, fixed seeds); the sizes are those of the workloads below.
"""
from __future__ import annotations

import numpy as np

_CHUNK = 1 << 22  # elements drawn per call


def rng_for(workload: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload, tensor])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng, dist: str, n: int, scale: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        if dist == "laplace":
            v = rng.laplace(0.0, scale, size=hi - lo)
        elif dist == "normal":
            v = rng.standard_normal(size=hi - lo) * scale
        elif dist == "t5":  # 0.42 * Student-t(5) activations body
            v = scale * rng.standard_t(5, size=hi - lo)
        else:
            raise ValueError(dist)
        out[lo:hi] = v.astype(np.float32)
    return out


def tensor(workload: int, tensor_id: int, rows: int, k: int, dist: str = "laplace",
           scale: float = 1.0, outlier_frac: float = 0.0, outlier_mult: float = 1.0,
           dtype: str = "bf16") -> np.ndarray:
    """[rows][k] tensor; dtype 'f32' -> float32, 'bf16' -> uint16 bf16 bits."""
    rng = rng_for(workload, tensor_id)
    n = rows * k
    x = _draw(rng, dist, n, scale)
    n_out = int(round(outlier_frac * n))
    if n_out:
        pos = rng.choice(n, size=n_out, replace=False)
        x[pos] = (x[pos].astype(np.float64) * outlier_mult).astype(np.float32)
    x = x.reshape(rows, k)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def channel_outliers(x_bits: np.ndarray, workload: int, tensor_id: int, n_channels: int,
                     mult: float) -> np.ndarray:
    """Scale n_channels distinct seeded columns of a bf16 tensor by mult (in fp32, then RNE to bf16)."""
    rng = rng_for(workload, 1000 + tensor_id)
    cols = np.sort(rng.choice(x_bits.shape[1], size=n_channels, replace=False))
    x = bf16_bits_to_f32(x_bits[:, cols]).astype(np.float64) * mult
    out = x_bits.copy()
    out[:, cols] = f32_to_bf16_bits(x.astype(np.float32))
    return out


# ------------------------------------------------------------ the workloads
# Workload ids: 1 tiny reference, 2 decode GEMV, 3 dynamic quantize,
# 4 W4A4 GEMM, 5 NVFP4 vs MXFP4, 6 Table-4-style activations.

def tiny_ref():
    """W fp32 [256][512] ~ Laplace(0,1), 1% entries x50; x bf16 [1][512] ~ N(0,1)."""
    w = tensor(1, 0, 256, 512, "laplace", 1.0, 0.01, 50.0, "f32")
    x = tensor(1, 1, 1, 512, "normal", 1.0, 0.0, 1.0, "bf16")
    return w, x


def decode_gemv(m: int, n: int = 28672, k: int = 8192):
    """W bf16 [n][k] ~ Laplace(0,0.02), 0.5% entries x30 (quantized later); x bf16 [m][k] ~ N(0,1)."""
    w = tensor(2, 0, n, k, "laplace", 0.02, 0.005, 30.0, "bf16")
    x = tensor(2, 10 + m, m, k, "normal", 1.0, 0.0, 1.0, "bf16")
    return w, x


def dynamic_quantize(rows: int = 16384, k: int = 8192):
    """X bf16 [rows][k] ~ Laplace(0,1) with 8 seeded channels scaled x100."""
    x = tensor(3, 0, rows, k, "laplace", 1.0, 0.0, 1.0, "bf16")
    return channel_outliers(x, 3, 0, 8, 100.0)


def w4a4_operands(m: int = 8192, n: int = 8192, k: int = 8192):
    """A [m][k], B [n][k] bf16 ~ N(0,1) with 1% entries x20 (independent streams)."""
    a = tensor(4, 0, m, k, "normal", 1.0, 0.01, 20.0, "bf16")
    b = tensor(4, 1, n, k, "normal", 1.0, 0.01, 20.0, "bf16")
    return a, b


def nv_vs_mx(n: int = 8192, m: int = 4096, k: int = 4096):
    """W bf16 [n][k], X bf16 [m][k] ~ Laplace(0,1) with 1% entries x50."""
    w = tensor(5, 0, n, k, "laplace", 1.0, 0.01, 50.0, "bf16")
    x = tensor(5, 1, m, k, "laplace", 1.0, 0.01, 50.0, "bf16")
    return w, x


def table4_activations(n: int = 131072, outlier_frac: float = 0.01, seed: int = 0) -> np.ndarray:
    """0.42 * t(5) body with round(p*n) positions replaced by body + N(0, 6^2) (fp32, 1 x n)."""
    rng = rng_for(6, seed)
    x = 0.42 * rng.standard_t(5, size=n)
    k = int(round(outlier_frac * n))
    pos = rng.choice(n, size=k, replace=False)
    x[pos] += rng.standard_normal(size=k) * 6.0
    return x.astype(np.float32).reshape(1, n)
