"""CPU oracle for OCP MXFP4 / NVFP4 microscaling (numpy front end).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module; the product path
(the HIP library and its binding) never does.  The arithmetic lives in
``mxq_oracle.c`` (plain C, built with gcc) and shares no code with the GPU
sources.  This module only marshals numpy arrays to it.

Every function cites the passage of the pages it follows in the C source;
the short versions are repeated here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmxq_oracle.so")

F32 = 0
BF16 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, no fp contraction, no fast-math."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = [
            "gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
            "-fopenmp", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.or_e2m1_decode.argtypes = [ctypes.c_uint8]
    lib.or_e2m1_decode.restype = ctypes.c_double
    lib.or_e2m1_encode.argtypes = [ctypes.c_double, I]
    lib.or_e2m1_encode.restype = ctypes.c_uint8
    lib.or_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.or_e4m3_decode.restype = ctypes.c_double
    lib.or_e4m3_encode.argtypes = [ctypes.c_float]
    lib.or_e4m3_encode.restype = ctypes.c_uint8
    lib.or_e8m0_exponent.argtypes = [ctypes.c_double]
    lib.or_e8m0_exponent.restype = I
    lib.or_e8m0_decode.argtypes = [ctypes.c_uint8]
    lib.or_e8m0_decode.restype = ctypes.c_double
    lib.or_to_f64.argtypes = [P, I, I64, P]
    lib.or_mx_quantize.argtypes = [P, I, I64, I64, P, P, I]
    lib.or_mx_dequantize.argtypes = [P, P, I64, I64, P]
    lib.or_nv_tensor_scale.argtypes = [ctypes.c_float]
    lib.or_nv_tensor_scale.restype = ctypes.c_float
    lib.or_nv_quantize.argtypes = [P, I, I64, I64, P, I, P, P]
    lib.or_nv_dequantize.argtypes = [P, P, ctypes.c_float, I64, I64, P]
    lib.or_gemm_nt.argtypes = [P, P, I64, I64, I64, P, P]
    lib.or_metrics.argtypes = [P, P, I64, P, P]
    lib.or_e8m0_exponent_e4m3.argtypes = [ctypes.c_double]
    lib.or_e8m0_exponent_e4m3.restype = I
    lib.or_mx8_quantize.argtypes = [P, I, I64, I64, P, P]
    lib.or_mx8_dequantize.argtypes = [P, P, I64, I64, P]
    lib.or_hadamard_norm.argtypes = [I]
    lib.or_hadamard_norm.restype = ctypes.c_float
    lib.or_hadamard_rotate.argtypes = [P, I, I64, I64, I, P]
    lib.or_int4_decode.argtypes = [ctypes.c_uint8]
    lib.or_int4_decode.restype = ctypes.c_double
    lib.or_int4_encode.argtypes = [ctypes.c_double]
    lib.or_int4_encode.restype = ctypes.c_uint8
    lib.or_tf4_encode_rotated.argtypes = [P, I64, I64, P, I, P, P, P, P]
    lib.or_tf4_quantize.argtypes = [P, I, I64, I64, P, I, P, P, P, P]
    lib.or_tf4_decode_rotated.argtypes = [P, P, P, P, ctypes.c_float, I64, I64, P]
    lib.or_tf4_dequantize.argtypes = [P, P, P, P, ctypes.c_float, I64, I64, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_input(x: np.ndarray):
    """Accept fp32 arrays, or bf16 given as uint16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError("oracle inputs are float32 or bf16 bit patterns (uint16)")


# ---------------------------------------------------------------- scalars

def e2m1_decode(code: int) -> float:
    return _load().or_e2m1_decode(code)


def e2m1_encode(v: float, ties_away: bool = False) -> int:
    return _load().or_e2m1_encode(float(v), int(ties_away))


def e4m3_decode(code: int) -> float:
    return _load().or_e4m3_decode(code)


def e4m3_encode(r: float) -> int:
    return _load().or_e4m3_encode(float(r))


def e8m0_exponent(amax: float) -> int:
    return _load().or_e8m0_exponent(float(amax))


def e8m0_decode(code: int) -> float:
    return _load().or_e8m0_decode(code)


def nv_tensor_scale(amax: float) -> float:
    return _load().or_nv_tensor_scale(float(amax))


# ---------------------------------------------------------------- tensors

def to_f64(x: np.ndarray) -> np.ndarray:
    x, dt = _as_input(x)
    y = np.empty(x.shape, dtype=np.float64)
    _load().or_to_f64(_ptr(x), dt, x.size, _ptr(y))
    return y


def mx_quantize(x: np.ndarray, ties_away: bool = False):
    """x[rows][k] (fp32 or bf16 bits) -> (q[rows][k/2] uint8, s[rows][k/32] uint8)."""
    x, dt = _as_input(x)
    rows, k = x.shape
    assert k % 32 == 0
    q = np.empty((rows, k // 2), dtype=np.uint8)
    s = np.empty((rows, k // 32), dtype=np.uint8)
    _load().or_mx_quantize(_ptr(x), dt, rows, k, _ptr(q), _ptr(s), int(ties_away))
    return q, s


def mx_dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    rows, half = q.shape
    k = 2 * half
    assert s.shape == (rows, k // 32)
    y = np.empty((rows, k), dtype=np.float64)
    _load().or_mx_dequantize(_ptr(q), _ptr(s), rows, k, _ptr(y))
    return y


def e8m0_exponent_e4m3(amax: float) -> int:
    """MXFP8 block exponent floor(log2 amax) - 8, clamped."""
    return _load().or_e8m0_exponent_e4m3(float(amax))


def mx8_quantize(x: np.ndarray):
    """MXFP8: x[rows][k] -> (q[rows][k] E4M3 codes uint8, s[rows][k/32] E8M0)."""
    x, dt = _as_input(x)
    rows, k = x.shape
    assert k % 32 == 0
    q = np.empty((rows, k), dtype=np.uint8)
    s = np.empty((rows, k // 32), dtype=np.uint8)
    _load().or_mx8_quantize(_ptr(x), dt, rows, k, _ptr(q), _ptr(s))
    return q, s


def mx8_dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    rows, k = q.shape
    assert s.shape == (rows, k // 32)
    y = np.empty((rows, k), dtype=np.float64)
    _load().or_mx8_dequantize(_ptr(q), _ptr(s), rows, k, _ptr(y))
    return y


def nv_quantize(x: np.ndarray, gscale: float | None = None):
    """x[rows][k] -> (q[rows][k/2], s[rows][k/16] E4M3 codes, s_t fp32).

    gscale=None computes the tensor scale from the tensor's amax; a number
    is used as the (fp32) tensor scale as given."""
    x, dt = _as_input(x)
    rows, k = x.shape
    assert k % 16 == 0
    q = np.empty((rows, k // 2), dtype=np.uint8)
    s = np.empty((rows, k // 16), dtype=np.uint8)
    g = np.zeros(1, dtype=np.float32)
    compute = gscale is None
    if not compute:
        g[0] = np.float32(gscale)
    _load().or_nv_quantize(_ptr(x), dt, rows, k, _ptr(g), int(compute), _ptr(q), _ptr(s))
    return q, s, float(g[0])


def nv_dequantize(q: np.ndarray, s: np.ndarray, gscale: float) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    rows, half = q.shape
    k = 2 * half
    assert s.shape == (rows, k // 16)
    y = np.empty((rows, k), dtype=np.float64)
    _load().or_nv_dequantize(_ptr(q), _ptr(s), float(np.float32(gscale)), rows, k, _ptr(y))
    return y


HADAMARD_SIZES = (16, 32, 64, 128)


def hadamard_norm(hk: int) -> float:
    """The fp32 factor 1/sqrt(hk) of the orthonormal block Hadamard."""
    return float(_load().or_hadamard_norm(int(hk)))


def hadamard_rotate(x: np.ndarray, hk: int) -> np.ndarray:
    """x[rows][k] -> fp32 x rotated block by block along k with the
    orthonormal Sylvester Hadamard H_hk, in the fixed fp32 butterfly order
    [TransFP4 page sec. 2.3 eq. (2); FP4 analysis page sec. 3.2.3]."""
    x, dt = _as_input(x)
    rows, k = x.shape
    assert hk in HADAMARD_SIZES and k % hk == 0
    y = np.empty((rows, k), dtype=np.float32)
    _load().or_hadamard_rotate(_ptr(x), dt, rows, k, int(hk), _ptr(y))
    return y


def mx_quantize_hadamard(x: np.ndarray, hk: int = 32):
    """Rotated MXFP4: MXFP4 codes and scales of hadamard_rotate(x, hk)."""
    return mx_quantize(hadamard_rotate(x, hk))


def int4_decode(code: int) -> float:
    """Sign-magnitude INT4 code -> value in {-7..7}."""
    return _load().or_int4_decode(code)


def int4_encode(v: float) -> int:
    """Nearest INT4 magnitude (ties to even), saturating at 7, sign kept."""
    return _load().or_int4_encode(float(v))


def _tf4_outputs(rows, k):
    return (np.empty((rows, k // 2), dtype=np.uint8), np.empty((rows, k // 16), dtype=np.uint8),
            np.empty((rows, k // 32), dtype=np.uint8), np.empty((rows, k // 32), dtype=np.uint16))


def tf4_encode_rotated(y: np.ndarray, gscale: float | None = None):
    """TransFP4 encode of already rotated fp32 values y[rows][k]:
    (q, s E4M3 [rows][k/16], meta [rows][k/32], res bf16 bits [rows][k/32], s_t)
    [TransFP4 page sec. 2.3 eq. (3), sec. 3.1]."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    rows, k = y.shape
    assert k % 32 == 0
    q, s, meta, res = _tf4_outputs(rows, k)
    g = np.zeros(1, dtype=np.float32)
    compute = gscale is None
    if not compute:
        g[0] = np.float32(gscale)
    _load().or_tf4_encode_rotated(_ptr(y), rows, k, _ptr(g), int(compute), _ptr(q), _ptr(s), _ptr(meta),
                                  _ptr(res))
    return q, s, meta, res, float(g[0])


def tf4_quantize(x: np.ndarray, gscale: float | None = None):
    """TransFP4 quantize of x[rows][k]: 32-point Hadamard, one bf16 residual
    per 32, per-block NVFP4-or-INT4 codes under E4M3 scales and s_t."""
    x, dt = _as_input(x)
    rows, k = x.shape
    assert k % 32 == 0
    q, s, meta, res = _tf4_outputs(rows, k)
    g = np.zeros(1, dtype=np.float32)
    compute = gscale is None
    if not compute:
        g[0] = np.float32(gscale)
    _load().or_tf4_quantize(_ptr(x), dt, rows, k, _ptr(g), int(compute), _ptr(q), _ptr(s), _ptr(meta), _ptr(res))
    return q, s, meta, res, float(g[0])


def _tf4_inputs(q, s, meta, res):
    q = np.ascontiguousarray(q, dtype=np.uint8)
    rows, half = q.shape
    k = 2 * half
    s = np.ascontiguousarray(s, dtype=np.uint8)
    meta = np.ascontiguousarray(meta, dtype=np.uint8)
    res = np.ascontiguousarray(res, dtype=np.uint16)
    assert s.shape == (rows, k // 16) and meta.shape == (rows, k // 32) and res.shape == (rows, k // 32)
    return q, s, meta, res, rows, k


def tf4_decode_rotated(q, s, meta, res, gscale: float) -> np.ndarray:
    """Rotated-domain reconstruction (fp32): codes times block scales, plus
    the residual at its position."""
    q, s, meta, res, rows, k = _tf4_inputs(q, s, meta, res)
    y = np.empty((rows, k), dtype=np.float32)
    _load().or_tf4_decode_rotated(_ptr(q), _ptr(s), _ptr(meta), _ptr(res), float(np.float32(gscale)), rows, k,
                                  _ptr(y))
    return y


def tf4_dequantize(q, s, meta, res, gscale: float) -> np.ndarray:
    """x_hat = H^T y_hat per 32-block, fp32 (eq. (3))."""
    q, s, meta, res, rows, k = _tf4_inputs(q, s, meta, res)
    y = np.empty((rows, k), dtype=np.float32)
    _load().or_tf4_dequantize(_ptr(q), _ptr(s), _ptr(meta), _ptr(res), float(np.float32(gscale)), rows, k, _ptr(y))
    return y


def gemm_nt(a: np.ndarray, b: np.ndarray):
    """Y = A B^T and S = |A| |B|^T (elementwise sum of |products|), in double."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    m, k = a.shape
    n, k2 = b.shape
    assert k == k2
    y = np.empty((m, n), dtype=np.float64)
    s = np.empty((m, n), dtype=np.float64)
    _load().or_gemm_nt(_ptr(a), _ptr(b), m, n, k, _ptr(y), _ptr(s))
    return y, s


def metrics(x: np.ndarray, xh: np.ndarray):
    """(NMSE, cosine) in double over the flattened tensors."""
    x = np.ascontiguousarray(x, dtype=np.float64).ravel()
    xh = np.ascontiguousarray(xh, dtype=np.float64).ravel()
    assert x.size == xh.size
    out = np.zeros(2, dtype=np.float64)
    _load().or_metrics(_ptr(x), _ptr(xh), x.size,
                       out[0:].ctypes.data_as(ctypes.c_void_p),
                       out[1:].ctypes.data_as(ctypes.c_void_p))
    return float(out[0]), float(out[1])
