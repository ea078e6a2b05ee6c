"""MXFP4 / NVFP4 microscaling on AMD MI355X (gfx950): Python binding.

Thin ctypes layer over ``libmxq.so`` (the C ABI in ``include/mxq.h``).  It
only checks shapes/dtypes, allocates outputs with ``torch.empty`` and passes
raw device pointers plus the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is not built, or the device is not gfx950, calls raise.

    q, s = quantize(x)                  # MXFP4: x [rows, k] bf16/fp32, k % 32 == 0
    y = dequantize(q, s, torch.float32)
    y = gemv_w4a16(wq, ws, x)           # y[m, n] = x @ deq(W)^T, x bf16
    c = gemm_w4a4(aq, as_, bq, bs)      # c[m, n] = deq(A) @ deq(B)^T
    q, s, g = nv_quantize(x)            # NVFP4: k % 16 == 0, g = fp32 tensor scale
    y = nv_dequantize(q, s, g)
    y = nv_gemm(wq, ws, g, x)
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxq.so")

MXQ_F32 = 0
MXQ_BF16 = 1
STATUS = {
    0: "MXQ_SUCCESS",
    1: "MXQ_ERROR_INVALID_VALUE",
    2: "MXQ_ERROR_MISALIGNED",
    3: "MXQ_ERROR_NOT_SUPPORTED",
    4: "MXQ_ERROR_LAUNCH_FAILURE",
}
API = (
    "mxq_status_string", "mxq_version", "mxq_quantize", "mxq_quantize_hadamard", "mxq_quantize_fp8",
    "mxq_dequantize", "mxq_gemv_w4a16", "mxq_gemm_w4a4", "mxq_gemm_w4a4_quant", "mxq_gemm_w4a4_dynamic",
    "mxq_gemm_w4a8", "mxq_gemm_w4a8_dynamic", "nvq_quantize", "nvq_dequantize", "nvq_gemm", "mxq_transfp4_quantize", "mxq_transfp4_dequantize",
)


class MXQError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)} ({status_string(code)})")


_lib = None


def capi() -> ctypes.CDLL:
    """The loaded C library with argument types set (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m mxfp4_microscaling_quantization_mxq_amd.build` (hipcc, gfx950)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.mxq_status_string.argtypes = [I]
    lib.mxq_status_string.restype = ctypes.c_char_p
    lib.mxq_version.argtypes = []
    lib.mxq_version.restype = I
    lib.mxq_quantize.argtypes = [P, I, I64, I64, P, P, P]
    lib.mxq_quantize_hadamard.argtypes = [P, I, I64, I64, I, P, P, P]
    lib.mxq_quantize_fp8.argtypes = [P, I, I64, I64, P, P, P]
    lib.mxq_gemm_w4a8.argtypes = [P, P, P, P, I64, I64, I64, P, I, P]
    lib.mxq_dequantize.argtypes = [P, P, I64, I64, P, I, P]
    lib.mxq_gemv_w4a16.argtypes = [P, P, I64, I64, P, I64, P, I, P]
    lib.mxq_gemm_w4a4.argtypes = [P, P, P, P, I64, I64, I64, P, I, P]
    lib.mxq_gemm_w4a4_quant.argtypes = [P, P, P, P, I64, I64, I64, P, P, P]
    lib.mxq_gemm_w4a4_dynamic.argtypes = [P, P, P, I64, I64, I64, P, I, P]
    lib.mxq_gemm_w4a8_dynamic.argtypes = [P, P, P, I64, I64, I64, P, I, P]
    lib.nvq_quantize.argtypes = [P, I, I64, I64, P, I, P, P, P]
    lib.nvq_dequantize.argtypes = [P, P, P, I64, I64, P, I, P]
    lib.nvq_gemm.argtypes = [P, P, P, I64, I64, P, I64, P, I, P]
    lib.mxq_transfp4_quantize.argtypes = [P, I, I64, I64, P, I, P, P, P, P, P]
    lib.mxq_transfp4_dequantize.argtypes = [P, P, P, P, P, I64, I64, P, I, P]
    for name in API[2:]:
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return capi().mxq_status_string(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise MXQError(code, what)


# ------------------------------------------------------------------ helpers

def _torch():
    import torch

    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return MXQ_F32
    if dt == torch.bfloat16:
        return MXQ_BF16
    raise TypeError(f"unsupported dtype {dt}: use torch.float32 or torch.bfloat16")


def _p(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, ndim=2):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda/hip) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


# ------------------------------------------------------------------ MXFP4

def quantize(x, q=None, s=None):
    """MXFP4 quantize x[rows, k] (bf16 or fp32) -> (q[rows, k/2] u8, s[rows, k/32] u8)."""
    torch = _torch()
    _need(x, "x")
    rows, k = x.shape
    if q is None:
        q = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, k // 32), dtype=torch.uint8, device=x.device)
    _check(capi().mxq_quantize(_p(x), _dtype_code(x.dtype), rows, k, _p(q), _p(s), _stream()), "mxq_quantize")
    return q, s


def quantize_hadamard(x, hk=32, q=None, s=None):
    """Rotated MXFP4: quantize x[rows, k] after the orthonormal block Hadamard
    H_hk along k (hk in 16, 32, 64, 128) -> (q[rows, k/2] u8, s[rows, k/32] u8)."""
    torch = _torch()
    _need(x, "x")
    rows, k = x.shape
    if q is None:
        q = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, k // 32), dtype=torch.uint8, device=x.device)
    _check(capi().mxq_quantize_hadamard(_p(x), _dtype_code(x.dtype), rows, k, int(hk), _p(q), _p(s), _stream()),
           "mxq_quantize_hadamard")
    return q, s


def quantize_fp8(x, q=None, s=None):
    """MXFP8 quantize x[rows, k] -> (q[rows, k] E4M3 codes u8, s[rows, k/32] E8M0 u8)."""
    torch = _torch()
    _need(x, "x")
    rows, k = x.shape
    if q is None:
        q = torch.empty((rows, k), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, k // 32), dtype=torch.uint8, device=x.device)
    _check(capi().mxq_quantize_fp8(_p(x), _dtype_code(x.dtype), rows, k, _p(q), _p(s), _stream()), "mxq_quantize_fp8")
    return q, s


def dequantize(q, s, dtype=None, y=None):
    """(q[rows, k/2], s[rows, k/32]) -> y[rows, k] in dtype (default bf16)."""
    torch = _torch()
    dtype = dtype or torch.bfloat16
    _need(q, "q", torch.uint8)
    _need(s, "s", torch.uint8)
    rows, k = q.shape[0], q.shape[1] * 2
    if y is None:
        y = torch.empty((rows, k), dtype=dtype, device=q.device)
    _check(capi().mxq_dequantize(_p(q), _p(s), rows, k, _p(y), _dtype_code(y.dtype), _stream()), "mxq_dequantize")
    return y


def gemv_w4a16(wq, ws, x, out_dtype=None, y=None):
    """y[m, n] = x[m, k] @ deq(W)^T with W = (wq[n, k/2], ws[n, k/32]); x bf16."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    _need(wq, "wq", torch.uint8)
    _need(ws, "ws", torch.uint8)
    _need(x, "x", torch.bfloat16)
    n, k = wq.shape[0], wq.shape[1] * 2
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError(f"x has k={x.shape[1]}, weight has k={k}")
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _check(capi().mxq_gemv_w4a16(_p(wq), _p(ws), n, k, _p(x), m, _p(y), _dtype_code(y.dtype), _stream()),
           "mxq_gemv_w4a16")
    return y


def gemm_w4a4(aq, as_, bq, bs, out_dtype=None, c=None):
    """c[m, n] = deq(A)[m, k] @ deq(B)[n, k]^T, both MXFP4."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    for t, nm in ((aq, "aq"), (as_, "as"), (bq, "bq"), (bs, "bs")):
        _need(t, nm, torch.uint8)
    m, k = aq.shape[0], aq.shape[1] * 2
    n = bq.shape[0]
    if bq.shape[1] * 2 != k:
        raise ValueError("A and B disagree on k")
    if c is None:
        c = torch.empty((m, n), dtype=out_dtype, device=aq.device)
    _check(capi().mxq_gemm_w4a4(_p(aq), _p(as_), _p(bq), _p(bs), m, n, k, _p(c), _dtype_code(c.dtype), _stream()),
           "mxq_gemm_w4a4")
    return c


def _gemm_dynamic(entry, x, bq, bs, out_dtype, c):
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    _need(x, "x", torch.bfloat16)
    for t, nm in ((bq, "bq"), (bs, "bs")):
        _need(t, nm, torch.uint8)
    m, k = x.shape
    n = bq.shape[0]
    if bq.shape[1] * 2 != k:
        raise ValueError("x and B disagree on k")
    if c is None:
        c = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _check(getattr(capi(), entry)(_p(x), _p(bq), _p(bs), m, n, k, _p(c), _dtype_code(c.dtype), _stream()), entry)
    return c


def gemm_w4a4_dynamic(x, bq, bs, out_dtype=None, c=None):
    """c[m, n] = MXFP4(x)[m, k] @ deq(B)[n, k]^T with bf16 x quantized inside
    the kernel (bit-identical to gemm_w4a4(*quantize(x), bq, bs)); m <= 16,
    k % 512 == 0."""
    return _gemm_dynamic("mxq_gemm_w4a4_dynamic", x, bq, bs, out_dtype, c)


def gemm_w4a8_dynamic(x, bq, bs, out_dtype=None, c=None):
    """c[m, n] = MXFP8(x)[m, k] @ deq(B)[n, k]^T with bf16 x quantized to MXFP8
    inside the kernel (bit-identical to gemm_w4a8(*quantize_fp8(x), bq, bs));
    m <= 16, k % 512 == 0."""
    return _gemm_dynamic("mxq_gemm_w4a8_dynamic", x, bq, bs, out_dtype, c)


def gemm_w4a8(aq8, as_, bq, bs, out_dtype=None, c=None):
    """c[m, n] = deq8(A)[m, k] @ deq4(B)[n, k]^T: MXFP8 activations, MXFP4 weights."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    for t, nm in ((aq8, "aq8"), (as_, "as"), (bq, "bq"), (bs, "bs")):
        _need(t, nm, torch.uint8)
    m, k = aq8.shape
    n = bq.shape[0]
    if bq.shape[1] * 2 != k:
        raise ValueError("A and B disagree on k")
    if c is None:
        c = torch.empty((m, n), dtype=out_dtype, device=aq8.device)
    _check(capi().mxq_gemm_w4a8(_p(aq8), _p(as_), _p(bq), _p(bs), m, n, k, _p(c), _dtype_code(c.dtype), _stream()),
           "mxq_gemm_w4a8")
    return c


def gemm_w4a4_quant(aq, as_, bq, bs, cq=None, cs=None):
    """W4A4 with MXFP4 output: (cq[m, n/2], cs[m, n/32]) = MXFP4 of the
    bf16-rounded deq(A) @ deq(B)^T, quantized in the GEMM epilogue."""
    torch = _torch()
    for t, nm in ((aq, "aq"), (as_, "as"), (bq, "bq"), (bs, "bs")):
        _need(t, nm, torch.uint8)
    m, k = aq.shape[0], aq.shape[1] * 2
    n = bq.shape[0]
    if bq.shape[1] * 2 != k:
        raise ValueError("A and B disagree on k")
    if cq is None:
        cq = torch.empty((m, n // 2), dtype=torch.uint8, device=aq.device)
    if cs is None:
        cs = torch.empty((m, n // 32), dtype=torch.uint8, device=aq.device)
    _check(capi().mxq_gemm_w4a4_quant(_p(aq), _p(as_), _p(bq), _p(bs), m, n, k, _p(cq), _p(cs), _stream()),
           "mxq_gemm_w4a4_quant")
    return cq, cs


# ------------------------------------------------------------------ NVFP4

def nv_quantize(x, gscale=None, q=None, s=None, g=None):
    """NVFP4 quantize x[rows, k] -> (q[rows, k/2], s[rows, k/16] E4M3, g[1] fp32 tensor scale).

    gscale=None computes the tensor scale on the device (into g if given); a
    float or a 1-element fp32 tensor is used as given."""
    torch = _torch()
    _need(x, "x")
    rows, k = x.shape
    compute = gscale is None
    if compute:
        if g is None:
            g = torch.empty(1, dtype=torch.float32, device=x.device)
    elif isinstance(gscale, (float, int)):
        g = torch.tensor([float(gscale)], dtype=torch.float32, device=x.device)
    else:
        g = gscale
    if q is None:
        q = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, k // 16), dtype=torch.uint8, device=x.device)
    _check(capi().nvq_quantize(_p(x), _dtype_code(x.dtype), rows, k, _p(g), int(compute), _p(q), _p(s),
                               _stream()), "nvq_quantize")
    return q, s, g


def nv_dequantize(q, s, g, dtype=None, y=None):
    torch = _torch()
    dtype = dtype or torch.bfloat16
    _need(q, "q", torch.uint8)
    _need(s, "s", torch.uint8)
    rows, k = q.shape[0], q.shape[1] * 2
    if y is None:
        y = torch.empty((rows, k), dtype=dtype, device=q.device)
    _check(capi().nvq_dequantize(_p(q), _p(s), _p(g), rows, k, _p(y), _dtype_code(y.dtype), _stream()),
           "nvq_dequantize")
    return y


# ------------------------------------------------------------------ TransFP4 blocks

def transfp4_quantize(x, gscale=None, q=None, s=None, meta=None, res=None, g=None):
    """TransFP4 quantize x[rows, k] -> (q[rows, k/2], s[rows, k/16] E4M3,
    meta[rows, k/32] (bit 7 INT4 tag, bits 0-4 residual position),
    res[rows, k/32] bf16 residuals, g[1] fp32 tensor scale).  gscale as in
    nv_quantize."""
    torch = _torch()
    _need(x, "x")
    rows, k = x.shape
    compute = gscale is None
    if compute:
        if g is None:
            g = torch.empty(1, dtype=torch.float32, device=x.device)
    elif isinstance(gscale, (float, int)):
        g = torch.tensor([float(gscale)], dtype=torch.float32, device=x.device)
    else:
        g = gscale
    dev = x.device
    q = q if q is not None else torch.empty((rows, k // 2), dtype=torch.uint8, device=dev)
    s = s if s is not None else torch.empty((rows, k // 16), dtype=torch.uint8, device=dev)
    meta = meta if meta is not None else torch.empty((rows, k // 32), dtype=torch.uint8, device=dev)
    res = res if res is not None else torch.empty((rows, k // 32), dtype=torch.bfloat16, device=dev)
    _check(capi().mxq_transfp4_quantize(_p(x), _dtype_code(x.dtype), rows, k, _p(g), int(compute), _p(q), _p(s),
                                        _p(meta), _p(res), _stream()), "mxq_transfp4_quantize")
    return q, s, meta, res, g


def transfp4_dequantize(q, s, meta, res, g, dtype=None, y=None):
    """x_hat[rows, k] (fp32 or bf16) from the TransFP4 arrays."""
    torch = _torch()
    dtype = dtype or torch.float32
    _need(q, "q", torch.uint8)
    _need(s, "s", torch.uint8)
    _need(meta, "meta", torch.uint8)
    _need(res, "res", torch.bfloat16)
    rows, k = q.shape[0], q.shape[1] * 2
    if y is None:
        y = torch.empty((rows, k), dtype=dtype, device=q.device)
    _check(capi().mxq_transfp4_dequantize(_p(q), _p(s), _p(meta), _p(res), _p(g), rows, k, _p(y),
                                          _dtype_code(y.dtype), _stream()), "mxq_transfp4_dequantize")
    return y


def nv_gemm(wq, ws, g, x, out_dtype=None, y=None):
    """y[m, n] = s_t * x[m, k] @ (s_b * q)[n, k]^T with an NVFP4 weight; x bf16."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    _need(wq, "wq", torch.uint8)
    _need(ws, "ws", torch.uint8)
    _need(x, "x", torch.bfloat16)
    n, k = wq.shape[0], wq.shape[1] * 2
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError(f"x has k={x.shape[1]}, weight has k={k}")
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _check(capi().nvq_gemm(_p(wq), _p(ws), _p(g), n, k, _p(x), m, _p(y), _dtype_code(y.dtype), _stream()),
           "nvq_gemm")
    return y
