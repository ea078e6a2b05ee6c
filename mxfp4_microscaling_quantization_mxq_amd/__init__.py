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
    q, s, g = nvq.quantize(x)           # NVFP4: k % 16 == 0, g = fp32 tensor scale
    y = nvq.dequantize(q, s, g)         # (also nv_quantize / nv_dequantize / nv_gemm)
    y = nvq.gemm(wq, ws, g, x)

Every tensor argument is checked before anything is enqueued: dtype, shape
(scales and caller-supplied outputs must match the operands exactly),
contiguity, and that it lives on the operands' device; the NVFP4 tensor
scale must be a 1-element fp32 device tensor.
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


def _need(t, name, dtype=None, shape=None, ndim=2, device=None):
    """Validate one tensor argument's type, dtype, shape and contiguity
    (where it lives is checked by _on_device, after every shape check).
    Raises TypeError / ValueError; `device` is accepted for symmetry only."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if dtype is not None:
        allowed = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in allowed:
            raise TypeError(f"{name} must be {' or '.join(str(d) for d in allowed)}, got {t.dtype}")
    if shape is not None:
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    elif t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(**tensors):
    """Every tensor of the call on one and the same device (cuda/hip)."""
    dev = None
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device (cuda/hip) tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other operands on {dev}")


def _floats():
    torch = _torch()
    return (torch.float32, torch.bfloat16)


def _out(t, name, shape, dtype, device, real=False):
    """An output tensor: allocated if None, else validated like an input.
    `real` outputs (unquantized values) must be float32 or bfloat16."""
    torch = _torch()
    if real and dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"{name} must be torch.float32 or torch.bfloat16, got {dtype}")
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(t, name, dtype, shape, device=device)
    return t


def _gscale(g, name, device):
    """The NVFP4 tensor scale: a 1-element fp32 device tensor."""
    torch = _torch()
    _need(g, name, torch.float32, (1,), device=device)
    return g


# ------------------------------------------------------------------ MXFP4

def _k_blocks(k, blk, what):
    if k % blk != 0:
        raise ValueError(f"{what}: k = {k} is not a multiple of {blk}")


def quantize(x, q=None, s=None):
    """MXFP4 quantize x[rows, k] (bf16 or fp32) -> (q[rows, k/2] u8, s[rows, k/32] u8)."""
    torch = _torch()
    _need(x, "x", _floats())
    rows, k = x.shape
    _k_blocks(k, 32, "quantize")
    q = _out(q, "q", (rows, k // 2), torch.uint8, x.device)
    s = _out(s, "s", (rows, k // 32), torch.uint8, x.device)
    _on_device(x=x, q=q, s=s)
    _check(capi().mxq_quantize(_p(x), _dtype_code(x.dtype), rows, k, _p(q), _p(s), _stream()), "mxq_quantize")
    return q, s


def quantize_hadamard(x, hk=32, q=None, s=None):
    """Rotated MXFP4: quantize x[rows, k] after the orthonormal block Hadamard
    H_hk along k (hk in 16, 32, 64, 128) -> (q[rows, k/2] u8, s[rows, k/32] u8)."""
    torch = _torch()
    _need(x, "x", _floats())
    rows, k = x.shape
    _k_blocks(k, 32, "quantize_hadamard")
    q = _out(q, "q", (rows, k // 2), torch.uint8, x.device)
    s = _out(s, "s", (rows, k // 32), torch.uint8, x.device)
    _on_device(x=x, q=q, s=s)
    _check(capi().mxq_quantize_hadamard(_p(x), _dtype_code(x.dtype), rows, k, int(hk), _p(q), _p(s), _stream()),
           "mxq_quantize_hadamard")
    return q, s


def quantize_fp8(x, q=None, s=None):
    """MXFP8 quantize x[rows, k] -> (q[rows, k] E4M3 codes u8, s[rows, k/32] E8M0 u8)."""
    torch = _torch()
    _need(x, "x", _floats())
    rows, k = x.shape
    _k_blocks(k, 32, "quantize_fp8")
    q = _out(q, "q", (rows, k), torch.uint8, x.device)
    s = _out(s, "s", (rows, k // 32), torch.uint8, x.device)
    _on_device(x=x, q=q, s=s)
    _check(capi().mxq_quantize_fp8(_p(x), _dtype_code(x.dtype), rows, k, _p(q), _p(s), _stream()), "mxq_quantize_fp8")
    return q, s


def dequantize(q, s, dtype=None, y=None):
    """(q[rows, k/2], s[rows, k/32]) -> y[rows, k] in dtype (default bf16; y's dtype if y is given)."""
    torch = _torch()
    _need(q, "q", torch.uint8)
    rows, k = q.shape[0], q.shape[1] * 2
    _k_blocks(k, 32, "dequantize")
    _need(s, "s", torch.uint8, (rows, k // 32), device=q.device)
    dtype = dtype or (y.dtype if y is not None else torch.bfloat16)
    y = _out(y, "y", (rows, k), dtype, q.device, real=True)
    _on_device(q=q, s=s, y=y)
    _check(capi().mxq_dequantize(_p(q), _p(s), rows, k, _p(y), _dtype_code(y.dtype), _stream()), "mxq_dequantize")
    return y


def _weight(wq, ws, blk, what):
    """An MXFP4 (blk 32) or NVFP4 (blk 16) weight: (n, k) after validation."""
    torch = _torch()
    _need(wq, "wq", torch.uint8)
    n, k = wq.shape[0], wq.shape[1] * 2
    _k_blocks(k, blk, what)
    _need(ws, "ws", torch.uint8, (n, k // blk), device=wq.device)
    return n, k


def _activations(x, k, dev):
    torch = _torch()
    _need(x, "x", torch.bfloat16, device=dev)
    if x.shape[1] != k:
        raise ValueError(f"x has k={x.shape[1]}, weight has k={k}")
    return x.shape[0]


def gemv_w4a16(wq, ws, x, out_dtype=None, y=None):
    """y[m, n] = x[m, k] @ deq(W)^T with W = (wq[n, k/2], ws[n, k/32]); x bf16."""
    torch = _torch()
    n, k = _weight(wq, ws, 32, "gemv_w4a16")
    m = _activations(x, k, wq.device)
    out_dtype = out_dtype or (y.dtype if y is not None else torch.bfloat16)
    y = _out(y, "y", (m, n), out_dtype, wq.device, real=True)
    _on_device(wq=wq, ws=ws, x=x, y=y)
    _check(capi().mxq_gemv_w4a16(_p(wq), _p(ws), n, k, _p(x), m, _p(y), _dtype_code(y.dtype), _stream()),
           "mxq_gemv_w4a16")
    return y


def _ab(aq, as_, bq, bs, a_bytes_per_k, what):
    """Block-scaled operands A (aq[m, k * a_bytes_per_k], as_[m, k/32]) and
    B (bq[n, k/2], bs[n, k/32]): (m, n, k) after validation."""
    torch = _torch()
    _need(aq, "aq", torch.uint8)
    m = aq.shape[0]
    k = int(aq.shape[1] / a_bytes_per_k)
    _k_blocks(k, 32, what)
    dev = aq.device
    _need(as_, "as", torch.uint8, (m, k // 32), device=dev)
    _need(bq, "bq", torch.uint8, device=dev)
    if bq.shape[1] * 2 != k:
        raise ValueError(f"{what}: A has k={k}, B has k={bq.shape[1] * 2}")
    n = bq.shape[0]
    _need(bs, "bs", torch.uint8, (n, k // 32), device=dev)
    return m, n, k


def gemm_w4a4(aq, as_, bq, bs, out_dtype=None, c=None):
    """c[m, n] = deq(A)[m, k] @ deq(B)[n, k]^T, both MXFP4."""
    torch = _torch()
    m, n, k = _ab(aq, as_, bq, bs, 0.5, "gemm_w4a4")
    out_dtype = out_dtype or (c.dtype if c is not None else torch.bfloat16)
    c = _out(c, "c", (m, n), out_dtype, aq.device, real=True)
    _on_device(aq=aq, as_=as_, bq=bq, bs=bs, c=c)
    _check(capi().mxq_gemm_w4a4(_p(aq), _p(as_), _p(bq), _p(bs), m, n, k, _p(c), _dtype_code(c.dtype), _stream()),
           "mxq_gemm_w4a4")
    return c


def _gemm_dynamic(entry, x, bq, bs, out_dtype, c):
    torch = _torch()
    n, k = _weight(bq, bs, 32, entry)
    m = _activations(x, k, bq.device)
    out_dtype = out_dtype or (c.dtype if c is not None else torch.bfloat16)
    c = _out(c, "c", (m, n), out_dtype, bq.device, real=True)
    _on_device(x=x, bq=bq, bs=bs, c=c)
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
    m, n, k = _ab(aq8, as_, bq, bs, 1, "gemm_w4a8")
    out_dtype = out_dtype or (c.dtype if c is not None else torch.bfloat16)
    c = _out(c, "c", (m, n), out_dtype, aq8.device, real=True)
    _on_device(aq8=aq8, as_=as_, bq=bq, bs=bs, c=c)
    _check(capi().mxq_gemm_w4a8(_p(aq8), _p(as_), _p(bq), _p(bs), m, n, k, _p(c), _dtype_code(c.dtype), _stream()),
           "mxq_gemm_w4a8")
    return c


def gemm_w4a4_quant(aq, as_, bq, bs, cq=None, cs=None):
    """W4A4 with MXFP4 output: (cq[m, n/2], cs[m, n/32]) = MXFP4 of the
    bf16-rounded deq(A) @ deq(B)^T, quantized in the GEMM epilogue."""
    torch = _torch()
    m, n, k = _ab(aq, as_, bq, bs, 0.5, "gemm_w4a4_quant")
    if n % 32 != 0:
        raise ValueError(f"gemm_w4a4_quant: n = {n} is not a multiple of 32")
    cq = _out(cq, "cq", (m, n // 2), torch.uint8, aq.device)
    cs = _out(cs, "cs", (m, n // 32), torch.uint8, aq.device)
    _on_device(aq=aq, as_=as_, bq=bq, bs=bs, cq=cq, cs=cs)
    _check(capi().mxq_gemm_w4a4_quant(_p(aq), _p(as_), _p(bq), _p(bs), m, n, k, _p(cq), _p(cs), _stream()),
           "mxq_gemm_w4a4_quant")
    return cq, cs


# ------------------------------------------------------------------ NVFP4

def _tensor_scale_arg(gscale, g, device):
    """(compute, g): gscale None -> computed on the device into g (allocated
    if None); a float -> a new device tensor; a tensor -> used as given."""
    torch = _torch()
    if gscale is None:
        if g is None:
            g = torch.empty(1, dtype=torch.float32, device=device)
        return True, _gscale(g, "g", device)
    if isinstance(gscale, (float, int)):
        return False, torch.tensor([float(gscale)], dtype=torch.float32, device=device)
    return False, _gscale(gscale, "gscale", device)


def nv_quantize(x, gscale=None, q=None, s=None, g=None):
    """NVFP4 quantize x[rows, k] -> (q[rows, k/2], s[rows, k/16] E4M3, g[1] fp32 tensor scale).

    gscale=None computes the tensor scale on the device (into g if given); a
    float or a 1-element fp32 tensor is used as given."""
    torch = _torch()
    _need(x, "x", _floats())
    rows, k = x.shape
    _k_blocks(k, 16, "nv_quantize")
    compute, g = _tensor_scale_arg(gscale, g, x.device)
    q = _out(q, "q", (rows, k // 2), torch.uint8, x.device)
    s = _out(s, "s", (rows, k // 16), torch.uint8, x.device)
    _on_device(x=x, g=g, q=q, s=s)
    _check(capi().nvq_quantize(_p(x), _dtype_code(x.dtype), rows, k, _p(g), int(compute), _p(q), _p(s),
                               _stream()), "nvq_quantize")
    return q, s, g


def nv_dequantize(q, s, g, dtype=None, y=None):
    """(q[rows, k/2], s[rows, k/16], g[1]) -> y[rows, k] = g * E4M3(s) * E2M1(q), rounded once to dtype."""
    torch = _torch()
    _need(q, "q", torch.uint8)
    rows, k = q.shape[0], q.shape[1] * 2
    _k_blocks(k, 16, "nv_dequantize")
    _need(s, "s", torch.uint8, (rows, k // 16), device=q.device)
    _gscale(g, "g", q.device)
    dtype = dtype or (y.dtype if y is not None else torch.bfloat16)
    y = _out(y, "y", (rows, k), dtype, q.device, real=True)
    _on_device(q=q, s=s, g=g, y=y)
    _check(capi().nvq_dequantize(_p(q), _p(s), _p(g), rows, k, _p(y), _dtype_code(y.dtype), _stream()),
           "nvq_dequantize")
    return y


def nv_gemm(wq, ws, g, x, out_dtype=None, y=None):
    """y[m, n] = s_t * x[m, k] @ (s_b * q)[n, k]^T with an NVFP4 weight; x bf16."""
    torch = _torch()
    n, k = _weight(wq, ws, 16, "nv_gemm")
    _gscale(g, "g", wq.device)
    m = _activations(x, k, wq.device)
    out_dtype = out_dtype or (y.dtype if y is not None else torch.bfloat16)
    y = _out(y, "y", (m, n), out_dtype, wq.device, real=True)
    _on_device(wq=wq, ws=ws, g=g, x=x, y=y)
    _check(capi().nvq_gemm(_p(wq), _p(ws), _p(g), n, k, _p(x), m, _p(y), _dtype_code(y.dtype), _stream()),
           "nvq_gemm")
    return y


# ------------------------------------------------------------------ TransFP4 blocks

def transfp4_quantize(x, gscale=None, q=None, s=None, meta=None, res=None, g=None):
    """TransFP4 quantize x[rows, k] -> (q[rows, k/2], s[rows, k/16] E4M3,
    meta[rows, k/32] (bit 7 INT4 tag, bits 0-4 residual position),
    res[rows, k/32] bf16 residuals, g[1] fp32 tensor scale).  gscale as in
    nv_quantize."""
    torch = _torch()
    _need(x, "x", _floats())
    rows, k = x.shape
    _k_blocks(k, 32, "transfp4_quantize")
    dev = x.device
    compute, g = _tensor_scale_arg(gscale, g, dev)
    q = _out(q, "q", (rows, k // 2), torch.uint8, dev)
    s = _out(s, "s", (rows, k // 16), torch.uint8, dev)
    meta = _out(meta, "meta", (rows, k // 32), torch.uint8, dev)
    res = _out(res, "res", (rows, k // 32), torch.bfloat16, dev)
    _on_device(x=x, g=g, q=q, s=s, meta=meta, res=res)
    _check(capi().mxq_transfp4_quantize(_p(x), _dtype_code(x.dtype), rows, k, _p(g), int(compute), _p(q), _p(s),
                                        _p(meta), _p(res), _stream()), "mxq_transfp4_quantize")
    return q, s, meta, res, g


def transfp4_dequantize(q, s, meta, res, g, dtype=None, y=None):
    """x_hat[rows, k] (fp32 or bf16) from the TransFP4 arrays."""
    torch = _torch()
    _need(q, "q", torch.uint8)
    rows, k = q.shape[0], q.shape[1] * 2
    _k_blocks(k, 32, "transfp4_dequantize")
    dev = q.device
    _need(s, "s", torch.uint8, (rows, k // 16), device=dev)
    _need(meta, "meta", torch.uint8, (rows, k // 32), device=dev)
    _need(res, "res", torch.bfloat16, (rows, k // 32), device=dev)
    _gscale(g, "g", dev)
    dtype = dtype or (y.dtype if y is not None else torch.float32)
    y = _out(y, "y", (rows, k), dtype, dev, real=True)
    _on_device(q=q, s=s, meta=meta, res=res, g=g, y=y)
    _check(capi().mxq_transfp4_dequantize(_p(q), _p(s), _p(meta), _p(res), _p(g), rows, k, _p(y),
                                          _dtype_code(y.dtype), _stream()), "mxq_transfp4_dequantize")
    return y


from . import nvq  # noqa: E402  (the NVFP4 names: nvq.quantize / nvq.dequantize / nvq.gemm)
