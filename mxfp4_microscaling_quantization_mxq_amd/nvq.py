"""NVFP4 names of the binding: ``nvq.quantize``, ``nvq.dequantize`` and
``nvq.gemm`` are the package's ``nv_quantize``, ``nv_dequantize`` and
``nv_gemm`` (the C entry points nvq_quantize, nvq_dequantize, nvq_gemm)."""
from . import nv_dequantize as dequantize  # noqa: F401
from . import nv_gemm as gemm  # noqa: F401
from . import nv_quantize as quantize  # noqa: F401
