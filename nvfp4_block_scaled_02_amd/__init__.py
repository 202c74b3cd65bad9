"""NVFP4 block-scaled quantization for AMD Instinct MI355X (gfx950).

The computation lives in libnvfp4.so (hand-written HIP kernels behind the C
ABI of include/nvfp4.h); this package is its Python binding.  Importing it
does not load the library; the first call does, and raises if it is not built.
"""
from .api import (Launch, Quantized, default_global_max, dequantize, dequantize_rowscaled,
                  dequantize_rht, dequantized_amax, fakequant_bwd, fakequant_fwd, quantize,
                  quantize_2d, quantize_pertoken, quantize_rht, quantize_rowscaled, requantize_t,
                  rht_amax, row_amax, tensor_amax, workspace, prepare, prepare_quantize,
                  prepare_dequantize, prepare_tensor_amax)

__all__ = ["Launch", "Quantized", "default_global_max", "dequantize", "dequantize_rowscaled",
           "dequantize_rht", "dequantized_amax", "fakequant_bwd", "fakequant_fwd", "quantize",
           "quantize_2d", "quantize_pertoken", "quantize_rht", "quantize_rowscaled", "requantize_t",
           "rht_amax", "row_amax", "tensor_amax", "workspace", "prepare", "prepare_quantize",
           "prepare_dequantize", "prepare_tensor_amax"]
