"""Weight-only NVFP4 fused MoE layer for AMD MI355X (gfx950).

The layer's steps run in hand-written HIP kernels behind the C ABI of libmoe_nvfp4.so
(include/moe_nvfp4.h); this package only marshals torch tensors and streams into it.
"""

from . import synth
from ._lib import LIB_PATH, MoeError
from .ops import (NvFp4Experts, NvFp4MoELayer, combine, forward, forward_workspace_size, gscale_from_quant_scale,
                  grouped_gemm, grouped_gemm_w4a4, pack_tiles, permute, quantize, quantize_act_nv, route,
                  route_from_logits, validate_forward, workspace_for)
from .workloads import build_bank, build_layer

__all__ = ["synth", "LIB_PATH", "MoeError", "NvFp4Experts", "NvFp4MoELayer", "combine", "forward",
           "forward_workspace_size", "gscale_from_quant_scale", "grouped_gemm", "grouped_gemm_w4a4", "pack_tiles",
           "permute", "quantize", "quantize_act_nv", "route", "route_from_logits", "validate_forward",
           "workspace_for", "build_bank", "build_layer"]
