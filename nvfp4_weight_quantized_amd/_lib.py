"""ctypes view of libmoe_nvfp4.so (the C ABI declared in include/moe_nvfp4.h).

The library is loaded on first use.  If it is missing the import of an op fails loudly:
there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_nvfp4.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED_DEVICE = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4

MOE_ROUTE_LOGITS_GIVEN = 1
MOE_GEMM_GATE_UP = 0
MOE_GEMM_DOWN = 1

c_void_p = ctypes.c_void_p
i32 = ctypes.c_int32
u32 = ctypes.c_uint32
size_t = ctypes.c_size_t


class Experts(ctypes.Structure):
    """moe_nvfp4_experts_t"""
    _fields_ = [
        ("num_experts", i32), ("hidden", i32), ("inter", i32), ("format", i32),
        ("w13", c_void_p), ("w13_scale", c_void_p), ("w13_gscale", c_void_p),
        ("w2", c_void_p), ("w2_scale", c_void_p), ("w2_gscale", c_void_p),
    ]


class Layer(ctypes.Structure):
    """moe_nvfp4_layer_t"""
    _fields_ = [
        ("hidden", i32), ("num_experts", i32), ("top_k", i32),
        ("w_router", c_void_p), ("router_bias", c_void_p),
        ("routed", Experts), ("shared", Experts),
        ("h16_norm", ctypes.c_float * 2),
    ]


class ForwardAux(ctypes.Structure):
    """moe_forward_aux_t"""
    _fields_ = [("logits", c_void_p), ("topk_ids", c_void_p), ("topk_w", c_void_p), ("expert_counts", c_void_p),
                ("stage_events", ctypes.POINTER(c_void_p)), ("y_rows", c_void_p), ("flags", u32)]


MOE_FORWARD_FUSED_DECODE = 1


NUM_STAGE_EVENTS = 6


# name -> (restype, argtypes)
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [i32]),
    "moe_route": (i32, [c_void_p, c_void_p, c_void_p, i32, i32, i32, i32, u32, c_void_p, c_void_p, c_void_p,
                        c_void_p]),
    "moe_permute_workspace_size": (size_t, [i32, i32, i32]),
    "moe_permute": (i32, [c_void_p, i32, i32, i32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, size_t,
                          c_void_p]),
    "moe_nvfp4_grouped_gemm": (i32, [i32, ctypes.POINTER(Experts), c_void_p, c_void_p, i32, c_void_p, i32,
                                     c_void_p, c_void_p]),
    "moe_combine": (i32, [c_void_p, c_void_p, c_void_p, c_void_p, i32, i32, i32, c_void_p, c_void_p]),
    "moe_nvfp4_forward_workspace_size": (size_t, [i32, i32, i32, i32, i32, i32]),
    "moe_nvfp4_forward": (i32, [ctypes.POINTER(Layer), c_void_p, i32, c_void_p, c_void_p, size_t,
                                ctypes.POINTER(ForwardAux), c_void_p]),
    "moe_validate_forward": (i32, [ctypes.POINTER(Layer), i32, size_t, ctypes.c_char_p]),
    "moe_gscale_from_quant_scale": (i32, [c_void_p, c_void_p, i32]),
    "moe_nvfp4_pack_tiles": (i32, [c_void_p, c_void_p, i32, i32, i32, c_void_p, c_void_p, c_void_p]),
    "moe_nvfp4_quantize": (i32, [c_void_p, i32, i32, i32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_mxfp4_pack_tiles": (i32, [c_void_p, c_void_p, i32, i32, i32, c_void_p, c_void_p, c_void_p]),
    "moe_mxfp4_quantize": (i32, [c_void_p, i32, i32, i32, c_void_p, c_void_p, c_void_p]),
    "moe_mxfp4_quantize_act": (i32, [c_void_p, i32, i32, c_void_p, c_void_p, c_void_p]),
    "moe_mxfp4_pack_tiles_a4": (i32, [c_void_p, c_void_p, i32, i32, i32, c_void_p, c_void_p, c_void_p]),
    "moe_mxfp4_w4a4_grouped_gemm": (i32, [i32, ctypes.POINTER(Experts), c_void_p, c_void_p, c_void_p, i32, c_void_p,
                                          i32, c_void_p, c_void_p]),
    "moe_mxfp4_w4a4_forward_workspace_size": (size_t, [i32, i32, i32, i32, i32, i32]),
    "moe_mxfp4_w4a4_validate_forward": (i32, [ctypes.POINTER(Layer), i32, size_t, ctypes.c_char_p]),
    "moe_mxfp4_w4a4_forward": (i32, [ctypes.POINTER(Layer), c_void_p, i32, c_void_p, c_void_p, size_t,
                                     ctypes.POINTER(ForwardAux), c_void_p]),
    "moe_nvfp4_quantize_act": (i32, [c_void_p, i32, i32, ctypes.c_float, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_nvfp4_w4a4_grouped_gemm": (i32, [i32, ctypes.POINTER(Experts), c_void_p, ctypes.c_float, c_void_p, i32,
                                          c_void_p, i32, c_void_p, c_void_p]),
    "moe_nvfp4_w4a4_forward_workspace_size": (size_t, [i32, i32, i32, i32, i32, i32]),
    "moe_nvfp4_w4a4_validate_forward": (i32, [ctypes.POINTER(Layer), i32, size_t, ctypes.c_float, ctypes.c_float,
                                              ctypes.c_char_p]),
    "moe_nvfp4_w4a4_forward": (i32, [ctypes.POINTER(Layer), c_void_p, i32, ctypes.c_float, ctypes.c_float, c_void_p,
                                     c_void_p, size_t, ctypes.POINTER(ForwardAux), c_void_p]),
    "moe_hbm_read_probe": (i32, [c_void_p, size_t, c_void_p, i32, c_void_p]),
    "moe_nvfp4_h16_bound": (i32, [ctypes.POINTER(Experts), c_void_p, c_void_p]),
    "moe_nvfp4_forward_noalloc": (i32, [ctypes.POINTER(Layer), c_void_p, i32, c_void_p, ctypes.POINTER(ForwardAux),
                                        c_void_p]),
}

NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES

# weight formats of an expert bank (moe_nvfp4_experts_t.format)
MOE_WEIGHT_NVFP4 = 0
MOE_WEIGHT_MXFP4 = 1
MOE_WEIGHT_MXFP4_A4 = 2
# bank layouts of the Python side: "mxfp4_a4" is MXFP4 in the W4A4 tile layout (the W4A4 layer)
FORMATS = {"nvfp4": MOE_WEIGHT_NVFP4, "mxfp4": MOE_WEIGHT_MXFP4, "mxfp4_a4": MOE_WEIGHT_MXFP4_A4}
SCALE_GROUP = {"nvfp4": 16, "mxfp4": 32, "mxfp4_a4": 32}
PACK_FN = {"nvfp4": "moe_nvfp4_pack_tiles", "mxfp4": "moe_mxfp4_pack_tiles", "mxfp4_a4": "moe_mxfp4_pack_tiles_a4"}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m nvfp4_weight_quantized_amd.build` "
                               "(there is no CPU fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)
