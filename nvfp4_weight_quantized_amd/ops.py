"""torch-facing wrappers of the C ABI: argument checks and marshalling only.

PyTorch supplies device memory and the current stream; every step of the layer runs in the
HIP kernels of libmoe_nvfp4.so.  There is no fallback path.
"""

from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

from . import _lib as L


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, ndim: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")


def _shape(t: torch.Tensor, name: str, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(ref: torch.Tensor, *named) -> None:
    for name, t in named:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name}: on {t.device}, expected {ref.device}")


# ----------------------------------------------------------------------------- weights

@dataclass
class NvFp4Experts:
    """A bank of 4-bit experts on the GPU, weights and scales in the MFMA tile layout.

    ``fmt`` "nvfp4": E4M3 scales per 16 elements along K plus fp32 global scales; "mxfp4": E8M0
    scales per 32 elements and no global scale (the gscale tensors are None); "mxfp4_a4": MXFP4 in
    the W4A4 tile layout, which makes a layer run the W4A4 path.  Shapes are those of
    the canonical tensors (include/moe_nvfp4.h); the bytes of each expert's tensors are permuted by
    ``pack_tiles``.  Use ``NvFp4Experts.from_canonical`` to build one from checkpoint-layout tensors.

    An NVFP4 bank on the GPU also carries ``h16_bound``, the largest Euclidean norm of its dequantized
    gate rows and of its up rows (``moe_nvfp4_h16_bound``), computed when the bank is made (or when
    its weight tensors are replaced); the layer hands it to the forward, which then holds h as fp16.
    After changing weight values in place, call ``refresh_h16_bound()``.
    """
    w13: torch.Tensor                    # uint8 [E, 2I, H/2]
    w13_scale: torch.Tensor              # uint8 [E, 2I, H/16] (nvfp4) or [E, 2I, H/32] (mxfp4)
    w13_gscale: Optional[torch.Tensor]   # float32 [E, 2] (nvfp4) or None
    w2: torch.Tensor                     # uint8 [E, H, I/2]
    w2_scale: torch.Tensor               # uint8 [E, H, I/16] or [E, H, I/32]
    w2_gscale: Optional[torch.Tensor]    # float32 [E] (nvfp4) or None
    fmt: str = "nvfp4"
    h16_bound: tuple = field(default=(0.0, 0.0), init=False, compare=False, repr=False)
    _h16_key: tuple = field(default=(), init=False, compare=False, repr=False)

    def __post_init__(self):
        self.refresh_h16_bound()

    def _tensors_key(self):
        return (id(self.w13), id(self.w13_scale), id(self.w13_gscale), self.fmt)

    def refresh_h16_bound(self) -> tuple:
        """(gate, up) weight-row norm bounds of an NVFP4 bank on the GPU, (0, 0) otherwise."""
        self._h16_key = self._tensors_key()
        self.h16_bound = (0.0, 0.0)
        if self.fmt != "nvfp4" or not isinstance(self.w13, torch.Tensor) or not self.w13.is_cuda:
            return self.h16_bound
        try:
            self.check()
        except (ValueError, TypeError):
            return self.h16_bound   # the layer's own check reports it
        bound = torch.zeros(2, dtype=torch.float32, device=self.w13.device)
        st = self.c_struct()
        L.check("moe_nvfp4_h16_bound", L.lib().moe_nvfp4_h16_bound(ctypes.byref(st), _ptr(bound),
                                                                   _stream(self.w13.device)))
        self.h16_bound = tuple(float(v) for v in bound.cpu().tolist())
        return self.h16_bound

    def current_h16_bound(self) -> tuple:
        """h16_bound, recomputed if the weight tensors were replaced since."""
        if self._h16_key != self._tensors_key():
            self.refresh_h16_bound()
        return self.h16_bound

    @property
    def num_experts(self) -> int:
        return self.w13.shape[0]

    @property
    def hidden(self) -> int:
        return self.w13.shape[2] * 2

    @property
    def inter(self) -> int:
        return self.w13.shape[1] // 2

    def check(self) -> None:
        if self.fmt not in L.FORMATS:
            raise ValueError(f"unknown weight format {self.fmt!r}")
        e, h, i, g = self.num_experts, self.hidden, self.inter, L.SCALE_GROUP[self.fmt]
        specs = [("w13", self.w13, torch.uint8, (e, 2 * i, h // 2)),
                 ("w13_scale", self.w13_scale, torch.uint8, (e, 2 * i, h // g)),
                 ("w2", self.w2, torch.uint8, (e, h, i // 2)),
                 ("w2_scale", self.w2_scale, torch.uint8, (e, h, i // g))]
        if self.fmt == "nvfp4":
            specs += [("w13_gscale", self.w13_gscale, torch.float32, (e, 2)),
                      ("w2_gscale", self.w2_gscale, torch.float32, (e,))]
        for name, t, dt, shape in specs:
            if t is None:
                raise ValueError(f"{name} is required for {self.fmt}")
            _need(t, name, dt)
            if tuple(t.shape) != shape:
                raise ValueError(f"{name}: expected shape {shape}, got {tuple(t.shape)}")

    @classmethod
    def from_canonical(cls, w13, w13_scale, w13_gscale, w2, w2_scale, w2_gscale, fmt: str = "nvfp4") -> "NvFp4Experts":
        """Repack canonical-layout device tensors into the tile layout (new tensors)."""
        t13, s13 = pack_tiles(w13, w13_scale, fmt=fmt)
        t2, s2 = pack_tiles(w2, w2_scale, fmt=fmt)
        return cls(t13, s13, w13_gscale, t2, s2, w2_gscale, fmt)

    def c_struct(self) -> L.Experts:
        def addr(t):
            return t.data_ptr() if t is not None else None
        return L.Experts(self.num_experts, self.hidden, self.inter, L.FORMATS[self.fmt],
                         self.w13.data_ptr(), self.w13_scale.data_ptr(), addr(self.w13_gscale),
                         self.w2.data_ptr(), self.w2_scale.data_ptr(), addr(self.w2_gscale))


@dataclass
class NvFp4MoELayer:
    """Router + routed experts + optional shared expert, all on one GPU."""
    w_router: torch.Tensor                 # bf16 [E, H]
    router_bias: Optional[torch.Tensor]    # float32 [E] or None
    routed: NvFp4Experts
    shared: Optional[NvFp4Experts]
    top_k: int
    # hold h as fp16 on the 128-row path (with the banks' weight-row norm bounds; NVFP4 only)
    fp16_h: bool = True

    @property
    def hidden(self) -> int:
        return self.routed.hidden

    @property
    def num_experts(self) -> int:
        return self.routed.num_experts

    @property
    def is_w4a4(self) -> bool:
        """True for banks in the W4A4 layout: forward() then quantizes the activations too."""
        return self.routed.fmt == "mxfp4_a4"

    def check(self) -> None:
        """Shapes, dtypes and devices of every tensor of the layer (raises before any launch)."""
        self.routed.check()
        e, h = self.routed.num_experts, self.routed.hidden
        _need(self.w_router, "w_router", torch.bfloat16, 2)
        _shape(self.w_router, "w_router", (e, h))
        if self.router_bias is not None:
            _need(self.router_bias, "router_bias", torch.float32, 1)
            _shape(self.router_bias, "router_bias", (e,))
        if self.shared is not None:
            self.shared.check()
            if self.shared.num_experts != 1 or self.shared.hidden != h:
                raise ValueError("shared expert bank: expected one expert of the routed hidden size")
            if self.shared.fmt != self.routed.fmt:
                raise ValueError("routed and shared banks must share one weight format")
        if not 1 <= self.top_k <= e:
            raise ValueError(f"top_k {self.top_k} outside [1, {e}]")
        b = self.routed
        _same_device(self.w_router, ("router_bias", self.router_bias), ("routed.w13", b.w13),
                     ("routed.w2", b.w2), ("shared.w13", self.shared.w13 if self.shared is not None else None))

    def _key(self):
        banks = [b for b in (self.routed, self.shared) if b is not None]
        return (id(self.w_router), id(self.router_bias), self.top_k, self.fp16_h,
                *[(id(t), b.fmt) for b in banks for t in (b.w13, b.w13_scale, b.w13_gscale, b.w2, b.w2_scale,
                                                          b.w2_gscale)],
                *[b.h16_bound for b in banks])

    def checked_struct(self) -> L.Layer:
        """check() + c_struct(), cached while the layer holds the same tensors."""
        key = self._key()
        cached = self.__dict__.get("_checked")
        if cached is None or cached[0] != key:
            self.check()
            cached = (key, self.c_struct())
            self.__dict__["_checked"] = cached
        return cached[1]

    def h16_norm(self) -> tuple:
        """The (gate, up) bounds the forward gets: the larger of the banks', (0, 0) when off."""
        if not self.fp16_h:
            return (0.0, 0.0)
        banks = [b for b in (self.routed, self.shared) if b is not None]
        bounds = [b.current_h16_bound() for b in banks]
        if any(not (b[0] > 0.0 and b[1] > 0.0 and math.isfinite(b[0]) and math.isfinite(b[1])) for b in bounds):
            return (0.0, 0.0)
        return (max(b[0] for b in bounds), max(b[1] for b in bounds))

    def c_struct(self) -> L.Layer:
        empty = L.Experts()
        norm = self.h16_norm()
        return L.Layer(self.hidden, self.num_experts, self.top_k, self.w_router.data_ptr(),
                       self.router_bias.data_ptr() if self.router_bias is not None else None,
                       self.routed.c_struct(), self.shared.c_struct() if self.shared is not None else empty,
                       (ctypes.c_float * 2)(*norm))

    @classmethod
    def from_tensors(cls, tensors: dict, top_k: int, global_scale_convention: str = "modelopt",
                     device="cuda", weight_format: str = "nvfp4") -> "NvFp4MoELayer":
        """Build a layer from a checkpoint-like dict.

        Keys: router.weight, router.bias (optional), experts.{w13, w13_scale, w13_global_scale,
        w2, w2_scale, w2_global_scale} and the same under shared_expert.* (optional).
        Global scales in the "compressed_tensors" convention are quant scales (448*6)/amax and are
        inverted on load; "modelopt" global scales are dequant scales and are used as stored.
        With ``weight_format="mxfp4"`` the scales are E8M0 per 32 elements and there are no
        global-scale keys.  Any activation-scale key (``*input_scale*``) is ignored: the layer is
        weight-only.
        """
        if global_scale_convention not in ("modelopt", "compressed_tensors"):
            raise ValueError(global_scale_convention)
        if weight_format not in L.FORMATS:
            raise ValueError(weight_format)

        def dev(t, dtype):
            return torch.as_tensor(t).to(device=device, dtype=dtype).contiguous()

        def gscale(t):
            a = torch.as_tensor(t).detach().to("cpu", torch.float32).contiguous()
            if global_scale_convention == "compressed_tensors":
                a = torch.from_numpy(gscale_from_quant_scale(a.numpy()))
            return a.to(device)

        def bank(prefix):
            if prefix + "w13" not in tensors:
                return None
            nv = weight_format == "nvfp4"
            return NvFp4Experts.from_canonical(
                dev(tensors[prefix + "w13"], torch.uint8), dev(tensors[prefix + "w13_scale"], torch.uint8),
                gscale(tensors[prefix + "w13_global_scale"]) if nv else None,
                dev(tensors[prefix + "w2"], torch.uint8), dev(tensors[prefix + "w2_scale"], torch.uint8),
                gscale(tensors[prefix + "w2_global_scale"]) if nv else None, fmt=weight_format)

        routed = bank("experts.")
        shared = bank("shared_expert.")
        bias = tensors.get("router.bias")
        layer = cls(dev(tensors["router.weight"], torch.bfloat16),
                    dev(bias, torch.float32) if bias is not None else None, routed, shared, top_k)
        routed.check()
        if shared is not None:
            shared.check()
        return layer


# ----------------------------------------------------------------------------- stages

def route(x: torch.Tensor, w_router: torch.Tensor, router_bias: Optional[torch.Tensor], k: int):
    """S1+S2: (logits fp32 [T, E], topk_ids int32 [T, k], topk_w fp32 [T, k])."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w_router, "w_router", torch.bfloat16, 2)
    t, h = x.shape
    e = w_router.shape[0]
    _shape(w_router, "w_router", (e, h))
    if router_bias is not None:
        _need(router_bias, "router_bias", torch.float32, 1)
        _shape(router_bias, "router_bias", (e,))
    _same_device(x, ("w_router", w_router), ("router_bias", router_bias))
    logits = torch.empty(t, e, dtype=torch.float32, device=x.device)
    ids = torch.empty(t, k, dtype=torch.int32, device=x.device)
    w = torch.empty(t, k, dtype=torch.float32, device=x.device)
    L.check("moe_route", L.lib().moe_route(_ptr(x), _ptr(w_router), _ptr(router_bias), t, h, e, k, 0,
                                           _ptr(logits), _ptr(ids), _ptr(w), _stream(x.device)))
    return logits, ids, w


def route_from_logits(logits: torch.Tensor, k: int):
    """S2 only, on given fp32 logits [T, E]: (topk_ids, topk_w)."""
    _need(logits, "logits", torch.float32, 2)
    t, e = logits.shape
    ids = torch.empty(t, k, dtype=torch.int32, device=logits.device)
    w = torch.empty(t, k, dtype=torch.float32, device=logits.device)
    L.check("moe_route", L.lib().moe_route(None, None, None, t, 0, e, k, L.MOE_ROUTE_LOGITS_GIVEN, _ptr(logits),
                                           _ptr(ids), _ptr(w), _stream(logits.device)))
    return ids, w


def permute(topk_ids: torch.Tensor, num_experts: int):
    """S3: (counts [E], offsets [E+1], sorted_slot [S], slot_to_row [S]), all int32."""
    _need(topk_ids, "topk_ids", torch.int32, 2)
    t, k = topk_ids.shape
    if not 1 <= num_experts <= 1024:
        raise ValueError(f"num_experts {num_experts} outside [1, 1024]")
    dev = topk_ids.device
    counts = torch.empty(num_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    sorted_slot = torch.empty(t * k, dtype=torch.int32, device=dev)
    slot_to_row = torch.empty(t * k, dtype=torch.int32, device=dev)
    ws_bytes = L.lib().moe_permute_workspace_size(t, k, num_experts)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    L.check("moe_permute", L.lib().moe_permute(_ptr(topk_ids), t, k, num_experts, _ptr(counts), _ptr(offsets),
                                               _ptr(sorted_slot), _ptr(slot_to_row), _ptr(ws), ws_bytes,
                                               _stream(dev)))
    return counts, offsets, sorted_slot, slot_to_row


def grouped_gemm(stage: int, experts: NvFp4Experts, a: torch.Tensor, expert_offsets: torch.Tensor, m_total: int,
                 row_index: Optional[torch.Tensor] = None, row_divisor: int = 1) -> torch.Tensor:
    """S4 (stage 0: gate/up + SiLU*up -> [M, I]) or S5 (stage 1: down -> [M, H]), bf16."""
    if experts.fmt == "mxfp4_a4":
        raise ValueError("a bank in the W4A4 layout runs through grouped_gemm_a4")
    experts.check()
    if stage not in (L.MOE_GEMM_GATE_UP, L.MOE_GEMM_DOWN):
        raise ValueError(f"unknown stage {stage}")
    _need(a, "a", torch.bfloat16, 2)
    _need(expert_offsets, "expert_offsets", torch.int32, 1)
    _shape(expert_offsets, "expert_offsets", (experts.num_experts + 1,))
    kdim = experts.hidden if stage == L.MOE_GEMM_GATE_UP else experts.inter
    if a.shape[1] != kdim:
        raise ValueError(f"a: expected {kdim} columns, got {a.shape[1]}")
    if row_index is not None:
        _need(row_index, "row_index", torch.int32, 1)
        if stage != L.MOE_GEMM_GATE_UP:
            raise ValueError("row_index applies to the gate/up stage only")
        if row_index.numel() < m_total:
            raise ValueError(f"row_index: {row_index.numel()} entries for {m_total} rows")
    elif a.shape[0] < m_total:
        raise ValueError(f"a: {a.shape[0]} rows for {m_total} output rows")
    _same_device(a, ("expert_offsets", expert_offsets), ("row_index", row_index), ("experts.w13", experts.w13))
    n = experts.inter if stage == L.MOE_GEMM_GATE_UP else experts.hidden
    out = torch.empty(m_total, n, dtype=torch.bfloat16, device=a.device)
    st = experts.c_struct()
    L.check("moe_nvfp4_grouped_gemm",
            L.lib().moe_nvfp4_grouped_gemm(stage, ctypes.byref(st), _ptr(a), _ptr(row_index), row_divisor,
                                           _ptr(expert_offsets), m_total, _ptr(out), _stream(a.device)))
    return out


def quantize_act(a: torch.Tensor, packed: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None):
    """MXFP4 quantization of bf16 rows [M, K] -> (codes uint8 [M, K/2], E8M0 scales uint8 [M, K/32])."""
    _need(a, "a", torch.bfloat16, 2)
    m, k = a.shape
    if packed is None:
        packed = torch.empty(m, k // 2, dtype=torch.uint8, device=a.device)
    if scales is None:
        scales = torch.empty(m, k // 32, dtype=torch.uint8, device=a.device)
    _need(packed, "packed", torch.uint8)
    _need(scales, "scales", torch.uint8)
    L.check("moe_mxfp4_quantize_act", L.lib().moe_mxfp4_quantize_act(_ptr(a), m, k, _ptr(packed), _ptr(scales),
                                                                     _stream(a.device)))
    return packed, scales


def _act_gscale(d, name: str) -> float:
    d = float(np.float32(d))
    if not (math.isfinite(d) and d > 0.0):
        raise ValueError(f"{name}: an activation global scale must be finite and positive, got {d!r}")
    return d


def quantize_act_nv(a: torch.Tensor, gscale: float, packed: bool = True, scales: bool = True,
                    values: bool = True, in_place: bool = False):
    """NVFP4 quantization of bf16 rows [M, K] with dequant global scale ``gscale``.

    Returns (codes uint8 [M, K/2] or None, E4M3 scales uint8 [M, K/16] or None, values bf16 [M, K] or
    None): ``values`` are e2m1(code) * e4m3(scale) without the global scale, the rows the NVFP4 W4A4
    GEMMs take.  ``in_place``: the values overwrite ``a``.
    """
    _need(a, "a", torch.bfloat16, 2)
    d = _act_gscale(gscale, "gscale")
    m, k = a.shape
    if k % 16:
        raise ValueError(f"a: {k} columns, not a multiple of 16")
    pk = torch.empty(m, k // 2, dtype=torch.uint8, device=a.device) if packed else None
    sc = torch.empty(m, k // 16, dtype=torch.uint8, device=a.device) if scales else None
    vals = (a if in_place else torch.empty_like(a)) if (values or in_place) else None
    L.check("moe_nvfp4_quantize_act", L.lib().moe_nvfp4_quantize_act(_ptr(a), m, k, d, _ptr(pk), _ptr(sc), _ptr(vals),
                                                                     _stream(a.device)))
    return pk, sc, vals


def grouped_gemm_w4a4(stage: int, experts: NvFp4Experts, a_values: torch.Tensor, act_gscale: float,
                      expert_offsets: torch.Tensor, m_total: int, row_index: Optional[torch.Tensor] = None,
                      row_divisor: int = 1) -> torch.Tensor:
    """NVFP4 W4A4 S4/S5: ``a_values`` from ``quantize_act_nv`` with dequant global scale ``act_gscale``,
    an "nvfp4" bank; shapes and checks as ``grouped_gemm``, bf16 out."""
    if experts.fmt != "nvfp4":
        raise ValueError("the NVFP4 W4A4 GEMM needs an nvfp4 bank")
    d = _act_gscale(act_gscale, "act_gscale")
    experts.check()
    if stage not in (L.MOE_GEMM_GATE_UP, L.MOE_GEMM_DOWN):
        raise ValueError(f"unknown stage {stage}")
    _need(a_values, "a_values", torch.bfloat16, 2)
    _need(expert_offsets, "expert_offsets", torch.int32, 1)
    _shape(expert_offsets, "expert_offsets", (experts.num_experts + 1,))
    kdim = experts.hidden if stage == L.MOE_GEMM_GATE_UP else experts.inter
    if a_values.shape[1] != kdim:
        raise ValueError(f"a_values: expected {kdim} columns, got {a_values.shape[1]}")
    if row_index is not None:
        _need(row_index, "row_index", torch.int32, 1)
        if stage != L.MOE_GEMM_GATE_UP:
            raise ValueError("row_index applies to the gate/up stage only")
        if row_index.numel() < m_total:
            raise ValueError(f"row_index: {row_index.numel()} entries for {m_total} rows")
    elif a_values.shape[0] < m_total:
        raise ValueError(f"a_values: {a_values.shape[0]} rows for {m_total} output rows")
    _same_device(a_values, ("expert_offsets", expert_offsets), ("row_index", row_index), ("experts.w13", experts.w13))
    n = experts.inter if stage == L.MOE_GEMM_GATE_UP else experts.hidden
    out = torch.empty(m_total, n, dtype=torch.bfloat16, device=a_values.device)
    st = experts.c_struct()
    L.check("moe_nvfp4_w4a4_grouped_gemm",
            L.lib().moe_nvfp4_w4a4_grouped_gemm(stage, ctypes.byref(st), _ptr(a_values), d, _ptr(row_index),
                                                row_divisor, _ptr(expert_offsets), m_total, _ptr(out),
                                                _stream(a_values.device)))
    return out


def grouped_gemm_a4(stage: int, experts: NvFp4Experts, a_codes: torch.Tensor, a_scales: torch.Tensor,
                    expert_offsets: torch.Tensor, m_total: int, row_index: Optional[torch.Tensor] = None,
                    row_divisor: int = 1) -> torch.Tensor:
    """W4A4 S4/S5 on MXFP4 activations (from ``quantize_act``) and an "mxfp4_a4" bank, bf16 out."""
    if experts.fmt != "mxfp4_a4":
        raise ValueError("the W4A4 GEMM needs a bank in the mxfp4_a4 layout")
    experts.check()
    _need(a_codes, "a_codes", torch.uint8, 2)
    _need(a_scales, "a_scales", torch.uint8, 2)
    _need(expert_offsets, "expert_offsets", torch.int32, 1)
    if row_index is not None:
        _need(row_index, "row_index", torch.int32, 1)
    n = experts.inter if stage == L.MOE_GEMM_GATE_UP else experts.hidden
    out = torch.empty(m_total, n, dtype=torch.bfloat16, device=a_codes.device)
    st = experts.c_struct()
    L.check("moe_mxfp4_w4a4_grouped_gemm",
            L.lib().moe_mxfp4_w4a4_grouped_gemm(stage, ctypes.byref(st), _ptr(a_codes), _ptr(a_scales),
                                                _ptr(row_index), row_divisor, _ptr(expert_offsets), m_total,
                                                _ptr(out), _stream(a_codes.device)))
    return out


def combine(y_rows: torch.Tensor, slot_to_row: torch.Tensor, topk_w: torch.Tensor,
            y_shared: Optional[torch.Tensor] = None) -> torch.Tensor:
    """S6: out [T, H] bf16."""
    _need(y_rows, "y_rows", torch.bfloat16, 2)
    _need(slot_to_row, "slot_to_row", torch.int32, 1)
    _need(topk_w, "topk_w", torch.float32, 2)
    t, k = topk_w.shape
    h = y_rows.shape[1]
    _shape(slot_to_row, "slot_to_row", (t * k,))
    if y_shared is not None:
        _need(y_shared, "y_shared", torch.bfloat16, 2)
        _shape(y_shared, "y_shared", (t, h))
    _same_device(y_rows, ("slot_to_row", slot_to_row), ("topk_w", topk_w), ("y_shared", y_shared))
    out = torch.empty(t, h, dtype=torch.bfloat16, device=y_rows.device)
    L.check("moe_combine", L.lib().moe_combine(_ptr(y_rows), _ptr(slot_to_row), _ptr(topk_w), _ptr(y_shared), t, k,
                                               h, _ptr(out), _stream(y_rows.device)))
    return out


# ----------------------------------------------------------------------------- whole layer

def forward_workspace_size(T: int, H: int, I: int, I_shared: int, E: int, k: int, w4a4: bool = False,
                           nvfp4_a4: bool = False) -> int:
    """Workspace bytes of the W4A16 forward, the MXFP4 W4A4 one (``w4a4``) or the NVFP4 W4A4 one."""
    if nvfp4_a4:
        fn = L.lib().moe_nvfp4_w4a4_forward_workspace_size
    else:
        fn = L.lib().moe_mxfp4_w4a4_forward_workspace_size if w4a4 else L.lib().moe_nvfp4_forward_workspace_size
    return int(fn(T, H, I, I_shared, E, k))


_POOL = {}


def workspace_for(layer: NvFp4MoELayer, T: int, device, nvfp4_a4: bool = False) -> torch.Tensor:
    """One module-level workspace per device, grown on demand and shared by every layer."""
    i_sh = layer.shared.inter if layer.shared is not None else 0
    need = forward_workspace_size(T, layer.hidden, layer.routed.inter, i_sh, layer.num_experts, layer.top_k,
                                  layer.is_w4a4, nvfp4_a4)
    dev = torch.device(device)
    cur = _POOL.get(dev)
    if cur is None or cur.numel() < need:
        cur = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        _POOL[dev] = cur
    return cur


def forward(layer: NvFp4MoELayer, x: torch.Tensor, workspace: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, return_aux: bool = False, stage_events=None,
            return_rows: bool = False, fused_decode: bool = False, act_gscales=None):
    """The whole layer on x [T, H] bf16 -> [T, H] bf16 (and, if asked, logits/ids/weights/counts).

    Runs moe_nvfp4_forward, or moe_mxfp4_w4a4_forward when the layer's banks are "mxfp4_a4", or
    moe_nvfp4_w4a4_forward when ``act_gscales`` = (d_x, d_h) is given (NVFP4 banks; the dequant
    global scales of the gate/up and down activations, W4A4 in NVFP4).
    ``return_rows`` (with ``return_aux``): the aux dict also holds "y_rows", the expert outputs the
    combine reads (bf16 [T*k + T_shared, H], routed rows in expert-sorted order, then the shared
    expert's row of every token).
    ``fused_decode``: run the two-launch fused decode path where it applies (few tokens).

    ``stage_events``: optional sequence of 6 raw hipEvent_t handles (ints or None) recorded at the
    stage boundaries (before S1, after S1, after S2+S3, after S4, S5, S6) on the current stream.
    """
    _need(x, "x", torch.bfloat16, 2)
    st = layer.checked_struct()
    t = x.shape[0]
    if x.shape[1] != layer.hidden:
        raise ValueError(f"x: expected {layer.hidden} columns, got {x.shape[1]}")
    _same_device(x, ("w_router", layer.w_router))
    a4 = None
    if act_gscales is not None:
        if layer.routed.fmt != "nvfp4":
            raise ValueError("act_gscales (NVFP4 W4A4) needs nvfp4 banks")
        if len(act_gscales) != 2:
            raise ValueError("act_gscales: (d_x, d_h) expected")
        a4 = (_act_gscale(act_gscales[0], "act_gscales[0]"), _act_gscale(act_gscales[1], "act_gscales[1]"))
    if workspace is None:
        workspace = workspace_for(layer, t, x.device, nvfp4_a4=a4 is not None)
    _need(workspace, "workspace", torch.uint8)
    _same_device(x, ("workspace", workspace))
    if out is None:
        out = torch.empty_like(x)
    else:
        _need(out, "out", torch.bfloat16, 2)
        _shape(out, "out", x.shape)
        _same_device(x, ("out", out))
    aux = None
    aux_t = None
    if return_aux or stage_events is not None or fused_decode:
        aux = L.ForwardAux()
        aux.flags = L.MOE_FORWARD_FUSED_DECODE if fused_decode else 0
    if return_aux:
        e, k = layer.num_experts, layer.top_k
        aux_t = dict(logits=torch.empty(t, e, dtype=torch.float32, device=x.device),
                     topk_ids=torch.empty(t, k, dtype=torch.int32, device=x.device),
                     topk_w=torch.empty(t, k, dtype=torch.float32, device=x.device),
                     expert_counts=torch.empty(e, dtype=torch.int32, device=x.device))
        aux.logits, aux.topk_ids, aux.topk_w, aux.expert_counts = (v.data_ptr() for v in aux_t.values())
        if return_rows:
            rows = t * k + (t if layer.shared is not None else 0)
            aux_t["y_rows"] = torch.empty(rows, layer.hidden, dtype=torch.bfloat16, device=x.device)
            aux.y_rows = aux_t["y_rows"].data_ptr()
    if stage_events is not None:
        if len(stage_events) != L.NUM_STAGE_EVENTS:
            raise ValueError(f"stage_events: {L.NUM_STAGE_EVENTS} entries expected")
        arr = (ctypes.c_void_p * L.NUM_STAGE_EVENTS)(*stage_events)
        aux.stage_events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    aux_p = ctypes.byref(aux) if aux is not None else None
    if a4 is not None:
        L.check("moe_nvfp4_w4a4_forward",
                L.lib().moe_nvfp4_w4a4_forward(ctypes.byref(st), _ptr(x), t, a4[0], a4[1], _ptr(out), _ptr(workspace),
                                               workspace.numel(), aux_p, _stream(x.device)))
        return (out, aux_t) if return_aux else out
    fn = "moe_mxfp4_w4a4_forward" if layer.is_w4a4 else "moe_nvfp4_forward"
    L.check(fn, getattr(L.lib(), fn)(ctypes.byref(st), _ptr(x), t, _ptr(out), _ptr(workspace), workspace.numel(),
                                     aux_p, _stream(x.device)))
    return (out, aux_t) if return_aux else out


def validate_forward(layer_struct: L.Layer, T: int, workspace_bytes: int, arch: Optional[str] = "gfx950",
                     w4a4: bool = False, act_gscales=None) -> int:
    """Pure-host validation status (needs no GPU when ``arch`` is given).  ``act_gscales`` = (d_x, d_h):
    the NVFP4 W4A4 forward's validation (the scales are passed through unchecked)."""
    a = arch.encode() if arch is not None else None
    if act_gscales is not None:
        return int(L.lib().moe_nvfp4_w4a4_validate_forward(ctypes.byref(layer_struct), T, workspace_bytes,
                                                            float(act_gscales[0]), float(act_gscales[1]), a))
    fn = L.lib().moe_mxfp4_w4a4_validate_forward if w4a4 else L.lib().moe_validate_forward
    return int(fn(ctypes.byref(layer_struct), T, workspace_bytes, a))


# ----------------------------------------------------------------------------- weight preparation

def gscale_from_quant_scale(q) -> np.ndarray:
    """compressed-tensors quant scales -> dequant scales (host, fp32)."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float32))
    d = np.empty_like(q)
    L.check("moe_gscale_from_quant_scale",
            L.lib().moe_gscale_from_quant_scale(q.ctypes.data_as(ctypes.c_void_p), d.ctypes.data_as(ctypes.c_void_p),
                                                q.size))
    return d


def pack_tiles(packed: torch.Tensor, scales: torch.Tensor, tiled: Optional[torch.Tensor] = None,
               tiled_scales: Optional[torch.Tensor] = None, fmt: str = "nvfp4"):
    """Canonical [..., rows, cols/2] nibbles + [..., rows, cols/16] (nvfp4) or [..., rows, cols/32]
    (mxfp4, mxfp4_a4) scales -> the MFMA tile layout of ``fmt`` (same shapes)."""
    _need(packed, "packed", torch.uint8)
    _need(scales, "scales", torch.uint8)
    rows, half = packed.shape[-2], packed.shape[-1]
    cols = half * 2
    nt = int(np.prod(packed.shape[:-2])) if packed.dim() > 2 else 1
    if tuple(scales.shape) != tuple(packed.shape[:-1]) + (cols // L.SCALE_GROUP[fmt],):
        raise ValueError("scales shape does not match packed")
    tiled = torch.empty_like(packed) if tiled is None else tiled
    tiled_scales = torch.empty_like(scales) if tiled_scales is None else tiled_scales
    fn = L.PACK_FN[fmt]
    L.check(fn, getattr(L.lib(), fn)(_ptr(packed), _ptr(scales), nt, rows, cols, _ptr(tiled), _ptr(tiled_scales),
                                     _stream(packed.device)))
    return tiled, tiled_scales


def quantize(w: torch.Tensor, gscale: torch.Tensor, packed: Optional[torch.Tensor] = None,
             scales: Optional[torch.Tensor] = None):
    """On-device NVFP4 quantization of fp32 [..., rows, cols] with one dequant scale per leading index."""
    _need(w, "w", torch.float32)
    _need(gscale, "gscale", torch.float32)
    rows, cols = w.shape[-2], w.shape[-1]
    nt = int(np.prod(w.shape[:-2])) if w.dim() > 2 else 1
    if gscale.numel() != nt:
        raise ValueError("one global scale per tensor expected")
    lead = tuple(w.shape[:-2])
    if packed is None:
        packed = torch.empty(*lead, rows, cols // 2, dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(*lead, rows, cols // 16, dtype=torch.uint8, device=w.device)
    _need(packed, "packed", torch.uint8)
    _need(scales, "scales", torch.uint8)
    L.check("moe_nvfp4_quantize", L.lib().moe_nvfp4_quantize(_ptr(w), nt, rows, cols, _ptr(gscale), _ptr(packed),
                                                             _ptr(scales), _stream(w.device)))
    return packed, scales


def quantize_mx(w: torch.Tensor, packed: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None):
    """On-device MXFP4 quantization of fp32 [..., rows, cols] (E8M0 scale per 32 elements)."""
    _need(w, "w", torch.float32)
    rows, cols = w.shape[-2], w.shape[-1]
    nt = int(np.prod(w.shape[:-2])) if w.dim() > 2 else 1
    lead = tuple(w.shape[:-2])
    if packed is None:
        packed = torch.empty(*lead, rows, cols // 2, dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(*lead, rows, cols // 32, dtype=torch.uint8, device=w.device)
    _need(packed, "packed", torch.uint8)
    _need(scales, "scales", torch.uint8)
    L.check("moe_mxfp4_quantize", L.lib().moe_mxfp4_quantize(_ptr(w), nt, rows, cols, _ptr(packed), _ptr(scales),
                                                             _stream(w.device)))
    return packed, scales


def forward_noalloc(layer: NvFp4MoELayer, x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole layer through moe_nvfp4_forward_noalloc: no workspace argument (the library's own
    device array of ``_lib.NOALLOC_SCRATCH_BYTES``), for callers that cannot allocate.  Calls that
    overlap in time on one GPU race."""
    _need(x, "x", torch.bfloat16, 2)
    st = layer.checked_struct()
    if layer.is_w4a4:
        raise ValueError("the allocation-free entry point runs the W4A16 layer")
    if x.shape[1] != layer.hidden:
        raise ValueError(f"x: expected {layer.hidden} columns, got {x.shape[1]}")
    _same_device(x, ("w_router", layer.w_router))
    if out is None:
        out = torch.empty_like(x)
    else:
        _need(out, "out", torch.bfloat16, 2)
        _shape(out, "out", x.shape)
        _same_device(x, ("out", out))
    L.check("moe_nvfp4_forward_noalloc",
            L.lib().moe_nvfp4_forward_noalloc(ctypes.byref(st), _ptr(x), x.shape[0], _ptr(out), None,
                                              _stream(x.device)))
    return out
