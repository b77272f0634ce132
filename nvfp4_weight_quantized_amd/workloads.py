"""Synthetic NVFP4 (or MXFP4) MoE layers on the GPU: seeded fp32 weights quantized by the
library's own on-device quantizers (moe_nvfp4_quantize / moe_mxfp4_quantize), NVFP4 global scales
in the workload's checkpoint convention and converted on load like a real checkpoint."""

from __future__ import annotations

import torch

from . import ops, synth


def _dequant_scales(amax, convention: str):
    gs = synth.checkpoint_global_scales(amax, convention)
    if convention == "compressed_tensors":
        return ops.gscale_from_quant_scale(gs)
    return gs


def build_bank_mx(wl: synth.Workload, bank: str, device="cuda", fmt: str = "mxfp4") -> ops.NvFp4Experts:
    """The same seeded fp32 experts quantized to MXFP4 (E8M0 scales per 32, no global scale), in the
    tile layout of ``fmt`` ("mxfp4": W4A16 kernels, "mxfp4_a4": W4A4 kernels)."""
    count = wl.E if bank == "routed" else 1
    inter = wl.I if bank == "routed" else wl.I_shared
    h = wl.H
    dev = torch.device(device)
    w13 = torch.empty(count, 2 * inter, h // 2, dtype=torch.uint8, device=dev)
    w13_s = torch.empty(count, 2 * inter, h // 32, dtype=torch.uint8, device=dev)
    w2 = torch.empty(count, h, inter // 2, dtype=torch.uint8, device=dev)
    w2_s = torch.empty(count, h, inter // 32, dtype=torch.uint8, device=dev)
    c13 = torch.empty(2 * inter, h // 2, dtype=torch.uint8, device=dev)
    c13_s = torch.empty(2 * inter, h // 32, dtype=torch.uint8, device=dev)
    c2 = torch.empty(h, inter // 2, dtype=torch.uint8, device=dev)
    c2_s = torch.empty(h, inter // 32, dtype=torch.uint8, device=dev)
    for e in range(count):
        f13, f2 = synth.expert_fp32(wl, bank, e, dev)
        ops.quantize_mx(f13, packed=c13, scales=c13_s)
        ops.quantize_mx(f2, packed=c2, scales=c2_s)
        ops.pack_tiles(c13, c13_s, tiled=w13[e], tiled_scales=w13_s[e], fmt=fmt)
        ops.pack_tiles(c2, c2_s, tiled=w2[e], tiled_scales=w2_s[e], fmt=fmt)
        del f13, f2
    return ops.NvFp4Experts(w13, w13_s, None, w2, w2_s, None, fmt=fmt)


def build_bank(wl: synth.Workload, bank: str, device="cuda", fmt: str = "nvfp4") -> ops.NvFp4Experts:
    """Quantize every expert of a bank ("routed": E experts of width I; "shared": 1 of width I_shared)
    on the GPU and repack it into the MFMA tile layout."""
    if fmt in ("mxfp4", "mxfp4_a4"):
        return build_bank_mx(wl, bank, device, fmt)
    count = wl.E if bank == "routed" else 1
    inter = wl.I if bank == "routed" else wl.I_shared
    h = wl.H
    dev = torch.device(device)
    w13 = torch.empty(count, 2 * inter, h // 2, dtype=torch.uint8, device=dev)
    w13_s = torch.empty(count, 2 * inter, h // 16, dtype=torch.uint8, device=dev)
    w2 = torch.empty(count, h, inter // 2, dtype=torch.uint8, device=dev)
    w2_s = torch.empty(count, h, inter // 16, dtype=torch.uint8, device=dev)
    gs13 = torch.empty(count, 2, dtype=torch.float32)
    gs2 = torch.empty(count, dtype=torch.float32)
    c13 = torch.empty(2 * inter, h // 2, dtype=torch.uint8, device=dev)      # canonical staging
    c13_s = torch.empty(2 * inter, h // 16, dtype=torch.uint8, device=dev)
    c2 = torch.empty(h, inter // 2, dtype=torch.uint8, device=dev)
    c2_s = torch.empty(h, inter // 16, dtype=torch.uint8, device=dev)
    for e in range(count):
        f13, f2 = synth.expert_fp32(wl, bank, e, dev)
        d = _dequant_scales(synth.expert_amax(f13, f2), wl.gscale_convention)
        d_dev = torch.from_numpy(d).to(dev)
        ops.quantize(f13.view(2, inter, h), d_dev[0:2], packed=c13.view(2, inter, h // 2),
                     scales=c13_s.view(2, inter, h // 16))
        ops.quantize(f2, d_dev[2:3], packed=c2, scales=c2_s)
        ops.pack_tiles(c13, c13_s, tiled=w13[e], tiled_scales=w13_s[e])
        ops.pack_tiles(c2, c2_s, tiled=w2[e], tiled_scales=w2_s[e])
        gs13[e] = torch.from_numpy(d[0:2])
        gs2[e] = float(d[2])
        del f13, f2
    return ops.NvFp4Experts(w13, w13_s, gs13.to(dev), w2, w2_s, gs2.to(dev))


def build_layer(wl: synth.Workload, device="cuda", fmt: str = "nvfp4") -> ops.NvFp4MoELayer:
    bias = synth.router_bias(wl)
    return ops.NvFp4MoELayer(
        w_router=synth.router_weight(wl, device).contiguous(),
        router_bias=torch.from_numpy(bias).to(device) if bias is not None else None,
        routed=build_bank(wl, "routed", device, fmt),
        shared=build_bank(wl, "shared", device, fmt) if wl.I_shared > 0 else None,
        top_k=wl.k)
