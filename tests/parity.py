"""Parity helpers shared by the GPU tests: oracle layers -> GPU tensors, and the tolerance checks.

Tolerances (fixed by the layer's specification of "matching"):
  * router logits: |gpu - exact| <= H * 2^-24 * sum_h |x_h * w_h| + 2^-24 * |logit| (fp32 recursive
    summation bound plus the rounding of the bias add);
  * top-k ids: bit-exact against the oracle's selection applied to the GPU's own fp32 logits;
    weights within 1e-5;
  * permutation, counts, offsets: bit-exact;
  * layer / GEMM outputs: rel-L2 <= 5e-3 and max-abs <= 2e-2 * max|ref|.
"""

from __future__ import annotations

import numpy as np
import torch

import helpers
from nvfp4_weight_quantized_amd import ops
from oracle import moe as omoe

REL_L2 = 5e-3
MAX_ABS_FRAC = 2e-2


def to_gpu_bank(bank, device="cuda", w4a4: bool = False) -> ops.NvFp4Experts:
    """Upload canonical oracle-side experts and repack them on the GPU into the tile layout
    (``w4a4``: MXFP4 experts in the W4A4 tile layout)."""
    items = [bank[e] for e in range(len(bank))]

    def st(name, dtype):
        return torch.from_numpy(np.ascontiguousarray(np.stack([getattr(i, name) for i in items]))).to(device, dtype)

    fmt = getattr(items[0], "fmt", "nvfp4")
    if fmt == "mxfp4":
        lay = "mxfp4_a4" if w4a4 else "mxfp4"
        return ops.NvFp4Experts.from_canonical(st("w13", torch.uint8), st("w13_scale", torch.uint8), None,
                                               st("w2", torch.uint8), st("w2_scale", torch.uint8), None, fmt=lay)
    assert not w4a4, "the W4A4 layout holds MXFP4 weights"
    return ops.NvFp4Experts.from_canonical(
        st("w13", torch.uint8), st("w13_scale", torch.uint8),
        torch.tensor(np.stack([i.w13_gscale for i in items]), dtype=torch.float32, device=device),
        st("w2", torch.uint8), st("w2_scale", torch.uint8),
        torch.tensor([i.w2_gscale for i in items], dtype=torch.float32, device=device))


def tile_np(packed: np.ndarray, scales: np.ndarray):
    """Test-side statement of the MFMA tile layout: canonical [R, K/2] + [R, K/16] -> tiled bytes.

    Tile (nb, c) = rows [16nb, 16nb+16) x K [128c, 128c+128), tiles in (nb, c) order.  Nibbles:
    lane l = 16q + n, word j holds canonical row 16nb + n bytes [64c + 16j + 4q, +4).  Scales: row
    n's 8 bytes of the chunk, even-numbered groups first.
    """
    r, half = packed.shape
    k = half * 2
    # canonical chunk bytes b = 16j + 4q + u  ->  tile order (q, n, j, u)
    t = packed.reshape(r // 16, 16, k // 128, 4, 4, 4).transpose(0, 2, 4, 1, 3, 5).reshape(r, half)
    # canonical scale byte g = 2jj + parity  ->  tile order (n, parity, jj)
    ts = scales.reshape(r // 16, 16, k // 128, 4, 2).transpose(0, 2, 1, 4, 3).reshape(r, k // 16)
    return np.ascontiguousarray(t), np.ascontiguousarray(ts)


def tile_np_mx(packed: np.ndarray, scales: np.ndarray):
    """Test-side statement of the MXFP4 tile layout: nibbles as tile_np; scales [R, K/32] -> per tile
    (nb, c) the 16 rows' 4 scale bytes of the chunk (one per 32-wide MFMA step), row after row."""
    r, half = packed.shape
    k = half * 2
    t = packed.reshape(r // 16, 16, k // 128, 4, 4, 4).transpose(0, 2, 4, 1, 3, 5).reshape(r, half)
    ts = scales.reshape(r // 16, 16, k // 128, 4).transpose(0, 2, 1, 3).reshape(r, k // 32)
    return np.ascontiguousarray(t), np.ascontiguousarray(ts)


def tile_np_a4(packed: np.ndarray, scales: np.ndarray):
    """Test-side statement of the W4A4 tile layout: tile (nb, c), lane l = 16q + n holds canonical
    row 16nb + n bytes [64c + 16q, +16) (one 32-element block); scale byte l of the tile is that
    row's canonical scale byte 4c + q."""
    r, half = packed.shape
    k = half * 2
    t = packed.reshape(r // 16, 16, k // 128, 4, 16).transpose(0, 2, 3, 1, 4).reshape(r, half)
    ts = scales.reshape(r // 16, 16, k // 128, 4).transpose(0, 2, 3, 1).reshape(r, k // 32)
    return np.ascontiguousarray(t), np.ascontiguousarray(ts)


def bits_to_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_gpu_layer(layer: omoe.Layer, device="cuda", w4a4: bool = False) -> ops.NvFp4MoELayer:
    bias = None if layer.router_bias is None else torch.from_numpy(layer.router_bias).to(device)
    return ops.NvFp4MoELayer(bits_to_bf16(layer.w_router, device), bias, to_gpu_bank(layer.routed, device, w4a4),
                             to_gpu_bank(layer.shared, device, w4a4) if layer.shared is not None else None,
                             layer.top_k)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    mx = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300)
    return rel, mx


def assert_close(got, ref, what=""):
    rel, mx = errors(got, ref)
    assert rel <= REL_L2 and mx <= MAX_ABS_FRAC, f"{what}: rel-L2 {rel:.3e} (<= {REL_L2}), max-abs/max|ref| {mx:.3e}"
    return rel, mx


# margins of the full-size checks, printed in the pytest terminal summary (also under -q)
MARGINS = []


def record_margin(what: str, rel: float, mx: float) -> None:
    """Keep the worst rel-L2 and max-abs/max|ref| of a check for the end-of-run summary."""
    MARGINS.append((what, float(rel), float(mx)))


def logit_bound(x_bits, wr_bits, bias=None):
    x = np.abs(omoe.bf16_to_float(x_bits))
    w = np.abs(omoe.bf16_to_float(wr_bits))
    h = x.shape[1]
    b = h * 2.0 ** -24 * (x @ w.T) + 1e-30
    if bias is not None:
        exact = omoe.router_logits(x_bits, wr_bits, bias)
        b = b + 2.0 ** -24 * np.abs(exact)
    return b


def check_route(logits_gpu, ids_gpu, w_gpu, x_bits, wr_bits, bias, k):
    """GEMM logits within the fp32 bound; selection bit-exact on the GPU's logits; weights within 1e-5."""
    lg = logits_gpu.cpu().numpy().astype(np.float64)
    exact = omoe.router_logits(x_bits, wr_bits, bias)
    bound = logit_bound(x_bits, wr_bits, bias)
    assert np.all(np.abs(lg - exact) <= bound), f"logits off by {np.abs(lg - exact).max():.3e}"
    ids_ref, w_ref = omoe.topk(lg, k)
    ids = ids_gpu.cpu().numpy()
    assert np.array_equal(ids, ids_ref)
    np.testing.assert_allclose(w_gpu.cpu().numpy(), w_ref, rtol=0, atol=1e-5)
    return lg


def ambiguous(logits_exact, k, margin=1e-3):
    """Tokens whose k-th and (k+1)-th exact logits are closer than ``margin``."""
    s = -np.sort(-logits_exact, axis=1)
    if s.shape[1] <= k:
        return np.zeros(s.shape[0], bool)
    return (s[:, k - 1] - s[:, k]) < margin


def reference_for_selection(x_bits, layer, ids_gpu, forward=omoe.forward):
    """Oracle forward (``forward``: oracle.moe's or oracle.w4a4's) where tokens with an ambiguous
    k-th choice take the GPU's selection."""
    res = forward(x_bits, layer)
    amb = ambiguous(res["logits"], layer.top_k)
    ids = ids_gpu.copy()
    mismatch = np.any(ids != res["ids"], axis=1)
    assert not np.any(mismatch & ~amb), f"unambiguous tokens routed differently: {np.where(mismatch & ~amb)[0][:10]}"
    if np.any(mismatch):
        route = np.where(mismatch[:, None], ids, res["ids"])
        res = forward(x_bits, layer, route=route)
    return res
