"""W4A4 variant of the MoE layer in the MX format (oracle side; test infrastructure only).

Both GEMM operands are 4-bit: the expert weights are MXFP4 (oracle.mxfp4) and the
activations entering each GEMM -- the token rows x for gate/up, the intermediate
h for down -- are quantized to MXFP4 on the fly, per row, one E8M0 scale per 32
consecutive elements along K.

Sources:
  * "vLLM on the DGX Spark, the Hard Way: Seven Months of GB10 Field Notes",
    section "The one rule that explains all the FP4 confusion": a W4A4 checkpoint
    carries 4-bit weights and 4-bit activations and runs a native FP4 matmul,
    while W4A16 has no FP4 activations; section "Measured: native FP4 + MTP vs
    the published Marlin numbers": the native-FP4 gain is in prefill, the
    compute-bound regime.
  * "vLLM on the NVIDIA DGX Spark: A Complete Technical Guide", section 4.3: the
    fused MoE kernel takes bf16 hidden states and quantizes them (BF16 -> FP4)
    inside the kernel; section 6.4: the MXFP4 format (E2M1 elements, E8M0 scale
    per 32 elements, no global scale).

Readings where the pages are silent (listed in the design notes):
  * the activation quantizer is the MXFP4 rule of oracle.mxfp4.quantize applied
    to the exact values of the bf16 activations, row by row along K;
  * h is rounded to bf16 (as in the W4A16 layer) before it is quantized, so the
    quantizer always starts from bf16 values on both sides;
  * the pages' NVFP4 W4A4 activation format (E4M3 scale per 16 plus a global
    scale) is not what is computed here: both operands use the MX format.

Arithmetic: float64 on the exact dequantized values (every E2M1 * 2^e product is
exact), so the only rounding is the quantizers' own and the bf16 rounding of h.
"""

from __future__ import annotations

import numpy as np

from . import mxfp4
from .moe import bf16_to_float, combine, permute, router_logits, silu, topk, topk_weights


def float_to_bf16_bits(v) -> np.ndarray:
    """Round float64 values to bf16 (8 significant bits), ties to even; returns the bit patterns.

    The grid spacing of bf16 in the binade [2^e, 2^(e+1)) is 2^(e-7), and 2^-133 below
    2^-126 (subnormals); v / spacing is exact, np.rint rounds half to even, and the
    rounded value is exact in float32, whose upper 16 bits are then the bf16 pattern.
    Values that round past the largest bf16 become infinities.
    """
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(v)                                   # |v| in [2^(ex-1), 2^ex)
    q = np.exp2(np.maximum(ex - 1, -126) - 7.0)
    r = np.rint(v / q) * q
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)                          # exact, or inf past the float32 range
    bits = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    too_big = np.abs(r) > 3.3895313892515355e38           # largest finite bf16, 0x7F7F
    bits = np.where(too_big, np.where(r > 0, np.uint16(0x7F80), np.uint16(0xFF80)), bits)
    return np.where(np.isnan(v), np.uint16(0x7FC0), bits).astype(np.uint16)


def quantize_act(a) -> tuple:
    """MXFP4 codes and E8M0 scales of activation rows ``a`` (values [M, K], K % 32 == 0)."""
    return mxfp4.quantize(np.asarray(a, dtype=np.float64))


def fake_quant_act(a) -> np.ndarray:
    """The values the 4-bit activation operand stands for: dequantize(quantize(a)) (float64)."""
    a = np.asarray(a, dtype=np.float64)
    if a.shape[0] == 0:
        return a.copy()
    packed, scales = quantize_act(a)
    return mxfp4.dequantize(packed, scales)


def gate_up_a4(a_vals, ew) -> np.ndarray:
    """h = silu(A . Wg^T) * (A . Wu^T) on 4-bit activations A = fake_quant_act(a_vals) -> [M, I]."""
    w13 = ew.dequant_w13()
    i = w13.shape[0] // 2
    gu = fake_quant_act(a_vals) @ w13.T
    return silu(gu[:, :i]) * gu[:, i:]


def down_a4(h_vals, ew) -> np.ndarray:
    """y = H . Wd^T on 4-bit activations H = fake_quant_act(h_vals) -> [M, H]."""
    return fake_quant_act(h_vals) @ ew.dequant_w2().T


def round_h(h) -> np.ndarray:
    """h as the bf16 values the down GEMM's quantizer starts from."""
    return bf16_to_float(float_to_bf16_bits(h))


def expert_ffn_a4(a_vals, ew) -> np.ndarray:
    return down_a4(round_h(gate_up_a4(a_vals, ew)), ew)


def grouped_gate_up_a4(a_vals, offsets, bank) -> np.ndarray:
    """Gate/up stage over row groups on 4-bit activations: rows [offsets[e], offsets[e+1]) use expert e."""
    a_vals = np.asarray(a_vals, np.float64)
    i = bank[0].w13.shape[0] // 2 if len(bank) else 0
    out = np.zeros((a_vals.shape[0], i))
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            out[r0:r1] = gate_up_a4(a_vals[r0:r1], bank[e])
    return out


def grouped_down_a4(h_vals, offsets, bank) -> np.ndarray:
    """Down stage over row groups on 4-bit activations."""
    h_vals = np.asarray(h_vals, np.float64)
    hdim = bank[0].w2.shape[0] if len(bank) else 0
    out = np.zeros((h_vals.shape[0], hdim))
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            out[r0:r1] = down_a4(h_vals[r0:r1], bank[e])
    return out


def forward(x_bits, layer, route=None) -> dict:
    """The W4A4 layer for tokens ``x_bits`` (bf16 bits [T, H]); banks must be MXFP4.

    Routing (S1-S3) and the combine (S6) are those of oracle.moe.forward; the expert
    FFNs quantize their GEMM inputs.  Returns the same dict as oracle.moe.forward.
    """
    x = bf16_to_float(x_bits)
    t_count, hdim = x.shape
    e_count = len(layer.routed)
    k = layer.top_k
    logits = router_logits(x_bits, layer.w_router, layer.router_bias)
    if route is None:
        ids, w = topk(logits, k)
    else:
        ids = np.asarray(route, np.int32)
        w = topk_weights(logits, ids)
    counts, offsets, sorted_slot, slot_to_row = permute(ids, e_count)
    a_rows = x[sorted_slot // k]
    y_rows = np.zeros((t_count * k, hdim))
    for e in range(e_count):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            y_rows[r0:r1] = expert_ffn_a4(a_rows[r0:r1], layer.routed[e])
    y_shared = expert_ffn_a4(x, layer.shared[0]) if layer.shared is not None else None
    out = combine(y_rows, slot_to_row, w, y_shared)
    return dict(logits=logits, ids=ids, weights=w, counts=counts, offsets=offsets,
                sorted_slot=sorted_slot, slot_to_row=slot_to_row, out=out)


__all__ = ["float_to_bf16_bits", "quantize_act", "fake_quant_act", "gate_up_a4", "down_a4", "round_h",
           "expert_ffn_a4", "grouped_gate_up_a4", "grouped_down_a4", "forward"]
