"""W4A4 variant of the MoE layer in the NVFP4 format (oracle side; test infrastructure only).

Both GEMM operands are NVFP4.  The expert weights are the NVFP4 banks of the W4A16 layer
(oracle.nvfp4, oracle.moe); the activations entering each GEMM -- the token rows x for gate/up,
the intermediate h for down -- are quantized to NVFP4 on the fly, row by row: E2M1 elements, one
E4M3 block scale per 16 consecutive elements along K, and one fp32 global scale per GEMM input.

Sources:
  * "vLLM on the NVIDIA DGX Spark: A Complete Technical Guide", section 6.1: the NVFP4 format;
    the global scale is one fp32 number for the weights and one for the activations, and the
    kernel combines them as alpha = 1 / (input_global_scale * weight_global_scale); section 4.3
    and the table of section 4.5: the fused MoE kernel takes bf16 hidden states and quantizes them
    (BF16 -> FP4) itself.
  * "vLLM on the DGX Spark, the Hard Way: Seven Months of GB10 Field Notes", "The one rule that
    explains all the FP4 confusion": a W4A4 checkpoint carries 4-bit weights and 4-bit
    activations.
  * "GLM-5.3-Flash-NVFP4 deployment blocked on SM121" discussion: static activation scales are
    calibrated per projection (a placeholder of 1.0 was wrong); a missing activation scale folded
    into the alphas multiplies every expert by zero; the global scale is a reciprocal between the
    ModelOpt (dequant, amax / (448 * 6)) and compressed-tensors (quant, (448 * 6) / amax) forms.

Readings where the pages are silent (listed in the design notes):
  * global scales are passed in their dequant form d (ModelOpt convention; the compressed-tensors
    quant scale is 1 / d), so alpha = 1 / (input_global_scale * weight_global_scale) = d_a * d_w;
  * one static activation scale per GEMM input, shared by every expert (and the shared expert):
    d_x for the gate/up input, d_h for the down input;
  * the activation quantizer is the rule of oracle.nvfp4.quantize (the one the weights are built
    with), applied to the exact values of the bf16 activations, all decisions in fp32;
  * h is rounded to bf16 (as in the W4A16 layer) before it is quantized;
  * a zero, negative or non-finite activation scale is an error, never a silent zero.

Arithmetic: float64 on the exact dequantized values, so the only roundings are the quantizers'
own and the bf16 rounding of h.
"""

from __future__ import annotations

import math

import numpy as np

from . import nvfp4
from .moe import bf16_to_float, combine, permute, router_logits, silu, topk, topk_weights
from .w4a4 import float_to_bf16_bits


def check_act_gscale(d) -> np.float32:
    """The activation dequant global scale as fp32; anything but a finite positive number is an error."""
    d32 = np.float32(d)
    if not (math.isfinite(float(d32)) and float(d32) > 0.0):
        raise ValueError(f"activation global scale must be finite and positive, got {d!r}")
    return d32


def quantize_act(a, d) -> tuple:
    """NVFP4 codes [M, K/2] and E4M3 block scales [M, K/16] of activation rows ``a`` (values, K % 16 == 0)."""
    d32 = check_act_gscale(d)
    a = np.asarray(a, dtype=np.float64)
    a32 = a.astype(np.float32)
    assert np.array_equal(a32.astype(np.float64), a), "activation values must be fp32-exact (bf16 rows are)"
    return nvfp4.quantize(a32, d32)


def act_values(a, d) -> np.ndarray:
    """The 4-bit operand without its global scale: e2m1(code) * e4m3(block scale) (float64).

    Every such product has at most 6 significant bits and lies within [2^-10, 2688], so it is
    exact in bf16 and in fp16.
    """
    a = np.asarray(a, dtype=np.float64)
    if a.shape[0] == 0:
        return a.copy()
    packed, scales = quantize_act(a, d)
    return nvfp4.dequantize(packed, scales, 1.0)


def fake_quant_act(a, d) -> np.ndarray:
    """The values the 4-bit activation operand stands for: act_values(a, d) * d (float64)."""
    return act_values(a, d) * float(check_act_gscale(d))


def gate_up_a4(a_vals, ew, d_x) -> np.ndarray:
    """h = silu(A . Wg^T) * (A . Wu^T) on 4-bit activations A = fake_quant_act(a_vals, d_x) -> [M, I]."""
    w13 = ew.dequant_w13()
    i = w13.shape[0] // 2
    gu = fake_quant_act(a_vals, d_x) @ w13.T
    return silu(gu[:, :i]) * gu[:, i:]


def down_a4(h_vals, ew, d_h) -> np.ndarray:
    """y = H . Wd^T on 4-bit activations H = fake_quant_act(h_vals, d_h) -> [M, H]."""
    return fake_quant_act(h_vals, d_h) @ ew.dequant_w2().T


def round_h(h) -> np.ndarray:
    """h as the bf16 values the down GEMM's quantizer starts from."""
    return bf16_to_float(float_to_bf16_bits(h))


def expert_ffn_a4(a_vals, ew, d_x, d_h) -> np.ndarray:
    return down_a4(round_h(gate_up_a4(a_vals, ew, d_x)), ew, d_h)


def grouped_gate_up_a4(a_vals, offsets, bank, d_x) -> np.ndarray:
    """Gate/up stage over row groups: rows [offsets[e], offsets[e+1]) use expert e."""
    a_vals = np.asarray(a_vals, np.float64)
    i = bank[0].w13.shape[0] // 2 if len(bank) else 0
    out = np.zeros((a_vals.shape[0], i))
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            out[r0:r1] = gate_up_a4(a_vals[r0:r1], bank[e], d_x)
    return out


def grouped_down_a4(h_vals, offsets, bank, d_h) -> np.ndarray:
    """Down stage over row groups on 4-bit activations."""
    h_vals = np.asarray(h_vals, np.float64)
    hdim = bank[0].w2.shape[0] if len(bank) else 0
    out = np.zeros((h_vals.shape[0], hdim))
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            out[r0:r1] = down_a4(h_vals[r0:r1], bank[e], d_h)
    return out


def forward(x_bits, layer, d_x, d_h, route=None) -> dict:
    """The NVFP4 W4A4 layer for tokens ``x_bits`` (bf16 bits [T, H]) with activation scales d_x, d_h.

    Routing (S1-S3) and the combine (S6) are those of oracle.moe.forward on the bf16 tokens; the
    expert FFNs quantize their GEMM inputs.  Returns the same dict as oracle.moe.forward plus the
    expert output rows ``y_rows`` (sorted order) and ``y_shared``.
    """
    d_x, d_h = check_act_gscale(d_x), check_act_gscale(d_h)
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
            y_rows[r0:r1] = expert_ffn_a4(a_rows[r0:r1], layer.routed[e], d_x, d_h)
    y_shared = expert_ffn_a4(x, layer.shared[0], d_x, d_h) if layer.shared is not None else None
    out = combine(y_rows, slot_to_row, w, y_shared)
    return dict(logits=logits, ids=ids, weights=w, counts=counts, offsets=offsets, sorted_slot=sorted_slot,
                slot_to_row=slot_to_row, out=out, y_rows=y_rows, y_shared=y_shared)


__all__ = ["check_act_gscale", "quantize_act", "act_values", "fake_quant_act", "gate_up_a4", "down_a4", "round_h",
           "expert_ffn_a4", "grouped_gate_up_a4", "grouped_down_a4", "forward"]
