"""Weight-only NVFP4 fused MoE layer, whole-layer oracle (float64; test infrastructure only).

Stages follow the modular fused-MoE decomposition of "vLLM on the NVIDIA DGX
Spark: A Complete Technical Guide", section 7.1: router -> permute -> experts
(gate/up GEMM, SiLU(gate)*up, down GEMM) -> combine (top-k-weighted reduction,
as the fused b12x kernel of section 4 describes it).  The W4A16 variant has no
quantize-dispatch step: activations stay 16-bit and only the weights are NVFP4
(section 5 "Marlin": 16-bit activations times low-bit weights, dequantized to
16-bit inside the GEMM; the GLM discussion page: weight-only is chosen when the
checkpoint carries no input quantization).  Layer shape: routed experts with
top-k selection plus one always-on shared expert ("Serving Solar Open 2 on DGX
Spark", "Solar Open 2 in brief": 320 routed + 1 shared, top-8).

Readings where the pages are silent (listed in the design notes):
  * router: logits = x . Wr^T (+ bias); softmax over all E, keep the k largest,
    renormalise over the k kept -- identical to a softmax over the k kept logits;
    the k largest logits are taken in descending order, equal logits -> lower
    expert index first;
  * fused w13: rows [0, I) are gate, rows [I, 2I) are up, each with its own
    global scale;
  * shared expert: added with weight 1, no gate;
  * no routed scaling factor (1.0);
  * no activation scale exists anywhere: an expert can never be multiplied by 0.

All arithmetic here is float64 on the exact values of the bf16 activations and
the dequantized NVFP4 (or MXFP4, oracle.mxfp4) weights.  The GPU keeps fp32 accumulators and bf16
intermediates; the parity tolerances absorb that difference.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from . import mxfp4, nvfp4


def bf16_to_float(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


@dataclass
class ExpertWeights:
    """One expert: fused gate/up [2I, H] and down [H, I], packed as the C ABI stores them.

    fmt "nvfp4": E4M3 block scales per 16 elements along K and fp32 global scales;
    fmt "mxfp4": E8M0 block scales per 32 elements, no global scale (the gscale
    fields are ignored).
    """
    w13: np.ndarray          # uint8 [2I, H/2]
    w13_scale: np.ndarray    # uint8 [2I, H/16] E4M3 (NVFP4) or [2I, H/32] E8M0 (MXFP4)
    w13_gscale: np.ndarray   # fp32 [2]  dequant global scales (gate, up); NVFP4 only
    w2: np.ndarray           # uint8 [H, I/2]
    w2_scale: np.ndarray     # uint8 [H, I/16] or [H, I/32]
    w2_gscale: float         # fp32 dequant global scale; NVFP4 only
    fmt: str = "nvfp4"

    def _deq(self, packed, scales, gscale) -> np.ndarray:
        if self.fmt == "mxfp4":
            return mxfp4.dequantize(packed, scales)
        return nvfp4.dequantize(packed, scales, gscale)

    def dequant_w13(self) -> np.ndarray:
        two_i = self.w13.shape[0]
        i = two_i // 2
        gs = self.w13_gscale if self.fmt == "nvfp4" else (None, None)
        g = self._deq(self.w13[:i], self.w13_scale[:i], gs[0])
        u = self._deq(self.w13[i:], self.w13_scale[i:], gs[1])
        return np.concatenate([g, u], axis=0)

    def dequant_w2(self) -> np.ndarray:
        return self._deq(self.w2, self.w2_scale, self.w2_gscale)


class ArrayBank:
    """A bank of experts held as stacked arrays with a leading expert dimension."""

    def __init__(self, w13, w13_scale, w13_gscale, w2, w2_scale, w2_gscale, fmt="nvfp4"):
        self.fmt = fmt
        self.w13, self.w13_scale = w13, w13_scale
        self.w2, self.w2_scale = w2, w2_scale
        e = w13.shape[0]
        self.w13_gscale = np.asarray(w13_gscale if w13_gscale is not None else np.ones((e, 2)), np.float32)
        self.w2_gscale = np.asarray(w2_gscale if w2_gscale is not None else np.ones(e), np.float32)

    def __len__(self):
        return self.w13.shape[0]

    def __getitem__(self, e) -> ExpertWeights:
        return ExpertWeights(self.w13[e], self.w13_scale[e], self.w13_gscale[e],
                             self.w2[e], self.w2_scale[e], float(self.w2_gscale[e]), self.fmt)


@dataclass
class Layer:
    w_router: np.ndarray                 # uint16 bf16 bits [E, H]
    router_bias: Optional[np.ndarray]    # fp32 [E] or None
    routed: Sequence[ExpertWeights]      # E experts (sequence-like: len() and [e])
    shared: Optional[Sequence[ExpertWeights]]  # 1 expert, or None
    top_k: int


# ----------------------------------------------------------------------------- router

def router_logits(x_bits, w_router_bits, bias=None) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * Wr[e, h] (+ bias[e]), float64 on bf16 values."""
    logits = bf16_to_float(x_bits) @ bf16_to_float(w_router_bits).T
    if bias is not None:
        logits = logits + np.asarray(bias, np.float32).astype(np.float64)[None, :]
    return logits


def topk(logits, k):
    """Top-k experts per token and their renormalised softmax weights.

    Selection: the k largest logits, descending; equal logits -> lower index
    first (a stable sort of -logits).  Softmax is strictly increasing, so
    selecting on logits selects the same experts as selecting on probabilities.
    Weights: exp(l_j - l_max) / sum over the k selected of exp(l_i - l_max),
    which equals the full softmax renormalised over the selected experts.
    """
    logits = np.asarray(logits, dtype=np.float64)
    order = np.argsort(-logits, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    return ids, topk_weights(logits, ids)


def topk_weights(logits, ids) -> np.ndarray:
    """Renormalised softmax weights of the given selection (float64)."""
    sel = np.take_along_axis(np.asarray(logits, np.float64), np.asarray(ids, np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


# ----------------------------------------------------------------------------- permute

def permute(ids, num_experts):
    """Group the T*k slots (slot = t*k + j) by expert, keeping slot order inside a group.

    Returns counts [E], offsets [E+1] (exclusive prefix sum), sorted_slot [S]
    (slots in expert order) and slot_to_row [S] (inverse: slot -> row).
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=num_experts).astype(np.int32)
    offsets = np.zeros(num_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_slot = np.argsort(flat, kind="stable").astype(np.int32)
    slot_to_row = np.empty_like(sorted_slot)
    slot_to_row[sorted_slot] = np.arange(flat.size, dtype=np.int32)
    return counts, offsets, sorted_slot, slot_to_row


# ----------------------------------------------------------------------------- experts

def silu(g) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def gate_up(a_rows, ew: ExpertWeights) -> np.ndarray:
    """h = silu(a . Wg^T) * (a . Wu^T) for rows ``a_rows`` (float64 [M, H]) -> [M, I]."""
    w13 = ew.dequant_w13()
    i = w13.shape[0] // 2
    gu = a_rows @ w13.T
    return silu(gu[:, :i]) * gu[:, i:]


def down(h_rows, ew: ExpertWeights) -> np.ndarray:
    """y = h . Wd^T for rows ``h_rows`` (float64 [M, I]) -> [M, H]."""
    return h_rows @ ew.dequant_w2().T


def expert_ffn(a_rows, ew: ExpertWeights) -> np.ndarray:
    return down(gate_up(a_rows, ew), ew)


def grouped_gate_up(a_rows, offsets, bank) -> np.ndarray:
    """Gate/up stage over row groups: rows [offsets[e], offsets[e+1]) use expert e."""
    a_rows = np.asarray(a_rows, np.float64)
    i = bank[0].w13.shape[0] // 2 if len(bank) else 0
    out = np.zeros((a_rows.shape[0], i))
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            out[r0:r1] = gate_up(a_rows[r0:r1], bank[e])
    return out


def grouped_down(h_rows, offsets, bank) -> np.ndarray:
    """Down stage over row groups: rows [offsets[e], offsets[e+1]) use expert e."""
    h_rows = np.asarray(h_rows, np.float64)
    hdim = bank[0].w2.shape[0] if len(bank) else 0
    out = np.zeros((h_rows.shape[0], hdim))
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            out[r0:r1] = down(h_rows[r0:r1], bank[e])
    return out


# ----------------------------------------------------------------------------- combine / layer

def combine(y_rows, slot_to_row, weights, y_shared=None) -> np.ndarray:
    """out[t] = sum_j w[t, j] * y_rows[slot_to_row[t*k + j]] (+ y_shared[t])."""
    weights = np.asarray(weights, np.float64)
    t, k = weights.shape
    rows = np.asarray(y_rows, np.float64)[np.asarray(slot_to_row).reshape(t, k)]
    out = np.einsum("tj,tjh->th", weights, rows)
    if y_shared is not None:
        out = out + np.asarray(y_shared, np.float64)
    return out


def forward(x_bits, layer: Layer, route=None) -> dict:
    """The whole layer for tokens ``x_bits`` (bf16 bits [T, H]).

    ``route`` optionally overrides the selection with (ids [T, k]); the weights
    are then the renormalised softmax of this oracle's logits at those ids.
    Returns a dict with logits, ids, weights, counts, offsets, sorted_slot,
    slot_to_row and out (float64 [T, H]).
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
            y_rows[r0:r1] = expert_ffn(a_rows[r0:r1], layer.routed[e])
    y_shared = expert_ffn(x, layer.shared[0]) if layer.shared is not None else None
    out = combine(y_rows, slot_to_row, w, y_shared)
    return dict(logits=logits, ids=ids, weights=w, counts=counts, offsets=offsets,
                sorted_slot=sorted_slot, slot_to_row=slot_to_row, out=out)
