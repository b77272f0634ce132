"""MXFP4 codecs, quantizer and dequantizer (oracle side; test infrastructure only).

Format, as stated in "vLLM on the NVIDIA DGX Spark: A Complete Technical Guide",
section 6.4 "NVFP4 vs MXFP4" and the glossary entry MXFP4:
  * element: E2M1, the same 4-bit float as NVFP4 (two per byte);
  * block: 32 consecutive elements along K share one scale;
  * block scale: E8M0, exponent only; there is no per-tensor global scale.

Readings taken where the page is silent (each is listed in the design notes):
  * E8M0 is an unsigned biased exponent: byte b stands for 2^(b - 127), and
    0xFF is NaN (the OCP Microscaling v1.0 encoding);
  * nibble order and E2M1 decoding exactly as for NVFP4 (oracle.nvfp4);
  * the test-data quantizer takes, per 32-block, the shared exponent
    floor(log2(amax)) - 2 (2 = the exponent of E2M1's largest value 6 = 1.5 * 2^2),
    clamped to the E8M0 range, and rounds every element divided by 2^exponent to
    the nearest E2M1 value, ties to even, saturating at +-6 (the OCP conversion;
    values in (6, 8) * 2^exponent clip to 6).  A block whose amax is 0 gets the
    smallest scale and all-zero codes.
"""

from __future__ import annotations

import numpy as np

from .nvfp4 import E2M1_MAX, e2m1_decode, e2m1_encode, pack_nibbles, unpack_nibbles

GROUP = 32
E8M0_BIAS = 127
E2M1_EMAX = 2   # 6 = 1.5 * 2^2


def e8m0_decode(b) -> np.ndarray:
    """Value of each E8M0 byte (float64): 2^(b - 127); 0xFF is NaN."""
    b = np.asarray(b).astype(np.int64) & 0xFF
    v = np.ldexp(1.0, b - E8M0_BIAS)
    return np.where(b == 0xFF, np.nan, v)


def dequantize(packed, scales) -> np.ndarray:
    """W[n, k] = e2m1(code[n, k]) * e8m0(scale[n, k // 32]), in float64 (exact)."""
    v = e2m1_decode(unpack_nibbles(packed))
    s = e8m0_decode(scales)
    n, k = v.shape
    assert s.shape == (n, k // GROUP)
    return v * np.repeat(s, GROUP, axis=1)


def shared_exponent(amax) -> np.ndarray:
    """Per-block exponent floor(log2(amax)) - 2, clamped to [-127, 127]; -127 where amax == 0."""
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))   # a = f * 2^ex with f in [0.5, 1): floor(log2 a) = ex - 1
    e = ex - 1 - E2M1_EMAX
    e = np.where(a > 0, e, -E8M0_BIAS)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def quantize(w):
    """MXFP4-quantize a [N, K] fp32 tensor; returns (packed [N, K/2] uint8, scales [N, K/32] uint8).

    Division by a power of two is exact, so only the E2M1 rounding is inexact.
    """
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    n, k = w.shape
    assert k % GROUP == 0
    g = w.reshape(n, k // GROUP, GROUP)
    e = shared_exponent(np.max(np.abs(g), axis=2))
    q = g / np.ldexp(1.0, e)[:, :, None]
    codes = e2m1_encode(q).reshape(n, k)
    return pack_nibbles(codes), (e + E8M0_BIAS).astype(np.uint8)


def storage_bytes(n, k) -> int:
    """Bytes of one packed [N, K] MXFP4 tensor: N*K/2 nibble bytes + N*K/32 scale bytes."""
    return n * k // 2 + n * k // GROUP


__all__ = ["GROUP", "E2M1_MAX", "e8m0_decode", "dequantize", "shared_exponent", "quantize", "storage_bytes"]
