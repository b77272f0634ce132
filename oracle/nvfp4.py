"""NVFP4 codecs, quantizer and dequantizer (oracle side; test infrastructure only).

Format, as stated in "vLLM on the NVIDIA DGX Spark: A Complete Technical Guide",
section 6.1 "NVFP4 format" and the glossary:
  * element: E2M1, a 4-bit float with a 2-bit exponent and a 1-bit mantissa whose
    largest value is 6.0; two elements are packed per byte;
  * block scale: one FP8 E4M3 value per 16 consecutive elements along K;
  * global scale: one fp32 number per tensor;
  * the value of an element is element * block_scale * global_scale.

Readings taken where the page is silent (each is listed in the design notes):
  * sign: the top bit of a nibble is the sign; magnitude bits are EEM;
    a max of 6.0 = 1.5 * 2^2 with two exponent bits forces exponent bias 1, and
    exponent field 0 is subnormal (0 or 0.5);
  * nibble order: element 2j of a row is the low nibble of byte j, element 2j+1
    the high nibble;
  * E4M3 is the "FN" variant (bias 7, no infinities, S.1111.111 is NaN, largest
    finite 448 -- the 448 used by both the block-scale clamp of the Solar Open 2
    page and the amax/(448*6) global scale of the GLM discussion page);
  * the test-data quantizer rounds to nearest, ties to even, on both grids, and
    takes its decisions in fp32 (the precision of the GPU quantizer).

Global-scale conventions ("GLM-5.3-Flash-NVFP4" discussion, compressed-tensors
follow-up): ModelOpt stores the dequant scale amax/(448*6); compressed-tensors
stores its reciprocal, the quant scale (448*6)/amax.  The worked example there is
one expert with 4.650297705666162e-05 against 21504.0.
"""

from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0
GROUP = 16
FP4_FP8_RANGE = E4M3_MAX * E2M1_MAX  # 2688: the amax/(448*6) denominator


# ----------------------------------------------------------------------------- decode

def e2m1_decode(codes) -> np.ndarray:
    """Value of each 4-bit E2M1 code (float64), from the bit fields.

    code = s e1 e0 m.  Exponent field 0 is subnormal: 0.5*m.  Otherwise
    (1 + m/2) * 2^(e-1).  Sign bit set negates (so -0 decodes to -0.0 == 0).
    """
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return np.where(sign == 1, -mag, mag)


def e4m3_decode(b) -> np.ndarray:
    """Value of each E4M3FN byte (float64): bias 7, subnormals m/8 * 2^-6, NaN at S.1111.111."""
    b = np.asarray(b).astype(np.int64) & 0xFF
    sign = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def unpack_nibbles(packed) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes; element 2j = low nibble of byte j."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def pack_nibbles(codes) -> np.ndarray:
    """[..., K] codes -> [..., K/2] bytes (inverse of unpack_nibbles)."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def dequantize(packed, scales, gscale) -> np.ndarray:
    """W[n, k] = e2m1(code[n, k]) * e4m3(scale[n, k // 16]) * gscale, in float64.

    ``packed`` is [N, K/2] uint8, ``scales`` is [N, K/16] uint8, ``gscale`` the
    fp32 dequant global scale of this tensor.  float64 holds every product
    exactly (at most 2 + 4 + 24 significant bits).
    """
    v = e2m1_decode(unpack_nibbles(packed))
    s = e4m3_decode(scales)
    n, k = v.shape
    assert s.shape == (n, k // GROUP)
    return v * np.repeat(s, GROUP, axis=1) * float(np.float32(gscale))


# ----------------------------------------------------------------------------- encode

_E4M3_FINITE_NONNEG = e4m3_decode(np.arange(0x7F))  # codes 0x00..0x7E, increasing


def e4m3_round(t) -> np.ndarray:
    """Round non-negative values to the nearest E4M3FN value, ties to even mantissa.

    Values above 448 saturate to 448.  Done exactly in float64 on the grid:
    the quantum is 2^(exp-3) for normals (exp >= -6) and 2^-9 below.
    """
    t = np.asarray(t, dtype=np.float64)
    assert np.all(t >= 0), "e4m3_round takes non-negative values"
    _, ex = np.frexp(t)                     # t = f * 2^ex, f in [0.5, 1)
    ex = ex - 1                             # t in [2^ex, 2^(ex+1))
    q = np.exp2(np.maximum(ex, -6) - 3.0)   # grid spacing in this binade
    r = np.rint(t / q) * q                  # np.rint: round half to even
    return np.minimum(r, E4M3_MAX)


def e4m3_encode(t) -> np.ndarray:
    """Byte code of the E4M3FN value nearest to each non-negative ``t`` (RNE, saturating)."""
    r = e4m3_round(t)
    idx = np.searchsorted(_E4M3_FINITE_NONNEG, r)
    assert np.array_equal(_E4M3_FINITE_NONNEG[idx], r)
    return idx.astype(np.uint8)


def e2m1_round(q) -> np.ndarray:
    """Round to the nearest E2M1 value, ties to even mantissa, saturating at +-6.

    The grid spacing is 0.5 below 2, 1 in [2, 4) and 2 from 4 on; rounding the
    multiple of the spacing half-to-even picks the code with mantissa bit 0 on
    a tie.  Returns float64 values.
    """
    q = np.asarray(q, dtype=np.float64)
    mag = np.abs(q)
    step = np.where(mag < 2.0, 0.5, np.where(mag < 4.0, 1.0, 2.0))
    v = np.minimum(np.rint(mag / step) * step, E2M1_MAX)
    return np.where(q < 0, -v, v)


_E2M1_MAGS = e2m1_decode(np.arange(8))  # 0, .5, 1, 1.5, 2, 3, 4, 6


def e2m1_encode(q) -> np.ndarray:
    """4-bit code of the rounded value; the sign bit is set for negative inputs (even if they round to 0)."""
    q = np.asarray(q, dtype=np.float64)
    v = e2m1_round(q)
    mag_code = np.searchsorted(_E2M1_MAGS, np.abs(v)).astype(np.uint8)
    assert np.array_equal(_E2M1_MAGS[mag_code], np.abs(v))
    return np.where(q < 0, mag_code | 8, mag_code).astype(np.uint8)


# ----------------------------------------------------------------------------- global scales

def gscale_modelopt(amax) -> np.float32:
    """ModelOpt dequant global scale amax / (448*6), rounded once to fp32."""
    return np.float32(np.float32(amax) / np.float32(FP4_FP8_RANGE))


def gscale_compressed_tensors(amax) -> np.float32:
    """compressed-tensors quant global scale (448*6) / amax, rounded once to fp32."""
    return np.float32(np.float32(FP4_FP8_RANGE) / np.float32(amax))


def gscale_from_quant_scale(q) -> np.ndarray:
    """Dequant scale from a compressed-tensors quant scale: fp32(1 / q)."""
    q = np.asarray(q, dtype=np.float32)
    return (np.float32(1.0) / q).astype(np.float32)


# ----------------------------------------------------------------------------- quantizer

def quantize(w, gscale):
    """NVFP4-quantize a [N, K] fp32 tensor with dequant global scale ``gscale``.

    Used to build test weights (recipe of the GLM discussion page: group 16,
    symmetric, E4M3 block scales).  Per 16-group along K, all arithmetic in fp32:
      s_b  = E4M3_RNE(min(amax_b / (6 * d), 448))
      code = E2M1_RNE(w / (s_b * d))      (code 0 for every element when s_b == 0)
    Returns (packed [N, K/2] uint8, scales [N, K/16] uint8).
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    assert k % GROUP == 0
    d = np.float32(gscale)
    g = w.reshape(n, k // GROUP, GROUP)
    amax_b = np.max(np.abs(g), axis=2)                               # exact
    t = (amax_b / (np.float32(E2M1_MAX) * d)).astype(np.float32)     # fp32 RN
    t = np.minimum(t, np.float32(E4M3_MAX))
    s_code = e4m3_encode(t)
    s_val = e4m3_decode(s_code).astype(np.float32)                   # exact
    sd = (s_val * d).astype(np.float32)                              # fp32 RN
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (g / sd[:, :, None]).astype(np.float32)                  # fp32 RN
    q = np.where(sd[:, :, None] > 0, q, np.float32(0.0))
    codes = e2m1_encode(q).reshape(n, k)
    return pack_nibbles(codes), s_code


def storage_bytes(n, k) -> int:
    """Bytes of one packed [N, K] NVFP4 tensor: N*K/2 nibble bytes + N*K/16 scale bytes."""
    return n * k // 2 + n * k // GROUP
