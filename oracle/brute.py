"""Independent scalar float64 implementation of the layer, token by token (test infrastructure only).

Written separately from ``oracle.moe`` and ``oracle.nvfp4`` (it imports neither)
so that it can pin them: plain Python loops, a literal E2M1 value table, an
E4M3 decode written with ``math.ldexp``, and a per-token routing by sorting.
Only for tiny layers (seconds at H=256, I=128).

Definitions used (same sources as ``oracle.moe``):
  * E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, top bit of the nibble = sign;
    element 2j in the low nibble of byte j ("vLLM on the NVIDIA DGX Spark: A
    Complete Technical Guide", section 6.1);
  * E4M3 block scale per 16 elements along K; value = element * block scale *
    global scale (same section); for MXFP4 one E8M0 scale 2^(b - 127) per 32
    elements and no global scale (section 6.4, the reading of oracle.mxfp4);
  * top-k on router logits (ties -> lower expert index), softmax renormalised
    over the selected experts; SiLU(gate)*up; down projection; top-k-weighted
    sum; shared expert added with weight 1 (same readings as ``oracle.moe``);
  * W4A4 (``act="mxfp4"``): each GEMM input vector is quantized per 32 elements
    to an E8M0 shared exponent floor(log2 amax) - 2 (clamped to [-127, 127]) and
    the nearest E2M1 value, found by searching the value table (ties -> even
    code, i.e. mantissa bit 0); h is rounded to bf16 first (the readings of
    ``oracle.w4a4``);
  * W4A4 in NVFP4 (``act="nvfp4"``, activation dequant global scales d_x, d_h): per
    16 elements, t = amax / (6 d) rounded to fp32 (6 d rounded first), capped at
    448, the nearest E4M3 value s by searching all 127 finite codes (ties -> even
    code); each element v / (s d) (s d and the quotient rounded to fp32) to the
    nearest E2M1 value; fp32 rounding emulated through ``struct`` (the readings
    of ``oracle.nvfp4_w4a4``).
"""

from __future__ import annotations

import math
import struct

E2M1_TABLE = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def fp4(row_bytes, k: int) -> float:
    byte = int(row_bytes[k // 2])
    nib = (byte >> 4) if (k % 2) else (byte & 0xF)
    mag = E2M1_TABLE[nib & 7]
    return -mag if nib & 8 else mag


def fp8_e4m3(byte: int) -> float:
    byte = int(byte)
    sign = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sign * math.ldexp(m, -9)          # m/8 * 2^-6
    return sign * math.ldexp(8 + m, e - 10)      # (1 + m/8) * 2^(e-7)


def e8m0(byte: int) -> float:
    byte = int(byte)
    return math.nan if byte == 255 else math.ldexp(1.0, byte - 127)


def weight(packed, scales, gscale: float, n: int, k: int, fmt: str = "nvfp4") -> float:
    if fmt == "mxfp4":
        return fp4(packed[n], k) * e8m0(scales[n][k // 32])
    return fp4(packed[n], k) * fp8_e4m3(scales[n][k // 16]) * float(gscale)


def dequant_expert(ew):
    """(Wg, Wu, Wd) as lists of float rows, decoded element by element."""
    fmt = getattr(ew, "fmt", "nvfp4")
    inter = len(ew.w13) // 2
    hdim = 2 * len(ew.w13[0])
    wg = [[weight(ew.w13, ew.w13_scale, ew.w13_gscale[0], i, h, fmt) for h in range(hdim)] for i in range(inter)]
    wu = [[weight(ew.w13, ew.w13_scale, ew.w13_gscale[1], inter + i, h, fmt) for h in range(hdim)]
          for i in range(inter)]
    wd = [[weight(ew.w2, ew.w2_scale, ew.w2_gscale, h, i, fmt) for i in range(inter)] for h in range(hdim)]
    return wg, wu, wd


def bf16_round(v: float) -> float:
    """Nearest bf16 value of v (8 significant bits, ties to even), via frexp and round()."""
    if v == 0.0 or math.isnan(v) or math.isinf(v):
        return v
    _, e = math.frexp(v)                 # |v| in [2^(e-1), 2^e): spacing 2^(e-8)
    e = max(e, -125)                     # subnormal bf16 spacing is 2^-133
    r = math.ldexp(float(round(math.ldexp(v, 8 - e))), e - 8)   # round(): half to even
    return math.copysign(math.inf, r) if abs(r) > 3.3895313892515355e38 else r


def mx_group(vals):
    """MXFP4 of one 32-element group: (signed E2M1 values, scale exponent)."""
    amax = max(abs(v) for v in vals)
    if amax == 0.0:
        e = -127
    else:
        _, ex = math.frexp(amax)         # amax in [2^(ex-1), 2^ex)
        e = min(max(ex - 1 - 2, -127), 127)
    out = []
    for v in vals:
        t = abs(v) / math.ldexp(1.0, e)
        best = 0
        for c in range(8):
            d, db = abs(t - E2M1_TABLE[c]), abs(t - E2M1_TABLE[best])
            if d < db or (d == db and c % 2 == 0 and best % 2 == 1):
                best = c
        out.append(-E2M1_TABLE[best] if v < 0 else E2M1_TABLE[best])
    return out, e


def mx_fake_quant(vec) -> list:
    """The values a vector stands for after MXFP4 quantization in groups of 32."""
    res = []
    for g0 in range(0, len(vec), 32):
        vals, e = mx_group(vec[g0:g0 + 32])
        res.extend(v * math.ldexp(1.0, e) for v in vals)
    return res


def f32(v: float) -> float:
    """v rounded to the nearest fp32 value (ties to even), by packing it as a C float."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


E4M3_VALUES = tuple(fp8_e4m3(b) for b in range(0x7F))   # finite non-negative codes, increasing


def nearest_index(t: float, table) -> int:
    """Index of the table value nearest to t; on a tie the even index (mantissa bit 0)."""
    best = 0
    for c, v in enumerate(table):
        d, db = abs(t - v), abs(t - table[best])
        if d < db or (d == db and c % 2 == 0 and best % 2 == 1):
            best = c
    return best


def nv_group(vals, d: float):
    """NVFP4 of one 16-element group with dequant global scale d: (signed E2M1 values, E4M3 scale)."""
    amax = max(abs(v) for v in vals)
    t = min(f32(amax / f32(6.0 * d)), 448.0)
    s = E4M3_VALUES[nearest_index(t, E4M3_VALUES)]
    sd = f32(s * d)
    out = []
    for v in vals:
        q = f32(v / sd) if sd > 0.0 else 0.0
        mag = E2M1_TABLE[nearest_index(abs(q), E2M1_TABLE)]
        out.append(-mag if q < 0 else mag)
    return out, s


def nv_fake_quant(vec, d: float) -> list:
    """The values a vector stands for after NVFP4 quantization in groups of 16 (global scale d)."""
    res = []
    for g0 in range(0, len(vec), 16):
        vals, s = nv_group(vec[g0:g0 + 16], d)
        res.extend(v * s * d for v in vals)
    return res


def expert_out(xv, mats, act: str = "bf16", act_gscales=(1.0, 1.0)) -> list:
    """y = Wd (silu(Wg x) * (Wu x)) for one token, scalar loops (act "mxfp4" or "nvfp4": W4A4;
    act_gscales = (d_x, d_h) for "nvfp4")."""
    wg, wu, wd = mats
    if act == "mxfp4":
        xv = mx_fake_quant(xv)
    elif act == "nvfp4":
        xv = nv_fake_quant(xv, act_gscales[0])
    hvec = []
    for grow, urow in zip(wg, wu):
        g = 0.0
        u = 0.0
        for xh, a, b in zip(xv, grow, urow):
            g += xh * a
            u += xh * b
        sg = g / (1.0 + math.exp(-g)) if g > -700.0 else 0.0
        hvec.append(sg * u)
    if act == "mxfp4":
        hvec = mx_fake_quant([bf16_round(v) for v in hvec])
    elif act == "nvfp4":
        hvec = nv_fake_quant([bf16_round(v) for v in hvec], act_gscales[1])
    y = []
    for drow in wd:
        acc = 0.0
        for hv, c in zip(hvec, drow):
            acc += hv * c
        y.append(acc)
    return y


def forward(x_bits, layer, tokens=None, act: str = "bf16", act_gscales=(1.0, 1.0)):
    """Per-token results [(ids, weights, out row, logits)] for the given token indices
    (act "mxfp4": the W4A4 layer, MXFP4 weights and activations; act "nvfp4": NVFP4 weights
    and activations with activation dequant global scales act_gscales = (d_x, d_h))."""
    cache = {}

    def mats(bank, e):
        key = (id(bank), e)
        if key not in cache:
            cache[key] = dequant_expert(bank[e])
        return cache[key]

    results = []
    rows = range(len(x_bits)) if tokens is None else tokens
    for t in rows:
        xv = [bf16(b) for b in x_bits[t]]
        e_count = len(layer.routed)
        logits = []
        for e in range(e_count):
            acc = 0.0
            for xh, wb in zip(xv, layer.w_router[e]):
                acc += xh * bf16(wb)
            if layer.router_bias is not None:
                acc += float(layer.router_bias[e])
            logits.append(acc)
        chosen = sorted(range(e_count), key=lambda e: (-logits[e], e))[: layer.top_k]
        top = max(logits[e] for e in chosen)
        z = [math.exp(logits[e] - top) for e in chosen]
        total = sum(z)
        wts = [v / total for v in z]
        out = [0.0] * len(xv)
        for e, w in zip(chosen, wts):
            y = expert_out(xv, mats(layer.routed, e), act, act_gscales)
            for h in range(len(xv)):
                out[h] += w * y[h]
        if layer.shared is not None:
            y = expert_out(xv, mats(layer.shared, 0), act, act_gscales)
            for h in range(len(xv)):
                out[h] += y[h]
        results.append((chosen, wts, out, logits))
    return results
