"""Pins of the oracle's MXFP4 codec, quantizer and dequantizer (CPU only).

Each test checks the oracle against something other than itself: the format facts printed on
the pages (tests/golden/mxfp4_format.txt), closed forms built independently of the oracle's
code (fp32 bit patterns), brute-force nearest search, and exact round trips of representable
tensors.
"""

import os

import numpy as np

from oracle import brute
from oracle import moe as omoe
from oracle import mxfp4 as omx
from oracle import nvfp4 as onv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            key, val = line.split()
            vals[key] = float(val)
    return vals


def test_format_facts():
    fmt = golden("mxfp4_format.txt")
    assert omx.GROUP == fmt["block_size_along_k"] == 2 * fmt["nvfp4_block_size_along_k"]
    assert onv.GROUP == fmt["nvfp4_block_size_along_k"]
    # exponent-only 8-bit scale: 256 codes, every finite one a power of two
    vals = omx.e8m0_decode(np.arange(2 ** int(fmt["scale_bits"])))
    fin = vals[np.isfinite(vals)]
    assert len(fin) == 255
    m, _ = np.frexp(fin)
    assert np.all(m == 0.5), "exponent only: no mantissa bits"
    # the element grid is the NVFP4 one (same e2m1)
    assert 2 ** (1 + int(fmt["e2m1_exponent_bits"]) + int(fmt["e2m1_mantissa_bits"])) == 16


def test_e8m0_decode_against_fp32_bit_patterns():
    """Byte b in 1..254 is the fp32 number whose exponent field is b and mantissa 0; 0 is 2^-127
    (the fp32 subnormal 0x00400000); 255 is NaN."""
    b = np.arange(1, 255, dtype=np.uint32)
    ref = (b << np.uint32(23)).view(np.float32).astype(np.float64)
    assert np.array_equal(omx.e8m0_decode(b), ref)
    assert omx.e8m0_decode(0) == np.array([0x00400000], np.uint32).view(np.float32)[0]
    assert np.isnan(omx.e8m0_decode(255))
    # the scalar decode of the independent brute-force module agrees on every code
    for byte in range(255):
        assert brute.e8m0(byte) == float(omx.e8m0_decode(byte))


def test_representable_round_trip():
    """W = v * 2^e with v on the E2M1 grid and every block holding a magnitude of 4 or 6 (so its
    shared exponent is e): quantize(dequantize) returns the identical codes and scales."""
    rng = np.random.default_rng(7)
    n, k = 24, 256
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    codes[codes == 8] = 0                      # no -0: it re-encodes as +0
    blocks = codes.reshape(n, k // 32, 32)
    blocks[:, :, 5] = rng.choice([6, 7, 14, 15], size=(n, k // 32))   # magnitude 4 or 6 in every block
    codes = blocks.reshape(n, k)
    e = rng.integers(-20, 20, (n, k // 32))
    scales = (e + 127).astype(np.uint8)
    packed = onv.pack_nibbles(codes)
    w = omx.dequantize(packed, scales)
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)   # fp32-exact
    p2, s2 = omx.quantize(w.astype(np.float32))
    assert np.array_equal(s2, scales)
    assert np.array_equal(p2, packed)


def test_quantizer_matches_brute_force_nearest():
    """Every element is the nearest point of the block's grid {+-v * 2^e}, ties to the even code;
    the block exponent is floor(log2(amax)) - 2, found here by a search over exponents."""
    rng = np.random.default_rng(11)
    w = (rng.normal(0, 1, (8, 128)) * np.exp2(rng.integers(-6, 6, (8, 1)))).astype(np.float32)
    w[0, :32] = 0.0                                          # an all-zero block
    w[1, 3] = 7.5 * 2.0 ** -3; w[1, 0:32] = np.where(np.arange(32) == 3, w[1, 0:32], 0.1)  # clip case
    packed, scales = omx.quantize(w)
    deq = omx.dequantize(packed, scales)
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for r in range(w.shape[0]):
        for b in range(w.shape[1] // 32):
            blk = w[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            if amax == 0:
                assert scales[r, b] == 0 and np.all(deq[r, 32 * b:32 * b + 32] == 0)
                continue
            e = -200
            while 2.0 ** (e + 1) <= amax:     # largest e with 2^e <= amax, by search
                e += 1
            while 2.0 ** e > amax:
                e -= 1
            assert scales[r, b] == e - 2 + 127
            for j in range(32):
                x = blk[j] / 2.0 ** (e - 2)
                mag = min(abs(x), 6.0)
                best = min(range(8), key=lambda c: (abs(grid[c] - mag), c & 1))
                want = (-grid[best] if x < 0 else grid[best]) * 2.0 ** (e - 2)
                assert deq[r, 32 * b + j] == want, (r, b, j)


def test_storage_cost():
    # 4 bits per element plus one byte per 32 elements
    assert omx.storage_bytes(64, 256) == 64 * 256 * (0.5 + 1 / 32)


def _mx_bank(rng, e, h, i, sigma=0.05):
    w13 = rng.normal(0, sigma, (e, 2 * i, h)).astype(np.float32)
    w2 = rng.normal(0, sigma, (e, h, i)).astype(np.float32)
    q13 = [omx.quantize(w13[x]) for x in range(e)]
    q2 = [omx.quantize(w2[x]) for x in range(e)]
    return omoe.ArrayBank(np.stack([q[0] for q in q13]), np.stack([q[1] for q in q13]), None,
                          np.stack([q[0] for q in q2]), np.stack([q[1] for q in q2]), None, fmt="mxfp4")


def test_mxfp4_layer_matches_brute_force():
    """oracle.moe on MXFP4 banks against the independent scalar loop of oracle.brute."""
    rng = np.random.default_rng(3)
    h, i, e, k, t = 64, 32, 6, 2, 5
    routed = _mx_bank(rng, e, h, i)
    shared = _mx_bank(rng, 1, h, i)
    w_router = (np.frombuffer(rng.normal(0, 0.2, (e, h)).astype(np.float32).tobytes(), np.uint32) >> 16).astype(
        np.uint16).reshape(e, h)
    x = (np.frombuffer(rng.normal(0, 1, (t, h)).astype(np.float32).tobytes(), np.uint32) >> 16).astype(
        np.uint16).reshape(t, h)
    layer = omoe.Layer(w_router, None, routed, shared, k)
    res = omoe.forward(x, layer)
    ref = brute.forward(x, layer)
    for tok, (ids, wts, out, _) in enumerate(ref):
        assert res["ids"][tok].tolist() == ids
        np.testing.assert_allclose(res["weights"][tok], wts, rtol=1e-12, atol=1e-15)
        scale = max(np.abs(out).max(), 1e-300)
        np.testing.assert_allclose(res["out"][tok], out, rtol=1e-10, atol=1e-12 * scale)


def test_dense_special_case_is_swiglu_on_dequantized_weights():
    """E = 1, k = 1, no shared expert: the layer is SwiGLU with the dequantized MXFP4 matrices."""
    rng = np.random.default_rng(5)
    h, i, t = 64, 64, 4
    bank = _mx_bank(rng, 1, h, i)
    x = (np.frombuffer(rng.normal(0, 1, (t, h)).astype(np.float32).tobytes(), np.uint32) >> 16).astype(
        np.uint16).reshape(t, h)
    w_router = np.zeros((1, h), np.uint16)
    res = omoe.forward(x, omoe.Layer(w_router, None, bank, None, 1))
    xv = omoe.bf16_to_float(x)
    w13 = omx.dequantize(bank.w13[0], bank.w13_scale[0])
    wd = omx.dequantize(bank.w2[0], bank.w2_scale[0])
    g, u = xv @ w13[:i].T, xv @ w13[i:].T
    ref = (g / (1 + np.exp(-g)) * u) @ wd.T
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-12)
