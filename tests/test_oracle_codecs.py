"""Pins of the oracle's NVFP4 codecs, quantizer and global-scale conventions (CPU only).

Each test checks the oracle against something other than itself: facts printed
on the pages (tests/golden/*.txt), closed forms, a library routine (torch's
float8_e4m3fn), or brute force.
"""

import os

import numpy as np
import pytest
import torch

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


# ------------------------------------------------------------------------- E2M1

def test_e2m1_value_set_from_format_facts():
    """2 exponent bits + 1 mantissa bit with max 6.0 -> exactly {0,.5,1,1.5,2,3,4,6} and their negatives."""
    fmt = golden("nvfp4_format.txt")
    vals = onv.e2m1_decode(np.arange(16))
    mags = sorted(set(np.abs(vals).tolist()))
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.abs(vals).max() == fmt["e2m1_max"]
    # 16 codes = 2^(1 + exponent bits + mantissa bits)
    assert 2 ** (1 + int(fmt["e2m1_exponent_bits"]) + int(fmt["e2m1_mantissa_bits"])) == 16
    # top bit is the sign: code c and c|8 are negatives of each other
    assert np.array_equal(vals[8:], -vals[:8])
    # independent enumeration: every (e, m) with bias 1, subnormal at e == 0
    brute = []
    for e in range(4):
        for m in range(2):
            brute.append(m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1))
    assert np.array_equal(vals[:8], np.array(brute))


def _nearest_e2m1_brute(q):
    """Nearest grid value by exhaustive search; ties go to the code with mantissa bit 0; saturate."""
    grid = [(0.0, 0), (0.5, 1), (1.0, 0), (1.5, 1), (2.0, 0), (3.0, 1), (4.0, 0), (6.0, 1)]
    mag = min(abs(q), 6.0)
    best = min(grid, key=lambda gm: (abs(gm[0] - mag), gm[1]))
    return -best[0] if q < 0 else best[0]


def test_e2m1_rounding_matches_brute_force():
    rng = np.random.default_rng(5)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mids = (grid[1:] + grid[:-1]) / 2
    q = np.concatenate([rng.uniform(-8, 8, 4000), mids, -mids, grid, -grid, [6.5, 7.0, 100.0, -7.0, 1e-30]])
    q = q.astype(np.float32).astype(np.float64)
    got = onv.e2m1_round(q)
    want = np.array([_nearest_e2m1_brute(v) for v in q])
    assert np.array_equal(got, want)
    codes = onv.e2m1_encode(q)
    assert np.array_equal(onv.e2m1_decode(codes), got)
    # ties: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4
    assert onv.e2m1_round(mids).tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]


# ------------------------------------------------------------------------- E4M3

def test_e4m3_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = onv.e4m3_decode(np.arange(256))
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e4m3_extremes():
    fmt = golden("nvfp4_format.txt")
    v = onv.e4m3_decode(np.arange(256))
    assert np.nanmax(v) == fmt["e4m3_max"] == v[0x7E]
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isnan(v).sum() == 2
    assert v[0x01] == 2.0 ** -9
    assert v[0x08] == 2.0 ** -6


def test_e4m3_rounding_matches_torch_cast():
    """RNE onto the E4M3 grid == torch's float -> float8_e4m3fn cast, including exact ties."""
    rng = np.random.default_rng(7)
    grid = onv.e4m3_decode(np.arange(0x7F))
    mids = (grid[1:] + grid[:-1]) / 2
    t = np.concatenate([rng.uniform(0, 448, 3000), np.exp2(rng.uniform(-12, 8.8, 3000)), mids, grid,
                        [0.0, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -10]])
    t = np.minimum(t.astype(np.float32), np.float32(448))
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(onv.e4m3_encode(t.astype(np.float64)), ref)


def test_e4m3_saturates_at_448():
    assert onv.e4m3_round(np.array([448.0, 460.0, 500.0, 1e9])).tolist() == [448.0] * 4


# ------------------------------------------------------------------------- global scales

def test_global_scale_worked_example():
    """The discussion page's pair: amax/(448*6) vs (448*6)/amax are fp32 reciprocals."""
    g = golden("global_scale_reciprocal.txt")
    amax = 2688.0 / g["compressed_tensors_quant_scale"]
    assert amax == 0.125
    d = onv.gscale_modelopt(amax)
    q = onv.gscale_compressed_tensors(amax)
    assert float(d) == g["modelopt_dequant_scale"]
    assert float(q) == g["compressed_tensors_quant_scale"]
    assert np.float32(d * q) == np.float32(1.0)
    assert float(onv.gscale_from_quant_scale(q)) == g["modelopt_dequant_scale"]


def test_global_scale_reciprocal_invariant_random():
    rng = np.random.default_rng(3)
    amax = np.exp2(rng.uniform(-12, 4, 20000)).astype(np.float32)
    d = onv.gscale_modelopt(amax)
    q = onv.gscale_compressed_tensors(amax)
    prod = (d * q).astype(np.float32).astype(np.float64)
    assert np.all(np.abs(prod - 1.0) <= 2.0 ** -23)
    back = onv.gscale_from_quant_scale(q)
    ulp = np.spacing(d.astype(np.float32))
    assert np.all(np.abs(back.astype(np.float64) - d.astype(np.float64)) <= ulp)


# ------------------------------------------------------------------------- quantizer

def test_storage_cost_per_element():
    fmt = golden("nvfp4_format.txt")
    n, k = 48, 256
    assert onv.storage_bytes(n, k) == fmt["bytes_per_element_fp4_plus_scales"] * n * k
    p, s = onv.quantize(np.random.default_rng(0).normal(0, 1, (n, k)).astype(np.float32), 1e-3)
    assert p.nbytes + s.nbytes == onv.storage_bytes(n, k)
    assert p.shape == (n, k // int(fmt["elements_per_byte"])) and s.shape == (n, k // int(fmt["block_size_along_k"]))


def test_nibble_order_low_first():
    codes = np.array([[1, 2, 3, 4]], np.uint8)
    assert onv.pack_nibbles(codes).tolist() == [[0x21, 0x43]]
    assert np.array_equal(onv.unpack_nibbles(onv.pack_nibbles(codes)), codes)


def test_representable_round_trip_is_exact():
    """W = v*s*d with v in E2M1, s in E4M3, every group holding a +-6 and d a power of two
    -> quantize(W) returns the same codes and scales, and dequantize returns W bit for bit."""
    rng = np.random.default_rng(11)
    n, k = 64, 128
    codes = rng.choice([c for c in range(16) if c != 8], size=(n, k)).astype(np.uint8)
    codes[:, ::16] = rng.choice([7, 15], size=(n, k // 16))     # one +-6 per group
    scales = rng.integers(1, 0x7F, size=(n, k // 16)).astype(np.uint8)
    scales[0, 0] = 0x7E                                           # the tensor holds s = 448
    d = np.float32(2.0 ** -14)
    w = onv.dequantize(onv.pack_nibbles(codes), scales, d)
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)
    amax = np.abs(w).max()
    assert amax == 2688.0 * float(d)
    assert onv.gscale_modelopt(amax) == d
    p2, s2 = onv.quantize(w.astype(np.float32), d)
    assert np.array_equal(s2, scales)
    assert np.array_equal(onv.unpack_nibbles(p2), codes)
    assert np.array_equal(onv.dequantize(p2, s2, d), w)


def test_quantizer_idempotent_on_gaussian_weights():
    rng = np.random.default_rng(12)
    for sigma in (0.02, 0.015):
        w = rng.normal(0, sigma, (96, 512)).astype(np.float32)
        d = onv.gscale_modelopt(np.abs(w).max())
        p, s = onv.quantize(w, d)
        w1 = onv.dequantize(p, s, d).astype(np.float32)
        p2, s2 = onv.quantize(w1, d)
        # same scales and same values; codes may differ only by the sign of zero
        # (a small negative weight rounds to code 8 = -0, which dequantizes to -0.0 and re-encodes as 0)
        assert np.array_equal(s2, s)
        assert np.array_equal(onv.dequantize(p2, s2, d), onv.dequantize(p, s, d))
        diff = onv.unpack_nibbles(p2) != onv.unpack_nibbles(p)
        assert set(onv.unpack_nibbles(p)[diff].tolist()) <= {8}
        d2 = onv.gscale_modelopt(np.abs(w1).max())
        assert abs(float(d2) - float(d)) <= np.spacing(d)


def test_quantizer_error_bound_and_cosine():
    """|w - D(Q(w))| <= half an E2M1 step of the group (times the scale) unless saturated; cosine ~ 1."""
    rng = np.random.default_rng(13)
    w = rng.normal(0, 0.02, (128, 1024)).astype(np.float32)
    d = onv.gscale_modelopt(np.abs(w).max())
    p, s = onv.quantize(w, d)
    wq = onv.dequantize(p, s, d)
    sd = np.repeat(onv.e4m3_decode(s), 16, axis=1) * float(d)
    # largest E2M1 spacing below |q| is 2 (between 4 and 6): error <= 1 * s * d, tighter for small q
    q = np.abs(w) / sd
    half_step = np.where(q < 2, 0.25, np.where(q < 4, 0.5, 1.0))
    assert np.all(np.abs(wq - w) <= half_step * sd * (1 + 1e-6) + np.maximum(q - 6, 0) * sd)
    cos = (w.astype(np.float64) * wq).sum() / np.linalg.norm(w) / np.linalg.norm(wq)
    assert cos > 0.99
    assert (onv.e4m3_decode(s) > 0).all()


def test_zero_group_gives_zero_codes():
    w = np.zeros((2, 32), np.float32)
    w[1, 16:] = np.linspace(-1, 1, 16)
    p, s = onv.quantize(w, onv.gscale_modelopt(1.0))
    assert (s[0] == 0).all() and (p[0] == 0).all() and s[1, 0] == 0 and s[1, 1] != 0
    assert np.array_equal(onv.dequantize(p, s, onv.gscale_modelopt(1.0))[0], np.zeros(32))


def test_dequantize_one_element_by_hand():
    """code 0x5 (3.0) low nibble, 0xB (-1.5) high nibble; scale byte 0x3A = (1+2/8)*2^0; d = 0.5."""
    p = np.zeros((1, 8), np.uint8)
    p[0, 0] = 0xB5
    s = np.array([[0x3A]], np.uint8)
    w = onv.dequantize(p, s, np.float32(0.5))
    assert w[0, 0] == 3.0 * 1.25 * 0.5 and w[0, 1] == -1.5 * 1.25 * 0.5 and (w[0, 2:] == 0).all()
