"""Pins of the oracle's NVFP4 W4A4 layer (NVFP4 weights and activations; CPU only).

Each test checks oracle.nvfp4_w4a4 against something other than itself: the independent scalar
module oracle.brute (a nearest-value search over all finite E4M3 codes and the E2M1 table, fp32
rounding emulated through struct, its own per-token layer loop), exact round trips of
representable activations, the reduction to the W4A16 oracle when the activation quantization is
exact, the power-of-two scale equivariance that fixes where the global scale enters, and the
refusal of a missing activation scale (the pages' "every expert multiplied by zero" failure).
"""

import math

import numpy as np
import pytest

from oracle import brute
from oracle import moe as omoe
from oracle import nvfp4 as onv
from oracle import nvfp4_w4a4 as onw
from oracle import w4a4 as oa4

from helpers import random_layer, random_x


def _edge_rows(rng, m, k):
    """bf16-exact rows whose groups hit the quantizer's special cases."""
    x = rng.standard_normal((m, k)) * 10.0 ** rng.integers(-2, 3, (m, 1))
    x[0, :16] = 0.0                                            # all-zero group: scale 0, codes 0
    x[1, :16] = rng.standard_normal(16) * 1e-6                 # tiny group: E4M3 subnormal or zero scale
    x[2, :16] = rng.standard_normal(16) * 1e6                  # huge group: scale capped at 448, codes saturate
    x[3, 16:32] = np.array([6, -3, 2.5, 1.25, .25, .75, 5, -5, 0, 3.5, -1.75, 1, 2, 4, -6, .5]) * 0.125
    x[4, 16:32] = -0.0
    bits = oa4.float_to_bf16_bits(x)
    return omoe.bf16_to_float(bits)


@pytest.mark.parametrize("d", [None, 1.0, 2.0 ** -20, 3.0e-3, 7.5])
def test_activation_quantizer_against_brute(d):
    rng = np.random.default_rng(31)
    x = _edge_rows(rng, 6, 64)
    d = onv.gscale_modelopt(np.abs(x).max()) if d is None else np.float32(d)
    packed, scales = onw.quantize_act(x, d)
    assert packed.shape == (6, 32) and scales.shape == (6, 4)
    vals = onw.act_values(x, d)
    for r in range(x.shape[0]):
        for g in range(4):
            ref_v, ref_s = brute.nv_group([float(v) for v in x[r, 16 * g:16 * g + 16]], float(d))
            assert onv.e4m3_decode(scales[r, g]) == ref_s, (r, g)
            assert np.array_equal(vals[r, 16 * g:16 * g + 16], np.array(ref_v) * ref_s), (r, g)
    fq = onw.fake_quant_act(x, d)
    for r in range(x.shape[0]):
        assert np.array_equal(fq[r], np.array(brute.nv_fake_quant([float(v) for v in x[r]], float(d))))
    # the special cases did what they should
    assert not packed[0, :8].any() and scales[0, 0] == 0
    assert np.array_equal(vals[4, 16:32], np.zeros(16))


def test_saturation_and_cap():
    """A group far above 6 * 448 * d gets the largest scale and codes clamped to +-6."""
    x = np.zeros((1, 16))
    x[0, :4] = [1e6, -1e6, 3e5, 0.0]
    vals = onw.act_values(x, np.float32(1.0))
    assert list(vals[0, :4]) == [6 * 448.0, -6 * 448.0, 6 * 448.0, 0.0]


def test_representable_activations_are_kept():
    """x = v * s * d with v on the E2M1 grid, a magnitude of 6 in every group, s an E4M3 value and
    d a power of two: the quantizer returns the same values."""
    rng = np.random.default_rng(32)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    v = rng.choice(grid, (4, 128)) * rng.choice([-1.0, 1.0], (4, 128))
    v[:, ::16] = rng.choice([6.0, -6.0], (4, 8))
    s = onv.e4m3_decode(rng.integers(1, 0x7F, (4, 8)))
    d = 2.0 ** -7
    x = v * np.repeat(s, 16, axis=1) * d
    assert np.array_equal(oa4.float_to_bf16_bits(x).astype(np.float64) * 0 + x, x)
    assert np.array_equal(onw.fake_quant_act(x, d), x)
    assert np.array_equal(onw.act_values(x, d), v * np.repeat(s, 16, axis=1))


def test_act_values_are_exact_in_bf16_and_fp16():
    """e2m1 * e4m3 has at most 6 significant bits and lies in [2^-10, 2688]: exact in both 16-bit types."""
    rng = np.random.default_rng(33)
    x = _edge_rows(rng, 6, 64)
    vals = onw.act_values(x, onv.gscale_modelopt(np.abs(x).max()))
    assert np.array_equal(omoe.bf16_to_float(oa4.float_to_bf16_bits(vals)), vals)
    assert np.array_equal(vals.astype(np.float16).astype(np.float64), vals)
    nz = np.abs(vals[vals != 0])
    assert nz.max() <= 2688.0 and nz.min() >= 2.0 ** -10


def test_power_of_two_scale_equivariance():
    """Scaling the rows and the global scale by the same power of two leaves the 4-bit operand alone
    (the global scale divides the values before the block scale is chosen)."""
    rng = np.random.default_rng(34)
    x = rng.standard_normal((3, 64)) * 0.1
    x = omoe.bf16_to_float(oa4.float_to_bf16_bits(x))
    d = onv.gscale_modelopt(np.abs(x).max())
    for c in (2.0 ** 5, 2.0 ** -7):
        assert np.array_equal(onw.act_values(x * c, np.float32(d * c)), onw.act_values(x, d))
        assert np.array_equal(onw.fake_quant_act(x * c, np.float32(d * c)), onw.fake_quant_act(x, d) * c)


def test_gate_up_reduces_to_w4a16_when_quantization_is_exact():
    rng = np.random.default_rng(35)
    layer = random_layer(rng, 128, 64, 1, 1, shared=False)
    ew = layer.routed[0]
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    v = rng.choice(grid, (5, 128)) * rng.choice([-1.0, 1.0], (5, 128))
    v[:, ::16] = 6.0
    x = v * 2.0 ** -3
    assert np.array_equal(onw.gate_up_a4(x, ew, 2.0 ** -3), omoe.gate_up(x, ew))
    xg = rng.standard_normal((5, 128))
    xg = omoe.bf16_to_float(oa4.float_to_bf16_bits(xg))
    ref = omoe.gate_up(xg, ew)
    rel = np.linalg.norm(onw.gate_up_a4(xg, ew, onv.gscale_modelopt(np.abs(xg).max())) - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 0.2


def _scales_for(layer, x_bits):
    """d_x from the token rows, d_h from the W4A16 layer's h (a calibration, as a caller would do)."""
    x = omoe.bf16_to_float(x_bits)
    d_x = onv.gscale_modelopt(np.abs(x).max())
    h = onw.gate_up_a4(x, layer.routed[0], d_x)
    d_h = onv.gscale_modelopt(max(np.abs(h).max(), 1e-30))
    return d_x, d_h


def test_w4a4_layer_matches_brute_force():
    rng = np.random.default_rng(36)
    layer = random_layer(rng, 64, 64, 4, 2, shared=True, bias=True)
    x = random_x(rng, 6, 64)
    d_x, d_h = _scales_for(layer, x)
    res = onw.forward(x, layer, d_x, d_h)
    ref = brute.forward(x, layer, act="nvfp4", act_gscales=(float(d_x), float(d_h)))
    out = np.array([r[2] for r in ref])
    assert np.array_equal(res["ids"], np.array([r[0] for r in ref]))
    assert np.allclose(res["out"], out, rtol=1e-10, atol=1e-12 * np.abs(out).max())
    # the W4A16 layer on the same weights is measurably different (the activations are 4-bit)
    w16 = omoe.forward(x, layer)["out"]
    assert np.linalg.norm(w16 - out) / np.linalg.norm(out) > 1e-3


def test_w4a4_stages_compose_to_the_layer():
    """grouped gate/up -> bf16 h -> grouped down -> combine reproduces forward()."""
    rng = np.random.default_rng(37)
    layer = random_layer(rng, 64, 32, 3, 2, shared=False)
    x = random_x(rng, 7, 64)
    d_x, d_h = _scales_for(layer, x)
    res = onw.forward(x, layer, d_x, d_h)
    a_rows = omoe.bf16_to_float(x)[res["sorted_slot"] // 2]
    h = onw.grouped_gate_up_a4(a_rows, res["offsets"], layer.routed, d_x)
    y = onw.grouped_down_a4(onw.round_h(h), res["offsets"], layer.routed, d_h)
    assert np.array_equal(y, res["y_rows"])
    out = omoe.combine(y, res["slot_to_row"], res["weights"])
    assert np.array_equal(out, res["out"])


@pytest.mark.parametrize("bad", [0.0, -1e-3, math.nan, math.inf])
def test_missing_activation_scale_is_refused(bad):
    """A zero (or otherwise unusable) activation scale would multiply every expert by zero; the
    oracle refuses it instead of returning zeros."""
    rng = np.random.default_rng(38)
    layer = random_layer(rng, 64, 32, 2, 1, shared=False)
    x = random_x(rng, 3, 64)
    with pytest.raises(ValueError):
        onw.forward(x, layer, bad, 1.0)
    with pytest.raises(ValueError):
        onw.forward(x, layer, 1.0, bad)
    with pytest.raises(ValueError):
        onw.quantize_act(omoe.bf16_to_float(x), bad)
