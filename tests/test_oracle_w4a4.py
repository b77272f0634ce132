"""Pins of the oracle's W4A4 (MXFP4 weights and activations) layer (CPU only).

Each test checks oracle.w4a4 against something other than itself: torch's float32 -> bf16
conversion (a library routine), the independent scalar module oracle.brute (nearest-value
search over the E2M1 table, its own bf16 rounding and its own per-token layer loop), exact
round trips of representable activations, and the reduction to the W4A16 oracle when the
activation quantization is the identity.
"""

import numpy as np
import torch

from oracle import brute
from oracle import moe as omoe
from oracle import mxfp4 as omx
from oracle import w4a4 as oa4

from helpers import random_layer, random_x


def test_bf16_rounding_against_torch_and_brute():
    rng = np.random.default_rng(11)
    mags = 10.0 ** rng.integers(-44, 38, 20000)
    v32 = (rng.standard_normal(20000) * mags).astype(np.float32)
    v32[:50] = 0.0
    v32[50:60] = np.float32(3.0e38)        # rounds past the largest bf16 -> inf
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oa4.float_to_bf16_bits(v32.astype(np.float64))
    assert np.array_equal(got, ref)
    for x in v32[:3000]:
        b = brute.bf16_round(float(x))
        assert b == omoe.bf16_to_float(oa4.float_to_bf16_bits(np.array([x], np.float64)))[0]
    # a float64 value just above a bf16 tie: the nearest bf16 is the upper neighbour, although
    # rounding through float32 first would land on the tie and pick the even (lower) one
    v = 112896.0029525933
    assert oa4.float_to_bf16_bits(np.array([v]))[0] == 0x47DD
    assert brute.bf16_round(v) == omoe.bf16_to_float(np.array([0x47DD], np.uint16))[0]


def _rows_with_edge_groups(rng, m, k):
    x = rng.standard_normal((m, k)) * 10.0 ** rng.integers(-3, 4, (m, 1))
    x[0, :32] = 0.0                                   # all-zero group
    x[1, :32] = rng.standard_normal(32) * 1e-39       # bf16 subnormals: exponent clamps to -127
    x[2, :32] = 1e38 * rng.standard_normal(32)        # huge group
    x[3, 32:64] = 0.75 * 2.0 ** rng.integers(-5, 5)   # every element on an E2M1 tie
    x[3, 64:96] = np.array([6.0, -3.5, 2.5, 1.25, 0.25] + [0.0] * 27) * 2.0 ** -3
    bits = oa4.float_to_bf16_bits(x)
    return bits, omoe.bf16_to_float(bits)


def test_activation_quantizer_against_brute():
    rng = np.random.default_rng(12)
    bits, x = _rows_with_edge_groups(rng, 6, 128)
    packed, scales = oa4.quantize_act(x)
    assert packed.shape == (6, 64) and scales.shape == (6, 4)
    deq = omx.dequantize(packed, scales)
    for r in range(x.shape[0]):
        ref = brute.mx_fake_quant([float(v) for v in x[r]])
        assert np.array_equal(deq[r], np.array(ref)), r
        for g in range(4):
            _, e = brute.mx_group([float(v) for v in x[r, 32 * g:32 * g + 32]])
            assert int(scales[r, g]) == e + 127
    assert int(scales[0, 0]) == 0 and not packed[0, :16].any()   # zero group: smallest scale, zero codes


def test_representable_activations_are_kept():
    """x = v * 2^e with v on the E2M1 grid and a magnitude of 4 or 6 in every group: exact."""
    rng = np.random.default_rng(13)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    v = rng.choice(grid, (4, 256)) * rng.choice([-1.0, 1.0], (4, 256))
    v[:, ::32] = rng.choice([4.0, 6.0, -4.0, -6.0], (4, 8))
    x = v * np.repeat(2.0 ** rng.integers(-20, 20, (4, 8)), 32, axis=1)
    assert np.array_equal(oa4.fake_quant_act(x), x)


def test_gate_up_reduces_to_w4a16_when_quantization_is_exact():
    rng = np.random.default_rng(14)
    layer = random_layer(rng, 128, 64, 1, 1, shared=False, fmt="mxfp4")
    ew = layer.routed[0]
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    v = rng.choice(grid, (5, 128)) * rng.choice([-1.0, 1.0], (5, 128))
    v[:, ::32] = 6.0
    x = v * 2.0 ** -3
    assert np.array_equal(oa4.gate_up_a4(x, ew), omoe.gate_up(x, ew))
    # and with general inputs the 4-bit activations do change the result
    xg = rng.standard_normal((5, 128))
    rel = np.linalg.norm(oa4.gate_up_a4(xg, ew) - omoe.gate_up(xg, ew)) / np.linalg.norm(omoe.gate_up(xg, ew))
    assert rel > 1e-2


def test_w4a4_layer_matches_brute_force():
    rng = np.random.default_rng(15)
    layer = random_layer(rng, 64, 64, 4, 2, shared=True, fmt="mxfp4", bias=True)
    x = random_x(rng, 6, 64)
    res = oa4.forward(x, layer)
    ref = brute.forward(x, layer, act="mxfp4")
    out = np.array([r[2] for r in ref])
    assert np.array_equal(res["ids"], np.array([r[0] for r in ref]))
    assert np.allclose(res["out"], out, rtol=1e-10, atol=1e-12 * np.abs(out).max())
    # the W4A16 layer on the same weights is measurably different (the activations are 4-bit)
    w16 = omoe.forward(x, layer)["out"]
    assert np.linalg.norm(w16 - out) / np.linalg.norm(out) > 1e-2


def test_w4a4_stages_compose_to_the_layer():
    """grouped gate/up -> bf16 h -> grouped down -> combine reproduces forward()."""
    rng = np.random.default_rng(16)
    layer = random_layer(rng, 64, 32, 3, 2, shared=False, fmt="mxfp4")
    x = random_x(rng, 7, 64)
    res = oa4.forward(x, layer)
    a_rows = omoe.bf16_to_float(x)[res["sorted_slot"] // 2]
    h = oa4.grouped_gate_up_a4(a_rows, res["offsets"], layer.routed)
    y = oa4.grouped_down_a4(oa4.round_h(h), res["offsets"], layer.routed)
    out = omoe.combine(y, res["slot_to_row"], res["weights"])
    assert np.array_equal(out, res["out"])
