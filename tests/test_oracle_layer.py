"""Pins of the oracle's router, top-k, permutation and whole-layer forward (CPU only).

The layer oracle (oracle.moe) is checked against an independent scalar
implementation (oracle.brute), against brute-force selection and sorting,
against a textbook SwiGLU FFN in the E=1, k=1 special case, and against exact
one-hot products that pin nibble order, scale indexing and gate/up order.
"""

import numpy as np
import pytest
import torch

import helpers
from oracle import brute
from oracle import moe as omoe
from oracle import nvfp4 as onv


# ------------------------------------------------------------------------- top-k

def _brute_topk(row, k):
    return sorted(range(len(row)), key=lambda e: (-row[e], e))[:k]


def test_topk_matches_brute_force_with_ties():
    rng = np.random.default_rng(0)
    logits = rng.normal(0, 1, (200, 40)).round(1)          # many exact ties
    logits[0, :] = 0.5                                     # all equal -> lowest indices
    logits[1, :] = -0.0
    logits[1, 3] = 0.0
    ids, w = omoe.topk(logits, 8)
    for t in range(len(logits)):
        assert ids[t].tolist() == _brute_topk(logits[t].tolist(), 8)
    assert ids[0].tolist() == list(range(8))
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)                 # descending logits -> descending weights


def test_topk_weights_equal_renormalised_full_softmax():
    rng = np.random.default_rng(1)
    logits = rng.normal(0, 2, (50, 32))
    ids, w = omoe.topk(logits, 6)
    full = np.exp(logits - logits.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)


def test_router_logits_match_library_matmul_and_bias():
    rng = np.random.default_rng(2)
    x = helpers.random_x(rng, 7, 64)
    wr = helpers.random_x(rng, 12, 64)
    b = rng.normal(0, 1, 12).astype(np.float32)
    want = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double()
            @ torch.from_numpy(wr.view(np.int16)).view(torch.bfloat16).double().T).numpy() + b.astype(np.float64)
    np.testing.assert_allclose(omoe.router_logits(x, wr, b), want, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------------------- permute

def test_permute_matches_brute_force_and_invariants():
    rng = np.random.default_rng(3)
    for t, k, e in [(1, 1, 1), (5, 2, 4), (64, 8, 320), (33, 3, 7)]:
        ids = np.stack([rng.choice(e, size=k, replace=False) for _ in range(t)]).astype(np.int32)
        counts, offsets, sorted_slot, slot_to_row = omoe.permute(ids, e)
        flat = ids.ravel().tolist()
        want = [s for ex in range(e) for s in range(t * k) if flat[s] == ex]
        assert sorted_slot.tolist() == want
        assert counts.tolist() == [flat.count(ex) for ex in range(e)]
        assert offsets[0] == 0 and offsets[-1] == t * k and np.all(np.diff(offsets) == counts)
        assert np.array_equal(sorted_slot[slot_to_row], np.arange(t * k))
        sorted_ids = ids.ravel()[sorted_slot]
        assert np.all(np.diff(sorted_ids) >= 0)


# ------------------------------------------------------------------------- whole layer

def _compare_with_brute(x, layer, tokens=None):
    res = omoe.forward(x if tokens is None else x[tokens], layer)
    br = brute.forward(x, layer, tokens)
    for i, (chosen, wts, out, logits) in enumerate(br):
        np.testing.assert_allclose(res["logits"][i], logits, rtol=1e-12, atol=1e-12)
        assert res["ids"][i].tolist() == chosen
        np.testing.assert_allclose(res["weights"][i], wts, rtol=1e-12, atol=1e-15)
        scale = max(np.abs(out).max(), 1e-300)
        np.testing.assert_allclose(res["out"][i], out, rtol=1e-10, atol=1e-12 * scale)
    return res


def test_forward_matches_brute_on_small_random_layers():
    rng = np.random.default_rng(4)
    for (t, h, i, e, k, shared, bias) in [(5, 32, 16, 4, 2, True, False), (3, 48, 32, 6, 3, False, True),
                                           (4, 16, 16, 1, 1, False, False), (2, 32, 16, 5, 5, True, True)]:
        layer = helpers.random_layer(rng, h, i, e, k, shared=shared, bias=bias)
        x = helpers.random_x(rng, t, h)
        _compare_with_brute(x, layer)


@pytest.mark.slow
def test_forward_matches_brute_on_tiny_workload():
    """The T=16, H=256, I=128, E=8 top-2 + shared layer, generated on the CPU; all tokens."""
    from nvfp4_weight_quantized_amd import synth
    wl = synth.WORKLOADS["tiny"]
    layer = helpers.oracle_layer(wl)
    layer.routed = helpers.stack_bank(layer.routed)
    x = helpers.bf16_bits(synth.activations(wl))
    _compare_with_brute(x, layer, tokens=list(range(wl.T)))


def test_dense_special_case_is_a_textbook_swiglu():
    """E = 1, k = 1, no shared expert: out = (silu(x Wg^T) * (x Wu^T)) Wd^T on brute-decoded weights."""
    rng = np.random.default_rng(5)
    layer = helpers.random_layer(rng, 64, 32, 1, 1, shared=False)
    x = helpers.random_x(rng, 9, 64)
    res = omoe.forward(x, layer)
    assert np.all(res["ids"] == 0) and np.all(res["weights"] == 1.0)
    wg, wu, wd = (torch.tensor(m, dtype=torch.float64) for m in brute.dequant_expert(layer.routed[0]))
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double()
    want = (torch.nn.functional.silu(xt @ wg.T) * (xt @ wu.T)) @ wd.T
    np.testing.assert_allclose(res["out"], want.numpy(), rtol=1e-12, atol=1e-14)


def test_one_hot_rows_select_dequantized_columns_exactly():
    """x = e_h: gate/up pre-activations are column h of the dequantized gate and up matrices."""
    rng = np.random.default_rng(6)
    layer = helpers.random_layer(rng, 32, 16, 1, 1, shared=False)
    ew = layer.routed[0]
    wg, wu, wd = brute.dequant_expert(ew)
    for h in (0, 1, 15, 16, 31):
        a = np.zeros((1, 32))
        a[0, h] = 1.0
        got = omoe.gate_up(a, ew)[0]
        g = np.array([row[h] for row in wg])
        u = np.array([row[h] for row in wu])
        assert np.array_equal(got, omoe.silu(g) * u)
    hvec = np.zeros((1, 16))
    hvec[0, 5] = 1.0
    assert np.array_equal(omoe.down(hvec, ew)[0], np.array([row[5] for row in wd]))


def test_gate_up_order_is_observable():
    """Swapping the gate and up halves of w13 changes the output far beyond the parity tolerance."""
    rng = np.random.default_rng(7)
    layer = helpers.random_layer(rng, 64, 32, 3, 2, shared=True)
    x = helpers.random_x(rng, 6, 64)
    ref = omoe.forward(x, layer)["out"]
    swapped = []
    for ew in layer.routed:
        i = ew.w13.shape[0] // 2
        swapped.append(omoe.ExpertWeights(np.concatenate([ew.w13[i:], ew.w13[:i]]),
                                          np.concatenate([ew.w13_scale[i:], ew.w13_scale[:i]]),
                                          ew.w13_gscale[::-1].copy(), ew.w2, ew.w2_scale, ew.w2_gscale))
    layer.routed = swapped
    bad = omoe.forward(x, layer)["out"]
    rel = np.linalg.norm(bad - ref) / np.linalg.norm(ref)
    assert rel > 0.1


def test_every_routed_expert_contributes():
    """No activation scale exists, so no expert can be zeroed: each used expert's rows are nonzero."""
    rng = np.random.default_rng(8)
    layer = helpers.random_layer(rng, 32, 16, 4, 2, shared=True)
    x = helpers.random_x(rng, 12, 32)
    res = omoe.forward(x, layer)
    a_rows = omoe.bf16_to_float(x)[res["sorted_slot"] // 2]
    for e in range(4):
        r0, r1 = res["offsets"][e], res["offsets"][e + 1]
        if r1 > r0:
            y = omoe.expert_ffn(a_rows[r0:r1], layer.routed[e])
            assert np.all(np.abs(y).max(axis=1) > 0)
    assert np.all(np.abs(res["out"]).max(axis=1) > 0)


def test_grouped_stages_compose_to_forward():
    rng = np.random.default_rng(9)
    layer = helpers.random_layer(rng, 32, 16, 5, 2, shared=False)
    x = helpers.random_x(rng, 10, 32)
    res = omoe.forward(x, layer)
    a_rows = omoe.bf16_to_float(x)[res["sorted_slot"] // 2]
    h = omoe.grouped_gate_up(a_rows, res["offsets"], layer.routed)
    y = omoe.grouped_down(h, res["offsets"], layer.routed)
    out = omoe.combine(y, res["slot_to_row"], res["weights"])
    np.testing.assert_allclose(out, res["out"], rtol=1e-12, atol=1e-14)


def test_quantize_dequantize_layer_cosine():
    """Weights of the configs' recipe survive NVFP4 with cosine > 0.99 (page reports 0.998 on real weights)."""
    rng = np.random.default_rng(10)
    w = rng.normal(0, 0.02, (256, 512)).astype(np.float32)
    d = onv.gscale_modelopt(np.abs(w).max())
    wq = onv.dequantize(*onv.quantize(w, d), d)
    cos = (w.astype(np.float64) * wq).sum() / np.linalg.norm(w) / np.linalg.norm(wq)
    assert cos > 0.99
