"""GPU parity of the whole layer (moe_nvfp4_forward through the C ABI) against the oracle."""

import numpy as np
import pytest
import torch

import helpers
import parity
from nvfp4_weight_quantized_amd import _lib as L
from nvfp4_weight_quantized_amd import build_bank, build_layer, ops, synth
from oracle import moe as omoe

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


# ----------------------------------------------------------------------------- small layers

SMALL = [
    # T, H, I, E, k, shared, bias, I_shared
    (5, 256, 128, 8, 2, True, False, None),
    (64, 512, 256, 16, 4, True, True, None),
    (300, 512, 256, 16, 4, True, False, None),
    (37, 384, 256, 12, 3, False, True, None),
    (50, 256, 128, 6, 2, True, False, 256),
    (1, 256, 128, 4, 4, True, False, None),
    (129, 256, 128, 64, 8, True, True, None),
    (200, 256, 128, 4, 2, True, False, 256),     # 128-row tiles, shared expert of another width
    (400, 256, 128, 4, 2, True, False, None),    # 128-row tiles with 2 and 1 K chunks
    (700, 384, 256, 40, 8, False, True, None),   # 128-row tiles, multi-block permute, no shared
    (20, 256, 128, 64, 2, True, False, None),    # 8-row tiles; the shared expert spans 8 + 8 + 4 rows
    (300, 256, 256, 4, 2, True, False, 512),     # fp16-row gate/up for the routed experts, shared expert of another width on bf16
]


@pytest.mark.parametrize("case", SMALL, ids=[f"T{c[0]}_H{c[1]}_I{c[2]}_E{c[3]}_k{c[4]}" for c in SMALL])
def test_small_layer_end_to_end(case):
    T, H, I, E, k, shared, bias, i_sh = case
    rng = np.random.default_rng(sum(case[:5]))
    layer = helpers.random_layer(rng, H, I, E, k, shared=shared, bias=bias, i_shared=i_sh)
    x = helpers.random_x(rng, T, H)
    glayer = parity.to_gpu_layer(layer)
    xg = parity.bits_to_bf16(x)
    out, aux = ops.forward(glayer, xg, return_aux=True)
    parity.check_route(aux["logits"], aux["topk_ids"], aux["topk_w"], x, layer.w_router, layer.router_bias, k)
    ids = aux["topk_ids"].cpu().numpy()
    res = parity.reference_for_selection(x, layer, ids)
    assert np.array_equal(aux["expert_counts"].cpu().numpy(), omoe.permute(ids, E)[0])
    parity.assert_close(parity.f64(out), res["out"], "layer")
    out2 = ops.forward(glayer, xg)
    assert torch.equal(out, out2), "two runs differ"


# Shapes on the boundaries between the forward's paths (router kernel, router split along K, top-k
# launch, permutation, 128-row tiles, fp16 token rows and fp16 h); every token checked.
PATHS = [
    # T, H, I, E, k, shared, bias, what the case sits on
    (32, 512, 256, 8, 8, True, True, "few-token router (T = 32), one-workgroup top-k + permutation"),
    (33, 512, 256, 8, 8, True, False, "MFMA router from T = 33, one-workgroup top-k + permutation"),
    (256, 512, 256, 8, 8, True, True, "T*k = 2048: the last one-workgroup top-k + permutation, one router pass"),
    (257, 512, 256, 8, 8, True, True, "T*k = 2056: split router (4 runs), multi-block permutation, fp16 h"),
    (513, 256, 256, 8, 4, True, False, "split capped at H/128 = 2 runs; gate/up on fp16 rows, down on bf16 h (width 256)"),
    (520, 128, 128, 16, 4, True, True, "H = 128: one router pass, top-k launch, four-wave 128-row tiles"),
    (400, 384, 256, 100, 7, False, True, "E = 100, k = 7, 3 router runs (H = 384), no shared expert"),
    (2049, 256, 128, 4, 1, True, False, "k = 1 past one permutation chunk, 2 router runs"),
]


@pytest.mark.parametrize("case", PATHS, ids=[f"T{c[0]}_H{c[1]}_I{c[2]}_E{c[3]}_k{c[4]}" for c in PATHS])
def test_forward_path_boundaries(case):
    T, H, I, E, k, shared, bias, _ = case
    rng = np.random.default_rng(T * 7 + H + E)
    layer = helpers.random_layer(rng, H, I, E, k, shared=shared, bias=bias)
    x = helpers.random_x(rng, T, H)
    glayer = parity.to_gpu_layer(layer)
    xg = parity.bits_to_bf16(x)
    out, aux = ops.forward(glayer, xg, return_aux=True)
    parity.check_route(aux["logits"], aux["topk_ids"], aux["topk_w"], x, layer.w_router, layer.router_bias, k)
    ids = aux["topk_ids"].cpu().numpy()
    assert np.array_equal(aux["expert_counts"].cpu().numpy(), omoe.permute(ids, E)[0])
    res = parity.reference_for_selection(x, layer, ids)
    parity.assert_close(parity.f64(out), res["out"], "layer")
    assert torch.equal(ops.forward(glayer, xg), out), "two runs differ"


def test_skewed_routing_on_128_row_tiles():
    """A few experts take most rows and many take a handful: the XCD ranges of the 128-row GEMMs are
    cut by cost, so most tiles land on few XCDs' ranges; every token is checked."""
    T, H, I, E, k = 900, 256, 128, 24, 2
    rng = np.random.default_rng(4242)
    layer = helpers.random_layer(rng, H, I, E, k, shared=True, bias=True)
    layer.router_bias = (-6.0 * np.log(rng.permutation(E) + 1.0)).astype(np.float32)
    x = helpers.random_x(rng, T, H)
    glayer = parity.to_gpu_layer(layer)
    out, aux = ops.forward(glayer, parity.bits_to_bf16(x), return_aux=True)
    ids = aux["topk_ids"].cpu().numpy()
    counts = omoe.permute(ids, E)[0]
    assert counts.max() > 256 and (counts < 32).sum() >= 8, counts
    res = parity.reference_for_selection(x, layer, ids)
    parity.assert_close(parity.f64(out), res["out"], "layer")


def test_rows_of_widely_different_magnitude_on_128_row_tiles():
    """The 128-row NVFP4 gate/up path reads the tokens as fp16 rows scaled by a power of two each:
    rows from 2^-40 to 2^20, a row whose elements span 2^-30..1, and a row of zeros all match the
    oracle row by row."""
    T, H, I, E, k = 300, 256, 256, 8, 2
    rng = np.random.default_rng(777)
    layer = helpers.random_layer(rng, H, I, E, k, shared=True)
    xf = rng.normal(0, 1, (T, H))
    xf *= 2.0 ** rng.integers(-40, 21, T)[:, None]
    xf[1] *= 2.0 ** rng.integers(-30, 1, H)
    xf[2] = 0.0
    x = helpers.bf16_bits(torch.from_numpy(xf.astype(np.float32)).to(torch.bfloat16))
    glayer = parity.to_gpu_layer(layer)
    out, aux = ops.forward(glayer, parity.bits_to_bf16(x), return_aux=True)
    ids = aux["topk_ids"].cpu().numpy()
    res = parity.reference_for_selection(x, layer, ids)
    got = parity.f64(out)
    assert np.all(got[2] == 0.0)
    for t in range(T):
        if t != 2:
            parity.assert_close(got[t:t + 1], res["out"][t:t + 1], f"token {t}")


def _row_norm_bounds(layer: omoe.Layer):
    """Largest Euclidean norm of the dequantized gate rows and of the up rows over both banks
    (float64, from the canonical bytes through the oracle's dequantization)."""
    from oracle import nvfp4 as onv
    g = u = 0.0
    banks = [layer.routed] + ([layer.shared] if layer.shared is not None else [])
    for bank in banks:
        for e in range(len(bank)):
            ew = bank[e]
            i = ew.w13.shape[0] // 2
            wg = onv.dequantize(ew.w13[:i], ew.w13_scale[:i], ew.w13_gscale[0])
            wu = onv.dequantize(ew.w13[i:], ew.w13_scale[i:], ew.w13_gscale[1])
            g = max(g, float(np.sqrt((wg * wg).sum(axis=1)).max()))
            u = max(u, float(np.sqrt((wu * wu).sum(axis=1)).max()))
    return g, u


def test_fp16_h_bound_is_the_largest_weight_row_norm():
    """moe_nvfp4_h16_bound: the largest gate-row and up-row norms of both banks, rounded up to fp32."""
    rng = np.random.default_rng(31337)
    layer = helpers.random_layer(rng, 512, 256, 8, 2, shared=True)
    glayer = parity.to_gpu_layer(layer)
    got = glayer.h16_norm()
    ref = _row_norm_bounds(layer)
    for a, b in zip(got, ref):
        assert b <= a <= b * (1 + 2.0 ** -22), (got, ref)


def _h16_layer(seed, T, H, I, E, k):
    rng = np.random.default_rng(seed)
    layer = helpers.random_layer(rng, H, I, E, k, shared=True)
    return rng, layer, parity.to_gpu_layer(layer)


def test_fp16_h_equals_bf16_h_on_rows_of_widely_different_magnitude():
    """On 128-row tiles with both GEMMs on the eight-wave kernel, h travels as fp16 scaled per token
    by a power of two chosen from the weight-row norm bounds.  Rows from 2^-40 to 2^20, a row
    spanning 2^-30..1 and a row of zeros: the forward equals the one with bf16 h bitwise, and
    every token matches the oracle."""
    T, H, I, E, k = 300, 512, 256, 8, 2
    rng, layer, glayer = _h16_layer(778, T, H, I, E, k)
    assert glayer.h16_norm()[0] > 0
    xf = rng.normal(0, 1, (T, H))
    xf *= 2.0 ** rng.integers(-40, 21, T)[:, None]
    xf[1] *= 2.0 ** rng.integers(-30, 1, H)
    xf[2] = 0.0
    x = helpers.bf16_bits(torch.from_numpy(xf.astype(np.float32)).to(torch.bfloat16))
    xg = parity.bits_to_bf16(x)
    out, aux = ops.forward(glayer, xg, return_aux=True)
    glayer.fp16_h = False
    out_bf = ops.forward(glayer, xg)
    glayer.fp16_h = True
    assert torch.equal(out, out_bf), "fp16 h and bf16 h differ"
    ids = aux["topk_ids"].cpu().numpy()
    res = parity.reference_for_selection(x, layer, ids)
    got = parity.f64(out)
    assert np.all(got[2] == 0.0)
    for t in range(T):
        if t != 2:
            parity.assert_close(got[t:t + 1], res["out"][t:t + 1], f"token {t}")


def test_fp16_h_on_tiny_rows_that_take_the_unfolded_epilogues():
    """Rows near 2^-55 and 2^-60 get h powers of two so large that the down epilogue cannot fold
    them into the weight scale (the folded scale would be subnormal) and scales after the product
    instead; for a row near 2^-100 the gate/up epilogue cannot fold the token's power of two either.
    Such a row makes its whole 16-row block take the two-step form: the N(0,1) rows around them
    equal the bf16-h forward bitwise; the tiny rows match the oracle (the bf16-h forward itself
    loses bits there, its fp32 products of such h being subnormal); the 2^-100 row's output is 0,
    the bf16 rounding of the oracle's."""
    T, H, I, E, k = 300, 512, 256, 8, 2
    rng, layer, glayer = _h16_layer(781, T, H, I, E, k)
    xf = rng.normal(0, 1, (T, H))
    tiny = {3: -55, 4: -60, 150: -55, 299: -60, 5: -100}
    for t, e in tiny.items():
        xf[t] *= 2.0 ** e
    x = helpers.bf16_bits(torch.from_numpy(xf.astype(np.float32)).to(torch.bfloat16))
    xg = parity.bits_to_bf16(x)
    out, aux = ops.forward(glayer, xg, return_aux=True)
    glayer.fp16_h = False
    out_bf = ops.forward(glayer, xg)
    glayer.fp16_h = True
    others = [t for t in range(T) if t not in tiny]
    assert torch.equal(out[others], out_bf[others]), "fp16 h and bf16 h differ on the N(0,1) rows"
    ids = aux["topk_ids"].cpu().numpy()
    res = parity.reference_for_selection(x, layer, ids)
    got = parity.f64(out)
    # below half the smallest bf16 subnormal (2^-133): its bf16 value is 0
    assert np.abs(res["out"][5]).max() < 2.0 ** -134 and np.all(got[5] == 0.0)
    for t in range(T):
        if t != 5:
            if t in tiny:
                assert np.abs(res["out"][t]).max() > 2.0 ** -126, f"token {t} is not a normal bf16 output"
            parity.assert_close(got[t:t + 1], res["out"][t:t + 1], f"token {t}")


def test_fp16_h_bound_is_what_the_forward_uses():
    """A bound 2^20 above the true norms is valid (no fp16 overflow) but leaves most of h below the
    range it carries exactly: the output then moves off the bf16-h result, so the forward does take
    h through fp16 with the layer's bounds; with the true bounds it is back to bitwise equal."""
    T, H, I, E, k = 600, 1024, 256, 8, 2
    rng, layer, glayer = _h16_layer(779, T, H, I, E, k)
    xg = parity.bits_to_bf16(helpers.random_x(rng, T, H))
    out = ops.forward(glayer, xg)
    glayer.fp16_h = False
    out_bf = ops.forward(glayer, xg)
    glayer.fp16_h = True
    assert torch.equal(out, out_bf)
    true_bounds = (glayer.routed.h16_bound, glayer.shared.h16_bound)
    for b in (glayer.routed, glayer.shared):
        b.h16_bound = tuple(v * 2.0 ** 20 for v in b.h16_bound)
    loose = ops.forward(glayer, xg)
    glayer.routed.h16_bound, glayer.shared.h16_bound = true_bounds
    assert torch.isfinite(loose.float()).all()
    assert not torch.equal(loose, out_bf), "the forward ignored the layer's bounds"
    assert torch.equal(ops.forward(glayer, xg), out_bf)


def test_persistent_gemm_tiles_chain_and_steal():
    """More 128-row tiles than workgroups, down K at the six-chunk minimum for chaining, routing
    skewed so that the XCD windows hold very different work: the forward (tiles drawn from the
    workspace counters, stolen across windows) matches the per-stage entry points (fixed share per
    workgroup) on every token, two forwards in a row agree bitwise (the counters start at zero each
    time), and sampled tokens match the oracle."""
    T, H, I, E, k = 8192, 1024, 768, 16, 2
    rng = np.random.default_rng(8086)
    layer = helpers.random_layer(rng, H, I, E, k, shared=True, bias=True)
    layer.router_bias = (-4.0 * np.log(rng.permutation(E) + 1.0)).astype(np.float32)
    x = helpers.random_x(rng, T, H)
    glayer = parity.to_gpu_layer(layer)
    xg = parity.bits_to_bf16(x)
    out, aux = ops.forward(glayer, xg, return_aux=True)
    ids = aux["topk_ids"].cpu().numpy()
    counts = omoe.permute(ids, E)[0]
    # gate/up: 3 column tiles per m-tile, down: 2; both well past 256 tiles
    m_tiles = int(np.sum((counts + 127) // 128)) + (T + 127) // 128
    assert 2 * m_tiles > 256 and counts.max() > 4 * counts.min(), (m_tiles, counts)
    out2 = ops.forward(glayer, xg)
    assert torch.equal(out, out2), "two forwards differ"
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(DEV)
    _, offs2, sorted_slot, slot_to_row = ops.permute(aux["topk_ids"], E)
    assert torch.equal(offs2, offsets)
    S = T * k
    h = ops.grouped_gemm(L.MOE_GEMM_GATE_UP, glayer.routed, xg, offsets, S, sorted_slot, k)
    y = ops.grouped_gemm(L.MOE_GEMM_DOWN, glayer.routed, h, offsets, S)
    one = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    hs = ops.grouped_gemm(L.MOE_GEMM_GATE_UP, glayer.shared, xg, one, T)
    ys = ops.grouped_gemm(L.MOE_GEMM_DOWN, glayer.shared, hs, one, T)
    staged = ops.combine(y, slot_to_row, aux["topk_w"], ys)
    rel, mx = parity.assert_close(parity.f64(out), parity.f64(staged), "forward vs per-stage entry points")
    parity.record_margin(f"persistent tiles: forward vs staged, all {T} tokens", rel, mx)
    tokens = np.unique(np.concatenate([rng.choice(T, 24, replace=False), [0, T - 1]]))
    res = parity.reference_for_selection(x[tokens], layer, ids[tokens])
    rel, mx = parity.assert_close(parity.f64(out[torch.from_numpy(tokens).to(DEV)]), res["out"], "sampled tokens")
    parity.record_margin(f"persistent tiles: layer output, {len(tokens)} tokens", rel, mx)


def test_zero_tokens_is_a_no_op():
    rng = np.random.default_rng(1)
    glayer = parity.to_gpu_layer(helpers.random_layer(rng, 256, 128, 4, 2))
    out = ops.forward(glayer, torch.zeros(0, 256, dtype=torch.bfloat16, device=DEV))
    assert out.shape == (0, 256)


def test_forward_replays_from_a_hip_graph():
    """The forward only enqueues kernels (no allocation, synchronisation or memset), so it can be
    captured in a HIP graph: every replay, with eager work between replays, equals the eager output."""
    rng = np.random.default_rng(11)
    # 16-row tiles + fused top-k/permute; 128-row tiles + tiled h; multi-block permute
    for T, H, I, E, k in [(8, 256, 128, 16, 4), (300, 512, 256, 16, 4), (600, 512, 256, 16, 4)]:
        layer = helpers.random_layer(rng, H, I, E, k)
        glayer = parity.to_gpu_layer(layer)
        x = parity.bits_to_bf16(helpers.random_x(rng, T, H))
        ws = ops.workspace_for(glayer, T, DEV)
        ref = ops.forward(glayer, x, ws).clone()
        out = torch.empty_like(x)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            ops.forward(glayer, x, ws, out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ops.forward(glayer, x, ws, out)
        for r in range(3):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"T={T}: replay {r} differs from the eager forward"
            other = ops.forward(glayer, x, ws)
            torch.cuda.synchronize()
            assert torch.equal(other, ref)


# ----------------------------------------------------------------------------- tiny workload

def _oracle_bank_equal(gbank, obank, experts):
    """GPU-quantized, tile-packed bank bytes == the oracle quantizer's bytes put in the tile layout."""
    for e in experts:
        ow = obank[e]
        t13, s13 = parity.tile_np(ow.w13, ow.w13_scale)
        t2, s2 = parity.tile_np(ow.w2, ow.w2_scale)
        assert np.array_equal(gbank.w13[e].cpu().numpy(), t13), e
        assert np.array_equal(gbank.w13_scale[e].cpu().numpy(), s13), e
        assert np.array_equal(gbank.w2[e].cpu().numpy(), t2), e
        assert np.array_equal(gbank.w2_scale[e].cpu().numpy(), s2), e
        assert np.array_equal(gbank.w13_gscale[e].cpu().numpy(), ow.w13_gscale), e
        assert float(gbank.w2_gscale[e]) == ow.w2_gscale, e


def test_tiny_workload_end_to_end_and_staged():
    wl = synth.WORKLOADS["tiny"]
    glayer = build_layer(wl, DEV)
    olayer = helpers.oracle_layer(wl, DEV)
    _oracle_bank_equal(glayer.routed, olayer.routed, range(wl.E))
    _oracle_bank_equal(glayer.shared, olayer.shared, [0])
    x = synth.activations(wl, DEV)
    xb = helpers.bf16_bits(x)
    out, aux = ops.forward(glayer, x, return_aux=True)
    parity.check_route(aux["logits"], aux["topk_ids"], aux["topk_w"], xb, olayer.w_router, None, wl.k)
    res = parity.reference_for_selection(xb, olayer, aux["topk_ids"].cpu().numpy())
    parity.assert_close(parity.f64(out), res["out"], "forward")
    # the same layer through the per-stage entry points
    logits, ids, w = ops.route(x, glayer.w_router, None, wl.k)
    counts, offsets, sorted_slot, slot_to_row = ops.permute(ids, wl.E)
    S = wl.T * wl.k
    h = ops.grouped_gemm(L.MOE_GEMM_GATE_UP, glayer.routed, x, offsets, S, sorted_slot, wl.k)
    y = ops.grouped_gemm(L.MOE_GEMM_DOWN, glayer.routed, h, offsets, S)
    one = torch.tensor([0, wl.T], dtype=torch.int32, device=DEV)
    hs = ops.grouped_gemm(L.MOE_GEMM_GATE_UP, glayer.shared, x, one, wl.T)
    ys = ops.grouped_gemm(L.MOE_GEMM_DOWN, glayer.shared, hs, one, wl.T)
    staged = ops.combine(y, slot_to_row, w, ys)
    parity.assert_close(parity.f64(staged), res["out"], "staged")
    assert torch.equal(ids, aux["topk_ids"])


def test_loader_ignores_activation_scales_and_converts_reciprocal_scales():
    """A checkpoint dict with input_scale entries (even 0) gives the same nonzero output; a
    compressed-tensors checkpoint (quant scales) is inverted on load."""
    wl = synth.WORKLOADS["tiny"]
    glayer = build_layer(wl, DEV)
    x = synth.activations(wl, DEV)
    ref = ops.forward(glayer, x)
    # a checkpoint in the canonical layout: the oracle quantizer's bytes (equal to the GPU quantizer's)
    olayer = helpers.oracle_layer(wl, DEV)
    tensors = {"router.weight": glayer.w_router}
    for pre, ob, n in (("experts.", olayer.routed, wl.E), ("shared_expert.", olayer.shared, 1)):
        b = helpers.stack_bank(ob)
        tensors.update({pre + "w13": torch.from_numpy(b.w13), pre + "w13_scale": torch.from_numpy(b.w13_scale),
                        pre + "w13_global_scale": torch.from_numpy(b.w13_gscale),
                        pre + "w2": torch.from_numpy(b.w2), pre + "w2_scale": torch.from_numpy(b.w2_scale),
                        pre + "w2_global_scale": torch.from_numpy(b.w2_gscale),
                        pre + "w13_input_scale": torch.zeros(n, 2), pre + "w2_input_scale": torch.zeros(n)})
    lay = ops.NvFp4MoELayer.from_tensors(tensors, wl.k, "modelopt", DEV)
    out = ops.forward(lay, x)
    assert torch.equal(out, ref)
    assert bool((out.float().abs().amax(dim=1) > 0).all())
    ct = dict(tensors)
    for pre in ("experts.", "shared_expert."):
        ct[pre + "w13_global_scale"] = torch.from_numpy(np.float32(1) / tensors[pre + "w13_global_scale"].numpy())
        ct[pre + "w2_global_scale"] = torch.from_numpy(np.float32(1) / tensors[pre + "w2_global_scale"].numpy())
    lay_ct = ops.NvFp4MoELayer.from_tensors(ct, wl.k, "compressed_tensors", DEV)
    want = (np.float32(1) / (np.float32(1) / glayer.routed.w13_gscale.cpu().numpy())).astype(np.float32)
    assert np.array_equal(lay_ct.routed.w13_gscale.cpu().numpy(), want)


# ----------------------------------------------------------------------------- full-size workloads

_BANKS = {}


def _gpu_layer(wl):
    key = (wl.wseed, wl.H, wl.I, wl.E)
    if key not in _BANKS:
        _BANKS.clear()
        torch.cuda.empty_cache()
        _BANKS[key] = (build_bank(wl, "routed", DEV), build_bank(wl, "shared", DEV))
    routed, shared = _BANKS[key]
    bias = synth.router_bias(wl)
    return ops.NvFp4MoELayer(synth.router_weight(wl, DEV).contiguous(),
                             torch.from_numpy(bias).to(DEV) if bias is not None else None, routed, shared, wl.k)


def _xcd_sample_tiles(counts, T, has_shared, N, BN=256, BM=128, xcds=8):
    """The 128-row m-tiles (group, first sorted row, rows; group -1 = the shared expert) that hold
    the first, middle and last (m-tile, n-tile) pair of each XCD's contiguous range in the prefill
    GEMMs of output width N (n-tiles of BN columns; the shared expert's m-tiles numbered first)."""
    tiles = [(-1, r, min(BM, T - r)) for r in range(0, T, BM)] if has_shared else []
    off = 0
    for e, c in enumerate(counts):
        tiles += [(e, off + r, min(BM, int(c) - r)) for r in range(0, int(c), BM)]
        off += int(c)
    nt = N // BN
    total = len(tiles) * nt
    per = -(-total // xcds)
    picks = set()
    for x in range(xcds):
        lo, hi = x * per, min((x + 1) * per, total) - 1
        if lo <= hi:
            picks.update(L // nt for L in (lo, (lo + hi) // 2, hi))
    return [tiles[m] for m in sorted(picks)]


E2E_TOKENS = {"decode": 8, "prefill": 16, "skewed": 16, "long_prefill": 16}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode", "prefill", "skewed", "long_prefill"])
def test_full_size_workload(name):
    """A full-size workload in the launch configuration the bench times (one moe_nvfp4_forward):
      * selection bit-exact for every token, router logits on a token sample, permutation for every slot;
      * the expert outputs y the combine reads (returned by the forward itself): every routed row at
        decode; at the prefill shapes every row of the m-tiles that start, sit in the middle of and end
        each XCD's tile range in both GEMMs, and the shared expert's row of EVERY token (all of its
        m-tiles in both GEMMs), each against the oracle's gate/up -> SiLU*up -> down of those rows;
      * the combine for EVERY token on the forward's own y rows and weights (fp32 summation bound);
      * the layer output of every decode token and of 16 tokens spread over the sampled tiles at the
        prefill shapes against the oracle's whole forward;
      * every token of the forward against the per-stage entry points (bf16, row-major h);
      * the GPU-quantized bytes of the experts checked against the oracle quantizer's."""
    wl = synth.WORKLOADS[name]
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    S = T * k
    _say(f"[full-size {name}] building layer T={T} H={H} I={I} E={E} k={k}")
    glayer = _gpu_layer(wl)
    x = synth.activations(wl, DEV)
    out, aux = ops.forward(glayer, x, return_aux=True, return_rows=True)
    torch.cuda.synchronize()
    _say(f"[full-size {name}] forward done")
    xb = helpers.bf16_bits(x)
    wrb = helpers.bf16_bits(glayer.w_router)
    bias = synth.router_bias(wl)
    lg = aux["logits"].cpu().numpy().astype(np.float64)
    ids = aux["topk_ids"].cpu().numpy()
    wts = aux["topk_w"].cpu().numpy()
    # selection: bit-exact for every token on the GPU's logits
    ids_ref, w_ref = omoe.topk(lg, k)
    assert np.array_equal(ids, ids_ref)
    np.testing.assert_allclose(wts, w_ref, rtol=0, atol=1e-5)
    # router GEMM: a token sample within the fp32 bound
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([rng.choice(T, min(T, 48), replace=False), [0, T - 1]]))
    exact = omoe.router_logits(xb[rows], wrb, bias)
    assert np.all(np.abs(lg[rows] - exact) <= parity.logit_bound(xb[rows], wrb, bias))
    # permutation: bit-exact for every slot
    counts, offsets, sorted_slot, slot_to_row = ops.permute(aux["topk_ids"], E)
    c, o, srt, s2r = omoe.permute(ids, E)
    assert np.array_equal(aux["expert_counts"].cpu().numpy(), c)
    assert np.array_equal(counts.cpu().numpy(), c) and np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(sorted_slot.cpu().numpy(), srt) and np.array_equal(slot_to_row.cpu().numpy(), s2r)
    _say(f"[full-size {name}] route/permute exact; {int((c > 0).sum())} experts used, max count {int(c.max())}")

    y_gpu = aux["y_rows"]
    decode = (S + T) // (E + 1) <= 32   # the 8-, 16- and 64-row kernels: no XCD tile ranges
    if decode:
        sample = [(int(e), int(o[e]), int(c[e])) for e in range(E) if c[e] > 0] + [(-1, 0, T)]
        tokens = np.arange(T)
    else:
        sample = sorted(set(_xcd_sample_tiles(c, T, True, I) + _xcd_sample_tiles(c, T, True, H)))
        firsts = [srt[r0] // k for g, r0, n in sample if g >= 0] + [srt[r0 + n - 1] // k for g, r0, n in sample
                                                                      if g >= 0]
        cand = np.unique(np.concatenate([firsts, [0, T - 1]]))
        tokens = cand[np.unique(np.linspace(0, len(cand) - 1, E2E_TOKENS[name]).round().astype(int))]
    experts = sorted({g for g, _, _ in sample if g >= 0} | {int(e) for e in np.unique(ids[tokens])})
    olayer = helpers.oracle_layer(wl, DEV)
    _say(f"[full-size {name}] oracle quantizes {len(experts)} experts")
    olayer.routed.prefetch(experts, threads=16)
    _oracle_bank_equal(glayer.routed, olayer.routed, experts[:: max(1, len(experts) // 8)])

    # expert outputs y of the sampled m-tiles (routed) against the oracle, expert by expert
    worst = (0.0, 0.0)
    by_expert = {}
    for g, r0, n in sample:
        if g >= 0:
            by_expert.setdefault(g, []).append(np.arange(r0, r0 + n))
    for e, parts in by_expert.items():
        r = np.concatenate(parts)
        a_rows = omoe.bf16_to_float(xb[srt[r] // k])
        y_ref = omoe.expert_ffn(a_rows, olayer.routed[e])
        got = parity.f64(y_gpu[torch.from_numpy(r).to(DEV)])
        rel, mx = parity.assert_close(got, y_ref, f"y rows of expert {e}")
        worst = (max(worst[0], rel), max(worst[1], mx))
    parity.record_margin(f"{name}: routed y rows ({len(by_expert)} experts)", *worst)
    # the shared expert for every token, and tile by tile
    ys_ref = omoe.expert_ffn(omoe.bf16_to_float(xb), olayer.shared[0])
    ys_gpu = parity.f64(y_gpu[S:S + T])
    rel, mx = parity.assert_close(ys_gpu, ys_ref, "shared expert y, all tokens")
    for r0 in range(0, T, 128):
        parity.assert_close(ys_gpu[r0:r0 + 128], ys_ref[r0:r0 + 128], f"shared expert y rows {r0}..")
    parity.record_margin(f"{name}: shared expert y, all {T} tokens", rel, mx)
    _say(f"[full-size {name}] y rows match ({len(by_expert)} routed experts, shared expert on every token)")

    # the combine of every token on the forward's own y rows
    w64 = wts.astype(np.float64)
    worst = 0.0
    for t0 in range(0, T, 1024):
        t1 = min(T, t0 + 1024)
        rsel = s2r.reshape(T, k)[t0:t1]
        y_routed = parity.f64(y_gpu[torch.from_numpy(np.unique(rsel)).to(DEV)])
        lut = np.searchsorted(np.unique(rsel), rsel)
        ysh = ys_gpu[t0:t1]
        ref = np.einsum("tj,tjh->th", w64[t0:t1], y_routed[lut]) + ysh
        sabs = np.einsum("tj,tjh->th", np.abs(w64[t0:t1]), np.abs(y_routed[lut])) + np.abs(ysh)
        got = parity.f64(out[t0:t1])
        err = np.abs(got - ref)
        bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -20 * sabs + 1e-30
        assert np.all(err <= bound), f"combine tokens {t0}..{t1}: worst ratio {float((err / bound).max()):.3f}"
        worst = max(worst, float((err / bound).max()))
    _say(f"[full-size {name}] combine exact within the fp32 bound for all {T} tokens (worst {worst:.3f} of it)")

    # the whole layer on sampled tokens against the oracle's forward
    res = parity.reference_for_selection(xb[tokens], olayer, ids[tokens])
    rel, mx = parity.assert_close(parity.f64(out[torch.from_numpy(tokens).to(DEV)]), res["out"], "sampled tokens")
    parity.record_margin(f"{name}: layer output, {len(tokens)} tokens", rel, mx)
    _say(f"[full-size {name}] layer output of tokens {tokens.tolist()}: rel-L2 {rel:.2e}, max-abs {mx:.2e}")

    # every token against the per-stage entry points (bf16 operands, row-major h)
    h = ops.grouped_gemm(L.MOE_GEMM_GATE_UP, glayer.routed, x, offsets, S, sorted_slot, k)
    y = ops.grouped_gemm(L.MOE_GEMM_DOWN, glayer.routed, h, offsets, S)
    one = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    hs = ops.grouped_gemm(L.MOE_GEMM_GATE_UP, glayer.shared, x, one, T)
    ys = ops.grouped_gemm(L.MOE_GEMM_DOWN, glayer.shared, hs, one, T)
    staged = ops.combine(y, slot_to_row, aux["topk_w"], ys)
    rel, mx = parity.assert_close(parity.f64(out), parity.f64(staged), "forward vs per-stage entry points")
    parity.record_margin(f"{name}: forward vs staged, all {T} tokens", rel, mx)
    e_max = int(np.argmax(c))
    r0, r1 = int(o[e_max]), int(o[e_max + 1])
    h_ref = omoe.gate_up(omoe.bf16_to_float(xb[srt[r0:r1] // k]), olayer.routed[e_max])
    parity.assert_close(parity.f64(h[r0:r1]), h_ref, f"staged gate/up rows of expert {e_max}")
    del h, y, hs, ys, staged, y_gpu
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- fused decode path

FUSED = [
    # T, H, I, E, k, shared, bias: few tokens, where the forward runs as two launches
    (8, 256, 128, 16, 4, True, False),
    (1, 512, 256, 64, 8, True, True),
    (32, 256, 128, 320, 8, True, False),     # T*k = 256 slots, E = 320
    (5, 384, 256, 12, 3, False, True),       # no shared expert
    (16, 256, 128, 8, 2, True, False),       # the tiny workload's shape
    (3, 512, 384, 40, 40, True, False),      # k = E
    (4, 384, 128, 16, 2, True, False),       # 128-wide K chunks in both GEMMs
]


@pytest.mark.parametrize("case", FUSED, ids=[f"T{c[0]}_H{c[1]}_I{c[2]}_E{c[3]}_k{c[4]}" for c in FUSED])
def test_fused_decode_path_equals_staged_launches_and_the_oracle(case):
    """The two-launch fused decode path (router, then top-k + permutation + both GEMMs + combine in
    one kernel with counter hand-offs) gives bitwise the output, selection, counts and expert rows of
    the staged launches, matches the oracle, and repeats bitwise."""
    T, H, I, E, k, shared, bias = case
    rng = np.random.default_rng(sum(case[:5]) + 99)
    layer = helpers.random_layer(rng, H, I, E, k, shared=shared, bias=bias)
    x = helpers.random_x(rng, T, H)
    glayer = parity.to_gpu_layer(layer)
    xg = parity.bits_to_bf16(x)
    out_f, aux_f = ops.forward(glayer, xg, return_aux=True, return_rows=True, fused_decode=True)
    out_s, aux_s = ops.forward(glayer, xg, return_aux=True, return_rows=True)
    torch.cuda.synchronize()
    for key in ("logits", "topk_ids", "topk_w", "expert_counts", "y_rows"):
        assert torch.equal(aux_f[key], aux_s[key]), key
    assert torch.equal(out_f, out_s), "fused decode path differs from the staged launches"
    assert not torch.isnan(out_f.float()).any()
    ids = aux_f["topk_ids"].cpu().numpy()
    parity.check_route(aux_f["logits"], aux_f["topk_ids"], aux_f["topk_w"], x, layer.w_router, layer.router_bias, k)
    res = parity.reference_for_selection(x, layer, ids)
    parity.assert_close(parity.f64(out_f), res["out"], "fused decode path")
    for _ in range(3):
        assert torch.equal(ops.forward(glayer, xg, fused_decode=True), out_f), "repeated fused forward differs"


def test_fused_decode_path_replays_from_a_hip_graph_with_other_work_between():
    """Both launches of the fused decode path captured in a HIP graph: its hand-off counters are
    cleared by the captured router launch, so every replay, with eager forwards of other sizes on the
    same workspace between replays, equals the eager output."""
    rng = np.random.default_rng(21)
    T, H, I, E, k = 8, 512, 256, 64, 8
    layer = helpers.random_layer(rng, H, I, E, k, bias=True)
    glayer = parity.to_gpu_layer(layer)
    x = parity.bits_to_bf16(helpers.random_x(rng, T, H))
    x2 = parity.bits_to_bf16(helpers.random_x(rng, 24, H))
    ws = ops.workspace_for(glayer, 24, DEV)
    ref = ops.forward(glayer, x, ws).clone()
    ref2 = ops.forward(glayer, x2, ws).clone()
    out = torch.empty_like(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ops.forward(glayer, x, ws, out, fused_decode=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.forward(glayer, x, ws, out, fused_decode=True)
    for r in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r} differs from the eager forward"
        assert torch.equal(ops.forward(glayer, x2, ws, fused_decode=True), ref2)
        torch.cuda.synchronize()
