"""GPU parity of the MXFP4 weight path (E2M1 with one E8M0 scale per 32 elements, no global scale)
against the oracle, through the C ABI: quantizer, tile repack, grouped GEMMs on every tile path,
small layers end to end and the decode-shaped layer at full size."""

import numpy as np
import pytest
import torch

import helpers
import parity
from nvfp4_weight_quantized_amd import _lib as L
from nvfp4_weight_quantized_amd import ops, synth
from nvfp4_weight_quantized_amd.workloads import build_layer
from oracle import moe as omoe
from oracle import mxfp4 as omx

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _quant_cases(rng):
    yield "gauss", rng.normal(0, 0.02, (3, 64, 256)).astype(np.float32)
    w = rng.normal(0, 0.015, (2, 32, 512)).astype(np.float32)
    w[:, ::7, 5] = 0.3                                            # outliers
    yield "outliers", w
    z = rng.normal(0, 1, (1, 16, 128)).astype(np.float32)
    z[0, 3] = 0.0                                                 # all-zero blocks
    z[0, 4, :32] = np.float32(1e-40)                              # fp32 subnormal block
    z[0, 5, :32] = -np.float32(1e-45)                             # negative, rounds to -0 codes
    yield "zeros_and_subnormals", z
    # block max 6 * 2^e; the others on E2M1 midpoints (ties to the even code) or in the clip range
    grid = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -1.75, -5.0, 4.0, 0.5, -6.0, 3.0, 1.0] * 2)
    t = np.tile(grid, (1, 8, 4)) * np.exp2(np.arange(-4, 4)).reshape(1, 8, 1)
    yield "ties", t.astype(np.float32)
    c = rng.uniform(-1, 1, (1, 8, 128)).astype(np.float32)
    c[0, :, ::32] = 7.9                                            # block max in (6, 8) * 2^e: clipping
    yield "clip", c
    yield "wide_range", (rng.normal(0, 1, (1, 8, 128)) * np.exp2(rng.integers(-120, 120, (1, 8, 1)))).astype(np.float32)


def test_mx_quantizer_bit_exact_against_oracle():
    rng = np.random.default_rng(31)
    for name, w in _quant_cases(rng):
        p, s = ops.quantize_mx(torch.from_numpy(w).to(DEV))
        for t in range(w.shape[0]):
            pr, sr = omx.quantize(w[t])
            assert np.array_equal(s[t].cpu().numpy(), sr), name
            assert np.array_equal(p[t].cpu().numpy(), pr), name


def test_mx_pack_tiles_is_the_stated_permutation():
    rng = np.random.default_rng(32)
    for nt, r, k in [(1, 16, 128), (3, 48, 384), (2, 256, 1024)]:
        p = rng.integers(0, 256, (nt, r, k // 2), dtype=np.uint8)
        s = rng.integers(0, 256, (nt, r, k // 32), dtype=np.uint8)
        tp, ts = ops.pack_tiles(torch.from_numpy(p).to(DEV), torch.from_numpy(s).to(DEV), fmt="mxfp4")
        for t in range(nt):
            wp, ws = parity.tile_np_mx(p[t], s[t])
            assert np.array_equal(tp[t].cpu().numpy(), wp)
            assert np.array_equal(ts[t].cpu().numpy(), ws)


def _bank(rng, e, h, i):
    return helpers.random_layer(rng, h, i, e, 1, shared=False, sigma=0.05, fmt="mxfp4").routed


def _offsets(counts):
    o = np.zeros(len(counts) + 1, np.int32)
    o[1:] = np.cumsum(counts)
    return o


@pytest.mark.parametrize("H,I,counts", [
    (256, 128, [1, 0, 3, 2]),                       # 16-row tiles (few rows per expert)
    (512, 256, [0, 17, 16, 15, 1, 33, 0, 64]),       # 64-row tiles, ragged tails
    (384, 256, [129, 0, 128, 127, 300, 5]),          # 128-row tiles; H % 256 != 0 -> narrow down tiles
    (512, 256, [100, 0, 200, 77, 129]),             # 128-row tiles: eight-wave gate/up, four-wave down
    (256, 384, [200, 70, 0, 1]),
])
def test_mx_grouped_gemm_random_matches_oracle(H, I, counts):
    rng = np.random.default_rng(H + I + sum(counts) + 1)
    E = len(counts)
    bank = _bank(rng, E, H, I)
    gbank = parity.to_gpu_bank(bank)
    assert gbank.fmt == "mxfp4"
    off = _offsets(counts)
    M = int(off[-1])
    div = 3
    T = (M + div - 1) // div + 2
    x = helpers.random_x(rng, T, H)
    row_index = rng.integers(0, T * div, M).astype(np.int32)
    h = ops.grouped_gemm(L.MOE_GEMM_GATE_UP, gbank, parity.bits_to_bf16(x), torch.from_numpy(off).to(DEV), M,
                         torch.from_numpy(row_index).to(DEV), div)
    h_ref = omoe.grouped_gate_up(omoe.bf16_to_float(x)[row_index // div], off, bank)
    parity.assert_close(parity.f64(h), h_ref, "gate/up")
    hb = helpers.bf16_bits(h)
    y = ops.grouped_gemm(L.MOE_GEMM_DOWN, gbank, h, torch.from_numpy(off).to(DEV), M)
    parity.assert_close(parity.f64(y), omoe.grouped_down(omoe.bf16_to_float(hb), off, bank), "down")


@pytest.mark.parametrize("counts", [[1, 2], [5, 11], [40, 90]])
def test_mx_grouped_gemm_one_hot_pins_layout(counts):
    """A unit row e_h makes each output one dequantized weight v * 2^(s - 127): pins nibble order,
    the per-32 scale index and gate/up order on the 16-row, 64-row and 128-row paths."""
    rng = np.random.default_rng(40 + sum(counts))
    H, I = 512, 256
    bank = _bank(rng, 2, H, I)
    gbank = parity.to_gpu_bank(bank)
    off = _offsets(counts)
    M = int(off[-1])
    hs = rng.integers(0, H, M)
    a = np.zeros((M, H), np.float32)
    a[np.arange(M), hs] = 1.0
    h = ops.grouped_gemm(L.MOE_GEMM_GATE_UP, gbank, torch.from_numpy(a).to(torch.bfloat16).to(DEV),
                         torch.from_numpy(off).to(DEV), M)
    ref = omoe.grouped_gate_up(a.astype(np.float64), off, bank)
    assert np.all(np.abs(parity.f64(h) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    is_ = rng.integers(0, I, M)
    a2 = np.zeros((M, I), np.float32)
    a2[np.arange(M), is_] = 1.0
    y = ops.grouped_gemm(L.MOE_GEMM_DOWN, gbank, torch.from_numpy(a2).to(torch.bfloat16).to(DEV),
                         torch.from_numpy(off).to(DEV), M)
    ref2 = omoe.grouped_down(a2.astype(np.float64), off, bank)
    assert np.all(np.abs(parity.f64(y) - ref2) <= 2.0 ** -8 * np.abs(ref2) + 1e-30)


SMALL = [
    # T, H, I, E, k, shared, bias
    (5, 256, 128, 8, 2, True, False),
    (64, 512, 256, 16, 4, True, True),
    (300, 512, 256, 16, 4, True, False),
    (37, 384, 256, 12, 3, False, True),
    (600, 512, 256, 16, 4, True, False),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"T{c[0]}_H{c[1]}_I{c[2]}_E{c[3]}_k{c[4]}" for c in SMALL])
def test_mx_small_layer_end_to_end(case):
    T, H, I, E, k, shared, bias = case
    rng = np.random.default_rng(sum(case[:5]) + 7)
    layer = helpers.random_layer(rng, H, I, E, k, shared=shared, bias=bias, fmt="mxfp4")
    x = helpers.random_x(rng, T, H)
    glayer = parity.to_gpu_layer(layer)
    out, aux = ops.forward(glayer, parity.bits_to_bf16(x), return_aux=True)
    parity.check_route(aux["logits"], aux["topk_ids"], aux["topk_w"], x, layer.w_router, layer.router_bias, k)
    res = parity.reference_for_selection(x, layer, aux["topk_ids"].cpu().numpy())
    parity.assert_close(parity.f64(out), res["out"], "layer")
    assert torch.equal(out, ops.forward(glayer, parity.bits_to_bf16(x))), "two runs differ"


@pytest.mark.timeout(600)
def test_mx_decode_workload_full_size():
    """The decode-shaped layer (T=8, H=4096, I=1536, E=320 top-8 + shared) with MXFP4 weights quantized
    on the GPU: quantized bytes of every expert used equal the oracle quantizer's, selection is exact,
    every expert output row the combine reads matches the oracle, and so does every token's output."""
    wl = synth.WORKLOADS["decode"]
    T, k, E = wl.T, wl.k, wl.E
    S = T * k
    _say(f"[mxfp4 decode] building layer E={E} H={wl.H} I={wl.I}")
    glayer = build_layer(wl, DEV, fmt="mxfp4")
    x = synth.activations(wl, DEV)
    out, aux = ops.forward(glayer, x, return_aux=True, return_rows=True)
    torch.cuda.synchronize()
    xb = helpers.bf16_bits(x)
    ids = aux["topk_ids"].cpu().numpy()
    ids_ref, _ = omoe.topk(aux["logits"].cpu().numpy().astype(np.float64), k)
    assert np.array_equal(ids, ids_ref)
    olayer = helpers.oracle_layer(wl, DEV, fmt="mxfp4")
    used = np.unique(ids)
    olayer.routed.prefetch(used, threads=16)
    for e in used:
        ow = olayer.routed[int(e)]
        t13, s13 = parity.tile_np_mx(ow.w13, ow.w13_scale)
        assert np.array_equal(glayer.routed.w13[e].cpu().numpy(), t13), e
        assert np.array_equal(glayer.routed.w13_scale[e].cpu().numpy(), s13), e
        t2, s2 = parity.tile_np_mx(ow.w2, ow.w2_scale)
        assert np.array_equal(glayer.routed.w2[e].cpu().numpy(), t2), e
        assert np.array_equal(glayer.routed.w2_scale[e].cpu().numpy(), s2), e
    # every expert output row (routed rows in expert order, then the shared expert's)
    counts, offsets, srt, s2r = omoe.permute(ids, E)
    y = parity.f64(aux["y_rows"])
    xf = omoe.bf16_to_float(xb)
    worst = (0.0, 0.0)
    for e in used:
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        rel, mx = parity.assert_close(y[r0:r1], omoe.expert_ffn(xf[srt[r0:r1] // k], olayer.routed[int(e)]),
                                      f"y rows of expert {e}")
        worst = (max(worst[0], rel), max(worst[1], mx))
    parity.record_margin(f"mxfp4 decode: routed y rows ({len(used)} experts)", *worst)
    rel, mx = parity.assert_close(y[S:S + T], omoe.expert_ffn(xf, olayer.shared[0]), "shared expert y")
    parity.record_margin("mxfp4 decode: shared expert y", rel, mx)
    # every token's output
    res = parity.reference_for_selection(xb, olayer, ids)
    rel, mx = parity.assert_close(parity.f64(out), res["out"], "all tokens")
    parity.record_margin(f"mxfp4 decode: layer output, all {T} tokens", rel, mx)
    _say(f"[mxfp4 decode] all {T} tokens: rel-L2 {rel:.2e}, max-abs {mx:.2e}")
