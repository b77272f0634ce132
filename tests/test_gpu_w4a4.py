"""GPU parity of the W4A4 path (MXFP4 weights x MXFP4-quantized activations on the FP4 matrix
cores) against the oracle (oracle.w4a4), through the C ABI: activation quantizer, W4A4 tile
repack, grouped GEMMs on every tile width, small layers end to end and the decode- and
prefill-shaped layers at full size."""

import numpy as np
import pytest
import torch

import helpers
import parity
from nvfp4_weight_quantized_amd import _lib as L
from nvfp4_weight_quantized_amd import ops, synth
from nvfp4_weight_quantized_amd.workloads import build_layer
from oracle import moe as omoe
from oracle import w4a4 as oa4

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _act_cases(rng):
    yield "gauss", rng.normal(0, 1, (64, 256))
    x = rng.normal(0, 1, (32, 512)) * np.exp2(rng.integers(-30, 30, (32, 1)))
    yield "row_scales", x
    e = rng.normal(0, 1, (8, 128))
    e[0, :32] = 0.0                                              # all-zero group
    e[1, :32] = rng.normal(0, 1, 32) * 1e-39                    # bf16 subnormals
    e[2, :32] = rng.normal(0, 1, 32) * 1e38                     # huge group
    e[3, :32] = 0.75 * 2.0 ** -4                                # every element on a tie
    e[4, :32] = np.array([6.0, -3.5, 2.5, 1.25, 0.25, 5.0, 7.5, -1.75] * 4) * 2.0 ** 3   # ties and clipping
    e[5, :32] = -0.0
    yield "edges", e
    yield "prefill_rows", rng.normal(0, 1, (512, 4096))


def test_a4_activation_quantizer_bit_exact():
    rng = np.random.default_rng(51)
    for name, v in _act_cases(rng):
        bits = oa4.float_to_bf16_bits(v)
        p, s = ops.quantize_act(parity.bits_to_bf16(bits))
        pr, sr = oa4.quantize_act(omoe.bf16_to_float(bits))
        assert np.array_equal(s.cpu().numpy(), sr), name
        assert np.array_equal(p.cpu().numpy(), pr), name


def test_a4_pack_tiles_is_the_stated_permutation():
    rng = np.random.default_rng(52)
    for nt, r, k in [(1, 16, 128), (3, 48, 384), (2, 256, 1024)]:
        p = rng.integers(0, 256, (nt, r, k // 2), dtype=np.uint8)
        s = rng.integers(0, 256, (nt, r, k // 32), dtype=np.uint8)
        tp, ts = ops.pack_tiles(torch.from_numpy(p).to(DEV), torch.from_numpy(s).to(DEV), fmt="mxfp4_a4")
        for t in range(nt):
            wp, ws = parity.tile_np_a4(p[t], s[t])
            assert np.array_equal(tp[t].cpu().numpy(), wp)
            assert np.array_equal(ts[t].cpu().numpy(), ws)


def _bank(rng, e, h, i):
    return helpers.random_layer(rng, h, i, e, 1, shared=False, sigma=0.05, fmt="mxfp4").routed


def _offsets(counts):
    o = np.zeros(len(counts) + 1, np.int32)
    o[1:] = np.cumsum(counts)
    return o


@pytest.mark.parametrize("H,I,counts", [
    (256, 128, [1, 0, 3, 2]),                        # narrow tiles; one K chunk in the down GEMM
    (512, 256, [0, 17, 16, 15, 1, 33, 0, 64]),        # wide tiles, ragged row blocks, empty groups
    (384, 256, [129, 0, 128, 127, 300, 5]),           # several 128-row tiles per group; H % 256 != 0
    (512, 256, [100, 0, 200, 77, 129]),
    (256, 384, [200, 70, 0, 1]),                      # I % 256 != 0
])
def test_a4_grouped_gemm_matches_oracle(H, I, counts):
    rng = np.random.default_rng(H + I + sum(counts) + 3)
    E = len(counts)
    bank = _bank(rng, E, H, I)
    gbank = parity.to_gpu_bank(bank, w4a4=True)
    off = _offsets(counts)
    M = int(off[-1])
    div = 3
    T = (M + div - 1) // div + 2
    x = helpers.random_x(rng, T, H)
    row_index = rng.integers(0, T * div, M).astype(np.int32)
    xq, xs = ops.quantize_act(parity.bits_to_bf16(x))
    goff = torch.from_numpy(off).to(DEV)
    h = ops.grouped_gemm_a4(L.MOE_GEMM_GATE_UP, gbank, xq, xs, goff, M, torch.from_numpy(row_index).to(DEV), div)
    h_ref = oa4.grouped_gate_up_a4(omoe.bf16_to_float(x)[row_index // div], off, bank)
    parity.assert_close(parity.f64(h), h_ref, "gate/up")
    hq, hs = ops.quantize_act(h)
    y = ops.grouped_gemm_a4(L.MOE_GEMM_DOWN, gbank, hq, hs, goff, M)
    y_ref = oa4.grouped_down_a4(parity.f64(h), off, bank)
    parity.assert_close(parity.f64(y), y_ref, "down")


@pytest.mark.parametrize("counts", [[1, 2], [5, 11], [40, 90], [130, 7]])
def test_a4_grouped_gemm_one_hot_pins_layout(counts):
    """A unit row e_h quantizes exactly (code 4.0 at scale 2^-2, zero groups elsewhere), so each
    output is one weight v * 2^(s - 127): pins the W4A4 tile layout, both MFMA operand layouts,
    both scale operands and the gate/up order."""
    rng = np.random.default_rng(60 + sum(counts))
    H, I = 512, 256
    bank = _bank(rng, 2, H, I)
    gbank = parity.to_gpu_bank(bank, w4a4=True)
    off = _offsets(counts)
    M = int(off[-1])
    goff = torch.from_numpy(off).to(DEV)
    hs_ = rng.integers(0, H, M)
    a = np.zeros((M, H), np.float32)
    a[np.arange(M), hs_] = 1.0
    aq, as_ = ops.quantize_act(torch.from_numpy(a).to(torch.bfloat16).to(DEV))
    h = ops.grouped_gemm_a4(L.MOE_GEMM_GATE_UP, gbank, aq, as_, goff, M)
    ref = omoe.grouped_gate_up(a.astype(np.float64), off, bank)
    assert np.all(np.abs(parity.f64(h) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    is_ = rng.integers(0, I, M)
    a2 = np.zeros((M, I), np.float32)
    a2[np.arange(M), is_] = 1.0
    a2q, a2s = ops.quantize_act(torch.from_numpy(a2).to(torch.bfloat16).to(DEV))
    y = ops.grouped_gemm_a4(L.MOE_GEMM_DOWN, gbank, a2q, a2s, goff, M)
    ref2 = omoe.grouped_down(a2.astype(np.float64), off, bank)
    assert np.all(np.abs(parity.f64(y) - ref2) <= 2.0 ** -8 * np.abs(ref2) + 1e-30)


SMALL = [
    # T, H, I, E, k, shared, bias, I_shared
    (16, 256, 128, 8, 2, True, False, None),          # the tiny layer's shape
    (5, 256, 128, 8, 2, True, False, None),
    (64, 512, 256, 16, 4, True, True, None),
    (300, 512, 256, 16, 4, True, False, None),
    (37, 384, 256, 12, 3, False, True, None),
    (600, 512, 256, 16, 4, True, False, None),
    (40, 256, 128, 8, 2, True, False, 256),           # shared expert of another width: own launches
]


@pytest.mark.parametrize("case", SMALL, ids=[f"T{c[0]}_H{c[1]}_I{c[2]}_E{c[3]}_k{c[4]}_Is{c[7]}" for c in SMALL])
def test_a4_small_layer_end_to_end(case):
    T, H, I, E, k, shared, bias, i_sh = case
    rng = np.random.default_rng(sum(case[:5]) + 11)
    layer = helpers.random_layer(rng, H, I, E, k, shared=shared, bias=bias, fmt="mxfp4", i_shared=i_sh)
    x = helpers.random_x(rng, T, H)
    glayer = parity.to_gpu_layer(layer, w4a4=True)
    assert glayer.is_w4a4
    out, aux = ops.forward(glayer, parity.bits_to_bf16(x), return_aux=True)
    parity.check_route(aux["logits"], aux["topk_ids"], aux["topk_w"], x, layer.w_router, layer.router_bias, k)
    res = parity.reference_for_selection(x, layer, aux["topk_ids"].cpu().numpy(), forward=oa4.forward)
    parity.assert_close(parity.f64(out), res["out"], "layer")
    assert torch.equal(out, ops.forward(glayer, parity.bits_to_bf16(x))), "two runs differ"
    # the W4A16 kernels on the same weights give a measurably different layer: 4-bit activations
    w16 = ops.forward(parity.to_gpu_layer(layer), parity.bits_to_bf16(x))
    rel, _ = parity.errors(parity.f64(w16), res["out"])
    assert rel > 1e-2


def test_a4_no_tokens_is_a_no_op():
    rng = np.random.default_rng(70)
    layer = helpers.random_layer(rng, 256, 128, 4, 2, shared=True, fmt="mxfp4")
    glayer = parity.to_gpu_layer(layer, w4a4=True)
    x = torch.empty(0, 256, dtype=torch.bfloat16, device=DEV)
    assert ops.forward(glayer, x).shape == (0, 256)


def _full_size(name, tokens):
    wl = synth.WORKLOADS[name]
    _say(f"[w4a4 {name}] building layer T={wl.T} E={wl.E} H={wl.H} I={wl.I}")
    glayer = build_layer(wl, DEV, fmt="mxfp4_a4")
    x = synth.activations(wl, DEV)
    out, aux = ops.forward(glayer, x, return_aux=True)
    torch.cuda.synchronize()
    xb = helpers.bf16_bits(x)
    ids = aux["topk_ids"].cpu().numpy()
    ids_ref, _ = omoe.topk(aux["logits"].cpu().numpy().astype(np.float64), wl.k)
    assert np.array_equal(ids, ids_ref)
    olayer = helpers.oracle_layer(wl, DEV, fmt="mxfp4")
    used = np.unique(ids[tokens])
    olayer.routed.prefetch(used)
    for e in used[:4]:
        ow = olayer.routed[int(e)]
        t13, s13 = parity.tile_np_a4(ow.w13, ow.w13_scale)
        assert np.array_equal(glayer.routed.w13[e].cpu().numpy(), t13), e
        assert np.array_equal(glayer.routed.w13_scale[e].cpu().numpy(), s13), e
    res = parity.reference_for_selection(xb[tokens], olayer, ids[tokens], forward=oa4.forward)
    rel, mx = parity.assert_close(parity.f64(out[torch.from_numpy(tokens).to(DEV)]), res["out"], "sampled tokens")
    _say(f"[w4a4 {name}] tokens {tokens.tolist()}: rel-L2 {rel:.2e}, max-abs {mx:.2e}")
    assert torch.equal(out, ops.forward(glayer, x)), "two runs differ"


@pytest.mark.timeout(600)
def test_a4_decode_workload_full_size():
    _full_size("decode", np.array([0, 7]))


@pytest.mark.timeout(900)
def test_a4_prefill_workload_full_size_sampled():
    """The prefill-shaped layer (T=4096): every tile path at its real grid; sampled tokens against
    the oracle."""
    _full_size("prefill", np.array([0, 1234, 4095]))
