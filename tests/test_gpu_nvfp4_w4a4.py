"""GPU parity of the NVFP4 W4A4 path (NVFP4 weights x NVFP4-quantized activations, alpha = d_act *
d_w) against the oracle (oracle.nvfp4_w4a4), through the C ABI: the activation quantizer bit for
bit, the grouped GEMMs on every tile path (8-, 16-, 64- and 128-row tiles, fp16 and bf16
operands), small layers end to end, the decode- and prefill-shaped layers at full size, and the
refusal of a missing activation scale."""

import ctypes

import numpy as np
import pytest
import torch

import helpers
import parity
from nvfp4_weight_quantized_amd import _lib as L
from nvfp4_weight_quantized_amd import ops, synth
from nvfp4_weight_quantized_amd.workloads import build_layer
from oracle import moe as omoe
from oracle import nvfp4 as onv
from oracle import nvfp4_w4a4 as onw
from oracle import w4a4 as oa4

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _act_cases(rng):
    yield "gauss", rng.normal(0, 1, (64, 256)), None
    x = rng.normal(0, 1, (32, 512)) * np.exp2(rng.integers(-12, 12, (32, 1)))
    yield "row_scales", x, None
    e = rng.normal(0, 1, (8, 128))
    e[0, :16] = 0.0                                              # all-zero group
    e[1, :16] = rng.normal(0, 1, 16) * 1e-7                      # tiny group: E4M3 subnormal / zero scale
    e[2, :16] = rng.normal(0, 1, 16) * 1e5                       # huge group: scale capped at 448
    e[3, :16] = 0.75 * 2.0 ** -4                                 # every element on the same value
    e[4, :16] = np.array([6.0, -3.5, 2.5, 1.25, 0.25, 5.0, 7.5, -1.75] * 2) * 2.0 ** -2
    e[5, :16] = -0.0
    yield "edges", e, 1.0 / 2688.0
    yield "edges_small_d", e, 2.0 ** -24
    yield "prefill_rows", rng.normal(0, 1, (512, 4096)), None


def test_nv_activation_quantizer_bit_exact():
    rng = np.random.default_rng(81)
    for name, v, d in _act_cases(rng):
        bits = oa4.float_to_bf16_bits(v)
        xv = omoe.bf16_to_float(bits)
        d = onv.gscale_modelopt(np.abs(xv).max()) if d is None else np.float32(d)
        a = parity.bits_to_bf16(bits)
        p, s, vals = ops.quantize_act_nv(a, float(d))
        pr, sr = onw.quantize_act(xv, d)
        assert np.array_equal(s.cpu().numpy(), sr), name
        assert np.array_equal(p.cpu().numpy(), pr), name
        assert np.array_equal(parity.f64(vals), onw.act_values(xv, d)), name
        # in place: the same values overwrite the input
        a2 = a.clone()
        ops.quantize_act_nv(a2, float(d), packed=False, scales=False, in_place=True)
        assert torch.equal(a2, vals), name


def _bank(rng, e, h, i):
    return helpers.random_layer(rng, h, i, e, 1, shared=False, sigma=0.05).routed


def _offsets(counts):
    o = np.zeros(len(counts) + 1, np.int32)
    o[1:] = np.cumsum(counts)
    return o


@pytest.mark.parametrize("H,I,counts", [
    (256, 128, [1, 0, 3, 2]),                         # 8-row (skinny) tiles
    (512, 256, [0, 17, 16, 15, 1, 12, 0, 9]),         # 16-row tiles
    (512, 256, [30, 0, 25, 31, 20]),                  # 64-row tiles
    (512, 256, [129, 0, 128, 127, 300, 5]),           # 128-row tiles, fp16 gate/up operands
    (384, 384, [200, 70, 0, 1]),                      # 128-row tiles, I % 256 != 0: bf16 operands
])
def test_nv_w4a4_grouped_gemm_matches_oracle(H, I, counts):
    rng = np.random.default_rng(H + I + sum(counts) + 7)
    E = len(counts)
    bank = _bank(rng, E, H, I)
    gbank = parity.to_gpu_bank(bank)
    off = _offsets(counts)
    M = int(off[-1])
    div = 3
    T = (M + div - 1) // div + 2
    x = helpers.random_x(rng, T, H)
    xv = omoe.bf16_to_float(x)
    d_x = onv.gscale_modelopt(np.abs(xv).max())
    row_index = rng.integers(0, T * div, M).astype(np.int32)
    _, _, xa = ops.quantize_act_nv(parity.bits_to_bf16(x), float(d_x), packed=False, scales=False)
    goff = torch.from_numpy(off).to(DEV)
    h = ops.grouped_gemm_w4a4(L.MOE_GEMM_GATE_UP, gbank, xa, float(d_x), goff, M,
                              torch.from_numpy(row_index).to(DEV), div)
    h_ref = onw.grouped_gate_up_a4(xv[row_index // div], off, bank, d_x)
    rel, mx = parity.assert_close(parity.f64(h), h_ref, "gate/up")
    hv = parity.f64(h)
    d_h = onv.gscale_modelopt(max(np.abs(hv).max(), 1e-30))
    _, _, ha = ops.quantize_act_nv(h, float(d_h), packed=False, scales=False)
    y = ops.grouped_gemm_w4a4(L.MOE_GEMM_DOWN, gbank, ha, float(d_h), goff, M)
    y_ref = onw.grouped_down_a4(hv, off, bank, d_h)
    parity.assert_close(parity.f64(y), y_ref, "down")
    # the W4A16 GEMM on the same rows is a different computation
    h16 = ops.grouped_gemm(L.MOE_GEMM_GATE_UP, gbank, parity.bits_to_bf16(x), goff, M,
                           torch.from_numpy(row_index).to(DEV), div)
    assert parity.errors(parity.f64(h16), h_ref)[0] > 1e-3


def _calibrate(layer, x_bits):
    """Static scales as a caller would calibrate them: d_x from the tokens, d_h from the W4A4 h of
    expert 0 on every token."""
    x = omoe.bf16_to_float(x_bits)
    d_x = onv.gscale_modelopt(np.abs(x).max())
    h = onw.gate_up_a4(x, layer.routed[0], d_x)
    return d_x, onv.gscale_modelopt(max(np.abs(h).max(), 1e-30))


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
def test_nv_w4a4_small_layer_end_to_end(case):
    T, H, I, E, k, shared, bias, i_sh = case
    rng = np.random.default_rng(sum(case[:5]) + 13)
    layer = helpers.random_layer(rng, H, I, E, k, shared=shared, bias=bias, i_shared=i_sh)
    x = helpers.random_x(rng, T, H)
    d_x, d_h = _calibrate(layer, x)
    glayer = parity.to_gpu_layer(layer)
    xg = parity.bits_to_bf16(x)
    out, aux = ops.forward(glayer, xg, return_aux=True, return_rows=True, act_gscales=(d_x, d_h))
    parity.check_route(aux["logits"], aux["topk_ids"], aux["topk_w"], x, layer.w_router, layer.router_bias, k)

    def oracle_fwd(xb, lay, route=None):
        return onw.forward(xb, lay, d_x, d_h, route=route)

    res = parity.reference_for_selection(x, layer, aux["topk_ids"].cpu().numpy(), forward=oracle_fwd)
    parity.assert_close(parity.f64(out), res["out"], "layer")
    yr = parity.f64(aux["y_rows"])
    parity.assert_close(yr[:T * k], res["y_rows"], "routed expert rows")
    if shared:
        parity.assert_close(yr[T * k:], res["y_shared"], "shared expert rows")
    assert torch.equal(out, ops.forward(glayer, xg, act_gscales=(d_x, d_h))), "two runs differ"
    # the W4A16 layer on the same weights and tokens is measurably different
    w16 = ops.forward(glayer, xg)
    assert parity.errors(parity.f64(w16), res["out"])[0] > 1e-3


def test_nv_w4a4_refuses_a_missing_activation_scale():
    """A zero activation scale would zero every expert: the library refuses it before any launch."""
    rng = np.random.default_rng(90)
    layer = helpers.random_layer(rng, 256, 128, 4, 2, shared=True)
    glayer = parity.to_gpu_layer(layer)
    x = parity.bits_to_bf16(helpers.random_x(rng, 8, 256))
    out = torch.full_like(x, 7.0)
    ws = ops.workspace_for(glayer, 8, x.device, nvfp4_a4=True)
    st = glayer.checked_struct()
    torch.cuda.synchronize()
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        rc = L.lib().moe_nvfp4_w4a4_forward(ctypes.byref(st), x.data_ptr(), 8, bad, 1e-3, out.data_ptr(),
                                            ws.data_ptr(), ws.numel(), None, None)
        assert rc == L.MOE_ERR_INVALID_ARGUMENT, bad
        with pytest.raises(ValueError):
            ops.forward(glayer, x, act_gscales=(1e-3, bad))
    torch.cuda.synchronize()
    assert torch.all(out == 7.0), "a refused call wrote its output"


def test_nv_w4a4_no_tokens_is_a_no_op():
    rng = np.random.default_rng(91)
    layer = helpers.random_layer(rng, 256, 128, 4, 2, shared=True)
    glayer = parity.to_gpu_layer(layer)
    x = torch.empty(0, 256, dtype=torch.bfloat16, device=DEV)
    assert ops.forward(glayer, x, act_gscales=(1e-3, 1e-3)).shape == (0, 256)


def _full_size(name, tokens):
    wl = synth.WORKLOADS[name]
    _say(f"[nvfp4 w4a4 {name}] building layer T={wl.T} E={wl.E} H={wl.H} I={wl.I}")
    glayer = build_layer(wl, DEV)
    x = synth.activations(wl, DEV)
    xb = helpers.bf16_bits(x)
    olayer = helpers.oracle_layer(wl, DEV)
    # static scales: d_x from the tokens, d_h from the GPU's W4A4 gate/up of the shared expert
    d_x = onv.gscale_modelopt(float(x.abs().max()))
    _, _, xa = ops.quantize_act_nv(x, float(d_x), packed=False, scales=False)
    zero = torch.zeros(2, dtype=torch.int32, device=DEV)
    zero[1] = wl.T
    h_sh = ops.grouped_gemm_w4a4(L.MOE_GEMM_GATE_UP, glayer.shared, xa, float(d_x), zero, wl.T)
    d_h = onv.gscale_modelopt(float(h_sh.abs().max()))
    out, aux = ops.forward(glayer, x, return_aux=True, act_gscales=(d_x, d_h))
    torch.cuda.synchronize()
    ids = aux["topk_ids"].cpu().numpy()
    ids_ref, _ = omoe.topk(aux["logits"].cpu().numpy().astype(np.float64), wl.k)
    assert np.array_equal(ids, ids_ref)
    used = np.unique(ids[tokens])
    olayer.routed.prefetch(used)

    def oracle_fwd(xbits, lay, route=None):
        return onw.forward(xbits, lay, d_x, d_h, route=route)

    res = parity.reference_for_selection(xb[tokens], olayer, ids[tokens], forward=oracle_fwd)
    rel, mx = parity.assert_close(parity.f64(out[torch.from_numpy(tokens).to(DEV)]), res["out"], "sampled tokens")
    parity.record_margin(f"nvfp4 w4a4 {name}: layer output, tokens {tokens.tolist()}", rel, mx)
    _say(f"[nvfp4 w4a4 {name}] tokens {tokens.tolist()}: rel-L2 {rel:.2e}, max-abs {mx:.2e}")
    assert torch.equal(out, ops.forward(glayer, x, act_gscales=(d_x, d_h))), "two runs differ"


@pytest.mark.timeout(600)
def test_nv_w4a4_decode_workload_full_size():
    _full_size("decode", np.arange(8))


@pytest.mark.timeout(900)
def test_nv_w4a4_prefill_workload_full_size_sampled():
    """The prefill-shaped layer (T=4096): every tile path at its real grid (fp16 gate/up operands);
    sampled tokens against the oracle."""
    _full_size("prefill", np.array([0, 1234, 4095]))
