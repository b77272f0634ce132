"""GPU parity of each stage of the HIP path against the oracle, through the C ABI."""

import ctypes

import numpy as np
import pytest
import torch

import helpers
import parity
from nvfp4_weight_quantized_amd import _lib as L
from nvfp4_weight_quantized_amd import ops
from oracle import moe as omoe
from oracle import nvfp4 as onv

pytestmark = pytest.mark.gpu
DEV = "cuda"


# ----------------------------------------------------------------------------- quantizer

def _quant_cases(rng):
    yield "gauss", rng.normal(0, 0.02, (3, 64, 256)).astype(np.float32)
    w = rng.normal(0, 0.015, (2, 32, 512)).astype(np.float32)
    w[:, ::7, 5] = 0.3                                   # outliers -> E4M3 scale at 448
    yield "outliers", w
    z = rng.normal(0, 1, (1, 16, 64)).astype(np.float32)
    z[0, 3] = 0.0                                        # all-zero groups
    z[0, 4, :16] = 1e-12                                 # scale underflows to 0
    yield "zeros", z
    # exact E2M1 midpoints after scaling: ties must go to the even code on both sides
    grid = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -1.75, -5.0, 6.0, 0.5, -6.0, 3.0, 4.0])
    yield "ties", np.tile(grid, (1, 8, 4)).astype(np.float32)
    yield "tiny_scales", (rng.normal(0, 1, (1, 8, 128)) * np.exp2(rng.integers(-20, 4, (1, 8, 1)))).astype(np.float32)


def test_quantizer_bit_exact_against_oracle():
    rng = np.random.default_rng(21)
    for name, w in _quant_cases(rng):
        d = np.array([onv.gscale_modelopt(np.abs(t).max()) if np.abs(t).max() > 0 else np.float32(1e-3) for t in w],
                     np.float32)
        if name == "ties":
            d[:] = np.float32(1.0 / 2688.0 * 6.0)            # amax 6 -> group scale exactly 1... of 6*d
        p, s = ops.quantize(torch.from_numpy(w).to(DEV), torch.from_numpy(d).to(DEV))
        for t in range(w.shape[0]):
            pr, sr = onv.quantize(w[t], d[t])
            assert np.array_equal(s[t].cpu().numpy(), sr), name
            assert np.array_equal(p[t].cpu().numpy(), pr), name


def test_pack_tiles_is_the_stated_permutation():
    rng = np.random.default_rng(22)
    for nt, r, k in [(1, 16, 128), (3, 48, 384), (2, 256, 1024)]:
        p = rng.integers(0, 256, (nt, r, k // 2), dtype=np.uint8)
        s = rng.integers(0, 256, (nt, r, k // 16), dtype=np.uint8)
        tp, ts = ops.pack_tiles(torch.from_numpy(p).to(DEV), torch.from_numpy(s).to(DEV))
        for t in range(nt):
            wp, ws = parity.tile_np(p[t], s[t])
            assert np.array_equal(tp[t].cpu().numpy(), wp)
            assert np.array_equal(ts[t].cpu().numpy(), ws)


# ----------------------------------------------------------------------------- route

@pytest.mark.parametrize("T,H,E,k,bias", [(1, 128, 8, 1, False), (8, 4096, 320, 8, False), (16, 256, 8, 2, True),
                                          (32, 512, 64, 6, False), (33, 256, 320, 8, True), (200, 384, 256, 8, False),
                                          (130, 1024, 1024, 64, True), (100, 256, 72, 4, True)])
def test_route_matches_oracle(T, H, E, k, bias):
    rng = np.random.default_rng(T * 1000 + E)
    x = helpers.random_x(rng, T, H)
    wr = helpers.bf16_bits(torch.from_numpy(rng.normal(0, 0.05, (E, H)).astype(np.float32)).to(torch.bfloat16))
    b = rng.normal(0, 0.5, E).astype(np.float32) if bias else None
    logits, ids, w = ops.route(parity.bits_to_bf16(x), parity.bits_to_bf16(wr),
                               torch.from_numpy(b).to(DEV) if bias else None, k)
    parity.check_route(logits, ids, w, x, wr, b, k)


def test_topk_from_given_logits_ties_and_nonfinite():
    rng = np.random.default_rng(5)
    lg = rng.normal(0, 1, (97, 300)).round(1).astype(np.float32)    # many exact ties
    lg[0, :] = 1.0
    lg[1, :5] = -np.inf
    lg[2, 7] = np.inf
    ids, w = ops.route_from_logits(torch.from_numpy(lg).to(DEV), 8)
    ids_ref, w_ref = omoe.topk(lg.astype(np.float64), 8)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    ok = np.isfinite(w_ref).all(axis=1)
    np.testing.assert_allclose(w.cpu().numpy()[ok], w_ref[ok], rtol=0, atol=1e-5)
    assert ids.cpu().numpy()[0].tolist() == list(range(8))


# ----------------------------------------------------------------------------- permute

@pytest.mark.parametrize("T,k,E,skew", [(0, 8, 320, 0.0), (1, 1, 1, 0.0), (8, 8, 320, 0.0), (16, 2, 8, 0.0),
                                        (256, 8, 320, 0.0), (257, 8, 320, 0.0), (4096, 8, 320, 0.0),
                                        (2048, 8, 320, 1.2), (3001, 5, 1024, 0.0), (1000, 8, 16, 3.0),
                                        (16384, 8, 256, 0.0)])
def test_permute_bit_exact(T, k, E, skew):
    rng = np.random.default_rng(T + E)
    if T:
        p = np.arange(1, E + 1, dtype=np.float64) ** -skew
        p /= p.sum()
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    else:
        ids = np.zeros((0, k), np.int32)
    counts, offsets, sorted_slot, slot_to_row = ops.permute(torch.from_numpy(ids).to(DEV), E)
    c, o, s, r = omoe.permute(ids, E)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(sorted_slot.cpu().numpy(), s)
    assert np.array_equal(slot_to_row.cpu().numpy(), r)


# ----------------------------------------------------------------------------- grouped GEMMs

def _random_bank(rng, E, H, I, sigma=0.05):
    return helpers.random_layer(rng, H, I, E, 1, shared=False, sigma=sigma).routed


def _offsets(counts):
    o = np.zeros(len(counts) + 1, np.int32)
    o[1:] = np.cumsum(counts)
    return o


@pytest.mark.parametrize("H,I,counts", [
    (256, 128, [1, 0, 3, 2]),                      # decode-like: 8-row skinny tiles, K chunks of 256 / 128
    (512, 256, [8, 9, 2, 4, 0, 17, 3, 1, 6, 5]),    # skinny: 1, 2 and 4 accumulator registers, 8-row tails
    (384, 512, [7, 1, 1, 2, 3, 4, 8, 0]),          # skinny: K = 384 (128-wide chunks), narrow down output
    (256, 128, [12, 0, 9, 16, 20]),                # 16-row tiles
    (256, 128, [0] * 700 + [1, 0, 3] * 100 + [2] * 24),   # 1024 groups: 16 groups per lane in the tile scan
    (256, 128, [40] * 1000 + [0, 300, 129] * 8),   # 1024 groups, 128-row tiles
    (512, 256, [0, 17, 16, 15, 1, 33, 0, 64]),      # 64-row tiles, ragged tails
    (384, 256, [129, 0, 128, 127, 300, 5]),         # 128-row tiles; H % 256 != 0 -> narrow down tiles
    (256, 384, [200, 70, 0, 1]),
    (512, 256, [100, 0, 200, 77, 129]),            # eight-wave gate/up, four-wave down (128-row tiles)
    (128, 256, [100, 0, 200, 77, 129]),            # eight-wave gate/up with a single K chunk
    (512, 128, [100, 0, 200, 77, 129]),            # four-wave down, 512-column output, a single K chunk
    (1024, 384, [100, 0, 200, 77, 129]),           # four-wave down with three K chunks (odd count)
    (256, 1024, [100, 0, 200, 77, 129]),           # eight-wave gate/up with two K chunks, four-wave down with eight
])
def test_grouped_gemm_random_matches_oracle(H, I, counts):
    rng = np.random.default_rng(H + I + sum(counts))
    E = len(counts)
    bank = _random_bank(rng, E, H, I)
    gbank = parity.to_gpu_bank(bank)
    off = _offsets(counts)
    M = int(off[-1])
    # gate/up with a row gather: A rows = x[row_index // div]
    div = 3
    T = (M + div - 1) // div + 2
    x = helpers.random_x(rng, T, H)
    row_index = rng.integers(0, T * div, M).astype(np.int32)
    h = ops.grouped_gemm(L.MOE_GEMM_GATE_UP, gbank, parity.bits_to_bf16(x), torch.from_numpy(off).to(DEV), M,
                         torch.from_numpy(row_index).to(DEV), div)
    a_rows = omoe.bf16_to_float(x)[row_index // div]
    h_ref = omoe.grouped_gate_up(a_rows, off, bank)
    parity.assert_close(parity.f64(h), h_ref, "gate/up")
    # down on the GPU's own h (bf16) rows
    hb = helpers.bf16_bits(h)
    y = ops.grouped_gemm(L.MOE_GEMM_DOWN, gbank, h, torch.from_numpy(off).to(DEV), M)
    y_ref = omoe.grouped_down(omoe.bf16_to_float(hb), off, bank)
    parity.assert_close(parity.f64(y), y_ref, "down")


def test_grouped_gemm_one_hot_pins_layout():
    """A unit row e_h makes each output one dequantized weight: pins nibble order, scale index, gate/up order."""
    rng = np.random.default_rng(3)
    H, I = 256, 128
    bank = _random_bank(rng, 2, H, I)
    gbank = parity.to_gpu_bank(bank)
    hs = np.array([0, 1, 15, 16, 17, 31, 32, 100, 127, 128, 255] * 2)
    M = len(hs)
    counts = [11, 11]
    off = _offsets(counts)
    a = np.zeros((M, H), np.float32)
    a[np.arange(M), hs] = 1.0
    ab = torch.from_numpy(a).to(torch.bfloat16)
    h = ops.grouped_gemm(L.MOE_GEMM_GATE_UP, gbank, ab.to(DEV), torch.from_numpy(off).to(DEV), M)
    ref = omoe.grouped_gate_up(a.astype(np.float64), off, bank)
    got = parity.f64(h)
    # one product per output, then SiLU and one bf16 rounding: within one bf16 ulp
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    # down: unit rows over I
    is_ = np.array([0, 1, 15, 16, 64, 127] * 2)
    a2 = np.zeros((len(is_), I), np.float32)
    a2[np.arange(len(is_)), is_] = 1.0
    off2 = _offsets([6, 6])
    y = ops.grouped_gemm(L.MOE_GEMM_DOWN, gbank, torch.from_numpy(a2).to(torch.bfloat16).to(DEV),
                         torch.from_numpy(off2).to(DEV), len(is_))
    ref2 = omoe.grouped_down(a2.astype(np.float64), off2, bank)
    assert np.all(np.abs(parity.f64(y) - ref2) <= 2.0 ** -8 * np.abs(ref2) + 1e-30)


@pytest.mark.parametrize("H,I,counts", [
    (512, 256, [40, 0, 130]),      # 128-row tiles: eight-wave gate/up, four-wave down (4 fragments)
    (384, 256, [40, 0, 130]),      # eight-wave gate/up, four-wave down with 2 fragments per wave
    (256, 128, [40, 0, 130]),      # four waves for both GEMMs
])
def test_tall_grouped_gemm_one_hot_pins_layout(H, I, counts):
    """Unit rows on the 128-row tile paths: each output is one dequantized weight (gate/up: then
    SiLU(gate)*up), within one bf16 ulp -- pins nibble order, scale index and gate/up order there."""
    rng = np.random.default_rng(H + I + 7)
    bank = _random_bank(rng, len(counts), H, I)
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


@pytest.mark.parametrize("counts", [[1, 1], [2, 0], [3, 4], [5, 8]])
def test_skinny_grouped_gemm_one_hot_pins_layout(counts):
    """The same one-hot pin on the few-rows path (unscaled codes, block scale applied to the sums)."""
    rng = np.random.default_rng(4 + sum(counts))
    H, I = 512, 256
    bank = _random_bank(rng, 2, H, I)
    gbank = parity.to_gpu_bank(bank)
    off = _offsets(counts)
    M = int(off[-1])
    hs = rng.choice(H, M, replace=False)
    a = np.zeros((M, H), np.float32)
    a[np.arange(M), hs] = 1.0
    h = ops.grouped_gemm(L.MOE_GEMM_GATE_UP, gbank, torch.from_numpy(a).to(torch.bfloat16).to(DEV),
                         torch.from_numpy(off).to(DEV), M)
    ref = omoe.grouped_gate_up(a.astype(np.float64), off, bank)
    assert np.all(np.abs(parity.f64(h) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    is_ = rng.choice(I, M, replace=False)
    a2 = np.zeros((M, I), np.float32)
    a2[np.arange(M), is_] = 1.0
    y = ops.grouped_gemm(L.MOE_GEMM_DOWN, gbank, torch.from_numpy(a2).to(torch.bfloat16).to(DEV),
                         torch.from_numpy(off).to(DEV), M)
    ref2 = omoe.grouped_down(a2.astype(np.float64), off, bank)
    assert np.all(np.abs(parity.f64(y) - ref2) <= 2.0 ** -8 * np.abs(ref2) + 1e-30)


# ----------------------------------------------------------------------------- combine

@pytest.mark.parametrize("T,k,H,shared", [(1, 1, 128, False), (8, 8, 4096, True), (100, 3, 384, True),
                                          (37, 8, 6144, False)])
def test_combine_matches_oracle(T, k, H, shared):
    rng = np.random.default_rng(T * k)
    S = T * k
    y = helpers.random_x(rng, S, H)
    ys = helpers.random_x(rng, T, H) if shared else None
    perm = rng.permutation(S).astype(np.int32)
    w = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    out = ops.combine(parity.bits_to_bf16(y), torch.from_numpy(perm).to(DEV), torch.from_numpy(w).to(DEV),
                      parity.bits_to_bf16(ys) if shared else None)
    ref = omoe.combine(omoe.bf16_to_float(y), perm, w.astype(np.float64),
                       omoe.bf16_to_float(ys) if shared else None)
    got = parity.f64(out)
    # fp32 accumulation, one bf16 rounding at the end
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max())


# ----------------------------------------------------------------------------- errors

def test_bad_arguments_fail_loudly():
    x = torch.zeros(4, 256, dtype=torch.bfloat16, device=DEV)
    wr = torch.zeros(8, 256, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(L.MoeError):
        ops.route(x, wr, None, 9)                       # k > E
    with pytest.raises(L.MoeError):
        ops.route(torch.zeros(4, 200, dtype=torch.bfloat16, device=DEV),
                  torch.zeros(8, 200, dtype=torch.bfloat16, device=DEV), None, 2)   # H % 128 != 0


def test_mismatched_shapes_raise_before_any_launch():
    """Host-side checks of the binding: every shape, dtype and device mismatch raises ValueError (or
    TypeError) before the library is called, so a wrong tensor never turns into out-of-bounds access."""
    rng = np.random.default_rng(5)
    layer = helpers.random_layer(rng, 256, 128, 8, 2)
    glayer = parity.to_gpu_layer(layer)
    x = torch.zeros(4, 256, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        ops.forward(glayer, torch.zeros(4, 384, dtype=torch.bfloat16, device=DEV))     # x width != H
    with pytest.raises(ValueError):
        ops.forward(glayer, x, out=torch.empty(5, 256, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(TypeError):
        ops.forward(glayer, x, out=torch.empty(4, 256, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        ops.forward(glayer, x, out=torch.empty(4, 256, dtype=torch.bfloat16))           # host tensor
    bad = ops.NvFp4MoELayer(glayer.w_router[:, :128].contiguous(), None, glayer.routed, glayer.shared, 2)
    with pytest.raises(ValueError):
        ops.forward(bad, x)                                                              # router [E, H/2]
    bad = ops.NvFp4MoELayer(glayer.w_router, torch.zeros(9, device=DEV), glayer.routed, glayer.shared, 2)
    with pytest.raises(ValueError):
        ops.forward(bad, x)                                                              # bias [E+1]
    wr = glayer.w_router
    with pytest.raises(ValueError):
        ops.route(x, torch.zeros(8, 384, dtype=torch.bfloat16, device=DEV), None, 2)
    with pytest.raises(ValueError):
        ops.route(x, wr, torch.zeros(7, device=DEV), 2)
    ids = torch.zeros(4, 2, dtype=torch.int32, device=DEV)
    counts, offsets, sorted_slot, slot_to_row = ops.permute(ids, 8)
    with pytest.raises(ValueError):
        ops.grouped_gemm(L.MOE_GEMM_GATE_UP, glayer.routed, torch.zeros(4, 128, dtype=torch.bfloat16, device=DEV),
                         offsets, 8, sorted_slot, 2)                                     # a width != H
    with pytest.raises(ValueError):
        ops.grouped_gemm(L.MOE_GEMM_GATE_UP, glayer.routed, x, offsets[:5].contiguous(), 8, sorted_slot, 2)
    with pytest.raises(ValueError):
        ops.grouped_gemm(L.MOE_GEMM_DOWN, glayer.routed, torch.zeros(3, 128, dtype=torch.bfloat16, device=DEV),
                         offsets, 8)                                                     # fewer rows than M
    y = torch.zeros(8, 256, dtype=torch.bfloat16, device=DEV)
    w = torch.full((4, 2), 0.5, device=DEV)
    with pytest.raises(ValueError):
        ops.combine(y, slot_to_row[:7].contiguous(), w)
    with pytest.raises(ValueError):
        ops.combine(y, slot_to_row, w, torch.zeros(4, 128, dtype=torch.bfloat16, device=DEV))
    a4 = ops.NvFp4Experts(glayer.routed.w13, glayer.routed.w13_scale[..., :64].contiguous(), None, glayer.routed.w2,
                          glayer.routed.w2_scale[..., :4].contiguous(), None, fmt="mxfp4_a4")
    with pytest.raises(ValueError):
        ops.grouped_gemm(L.MOE_GEMM_GATE_UP, a4, x, offsets, 8, sorted_slot, 2)         # W4A4 bank


def test_permute_rejects_out_of_range_ids_without_writing_out_of_bounds():
    """ids outside [0, E) join no group: their slots get row -1, the offsets end below T*k, nothing is
    written past the output buffers, and the combine turns a token with such a slot into NaN."""
    T, k, E = 300, 4, 16
    rng = np.random.default_rng(9)
    for S_case in (T, 4000):   # one-workgroup and multi-block permutation
        t = S_case // k
        ids = rng.integers(0, E, (t, k)).astype(np.int32)
        ids[3, 1] = E
        ids[t - 1, 0] = -1
        ids[t // 2, k - 1] = 1 << 20
        guard = 1000
        dev_ids = torch.from_numpy(ids).to(DEV)
        counts = torch.empty(E, dtype=torch.int32, device=DEV)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        sorted_buf = torch.full((t * k + guard,), -7, dtype=torch.int32, device=DEV)
        s2r_buf = torch.full((t * k + guard,), -7, dtype=torch.int32, device=DEV)
        ws_bytes = L.lib().moe_permute_workspace_size(t, k, E)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=DEV)
        L.check("moe_permute", L.lib().moe_permute(
            ctypes.c_void_p(dev_ids.data_ptr()), t, k, E, ctypes.c_void_p(counts.data_ptr()),
            ctypes.c_void_p(offsets.data_ptr()), ctypes.c_void_p(sorted_buf.data_ptr()),
            ctypes.c_void_p(s2r_buf.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws_bytes,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
        torch.cuda.synchronize()
        valid = (ids >= 0) & (ids < E)
        n_valid = int(valid.sum())
        flat = ids.reshape(-1)
        want_counts = np.bincount(flat[valid.reshape(-1)], minlength=E)
        assert np.array_equal(counts.cpu().numpy(), want_counts)
        off = offsets.cpu().numpy()
        assert off[E] == n_valid < t * k
        srt = sorted_buf.cpu().numpy()
        s2r = s2r_buf.cpu().numpy()
        assert np.all(srt[t * k:] == -7) and np.all(s2r[t * k:] == -7), "write past the end"
        order = np.argsort(np.where(valid.reshape(-1), flat, E), kind="stable")[:n_valid]
        assert np.array_equal(srt[:n_valid], order)
        assert np.all(s2r[:t * k][~valid.reshape(-1)] == -1)
        assert np.array_equal(s2r[order], np.arange(n_valid))
        # the combine makes the affected tokens NaN (loud), the others finite
        y = torch.ones(t * k, 128, dtype=torch.bfloat16, device=DEV)
        w = torch.full((t, k), 1.0 / k, device=DEV)
        out = ops.combine(y, s2r_buf[:t * k].contiguous(), w).float().cpu().numpy()
        bad_tok = ~valid.all(axis=1)
        assert np.all(np.isnan(out[bad_tok])) and np.all(np.isfinite(out[~bad_tok]))
