"""The C-ABI library loads, exports every declared symbol, and its host-only logic is right (CPU only)."""

import ctypes
import os
import re

import numpy as np
import pytest

import nvfp4_weight_quantized_amd as moe
from nvfp4_weight_quantized_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_nvfp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 11
    lib = L.lib()
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(L.SIGNATURES), "binding and header disagree"


def test_status_strings():
    assert L.status_string(0) == "MOE_OK"
    assert "WORKSPACE" in L.status_string(3)
    assert "gfx950" in L.status_string(2)


def test_gscale_conversion_worked_example_and_errors():
    d = moe.gscale_from_quant_scale(np.array([21504.0], np.float32))
    assert float(d[0]) == 4.650297705666162e-05
    q = np.exp2(np.random.default_rng(0).uniform(-10, 14, 1000)).astype(np.float32)
    assert np.array_equal(moe.gscale_from_quant_scale(q), (np.float32(1) / q).astype(np.float32))
    for bad in (0.0, np.inf, np.nan):
        with pytest.raises(moe.MoeError):
            moe.gscale_from_quant_scale(np.array([1.0, bad], np.float32))


def _fake_bank(e, h, i, base=0x1000, fmt=L.MOE_WEIGHT_NVFP4):
    return L.Experts(num_experts=e, hidden=h, inter=i, format=fmt, w13=base, w13_scale=base + 0x10,
                     w13_gscale=base + 0x20, w2=base + 0x30, w2_scale=base + 0x40, w2_gscale=base + 0x50)


def _fake_layer(h=4096, e=320, k=8, i=1536, i_sh=1536, shared=True):
    return L.Layer(h, e, k, 0x2000, None, _fake_bank(e, h, i), _fake_bank(1, h, i_sh) if shared else L.Experts())


def test_validate_forward_host_only():
    lay = _fake_layer()
    need = moe.forward_workspace_size(8, 4096, 1536, 1536, 320, 8)
    assert moe.validate_forward(lay, 8, need) == L.MOE_OK
    assert moe.validate_forward(lay, 8, need - 1) == L.MOE_ERR_WORKSPACE_TOO_SMALL
    assert moe.validate_forward(lay, 8, need, arch="gfx942") == L.MOE_ERR_UNSUPPORTED_DEVICE
    assert moe.validate_forward(lay, 0, 0) == L.MOE_OK
    assert moe.validate_forward(lay, -1, need) == L.MOE_ERR_INVALID_ARGUMENT
    # k out of range, E too large, H/I not multiples of 128, bank/layer mismatch, null pointers
    for bad in (_fake_layer(k=0), _fake_layer(k=321), _fake_layer(k=65, e=100), _fake_layer(e=1025, k=8),
                _fake_layer(h=4000), _fake_layer(i=1500), _fake_layer(i_sh=100)):
        assert moe.validate_forward(bad, 8, 1 << 40) == L.MOE_ERR_INVALID_ARGUMENT
    lay2 = _fake_layer()
    lay2.routed.w2_scale = None
    assert moe.validate_forward(lay2, 8, 1 << 40) == L.MOE_ERR_INVALID_ARGUMENT
    lay3 = _fake_layer()
    lay3.w_router = None
    assert moe.validate_forward(lay3, 8, 1 << 40) == L.MOE_ERR_INVALID_ARGUMENT
    lay4 = _fake_layer()
    lay4.shared.hidden = 2048
    assert moe.validate_forward(lay4, 8, 1 << 40) == L.MOE_ERR_INVALID_ARGUMENT
    # device pointers the kernels read with 16-byte vectors must be 16-byte aligned
    lay6 = _fake_layer()
    lay6.routed.w13 = 0x1008
    assert moe.validate_forward(lay6, 8, 1 << 40) == L.MOE_ERR_INVALID_ARGUMENT
    lay7 = _fake_layer()
    lay7.w_router = 0x2004
    assert moe.validate_forward(lay7, 8, 1 << 40) == L.MOE_ERR_INVALID_ARGUMENT
    # activation matrices are addressed with 32-bit byte offsets: 4 GiB of x is rejected
    assert moe.validate_forward(_fake_layer(), 1 << 19, 1 << 62) == L.MOE_ERR_INVALID_ARGUMENT
    assert moe.validate_forward(_fake_layer(), (1 << 19) - 1, 1 << 62, arch="gfx950") in (L.MOE_OK,
                                                                                        L.MOE_ERR_INVALID_ARGUMENT)
    # weight formats: MXFP4 needs no global scales; unknown formats and mixed banks are rejected
    lay8 = _fake_layer()
    lay8.routed.format = lay8.shared.format = L.MOE_WEIGHT_MXFP4
    lay8.routed.w13_gscale = lay8.routed.w2_gscale = lay8.shared.w13_gscale = lay8.shared.w2_gscale = None
    assert moe.validate_forward(lay8, 8, need) == L.MOE_OK
    lay9 = _fake_layer()
    lay9.routed.w2_gscale = None
    assert moe.validate_forward(lay9, 8, 1 << 40) == L.MOE_ERR_INVALID_ARGUMENT   # NVFP4 needs them
    lay10 = _fake_layer()
    lay10.routed.format = L.MOE_WEIGHT_MXFP4
    assert moe.validate_forward(lay10, 8, 1 << 40) == L.MOE_ERR_INVALID_ARGUMENT  # shared is NVFP4
    lay11 = _fake_layer()
    lay11.routed.format = lay11.shared.format = 3
    assert moe.validate_forward(lay11, 8, 1 << 40) == L.MOE_ERR_INVALID_ARGUMENT
    # a bank in the W4A4 tile layout is not read by the W4A16 layer
    lay12 = _fake_layer()
    lay12.routed.format = lay12.shared.format = L.MOE_WEIGHT_MXFP4_A4
    assert moe.validate_forward(lay12, 8, 1 << 40) == L.MOE_ERR_INVALID_ARGUMENT
    # no shared expert is valid
    lay5 = _fake_layer(shared=False)
    assert moe.validate_forward(lay5, 8, moe.forward_workspace_size(8, 4096, 1536, 0, 320, 8)) == L.MOE_OK


def test_workspace_size_covers_intermediates():
    t, h, i, e, k = 4096, 4096, 1536, 320, 8
    s = t * k
    need = moe.forward_workspace_size(t, h, i, i, e, k)
    # h (row-major (S+T) rows, or one 128-row block per m-tile in the tiled layout) and the
    # y rows (S+T) x H bf16 dominate
    h_rows = max(s + t, (min(e, s) + s // 128 + (t + 127) // 128) * 128)
    assert need >= h_rows * i * 2 + (s + t) * h * 2 + t * e * 4
    assert need < 1.01 * (h_rows * i * 2 + (s + t) * h * 2) + (64 << 20)
    assert moe.forward_workspace_size(0, h, i, i, e, k) > 0
    assert L.lib().moe_permute_workspace_size(8, 8, 320) == 0
    assert L.lib().moe_permute_workspace_size(4096, 8, 320) >= (4096 * 8 // 2048) * 320 * 4


def test_h16_bound_validation_host_only():
    """moe_nvfp4_h16_bound refuses, before any launch, a NULL bank or output, a non-NVFP4 bank, a bank
    without its gate/up tensors, dimensions off the kernels' grid and a misaligned output; an empty
    bank is a no-op."""
    fn = L.lib().moe_nvfp4_h16_bound
    out = ctypes.c_void_p(0x3000)
    assert fn(None, out, None) == L.MOE_ERR_INVALID_ARGUMENT
    assert fn(ctypes.byref(_fake_bank(8, 512, 256)), None, None) == L.MOE_ERR_INVALID_ARGUMENT
    for fmt in (L.MOE_WEIGHT_MXFP4, L.MOE_WEIGHT_MXFP4_A4, 7):
        assert fn(ctypes.byref(_fake_bank(8, 512, 256, fmt=fmt)), out, None) == L.MOE_ERR_INVALID_ARGUMENT
    for h, i in ((500, 256), (512, 250), (0, 256), (512, 0)):
        assert fn(ctypes.byref(_fake_bank(8, h, i)), out, None) == L.MOE_ERR_INVALID_ARGUMENT, (h, i)
    for field in ("w13", "w13_scale", "w13_gscale"):
        b = _fake_bank(8, 512, 256)
        setattr(b, field, None)
        assert fn(ctypes.byref(b), out, None) == L.MOE_ERR_INVALID_ARGUMENT, field
    assert fn(ctypes.byref(_fake_bank(8, 512, 256)), ctypes.c_void_p(0x3002), None) == L.MOE_ERR_INVALID_ARGUMENT
    assert fn(ctypes.byref(_fake_bank(0, 512, 256)), out, None) == L.MOE_OK


def test_layer_struct_carries_the_fp16_h_bounds():
    """h16_norm sits at the end of moe_nvfp4_layer_t; a zero-initialised struct keeps fp16 h off."""
    lay = L.Layer()
    assert list(lay.h16_norm) == [0.0, 0.0]
    assert L.Layer.h16_norm.offset == L.Layer.shared.offset + ctypes.sizeof(L.Experts)


def test_product_path_has_no_oracle_dependency():
    """The package never imports the oracle (the oracle is test infrastructure only)."""
    pkg = os.path.join(ROOT, "nvfp4_weight_quantized_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_w4a4_validation_host_only():
    """The W4A4 layer needs MXFP4 banks (no global scales) and its own, larger workspace."""
    lay = _fake_layer()
    lay.routed.format = lay.shared.format = L.MOE_WEIGHT_MXFP4_A4
    lay.routed.w13_gscale = lay.routed.w2_gscale = lay.shared.w13_gscale = lay.shared.w2_gscale = None
    need = moe.forward_workspace_size(8, 4096, 1536, 1536, 320, 8, w4a4=True)
    assert moe.validate_forward(lay, 8, need, w4a4=True) == L.MOE_OK
    # MXFP4 banks in the W4A16 tile layout are not read by the W4A4 layer
    lay_w16 = _fake_layer()
    lay_w16.routed.format = lay_w16.shared.format = L.MOE_WEIGHT_MXFP4
    assert moe.validate_forward(lay_w16, 8, need, w4a4=True) == L.MOE_ERR_INVALID_ARGUMENT
    assert moe.validate_forward(lay, 8, need - 1, w4a4=True) == L.MOE_ERR_WORKSPACE_TOO_SMALL
    assert moe.validate_forward(lay, 8, need, arch="gfx942", w4a4=True) == L.MOE_ERR_UNSUPPORTED_DEVICE
    assert moe.validate_forward(_fake_layer(), 8, 1 << 40, w4a4=True) == L.MOE_ERR_INVALID_ARGUMENT  # NVFP4
    # the 4-bit copies of x and h, bf16 h and the y rows
    t, h, i, e, k = 4096, 4096, 1536, 320, 8
    s = t * k
    big = moe.forward_workspace_size(t, h, i, i, e, k, w4a4=True)
    floor = (s + t) * i * 2 + (s + t) * i // 2 + (s + t) * i // 32 + t * h // 2 + (s + t) * h * 2
    assert floor <= big < floor + (64 << 20)


def test_nvfp4_w4a4_validation_host_only():
    """The NVFP4 W4A4 layer takes the NVFP4 banks, a larger workspace, and refuses an activation
    scale that is zero, negative or not finite (a missing scale would zero every expert)."""
    lay = _fake_layer()
    need = moe.forward_workspace_size(8, 4096, 1536, 1536, 320, 8, nvfp4_a4=True)
    base = moe.forward_workspace_size(8, 4096, 1536, 1536, 320, 8)
    assert need >= base + 8 * 4096 * 2            # plus x's 4-bit values as bf16 rows
    good = (1.6e-3, 2.5e-4)
    assert moe.validate_forward(lay, 8, need, act_gscales=good) == L.MOE_OK
    assert moe.validate_forward(lay, 8, need - 1, act_gscales=good) == L.MOE_ERR_WORKSPACE_TOO_SMALL
    assert moe.validate_forward(lay, 8, need, arch="gfx942", act_gscales=good) == L.MOE_ERR_UNSUPPORTED_DEVICE
    for bad in (0.0, -1e-3, float("nan"), float("inf")):
        assert moe.validate_forward(lay, 8, need, act_gscales=(bad, 1.0)) == L.MOE_ERR_INVALID_ARGUMENT
        assert moe.validate_forward(lay, 8, need, act_gscales=(1.0, bad)) == L.MOE_ERR_INVALID_ARGUMENT
    # MXFP4 banks are not NVFP4 weights
    lay_mx = _fake_layer()
    lay_mx.routed.format = lay_mx.shared.format = L.MOE_WEIGHT_MXFP4
    assert moe.validate_forward(lay_mx, 8, need, act_gscales=good) == L.MOE_ERR_INVALID_ARGUMENT
    # the Python wrapper refuses a missing scale before anything reaches the library
    with pytest.raises(ValueError):
        moe.ops._act_gscale(0.0, "d_x")
