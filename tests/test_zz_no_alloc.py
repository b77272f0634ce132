"""moe_nvfp4_forward_noalloc (the allocation-free whole layer) through the C ABI: the same output as
moe_nvfp4_forward on two calls in a row, the second with fewer tokens, and a loud refusal of a size
beyond its device array."""

import ctypes

import numpy as np
import pytest
import torch

import helpers
import parity
from nvfp4_weight_quantized_amd import _lib as L
from nvfp4_weight_quantized_amd import ops

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _noalloc(glayer, x):
    out = torch.full_like(x, float("nan"))
    st = glayer.checked_struct()
    status = L.lib().moe_nvfp4_forward_noalloc(ctypes.byref(st), ctypes.c_void_p(x.data_ptr()), x.shape[0],
                                               ctypes.c_void_p(out.data_ptr()), None,
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    L.check("moe_nvfp4_forward_noalloc", status)
    return out


@pytest.mark.parametrize("case", [
    # T (first call), T (second call), H, I, E, k: 128-row tiles with the tiled h and the multi-block
    # permutation first, then 16-row tiles and the one-workgroup top-k + permutation
    (600, 40, 512, 256, 16, 4),
    # 8-row (skinny) tiles, then fewer tokens still
    (24, 3, 256, 128, 64, 2),
])
def test_noalloc_forward_equals_forward_on_two_calls(case):
    t1, t2, H, I, E, k = case
    rng = np.random.default_rng(sum(case))
    layer = helpers.random_layer(rng, H, I, E, k, shared=True, bias=True)
    glayer = parity.to_gpu_layer(layer)
    x = parity.bits_to_bf16(helpers.random_x(rng, t1, H))
    for T in (t1, t2):
        xs = x[:T].contiguous()
        ref = ops.forward(glayer, xs)
        got = _noalloc(glayer, xs)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"T={T}: allocation-free forward differs from moe_nvfp4_forward"
        got2 = ops.forward_noalloc(glayer, xs)
        torch.cuda.synchronize()
        assert torch.equal(got2, ref), f"T={T}: second allocation-free call differs"
    # and against the oracle at the second size
    ids = ops.forward(glayer, x[:t2].contiguous(), return_aux=True)[1]["topk_ids"].cpu().numpy()
    res = parity.reference_for_selection(helpers.bf16_bits(x[:t2]), layer, ids)
    parity.assert_close(parity.f64(got2), res["out"], "allocation-free forward")


def test_noalloc_refuses_a_workspace_beyond_its_array():
    rng = np.random.default_rng(3)
    layer = helpers.random_layer(rng, 256, 128, 8, 2)
    glayer = parity.to_gpu_layer(layer)
    # workspace grows ~linearly in T; find a T whose workspace exceeds the array
    T = 1
    while ops.forward_workspace_size(T, 256, 128, 128, 8, 2) <= L.NOALLOC_SCRATCH_BYTES:
        T *= 2
    x = torch.zeros(T, 256, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(L.MoeError) as err:
        ops.forward_noalloc(glayer, x)
    assert err.value.status == L.MOE_ERR_WORKSPACE_TOO_SMALL
    # zero tokens is a no-op
    ops.forward_noalloc(glayer, torch.zeros(0, 256, dtype=torch.bfloat16, device=DEV))
