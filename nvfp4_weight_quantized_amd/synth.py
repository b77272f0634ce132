"""Seeded synthetic inputs for the NVFP4 MoE layer (shared by tests, bench and smoke).

This module only draws random numbers with the shapes and distributions of the
workloads; it holds none of the layer's arithmetic and none of the NVFP4 codec.
It produces:
  * activations x (bf16 [T, H], N(0, sigma_x));
  * router weight (bf16 [E, H], N(0, sigma_router)) and, for the skewed
    workload, a per-expert additive router bias b_e = -s * ln(r_e), the log of a
    Zipf(s) pmf over a seeded random ranking r of the experts (up to a constant);
  * full-precision expert weights (fp32 w13 [2I, H] = gate rows then up rows,
    w2 [H, I]) from N(0, sigma_w), optionally with one outlier of +-mult*sigma_w
    planted in a seeded fraction of the 16-element groups along K;
  * the checkpoint's global scale per tensor in the workload's convention:
    ModelOpt stores amax/(448*6), compressed-tensors stores (448*6)/amax
    (the two conventions of the GLM-5.3-Flash-NVFP4 discussion page).

Every stream comes from a torch.Generator seeded from (workload seed, stream
name, index), so any single expert can be regenerated on its own.  The three
H=4096, I=1536, E=320 workloads (decode, prefill, skewed) share one expert bank
(same recipe, same weight seed) and differ in activations and router.  The same
seed gives different numbers on 'cpu' and on 'cuda' (different generators):
one test or bench run always draws everything on one device.
"""

from __future__ import annotations

import math
import zlib
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                  # tokens
    H: int                  # hidden size
    I: int                  # routed expert intermediate size
    E: int                  # routed experts
    k: int                  # experts per token
    I_shared: int           # shared expert intermediate size (0: no shared expert)
    sigma_router: float
    sigma_w: float
    seed: int
    sigma_x: float = 1.0
    zipf_s: float = 0.0     # > 0: Zipf(s) router bias
    outlier_frac: float = 0.0
    outlier_mult: float = 20.0
    gscale_convention: str = "modelopt"   # or "compressed_tensors"
    weight_seed: int = -1   # >= 0: expert weights drawn from this seed instead of ``seed``

    @property
    def slots(self) -> int:
        return self.T * self.k

    @property
    def wseed(self) -> int:
        return self.weight_seed if self.weight_seed >= 0 else self.seed


WORKLOADS = {
    "tiny": Workload("tiny", T=16, H=256, I=128, E=8, k=2, I_shared=128,
                     sigma_router=0.02, sigma_w=0.02, seed=1000),
    "decode": Workload("decode", T=8, H=4096, I=1536, E=320, k=8, I_shared=1536,
                       sigma_router=0.02, sigma_w=0.02, seed=1001),
    "prefill": Workload("prefill", T=4096, H=4096, I=1536, E=320, k=8, I_shared=1536,
                        sigma_router=1.0 / 64.0, sigma_w=0.02, seed=1002, weight_seed=1001),
    "skewed": Workload("skewed", T=2048, H=4096, I=1536, E=320, k=8, I_shared=1536,
                       sigma_router=1.0 / 64.0, sigma_w=0.02, seed=1003, zipf_s=1.2, weight_seed=1001),
    "long_prefill": Workload("long_prefill", T=16384, H=6144, I=2048, E=256, k=8, I_shared=2048,
                             sigma_router=0.015, sigma_w=0.015, seed=1004,
                             outlier_frac=0.01, outlier_mult=20.0,
                             gscale_convention="compressed_tensors"),
}


def _seed(wl_seed: int, stream: str, index: int = 0) -> int:
    ss = np.random.SeedSequence([wl_seed, zlib.crc32(stream.encode()), index])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gen(device, wl_seed: int, stream: str, index: int = 0) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(_seed(wl_seed, stream, index))
    return g


def activations(wl: Workload, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    """x: bf16 [T, H] ~ N(0, sigma_x), rounded to bf16."""
    t = wl.T if T is None else T
    g = _gen(device, wl.seed, "x")
    x = torch.randn(t, wl.H, generator=g, device=device, dtype=torch.float32)
    return (x * wl.sigma_x).to(torch.bfloat16)


def router_weight(wl: Workload, device="cpu") -> torch.Tensor:
    """Router weight: bf16 [E, H] ~ N(0, sigma_router)."""
    g = _gen(device, wl.seed, "router")
    w = torch.randn(wl.E, wl.H, generator=g, device=device, dtype=torch.float32)
    return (w * wl.sigma_router).to(torch.bfloat16)


def router_bias(wl: Workload) -> Optional[np.ndarray]:
    """fp32 [E] additive router bias for a Zipf-skewed routing, or None."""
    if wl.zipf_s <= 0.0:
        return None
    rng = np.random.default_rng(_seed(wl.seed, "router_bias"))
    rank = rng.permutation(wl.E) + 1
    return np.array([-wl.zipf_s * math.log(r) for r in rank], dtype=np.float32)


def _outliers(w: torch.Tensor, wl: Workload, g: torch.Generator) -> None:
    """Plant one +-mult*sigma_w element in a random fraction of the 16-groups along K (in place)."""
    n, kdim = w.shape
    groups = w.view(n, kdim // 16, 16)
    hit = torch.rand(n, kdim // 16, generator=g, device=w.device) < wl.outlier_frac
    pos = torch.randint(0, 16, (n, kdim // 16), generator=g, device=w.device)
    sign = torch.randint(0, 2, (n, kdim // 16), generator=g, device=w.device).float() * 2 - 1
    idx = hit.nonzero(as_tuple=True)
    groups[idx[0], idx[1], pos[idx]] = sign[idx] * (wl.outlier_mult * wl.sigma_w)


def expert_fp32(wl: Workload, bank: str, e: int, device="cpu"):
    """Full-precision weights of one expert: (w13 fp32 [2I, H], w2 fp32 [H, I]).

    ``bank`` is "routed" (I = wl.I) or "shared" (I = wl.I_shared, e = 0).
    """
    inter = wl.I if bank == "routed" else wl.I_shared
    g = _gen(device, wl.wseed, "w_" + bank, e)
    w13 = torch.randn(2 * inter, wl.H, generator=g, device=device, dtype=torch.float32) * wl.sigma_w
    w2 = torch.randn(wl.H, inter, generator=g, device=device, dtype=torch.float32) * wl.sigma_w
    if wl.outlier_frac > 0.0:
        _outliers(w13, wl, g)
        _outliers(w2, wl, g)
    return w13, w2


def checkpoint_global_scales(amax: np.ndarray, convention: str) -> np.ndarray:
    """Global scale a checkpoint stores for tensors with the given amax values (fp32).

    "modelopt": the dequant scale amax/(448*6); "compressed_tensors": the quant
    scale (448*6)/amax.  One fp32 division each.
    """
    a = np.asarray(amax, dtype=np.float32)
    if convention == "modelopt":
        return (a / np.float32(2688.0)).astype(np.float32)
    if convention == "compressed_tensors":
        return (np.float32(2688.0) / a).astype(np.float32)
    raise ValueError(convention)


def expert_amax(w13: torch.Tensor, w2: torch.Tensor):
    """Per-tensor amax of one expert: gate, up and down (exact maxima), as float32 numpy."""
    inter = w13.shape[0] // 2
    vals = torch.stack([w13[:inter].abs().amax(), w13[inter:].abs().amax(), w2.abs().amax()])
    return vals.float().cpu().numpy()
