"""Test-side glue: build oracle-side layers from the seeded generator (never used by the product path)."""

from __future__ import annotations

import numpy as np
import torch

from nvfp4_weight_quantized_amd import synth
from oracle import moe as omoe
from oracle import mxfp4 as omx
from oracle import nvfp4 as onv


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns (numpy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def dequant_scale_from_checkpoint(gs: np.ndarray, convention: str) -> np.ndarray:
    """Oracle-side loader: checkpoint global scale -> dequant scale."""
    gs = np.asarray(gs, np.float32)
    if convention == "modelopt":
        return gs
    return onv.gscale_from_quant_scale(gs)


def oracle_dequant_scales(w13: np.ndarray, w2: np.ndarray, convention: str) -> np.ndarray:
    """The oracle's own dequant global scales (gate, up, down) of one fp32 expert: amax of each
    tensor, the checkpoint scale of the convention (oracle.nvfp4), inverted on load for
    compressed-tensors."""
    inter = w13.shape[0] // 2
    amax = [np.abs(a).max() for a in (w13[:inter], w13[inter:], w2)]
    if convention == "modelopt":
        return np.array([onv.gscale_modelopt(a) for a in amax], np.float32)
    q = np.array([onv.gscale_compressed_tensors(a) for a in amax], np.float32)
    return onv.gscale_from_quant_scale(q)


def oracle_expert_mx(wl, bank: str, e: int, device="cpu") -> omoe.ExpertWeights:
    """Quantize one synthetic expert to MXFP4 with the oracle quantizer."""
    w13, w2 = synth.expert_fp32(wl, bank, e, device)
    p13, s13 = omx.quantize(w13.cpu().numpy())
    p2, s2 = omx.quantize(w2.cpu().numpy())
    return omoe.ExpertWeights(p13, s13, np.ones(2, np.float32), p2, s2, 1.0, fmt="mxfp4")


def oracle_expert(wl, bank: str, e: int, device="cpu", fmt: str = "nvfp4") -> omoe.ExpertWeights:
    """Quantize one synthetic expert with the oracle quantizer."""
    if fmt == "mxfp4":
        return oracle_expert_mx(wl, bank, e, device)
    w13, w2 = synth.expert_fp32(wl, bank, e, device)
    w13 = w13.cpu().numpy()
    w2 = w2.cpu().numpy()
    d = oracle_dequant_scales(w13, w2, wl.gscale_convention)
    inter = w13.shape[0] // 2
    pg, sg = onv.quantize(w13[:inter], d[0])
    pu, su = onv.quantize(w13[inter:], d[1])
    pd, sd = onv.quantize(w2, d[2])
    return omoe.ExpertWeights(np.concatenate([pg, pu]), np.concatenate([sg, su]),
                              np.array([d[0], d[1]], np.float32), pd, sd, float(d[2]))


_EXPERT_CACHE = {}


class LazyBank:
    """Sequence of oracle experts quantized on first access (for layers too big to hold).

    Experts are cached per (weight seed, bank, index, device) across tests, since several
    workloads share one bank.  ``prefetch`` quantizes a set of experts on a thread pool.
    """

    def __init__(self, wl, bank: str, count: int, device="cpu", fmt: str = "nvfp4"):
        self.wl, self.bank, self.count, self.device, self.fmt = wl, bank, count, device, fmt

    def _key(self, e):
        return (self.wl.wseed, self.wl.H, self.wl.I, self.bank, int(e), str(self.device), self.fmt)

    def __len__(self):
        return self.count

    def __getitem__(self, e):
        key = self._key(e)
        if key not in _EXPERT_CACHE:
            _EXPERT_CACHE[key] = oracle_expert(self.wl, self.bank, int(e), self.device, self.fmt)
        return _EXPERT_CACHE[key]

    def prefetch(self, experts, threads=8):
        from concurrent.futures import ThreadPoolExecutor
        todo = sorted({int(e) for e in experts if self._key(e) not in _EXPERT_CACHE})
        with ThreadPoolExecutor(max_workers=threads) as ex:
            for e, ew in zip(todo, ex.map(lambda i: oracle_expert(self.wl, self.bank, i, self.device, self.fmt),
                                          todo)):
                _EXPERT_CACHE[self._key(e)] = ew


def oracle_layer(wl, device="cpu", fmt: str = "nvfp4") -> omoe.Layer:
    routed = LazyBank(wl, "routed", wl.E, device, fmt)
    shared = LazyBank(wl, "shared", 1, device, fmt) if wl.I_shared > 0 else None
    return omoe.Layer(w_router=bf16_bits(synth.router_weight(wl, device)),
                      router_bias=synth.router_bias(wl), routed=routed, shared=shared, top_k=wl.k)


def stack_bank(bank) -> omoe.ArrayBank:
    items = [bank[e] for e in range(len(bank))]
    return omoe.ArrayBank(np.stack([i.w13 for i in items]), np.stack([i.w13_scale for i in items]),
                          np.stack([i.w13_gscale for i in items]), np.stack([i.w2 for i in items]),
                          np.stack([i.w2_scale for i in items]),
                          np.array([i.w2_gscale for i in items], np.float32))


def random_layer(rng, H, I, E, k, shared=True, sigma=0.05, bias=False, i_shared=None, fmt="nvfp4") -> omoe.Layer:
    """A small random layer quantized by the oracle (for brute-force comparisons)."""
    def one(i_dim):
        w13 = rng.normal(0, sigma, (2 * i_dim, H)).astype(np.float32)
        w2 = rng.normal(0, sigma, (H, i_dim)).astype(np.float32)
        if fmt == "mxfp4":
            p13, s13 = omx.quantize(w13)
            p2, s2 = omx.quantize(w2)
            return omoe.ExpertWeights(p13, s13, np.ones(2, np.float32), p2, s2, 1.0, fmt="mxfp4")
        d = [onv.gscale_modelopt(np.abs(a).max()) for a in (w13[:i_dim], w13[i_dim:], w2)]
        pg, sg = onv.quantize(w13[:i_dim], d[0])
        pu, su = onv.quantize(w13[i_dim:], d[1])
        pd, sd = onv.quantize(w2, d[2])
        return omoe.ExpertWeights(np.concatenate([pg, pu]), np.concatenate([sg, su]),
                                  np.array(d[:2], np.float32), pd, sd, float(d[2]))
    wr = torch.from_numpy(rng.normal(0, 0.3, (E, H)).astype(np.float32)).to(torch.bfloat16)
    b = rng.normal(0, 0.5, E).astype(np.float32) if bias else None
    return omoe.Layer(w_router=bf16_bits(wr), router_bias=b, routed=[one(I) for _ in range(E)],
                      shared=[one(i_shared or I)] if shared else None, top_k=k)


def random_x(rng, T, H) -> np.ndarray:
    return bf16_bits(torch.from_numpy(rng.normal(0, 1, (T, H)).astype(np.float32)).to(torch.bfloat16))
