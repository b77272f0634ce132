#!/usr/bin/env python3
"""Throughput of the weight-only NVFP4 fused MoE layer on one MI355X.

A step is one pass of the whole layer (router, top-k, permute, gate/up GEMM + SiLU*up, down
GEMM, combine, shared expert) over one batch of synthetic tokens already resident in HBM.
The default workload is the decode-shaped layer (T=8, H=4096, I=1536, E=320 top-8 + 1 shared).
The K timed steps are launched eagerly, with HIP events recorded by the library at the stage
boundaries of every step (they time the dominant kernel for the roofline); the same K forwards
replayed from HIP graphs are reported beside them.
Prints one JSON line with the layer tokens/s, the roofline of the dominant kernel and the CPU
oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense fp4 MFMA (the W4A4 layer)
BYTES_PER_WEIGHT = {"nvfp4": 0.5 + 1 / 16, "mxfp4": 0.5 + 1 / 32, "mxfp4_a4": 0.5 + 1 / 32}   # nibble + scale bytes

# HBM traffic of the gate/up GEMM per launch, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this
# script (profiles/traffic_<workload>.md), scaled by what the same counters read for the 1 GiB copy
# (FETCH x 2.0, WRITE x 1.0).  Valid only for the kernel code it was measured on: reported as null
# once the code of the W4A16 GEMM sources has changed (the fingerprint ignores comments and blank
# lines).
_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "nvfp4_weight_quantized_amd", "csrc")
_GEMM_SRCS = [os.path.join(_CSRC, f) for f in ("grouped_gemm.hip", "gemm_tiles.h")]
_TRAFFIC = {  # workload: (code fingerprint of the GEMM sources, bytes read, bytes written) per gate/up launch
    "decode": ("bd630153f235c241a85ffd7e08803462ec20142040e22b8f02bf815c411519d9", 432.57e6, 0.22e6),
    "prefill": ("bd630153f235c241a85ffd7e08803462ec20142040e22b8f02bf815c411519d9", 2782.99e6, 115.81e6),
}


def code_fingerprint(paths) -> str:
    """sha256 of C++ sources without their // comments, trailing spaces and blank lines."""
    import hashlib
    import re
    lines = []
    for path in paths:
        for line in open(path, encoding="utf-8"):
            line = re.sub(r"//.*$", "", line.rstrip("\n")).rstrip()
            if line:
                lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def gate_up_traffic(workload: str):
    rec = _TRAFFIC.get(workload)
    if rec is None or code_fingerprint(_GEMM_SRCS) != rec[0]:
        return None
    return rec[1] + rec[2]


_DEFAULTS = {  # steps, warmup, weight copies cycled through (decode: defeat the 256 MB last-level cache)
    "tiny": (200, 20, 1), "decode": (200, 20, 4), "prefill": (20, 3, 1), "skewed": (20, 3, 1),
    "long_prefill": (5, 2, 1),
}


class HipEvents:
    """Raw hipEvent_t handles (the library records them on the stream it launches on)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self) -> int:
        ev = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.made.append(ev.value)
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def destroy_all(self):
        for ev in self.made:
            self.lib.hipEventDestroy(ctypes.c_void_p(ev))
        self.made = []


def clone_layer(layer, ops):
    def bank(b):
        return ops.NvFp4Experts(*(t.clone() if t is not None else None
                                  for t in (b.w13, b.w13_scale, b.w13_gscale, b.w2, b.w2_scale, b.w2_gscale)),
                                fmt=b.fmt)
    return ops.NvFp4MoELayer(layer.w_router.clone(), None if layer.router_bias is None else layer.router_bias.clone(),
                             bank(layer.routed), bank(layer.shared) if layer.shared is not None else None, layer.top_k)


def cpu_baseline(wl, x_bits, ids, n_tokens, synth, fmt="nvfp4"):
    """The oracle as it stands, single-threaded, on the first ``n_tokens`` tokens of the workload."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import moe as omoe
    from oracle import mxfp4 as omx
    from oracle import nvfp4 as onv
    from oracle import w4a4 as oa4

    def oracle_expert(bank, e):
        w13, w2 = synth.expert_fp32(wl, bank, e, "cuda")
        if fmt in ("mxfp4", "mxfp4_a4"):
            (p13, s13), (p2, s2) = omx.quantize(w13.cpu().numpy()), omx.quantize(w2.cpu().numpy())
            return omoe.ExpertWeights(p13, s13, np.ones(2, np.float32), p2, s2, 1.0, fmt="mxfp4")
        gs = synth.checkpoint_global_scales(synth.expert_amax(w13, w2), wl.gscale_convention)
        d = onv.gscale_from_quant_scale(gs) if wl.gscale_convention == "compressed_tensors" else gs
        w13, w2 = w13.cpu().numpy(), w2.cpu().numpy()
        i = w13.shape[0] // 2
        (pg, sg), (pu, su), (pd, sd) = onv.quantize(w13[:i], d[0]), onv.quantize(w13[i:], d[1]), onv.quantize(w2, d[2])
        return omoe.ExpertWeights(np.concatenate([pg, pu]), np.concatenate([sg, su]), np.array(d[:2], np.float32),
                                  pd, sd, float(d[2]))

    used = sorted({int(e) for e in np.unique(ids[:n_tokens])})
    with ThreadPoolExecutor(max_workers=8) as ex:   # input preparation, not timed
        experts = dict(zip(used, ex.map(lambda e: oracle_expert("routed", e), used)))
        shared = [oracle_expert("shared", 0)] if wl.I_shared > 0 else None

    class Bank:
        def __len__(self):
            return wl.E

        def __getitem__(self, e):
            return experts[e]

    layer = omoe.Layer(w_router=x_bits["router"], router_bias=synth.router_bias(wl), routed=Bank(), shared=shared,
                       top_k=wl.k)
    forward = oa4.forward if fmt == "mxfp4_a4" else omoe.forward
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        forward(x_bits["x"][:n_tokens], layer)
        dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n_tokens} of {wl.T} tokens of the {wl.name} workload ({len(used)} routed experts + "
                      f"shared): float64 numpy oracle forward, one thread, {dt:.1f} s; weight quantization "
                      f"untimed"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode", choices=sorted(_DEFAULTS))
    ap.add_argument("--copies", type=int, default=None, help="weight copies cycled through")
    ap.add_argument("--cpu-tokens", type=int, default=5,
                    help="tokens in the CPU oracle sample, about 3 s of CPU each (0: skip)")
    ap.add_argument("--format", default="nvfp4", choices=["nvfp4", "mxfp4", "mxfp4_a4"],
                    help="weight format of the synthetic experts (the headline metric is NVFP4); mxfp4_a4: "
                         "the W4A4 layer (MXFP4 weights and activations on the FP4 matrix cores)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the layer on one GPU only: each layer runs whole on one MI355X "
              "(no expert or tensor sharding, no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    from nvfp4_weight_quantized_amd import _lib, build_layer, ops, synth

    _lib.lib()  # fail loudly now if the HIP library is missing
    wl = synth.WORKLOADS[args.workload]
    steps, warmup, copies = _DEFAULTS[args.workload]
    steps = args.steps if args.steps is not None else steps
    warmup = args.warmup if args.warmup is not None else warmup
    copies = args.copies if args.copies is not None else copies
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    print(f"[bench] building {wl.name} layer ({copies} weight copies, {args.format})", file=sys.stderr, flush=True)
    layer = build_layer(wl, dev, fmt=args.format)
    bytes_per_weight = BYTES_PER_WEIGHT[args.format]
    layers = [layer] + [clone_layer(layer, ops) for _ in range(copies - 1)]
    x = synth.activations(wl, dev)
    ws = ops.workspace_for(layer, wl.T, dev)
    out = torch.empty_like(x)
    _, aux = ops.forward(layer, x, ws, out, return_aux=True)
    counts = aux["expert_counts"].cpu().numpy()
    ids = aux["topk_ids"].cpu().numpy()
    touched = int((counts > 0).sum())

    # plain device-to-device copy of 1 GiB: the HBM bandwidth a streaming kernel reaches on this
    # box, and the known-size kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * src.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    # dense bf16 GEMM of the gate/up shape through the vendor library (torch.mm -> hipBLASLt): the
    # practical MFMA ceiling of this machine for that shape (context only; not part of the layer)
    dense_tflops = None
    w4a4 = args.format == "mxfp4_a4"
    if wl.name not in ("tiny", "decode") and not w4a4:
        m_rows, n_cols = wl.T * wl.k + wl.T, 2 * wl.I
        a_ = torch.randn(m_rows, wl.H, device=dev, dtype=torch.bfloat16)
        b_ = torch.randn(n_cols, wl.H, device=dev, dtype=torch.bfloat16)
        c_ = a_ @ b_.t()
        c0.record()
        for _ in range(3):
            c_ = a_ @ b_.t()
        c1.record()
        torch.cuda.synchronize()
        dense_tflops = 3 * 2.0 * m_rows * n_cols * wl.H / (c0.elapsed_time(c1) * 1e-3) / 1e12
        del a_, b_, c_
        torch.cuda.empty_cache()

    for i in range(warmup):
        ops.forward(layers[i % copies], x, ws, out)
    torch.cuda.synchronize()

    hip = HipEvents()
    evs = [[hip.create() for _ in range(3)] for _ in range(steps)]   # after S3, after S4, after S5
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    print(f"[bench] timing {steps} steps", file=sys.stderr, flush=True)
    start.record()
    for i in range(steps):
        e = evs[i]
        ops.forward(layers[i % copies], x, ws, out, stage_events=[None, None, e[0], e[1], e[2], None])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    gate_up_ms = float(np.mean([hip.elapsed_ms(e[0], e[1]) for e in evs]))
    down_ms = float(np.mean([hip.elapsed_ms(e[1], e[2]) for e in evs]))
    # the same forwards replayed from HIP graphs (one captured forward per weight copy): how a
    # serving loop runs the layer, without per-kernel launch overhead
    graph_ms = None
    try:
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for lay in layers:
                ops.forward(lay, x, ws, out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for lay in layers:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                ops.forward(lay, x, ws, out)
            graphs.append(g)
        for i in range(warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for i in range(steps):
            graphs[i % copies].replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / steps
        del graphs
    except RuntimeError as exc:  # capture unsupported: report the eager timing only
        print(f"[bench] graph replay unavailable: {exc}", file=sys.stderr, flush=True)
    # per-stage breakdown, outside the timed region: all six stage boundaries
    bevs = [[hip.create() for _ in range(6)] for _ in range(min(steps, 50))]
    torch.cuda.synchronize()
    for i, e in enumerate(bevs):
        ops.forward(layers[i % copies], x, ws, out, stage_events=e)
    torch.cuda.synchronize()
    names = ["router", "topk_permute", "gate_up", "down", "combine"]
    stages_us = {n: float(np.mean([hip.elapsed_ms(e[i], e[i + 1]) for e in bevs])) * 1e3 for i, n in enumerate(names)}
    hip.destroy_all()

    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    S = T * k
    ms_per_step = total_ms / steps
    value = T * steps / (total_ms / 1e3)
    # roofline of the gate/up GEMM, the dominant kernel (2/3 of the weight bytes and flops)
    n_banks = touched + (1 if wl.I_shared > 0 else 0)
    gu_weight_bytes = n_banks * 2 * I * H * bytes_per_weight
    # activations in: bf16 x (W4A16); for W4A4 the x read by its quantizer plus the 4-bit copy
    x_bytes = T * H * 2 + (T * H * bytes_per_weight * 2 if w4a4 else 0)
    gu_bytes = gu_weight_bytes + x_bytes + (S + T) * I * 2
    gu_flops = 2.0 * (S + T) * H * 2 * I
    mfma_peak = FP4_PEAK_TFLOPS if w4a4 else BF16_PEAK_TFLOPS
    if w4a4:   # bound by the algorithmic intensity against the fp4 ridge point
        hbm_bound = gu_bytes / (HBM_PEAK_GBS * 1e9) >= gu_flops / (mfma_peak * 1e12)
    else:
        hbm_bound = wl.name in ("tiny", "decode")
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": gu_bytes / (gate_up_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": gu_flops / (gate_up_ms * 1e-3) / 1e12, "peak": mfma_peak,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # the same against what this box measurably reaches: a streaming copy (HBM-bound case) or the
    # vendor library's dense bf16 GEMM of the same shape (MFMA-bound case)
    roof["peak_measured"] = copy_gbs if roof["bound"] == "hbm" else dense_tflops
    roof["peak_measured_source"] = ("1 GiB device-to-device copy (read + write)" if roof["bound"] == "hbm"
                                    else "dense bf16 GEMM of the gate/up shape via torch.mm (hipBLASLt)")
    roof["frac_of_measured"] = (roof["achieved"] / roof["peak_measured"]) if roof["peak_measured"] else None
    roof["traffic"] = gate_up_traffic(wl.name) if args.format == "nvfp4" else None
    roof["traffic_unit"] = "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)"
    roof["algorithmic_bytes"] = gu_bytes
    roof["kernel"] = ("gate/up stage (S4): x to MXFP4 + W4A4 grouped GEMM" if w4a4
                      else "gate/up grouped GEMM (S4)")
    roof["kernel_us"] = gate_up_ms * 1e3

    # whole layer: flops 2(S+T)*3HI + 2THE (MFMA-bound shapes) or the bytes of every touched
    # expert, the shared expert, the router weight and the activations (HBM-bound shapes)
    if roof["bound"] == "hbm":
        layer_bytes = ((touched * 3 * I + 3 * wl.I_shared) * H * bytes_per_weight + 2 * E * H + 4 * T * H)
        layer_roof = {"bound": "hbm", "achieved": layer_bytes / (ms_per_step * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                      "unit": "GB/s", "algorithmic_bytes": layer_bytes}
    else:
        layer_flops = 2.0 * S * 3 * H * I + 2.0 * T * 3 * H * wl.I_shared + 2.0 * T * H * E
        layer_roof = {"bound": "mfma", "achieved": layer_flops / (ms_per_step * 1e-3) / 1e12,
                      "peak": mfma_peak, "unit": "TFLOP/s", "algorithmic_flops": layer_flops}
    layer_roof["frac"] = layer_roof["achieved"] / layer_roof["peak"]

    cpu = None
    if args.cpu_tokens > 0:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)

        def bits(t):
            return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

        cpu = cpu_baseline(wl, {"x": bits(x), "router": bits(layer.w_router)}, ids, args.cpu_tokens, synth,
                           args.format)
    line = {
        "metric": "NVFP4 MoE layer tokens/s; decode HBM GB/s %peak, prefill MFMA %peak"
                  + {"nvfp4": "", "mxfp4": " (measured here on MXFP4 weights)",
                     "mxfp4_a4": " (measured here on the MXFP4 W4A4 layer)"}[args.format],
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4" if w4a4 else "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: T={T} H={H} I={I} E={E} top-{k} + 1 shared (I={wl.I_shared}), "
                               + ("MXFP4 W4A4" if w4a4 else f"{args.format.upper()} W4A16"),
                   "tokens": T, "hidden": H, "inter": I, "experts": E, "top_k": k,
                   "weight_copies": copies, "experts_touched": touched},
        "roofline": roof,
        "layer_roofline": layer_roof,
        "graph_replay_ms_per_step": graph_ms,
        "stages_us": stages_us,
        "measured_copy_GBs": copy_gbs,
        "timed_stages_us": {"gate_up": gate_up_ms * 1e3, "down": down_ms * 1e3},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
