#!/usr/bin/env python3
"""Throughput of the weight-only NVFP4 fused MoE layer on one MI355X.

A step is one pass of the whole layer (router, top-k, permute, gate/up GEMM + SiLU*up, down
GEMM, combine, shared expert) over one batch of synthetic tokens already resident in HBM.

The JSON line's top level is the decode-shaped layer (T=8, H=4096, I=1536, E=320 top-8 + 1 shared),
the configuration the metric's HBM half is quoted on; `configs` holds, in the same line, the
prefill-shaped layers the metric's MFMA half is quoted on (prefill T=4096, skewed routing T=2048,
long prefill T=16384 with H=6144, I=2048, E=256), each timed the same way.  For every layer:
  * forwards of the layer for 150 ms (the clock settles under load), then the W warm-up forwards;
  * K forwards launched eagerly, timed between two synchronisations with nothing else in between
    (the value and ms_per_step); then the same K forwards with one HIP event per step (the step
    periods: median, p10, p90), and again with events at the stage boundaries, which the library
    records on its launch stream (the gate/up and down GEMM intervals of the roofline); the
    per-stage breakdown comes from a run with all six events;
  * the roofline of the gate/up GEMM (the dominant kernel: 2/3 of weight bytes and flops) and of
    the whole layer, against the MI355X data-sheet peaks and against what this box measurably
    reaches (a streaming-read kernel of the library for HBM, the vendor dense bf16 GEMM of the same
    shape for MFMA);
  * the same K forwards replayed from HIP graphs;
  * the CPU oracle on the machine's host cores: routing of every token, a sample of routed experts on
    their rows, the shared expert and the combine on a token block, each 1 warm-up + 3 runs
    (median), scaled to the whole job.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense fp4 MFMA (the W4A4 layer)
BYTES_PER_WEIGHT = {"nvfp4": 0.5 + 1 / 16, "mxfp4": 0.5 + 1 / 32, "mxfp4_a4": 0.5 + 1 / 32,
                    "nvfp4_a4": 0.5 + 1 / 16}   # nibble + scale bytes

# HBM traffic of the gate/up GEMM per launch, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this
# script (profiles/traffic_<workload>.md), scaled by what the same counters read for a copy of known
# size (FETCH x 2.0, WRITE x 1.0).  Valid only for the kernel code it was measured on: reported as
# null once the code of the W4A16 GEMM sources has changed (the fingerprint ignores comments and
# blank lines).
_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "nvfp4_weight_quantized_amd", "csrc")
_GEMM_SRCS = [os.path.join(_CSRC, f) for f in ("grouped_gemm.hip", "gemm_tiles.h", "gemm_skinny.h")]
_TRAFFIC = {  # workload: (code fingerprint of the GEMM sources, bytes read, bytes written) per gate/up launch
    "decode": ("43f04cc0f3ee4e7e43eabb7761f144b6ccad315e393e345b5e2e5fca5504bfc9", 432.49e6, 0.22e6),
    "prefill": ("43f04cc0f3ee4e7e43eabb7761f144b6ccad315e393e345b5e2e5fca5504bfc9", 2869.87e6, 113.99e6),
}

PREFILL_CONFIGS = ["prefill", "skewed", "long_prefill"]
# steps, warmup, weight copies cycled through (decode: defeat the 256 MB last-level cache)
_DEFAULTS = {
    "tiny": (200, 50, 1), "decode": (200, 50, 4), "prefill": (20, 5, 1), "skewed": (20, 5, 1),
    "long_prefill": (5, 2, 1),
}
# Before the counted warm-up steps, forwards of the same workload run until this much wall time has
# passed: the first tens of milliseconds of full load run at a lower clock (measured: the first 20
# prefill forwards of a process 6% slower than later ones), whatever the warm-up count.
SETTLE_S = 0.15


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


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


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


def percentiles(v):
    a = np.asarray(v, np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "mean": float(a.mean())}


# ----------------------------------------------------------------------------- measured ceilings

def hbm_read_ceiling(lib, dev) -> float:
    """GB/s of the library's streaming-read kernel over 2 GiB (best of several workgroup counts)."""
    n = 2 << 30
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    best = 0.0
    for wgs in (2048, 4096, 8192):
        for _ in range(2):
            lib.moe_hbm_read_probe(ctypes.c_void_p(buf.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()), wgs, stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            st = lib.moe_hbm_read_probe(ctypes.c_void_p(buf.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()), wgs,
                                        stream)
            if st != 0:
                raise RuntimeError(f"moe_hbm_read_probe failed: {st}")
        b.record()
        torch.cuda.synchronize()
        best = max(best, 5 * n / (a.elapsed_time(b) * 1e-3) / 1e9)
    del buf
    return best


def dense_bf16_tflops(wl, dev) -> float:
    """Vendor dense bf16 GEMM (torch.mm -> hipBLASLt) of the gate/up shape: the practical MFMA ceiling
    of this box for that shape (context only; not part of the layer)."""
    m_rows, n_cols = wl.T * wl.k + wl.T, 2 * wl.I
    a_ = torch.randn(m_rows, wl.H, device=dev, dtype=torch.bfloat16)
    b_ = torch.randn(n_cols, wl.H, device=dev, dtype=torch.bfloat16)
    c_ = a_ @ b_.t()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(3):
        c_ = a_ @ b_.t()
    c1.record()
    torch.cuda.synchronize()
    out = 3 * 2.0 * m_rows * n_cols * wl.H / (c0.elapsed_time(c1) * 1e-3) / 1e12
    del a_, b_, c_
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- CPU oracle baseline

def host_info() -> dict:
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        blas = f"{b.get('name')} {b.get('version')}"
    except Exception:  # older numpy: no dict mode
        pass
    return {"nproc": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": model,
            "numpy": np.__version__, "blas": blas}


def cpu_baseline(wl, x_bits, wr_bits, synth, fmt="nvfp4", n_experts=4, token_block=1024, runs=3, act_gscales=None):
    """The oracle as it stands, on the host's cores, on a bounded sample of the whole job, scaled to it.

    Parts, each timed with 1 warm-up + ``runs`` runs (median): routing of every token (router GEMM,
    top-k, permutation); ``n_experts`` routed experts spread over the load distribution, each on all
    of its rows (dequantization + gate/up + SiLU*up + down); the shared expert and the combine on the
    first ``token_block`` tokens.  Job time = routing + routed * (experts used / sampled) +
    (shared + combine) * T / token_block.  Weight quantization is input preparation, not timed."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import moe as omoe
    from oracle import mxfp4 as omx
    from oracle import nvfp4 as onv
    from oracle import nvfp4_w4a4 as onw
    from oracle import w4a4 as oa4

    def oracle_expert(bank, e):
        w13, w2 = synth.expert_fp32(wl, bank, e, "cuda")
        w13, w2 = w13.cpu().numpy(), w2.cpu().numpy()
        if fmt in ("mxfp4", "mxfp4_a4"):
            (p13, s13), (p2, s2) = omx.quantize(w13), omx.quantize(w2)
            return omoe.ExpertWeights(p13, s13, np.ones(2, np.float32), p2, s2, 1.0, fmt="mxfp4")
        i = w13.shape[0] // 2
        amax = [np.abs(a).max() for a in (w13[:i], w13[i:], w2)]
        if wl.gscale_convention == "compressed_tensors":
            d = onv.gscale_from_quant_scale(np.array([onv.gscale_compressed_tensors(a) for a in amax], np.float32))
        else:
            d = np.array([onv.gscale_modelopt(a) for a in amax], np.float32)
        (pg, sg), (pu, su), (pd, sd) = onv.quantize(w13[:i], d[0]), onv.quantize(w13[i:], d[1]), onv.quantize(w2, d[2])
        return omoe.ExpertWeights(np.concatenate([pg, pu]), np.concatenate([sg, su]), np.array(d[:2], np.float32),
                                  pd, sd, float(d[2]))

    T, k, E = wl.T, wl.k, wl.E
    bias = synth.router_bias(wl)
    w4a4 = fmt == "mxfp4_a4"
    ffn = oa4.expert_ffn_a4 if w4a4 else omoe.expert_ffn
    if fmt == "nvfp4_a4":
        def ffn(a, ew):
            return onw.expert_ffn_a4(a, ew, act_gscales[0], act_gscales[1])
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        logits = omoe.router_logits(x_bits, wr_bits, bias)
        ids, w = omoe.topk(logits, k)
        counts, offsets, sorted_slot, slot_to_row = omoe.permute(ids, E)
        used = np.nonzero(counts)[0]
        by_load = used[np.argsort(counts[used], kind="stable")]
        pick = by_load[np.unique(np.linspace(0, len(by_load) - 1, min(n_experts, len(by_load))).round().astype(int))]
        with ThreadPoolExecutor(max_workers=min(8, cores)) as ex:   # input preparation, not timed
            experts = dict(zip(pick.tolist(), ex.map(lambda e: oracle_expert("routed", int(e)), pick.tolist())))
            shared = oracle_expert("shared", 0) if wl.I_shared > 0 else None
        x = omoe.bf16_to_float(x_bits)
        tb = min(T, token_block)
        y_block = np.zeros((tb * k, wl.H))
        rows_of = {int(e): sorted_slot[offsets[e]:offsets[e + 1]] // k for e in pick}

        def routing():
            lg = omoe.router_logits(x_bits, wr_bits, bias)
            i_, _ = omoe.topk(lg, k)
            omoe.permute(i_, E)

        def routed():
            for e, ew in experts.items():
                ffn(x[rows_of[e]], ew)

        def shared_part():
            if shared is not None:
                ffn(x[:tb], shared)

        def combine_part():
            omoe.combine(y_block, np.arange(tb * k), w[:tb])

        parts = {}
        for name, fn in (("routing", routing), ("routed_sample", routed), ("shared_block", shared_part),
                         ("combine_block", combine_part)):
            fn()
            ts = []
            for _ in range(runs):
                t0 = time.perf_counter()
                fn()
                ts.append(time.perf_counter() - t0)
            parts[name] = float(np.median(ts))
    job = (parts["routing"] + parts["routed_sample"] * len(used) / len(pick)
           + (parts["shared_block"] + parts["combine_block"]) * T / tb)
    return {"value": T / job, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"{wl.name} workload: routing of all {T} tokens; {len(pick)} of the {len(used)} routed experts "
                       f"in use (spread over the load distribution, {int(counts[pick].sum())} rows) scaled by "
                       f"{len(used)}/{len(pick)}; shared expert and combine on {tb} tokens scaled by {T}/{tb}; "
                       f"float64 numpy oracle, BLAS threads = {threads}; each part 1 warm-up + {runs} runs, median; "
                       f"weight quantization untimed"),
            "job_s": job, "parts_s": parts, **host_info()}


# ----------------------------------------------------------------------------- one workload

def calibrate_nvfp4_a4(wl, layer, x, ops_mod, dev):
    """Static activation scales of the NVFP4 W4A4 layer, as a caller calibrates them once: d_x =
    amax(x) / (448 * 6) over the batch, d_h the same over the W4A4 gate/up output of the shared
    expert (or of routed expert 0) on every token.  Not timed."""
    from nvfp4_weight_quantized_amd import _lib as L
    d_x = float(np.float32(float(x.abs().max()) / 2688.0))
    _, _, xa = ops_mod.quantize_act_nv(x, d_x, packed=False, scales=False)
    bank = layer.shared if layer.shared is not None else layer.routed
    offs = torch.zeros(bank.num_experts + 1, dtype=torch.int32, device=dev)
    offs[1:] = wl.T
    h = ops_mod.grouped_gemm_w4a4(L.MOE_GEMM_GATE_UP, bank, xa, d_x, offs, wl.T)
    d_h = float(np.float32(max(float(h.abs().max()), 1e-30) / 2688.0))
    log(f"{wl.name}: NVFP4 W4A4 activation scales d_x={d_x:.4g} d_h={d_h:.4g}")
    return (d_x, d_h)


def measure(wl, layers, steps, warmup, fmt, ops_mod, lib, dev, copy_gbs, cpu: bool, fused_decode: bool = False):
    """Time one workload; returns its record (the fields of a bench line)."""
    import functools
    import types
    w4a4 = fmt == "mxfp4_a4"
    layer = layers[0]
    copies = len(layers)
    x = synth_mod.activations(wl, dev)
    a4 = calibrate_nvfp4_a4(wl, layer, x, ops_mod, dev) if fmt == "nvfp4_a4" else None
    ops = types.SimpleNamespace(forward=functools.partial(ops_mod.forward, fused_decode=fused_decode,
                                                          act_gscales=a4),
                                workspace_for=ops_mod.workspace_for)
    ws = ops.workspace_for(layer, wl.T, dev, nvfp4_a4=a4 is not None)
    out = torch.empty_like(x)
    _, aux = ops.forward(layer, x, ws, out, return_aux=True)
    counts = aux["expert_counts"].cpu().numpy()
    touched = int((counts > 0).sum())
    settle, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(8):
            ops.forward(layers[settle % copies], x, ws, out)
            settle += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        ops.forward(layers[i % copies], x, ws, out)
    torch.cuda.synchronize()

    hip = HipEvents()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    # (1) the K timed steps, nothing but the forwards between the two synchronisations
    torch.cuda.synchronize()
    log(f"{wl.name}: timing {steps} steps")
    start.record()
    for i in range(steps):
        ops.forward(layers[i % copies], x, ws, out)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    # (2) the same K steps with one event per step (before S1): the step periods, for the spread
    pev = [hip.create() for _ in range(steps + 1)]
    torch.cuda.synchronize()
    for i in range(steps):
        ops.forward(layers[i % copies], x, ws, out, stage_events=[pev[i], None, None, None, None, None])
    ops.forward(layers[steps % copies], x, ws, out, stage_events=[pev[steps], None, None, None, None, None])
    torch.cuda.synchronize()
    step_ms = [hip.elapsed_ms(pev[i], pev[i + 1]) for i in range(steps)]
    # (3) the same K steps with events at the stage boundaries after S1, S3, S4 and S5 (HIP events on
    # the launch stream): the gate/up and down intervals (staged launches) or the fused S2-S6 launch
    evs = [[hip.create() for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        e = evs[i]
        ops.forward(layers[i % copies], x, ws, out, stage_events=[None, e[0], e[1], e[2], e[3], None])
    torch.cuda.synchronize()
    gate_up = [hip.elapsed_ms(e[1], e[2]) for e in evs]
    down = [hip.elapsed_ms(e[2], e[3]) for e in evs]
    fused_k = [hip.elapsed_ms(e[0], e[3]) for e in evs]
    # the library runs the fused launch on request for few tokens (NVFP4, T <= 32, T*k <= 256, E <= 320)
    fused = (fused_decode and fmt == "nvfp4" and wl.T <= 32 and wl.T * wl.k <= 256 and wl.E <= 320
             and wl.I_shared in (0, wl.I))
    kernel = fused_k if fused else gate_up
    kernel_ms = float(np.mean(kernel))
    # per-stage breakdown, outside the timed region: all six stage boundaries
    bevs = [[hip.create() for _ in range(6)] for _ in range(min(steps, 50))]
    torch.cuda.synchronize()
    for i, e in enumerate(bevs):
        ops.forward(layers[i % copies], x, ws, out, stage_events=e)
    torch.cuda.synchronize()
    names = (["router", "fused_topk_permute_gemms_combine", None, None, None] if fused
             else ["router", "topk_permute", "gate_up", "down", "combine"])
    stages_us = {n: float(np.mean([hip.elapsed_ms(e[i], e[i + 1]) for e in bevs])) * 1e3
                 for i, n in enumerate(names) if n}
    hip.destroy_all()

    # the same forwards replayed from HIP graphs (one captured forward per weight copy)
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
        log(f"graph replay unavailable: {exc}")

    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    S = T * k
    ms_per_step = total_ms / steps
    bpw = BYTES_PER_WEIGHT[fmt]
    n_banks = touched + (1 if wl.I_shared > 0 else 0)
    # activations in: bf16 x (W4A16); for W4A4 the x read by its quantizer plus the 4-bit copy
    x_bytes = T * H * 2 + (T * H * bpw * 2 if w4a4 else 0)
    if fused:   # the fused S2-S6 launch: every expert weight, x in and the output out
        gu_bytes = n_banks * 3 * I * H * bpw + 2 * T * H * 2
        gu_flops = 2.0 * (S + T) * 3 * H * I
    else:
        gu_bytes = n_banks * 2 * I * H * bpw + x_bytes + (S + T) * I * 2
        gu_flops = 2.0 * (S + T) * H * 2 * I
    mfma_peak = FP4_PEAK_TFLOPS if w4a4 else BF16_PEAK_TFLOPS
    if w4a4:   # bound by the algorithmic intensity against the fp4 ridge point
        hbm_bound = gu_bytes / (HBM_PEAK_GBS * 1e9) >= gu_flops / (mfma_peak * 1e12)
    else:
        hbm_bound = wl.name in ("tiny", "decode")
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": gu_bytes / (kernel_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": gu_flops / (kernel_ms * 1e-3) / 1e12, "peak": mfma_peak,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if roof["bound"] == "hbm":
        roof["peak_measured"] = copy_gbs
        roof["peak_measured_source"] = "streaming-read kernel of the library over 2 GiB (moe_hbm_read_probe)"
    else:
        roof["peak_measured"] = None if w4a4 else dense_bf16_tflops(wl, dev)
        roof["peak_measured_source"] = "dense bf16 GEMM of the gate/up shape via torch.mm (hipBLASLt)"
    roof["frac_of_measured"] = (roof["achieved"] / roof["peak_measured"]) if roof["peak_measured"] else None
    roof["traffic"] = gate_up_traffic(wl.name) if (fmt == "nvfp4" and not fused) else None
    roof["traffic_unit"] = "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)"
    roof["algorithmic_bytes"] = gu_bytes
    roof["algorithmic_flops"] = gu_flops
    if fused:
        roof["kernel"] = "fused decode kernel (S2-S6: top-k, permutation, gate/up, down, combine)"
    else:
        roof["kernel"] = ("gate/up stage (S4): x to MXFP4 + W4A4 grouped GEMM" if w4a4
                          else "gate/up stage (S4): x to NVFP4 values + grouped GEMM (alpha = d_x * d_w)"
                          + ("" if hbm_bound else " (+ fp16 row pass)") if a4 is not None
                          else "gate/up stage (S4): grouped GEMM")
    roof["kernel_us"] = kernel_ms * 1e3
    roof["kernel_us_median"] = float(np.median(kernel)) * 1e3

    # whole layer: flops 2(S+T)*3HI + 2THE (MFMA-bound shapes) or the bytes of every touched
    # expert, the shared expert, the router weight and the activations (HBM-bound shapes)
    if roof["bound"] == "hbm":
        layer_bytes = ((touched * 3 * I + 3 * wl.I_shared) * H * bpw + 2 * E * H + 4 * T * H)
        layer_roof = {"bound": "hbm", "achieved": layer_bytes / (ms_per_step * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                      "unit": "GB/s", "algorithmic_bytes": layer_bytes}
    else:
        layer_flops = 2.0 * S * 3 * H * I + 2.0 * T * 3 * H * wl.I_shared + 2.0 * T * H * E
        layer_roof = {"bound": "mfma", "achieved": layer_flops / (ms_per_step * 1e-3) / 1e12,
                      "peak": mfma_peak, "unit": "TFLOP/s", "algorithmic_flops": layer_flops}
    layer_roof["frac"] = layer_roof["achieved"] / layer_roof["peak"]
    layer_roof["frac_of_measured"] = (layer_roof["achieved"] / copy_gbs if roof["bound"] == "hbm" else
                                      (layer_roof["achieved"] / roof["peak_measured"]
                                       if roof["peak_measured"] else None))

    cpu_rec = None
    if cpu:
        log(f"{wl.name}: cpu oracle baseline")

        def bits(t):
            return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

        cpu_rec = cpu_baseline(wl, bits(x), bits(layer.w_router), synth_mod, fmt, act_gscales=a4)
    return {
        "value": T * steps / (total_ms / 1e3), "unit": "tokens/s", "steps": steps, "warmup": warmup,
        "settle_forwards": settle,
        "ms_per_step": ms_per_step,
        "step_ms": percentiles(step_ms),
        "config": {"workload": f"{wl.name}: T={T} H={H} I={I} E={E} top-{k} + 1 shared (I={wl.I_shared}), "
                               + ("MXFP4 W4A4" if w4a4 else "NVFP4 W4A4 (static activation scales)" if a4
                                  else f"{fmt.upper()} W4A16"),
                   "tokens": T, "hidden": H, "inter": I, "experts": E, "top_k": k,
                   "weight_copies": copies, "experts_touched": touched,
                   **({"activation_gscales": {"d_x": a4[0], "d_h": a4[1]}} if a4 else {})},
        "roofline": roof,
        "layer_roofline": layer_roof,
        "graph_replay_ms_per_step": graph_ms,
        "stages_us": stages_us,
        "timed_stages_us": ({"fused_S2_S6": percentiles([v * 1e3 for v in fused_k])} if fused else
                            {"gate_up": percentiles([v * 1e3 for v in gate_up]),
                             "down": percentiles([v * 1e3 for v in down])}),
        "cpu_baseline": cpu_rec,
    }


synth_mod = None


def main():
    global synth_mod
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode", choices=sorted(_DEFAULTS))
    ap.add_argument("--configs", default=None,
                    help="comma-separated workloads measured in the same line under 'configs' (default with the "
                         "decode workload: prefill,skewed,long_prefill; 'none' for none)")
    ap.add_argument("--copies", type=int, default=None, help="weight copies cycled through (main workload)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--fused-decode", action="store_true",
                    help="run few-token forwards on the two-launch fused decode path (opt-in; slower on MI355X)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB device to device three times (a kernel of known traffic, for "
                         "calibrating HBM byte counters)")
    ap.add_argument("--format", default="nvfp4", choices=["nvfp4", "mxfp4", "mxfp4_a4", "nvfp4_a4"],
                    help="weight format of the synthetic experts (the headline metric is NVFP4); mxfp4_a4: "
                         "the W4A4 layer (MXFP4 weights and activations on the FP4 matrix cores); nvfp4_a4: "
                         "the NVFP4 W4A4 layer (NVFP4 weights and activations, a numerics path)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the layer on one GPU only: each layer runs whole on one MI355X "
              "(no expert or tensor sharding, no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    from nvfp4_weight_quantized_amd import _lib, build_bank, ops, synth

    synth_mod = synth
    lib = _lib.lib()  # fail loudly now if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.configs is None:
        extra = PREFILL_CONFIGS if (args.workload == "decode" and args.format == "nvfp4") else []
    else:
        extra = [c for c in args.configs.split(",") if c and c != "none"]
    for c in extra:
        if c not in _DEFAULTS:
            raise SystemExit(f"unknown workload {c}")

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    copy_gbs = hbm_read_ceiling(lib, dev)
    log(f"streaming-read ceiling {copy_gbs:.0f} GB/s")

    banks = {}

    def layer_for(wl, copies):
        key = (wl.wseed, wl.H, wl.I, wl.E, wl.I_shared)
        if key not in banks:
            banks.clear()
            torch.cuda.empty_cache()
            log(f"building the {wl.name} expert bank ({args.format})")
            bfmt = "nvfp4" if args.format == "nvfp4_a4" else args.format
            banks[key] = (build_bank(wl, "routed", dev, bfmt),
                          build_bank(wl, "shared", dev, bfmt) if wl.I_shared > 0 else None)
        routed, shared = banks[key]
        bias = synth.router_bias(wl)
        lay = ops.NvFp4MoELayer(synth.router_weight(wl, dev).contiguous(),
                                torch.from_numpy(bias).to(dev) if bias is not None else None, routed, shared, wl.k)
        return [lay] + [clone_layer(lay, ops) for _ in range(copies - 1)]

    def run(name, main_line):
        wl = synth.WORKLOADS[name]
        d_steps, d_warmup, d_copies = _DEFAULTS[name]
        steps = args.steps if args.steps is not None else d_steps
        warmup = args.warmup if args.warmup is not None else d_warmup
        copies = (args.copies if args.copies is not None else d_copies) if main_line else d_copies
        layers = layer_for(wl, copies)
        rec = measure(wl, layers, steps, warmup, args.format, ops, lib, dev, copy_gbs, not args.no_cpu,
                      args.fused_decode)
        del layers
        torch.cuda.empty_cache()
        return rec

    main_rec = run(args.workload, True)
    configs = {name: run(name, False) for name in extra}

    w4a4 = args.format == "mxfp4_a4"
    line = {
        "metric": "NVFP4 MoE layer tokens/s; decode HBM GB/s %peak, prefill MFMA %peak"
                  + {"nvfp4": "", "mxfp4": " (measured here on MXFP4 weights)",
                     "mxfp4_a4": " (measured here on the MXFP4 W4A4 layer)",
                     "nvfp4_a4": " (measured here on the NVFP4 W4A4 layer)"}[args.format],
        "value": main_rec["value"], "unit": "tokens/s", "n_gpus": 1, "steps": main_rec["steps"],
        "warmup": main_rec["warmup"], "ms_per_step": main_rec["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp4" if w4a4 else "bf16", "data": "synthetic",
    }
    line.update({k: v for k, v in main_rec.items() if k not in line and k not in ("unit",)})
    line["measured_hbm_read_GBs"] = copy_gbs
    line["configs"] = configs
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
