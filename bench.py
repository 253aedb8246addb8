#!/usr/bin/env python3
"""Benchmark of the LM-head logits library on one MI355X.

A step is one pass of the hot path over the decode workload (H=4096,
V=128256, bf16 weight ~N(0, 0.02), hidden ~N(0, 1), fp32 logits, alpha=1/16):
one lmhead_logits call for each M in {1, 2, 8, 32, 64}. The headline value is
the whole step's algorithmic HBM throughput (weight read once + hidden +
output written, divided by the step time). The other workloads -- prefill
(M=2048), spec-decode (M=128 with bias), the NVFP4 head (M in 1, 16, 64,
256), fp16 inputs (M in 1, 64, 2048), the row-reduction epilogue (decode
M = 64, spec M = 128) and the BF16 -> NVFP4 quantiser -- are timed after it
and reported alongside.

Inputs are generated on the host from the seeded generator, copied to HBM
before timing, and never touched by the timed region. Timing uses HIP events
on the stream the library launches on (torch's current stream).

Output: one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

import numpy as np  # noqa: E402

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6       # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
METRIC = ("LM-head µs/call + HBM GB/s (M≤64) and TFLOP/s (M=2048), % of roofline")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# Algorithmic byte and flop models (W read once + hidden + bias + output).
# ----------------------------------------------------------------------------

def bytes_bf16(M, H, V, out_bytes, bias):
    return V * H * 2 + M * H * 2 + (V * 4 if bias else 0) + M * V * out_bytes


def bytes_nvfp4(M, H, V, bias=False):
    return V * H // 2 + V * H // 16 + M * H * 2 + (V * 4 if bias else 0) + M * V * 2


def flops(M, H, V):
    return 2 * M * H * V


# Sources the decode kernel's code and launch depend on: a counter reading is
# valid only while these are unchanged.
DECODE_SOURCES = ("kstep.hpp", "korder.hpp", "launch.hpp", "lmhead_api.cpp", "ring.hpp",
                  "skinny.hip")


def kernel_source_hash(files=DECODE_SOURCES):
    h = hashlib.sha256()
    for name in files:
        p = ROOT / "lm_head_logits_amd" / "csrc" / name
        h.update(name.encode())
        h.update(p.read_bytes())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    f = ROOT / "profiles" / "traffic_counters.md"
    if not f.exists():
        return None
    text = f.read_text()
    m = re.search(r"source-hash:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(rf"^\|\s*{re.escape(kernel)}\s*\|[^\n]*?\|\s*([0-9.]+)\s*\|\s*$", text, re.M)
    return float(m.group(1)) if m else None


# ----------------------------------------------------------------------------
# GPU timing
# ----------------------------------------------------------------------------

# Untimed load before each timed region. After any idle spell (input
# generation between workloads, host copies) the GPU's clocks ramp up over
# roughly the first 20 ms of load: a 43 us NVFP4 call took about 49 us
# through its first 220 calls, again after 2 s idle, and again on freshly
# allocated buffers.
WARM_MS = 50.0


def timed_calls(torch, fns, warmup, steps, batches=5):
    """Run `fns` (one step = each fn once) warmup + steps times. Each fn's
    `steps` calls run back to back in `batches` batches, one pair of events
    around each batch and none between calls, so a batch's time is that of
    its kernels (an event recorded between two kernels holds the second back
    by several microseconds). The untimed warm-up runs `warmup` steps, and
    more until at least WARM_MS of continuous work has run. Returns the step
    time (ms: events around all steps, divided by steps), the wall time per
    step (ms) and, per fn, the batches' average launch times (ms)."""
    t0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t0) * 1e3 < WARM_MS:
        for f in fns:
            f()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()  # so that the wall clock follows the GPU
    torch.cuda.synchronize()
    nb = max(1, min(batches, steps))
    sizes = [steps // nb + (1 if b < steps % nb else 0) for b in range(nb)]
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nb)] for _ in fns]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i, f in enumerate(fns):
        for b, n in enumerate(sizes):
            ev[i][b][0].record()
            for _ in range(n):
                f()
            ev[i][b][1].record()
    t1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) * 1e3
    total = t0.elapsed_time(t1)
    per = [[ev[i][b][0].elapsed_time(ev[i][b][1]) / n for b, n in enumerate(sizes)]
           for i in range(len(fns))]
    return total / steps, wall / steps, per


def rotating(fns):
    """One callable that calls `fns` in turn (copies of a head that fits the
    256 MB MALL: each call then reads its copy from HBM)."""
    it = itertools.cycle(fns)
    return lambda: next(it)()


def to_dev_bf16(torch, a, dev):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)


def bench_decode(torch, L, wl, dev, warmup, steps):
    w = wl.DECODE
    log("decode: generating inputs")
    h, W = wl.hidden(w), wl.weight(w)
    hd, Wd = to_dev_bf16(torch, h, dev), to_dev_bf16(torch, W, dev)
    alpha = w.alphas[1]
    outs = {M: torch.empty((M, w.V), dtype=torch.float32, device=dev) for M in w.Ms}
    fns = [(lambda M=M: L.logits(hd[:M], Wd, alpha, None, torch.float32, out=outs[M])) for M in w.Ms]
    step_ms, wall_ms, per = timed_calls(torch, fns, warmup, steps)
    per_m = {}
    tot_bytes = 0
    for M, ts in zip(w.Ms, per):
        b = bytes_bf16(M, w.H, w.V, 4, False)
        tot_bytes += b
        us_avg = 1e3 * float(np.mean(ts))
        per_m[str(M)] = {"us_avg": round(us_avg, 2), "us_min": round(1e3 * float(np.min(ts)), 2),
                         "GBps": round(b / us_avg / 1e3, 1),
                         "frac_hbm": round(b / us_avg / 1e3 / HBM_PEAK_GBPS, 4),
                         "roofline_us": round(b / HBM_PEAK_GBPS / 1e3, 2)}
    launches_ms = float(np.sum([np.mean(ts) for ts in per]))
    return {"w": w, "per_m": per_m, "step_ms": step_ms, "wall_ms": wall_ms,
            "bytes_per_step": tot_bytes, "launch_ms_sum": launches_ms, "h": h, "W": W,
            "hd": hd, "Wd": Wd}


def bench_tiny(torch, L, wl, dev, warmup, steps):
    """The tiny head (M = 4, H = 256, V = 4096, fp32 logits): 2 MB of weight,
    held in L2 between calls, so a call is bound by launch and ramp-up, not
    by HBM; reported in µs per call with its fraction of the HBM roofline
    for completeness."""
    w = wl.TINY
    log("tiny: generating inputs")
    h, W = wl.hidden(w), wl.weight(w)
    hd, Wd = to_dev_bf16(torch, h, dev), to_dev_bf16(torch, W, dev)
    M = w.Ms[0]
    out = torch.empty((M, w.V), dtype=torch.float32, device=dev)
    _, _, per = timed_calls(torch, [lambda: L.logits(hd, Wd, w.alphas[0], None, torch.float32,
                                                     out=out)], warmup, steps)
    us = 1e3 * float(np.mean(per[0]))
    by = bytes_bf16(M, w.H, w.V, 4, False)
    # The same calls replayed from a HIP graph (the entry points allocate and
    # synchronise nothing, so they can be captured): the per-call time without
    # the host's launch overhead between calls.
    calls = 20
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        L.logits(hd, Wd, w.alphas[0], None, torch.float32, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            L.logits(hd, Wd, w.alphas[0], None, torch.float32, out=out)
    _, _, gper = timed_calls(torch, [g.replay], max(1, warmup // 5), max(2, steps // 5))
    us_graph = 1e3 * float(np.mean(gper[0])) / calls
    return {"M": M, "H": w.H, "V": w.V, "us_avg": round(us, 2),
            "us_min": round(1e3 * float(np.min(per[0])), 2),
            "us_per_call_graph_replay": round(us_graph, 2), "GBps": round(by / us / 1e3, 1),
            "roofline_us": round(by / HBM_PEAK_GBPS / 1e3, 3),
            "frac_hbm": round(by / us / 1e3 / HBM_PEAK_GBPS, 4),
            "bound": "launch (the weight stays in L2)"}


def bench_shard(torch, L, w, hd, Wd, warmup, steps, shards=8, copies=4):
    """The decode head's one-GPU share when the vocabulary is split over
    `shards` GPUs (V/8 = 16032 rows, 131 MB): `copies` distinct row ranges of
    the decode weight in rotation, so successive calls cannot hit the 256 MB
    MALL."""
    vs = w.V // shards
    res = {"V_shard": vs, "H": w.H, "copies": copies}
    for M in (1, 64):
        out = torch.empty((M, vs), dtype=torch.float32, device=hd.device)
        fns = [(lambda i=i: L.logits(hd[:M], Wd[i * vs:(i + 1) * vs], w.alphas[1], None,
                                     torch.float32, out=out)) for i in range(copies)]
        _, _, per = timed_calls(torch, [rotating(fns)], warmup * copies, steps * copies)
        us = 1e3 * float(np.mean(per))
        b = bytes_bf16(M, w.H, vs, 4, False)
        res[str(M)] = {"us_avg": round(us, 2), "GBps": round(b / us / 1e3, 1),
                       "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBPS, 4),
                       "roofline_us": round(b / HBM_PEAK_GBPS / 1e3, 2)}
    return res


def bench_probes(torch, L, dev, warmup, steps, nbytes=1 << 30, mfma_iters=15000):
    """The practical ceilings on this part: a plain read of 1 GiB of HBM and
    the bf16 MFMA-only probe (include/lmhead_probes.h), timed like the
    projection (HIP events on the launch stream)."""
    buf = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).normal_()
    _, _, per = timed_calls(torch, [lambda: L.probe_hbm_read(buf)], warmup, steps)
    ms = np.asarray(per[0])
    fl = L.probe_mfma_bf16(mfma_iters, dev)
    _, _, perm = timed_calls(torch, [lambda: L.probe_mfma_bf16(mfma_iters, dev)], 2,
                             max(3, steps // 10))
    msm = np.asarray(perm[0])
    del buf
    return {"hbm_read_GBps": round(nbytes / float(np.mean(ms)) / 1e6, 1),
            "hbm_read_GBps_best": round(nbytes / float(np.min(ms)) / 1e6, 1),
            "mfma_bf16_TFLOPs": round(fl / float(np.mean(msm)) / 1e9, 1),
            "mfma_bf16_TFLOPs_best": round(fl / float(np.min(msm)) / 1e9, 1),
            "read_bytes": nbytes, "mfma_flops_per_launch": fl}


def bench_prefill(torch, L, wl, dev, warmup, steps):
    w = wl.PREFILL
    log("prefill: generating inputs")
    h, W = wl.hidden(w), wl.weight(w)
    hd, Wd = to_dev_bf16(torch, h, dev), to_dev_bf16(torch, W, dev)
    out = torch.empty((w.M, w.V), dtype=torch.float32, device=dev)
    step_ms, _, per = timed_calls(torch, [lambda: L.logits(hd, Wd, w.alphas[0], None, out=out)],
                                  warmup, steps)
    us = 1e3 * float(np.mean(per[0]))
    f = flops(w.M, w.H, w.V)
    del hd, Wd, out
    return {"M": w.M, "H": w.H, "V": w.V, "us_avg": round(us, 1),
            "us_min": round(1e3 * float(np.min(per[0])), 1),
            "TFLOPs": round(f / us / 1e6, 1), "frac_mfma": round(f / us / 1e6 / BF16_PEAK_TFLOPS, 4),
            "roofline_us": round(max(f / BF16_PEAK_TFLOPS / 1e6,
                                     bytes_bf16(w.M, w.H, w.V, 4, False) / HBM_PEAK_GBPS / 1e3), 1)}


def bench_spec(torch, L, wl, dev, warmup, steps):
    w = wl.SPEC
    log("spec: generating inputs")
    h, W, b = wl.hidden(w), wl.weight(w), wl.bias(w)
    hd, Wd = to_dev_bf16(torch, h, dev), to_dev_bf16(torch, W, dev)
    bd = torch.from_numpy(b).to(dev)
    res = {}
    for M in (w.M, 32):
        out = torch.empty((M, w.V), dtype=torch.float32, device=dev)
        _, _, per = timed_calls(torch, [lambda: L.logits(hd[:M], Wd, w.alphas[0], bd, out=out)],
                                warmup, steps)
        us = 1e3 * float(np.mean(per[0]))
        by = bytes_bf16(M, w.H, w.V, 4, True)
        res[str(M)] = {"us_avg": round(us, 2), "GBps": round(by / us / 1e3, 1),
                       "frac_hbm": round(by / us / 1e3 / HBM_PEAK_GBPS, 4),
                       "roofline_us": round(by / HBM_PEAK_GBPS / 1e3, 2)}
    return res


def bench_nvfp4(torch, L, wl, dev, warmup, steps, copies=4):
    w = wl.NVFP4
    log("nvfp4: generating inputs")
    h, c, s = wl.hidden(w), wl.codes(w), wl.scales(w)
    hd = to_dev_bf16(torch, h, dev)
    # several copies of the 175 MB head so successive calls cannot hit the 256 MB MALL
    cs = [torch.from_numpy(c).to(dev) for _ in range(copies)]
    ss = [torch.from_numpy(s).to(dev) for _ in range(copies)]
    res = {}
    for M in w.Ms:
        out = torch.empty((M, w.V), dtype=torch.bfloat16, device=dev)
        fns = [(lambda i=i: L.logits_nvfp4(hd[:M], cs[i], ss[i], w.g, 1.0, out=out))
               for i in range(copies)]
        _, _, per = timed_calls(torch, [rotating(fns)], warmup * copies, steps * copies)
        us = 1e3 * float(np.mean(per))
        by = bytes_nvfp4(M, w.H, w.V)
        f = flops(M, w.H, w.V)
        roof = max(by / HBM_PEAK_GBPS / 1e3, f / BF16_PEAK_TFLOPS / 1e6)
        res[str(M)] = {"us_avg": round(us, 2), "GBps": round(by / us / 1e3, 1),
                       "TFLOPs": round(f / us / 1e6, 1), "roofline_us": round(roof, 2),
                       "frac_roofline": round(roof / us, 4)}
    del cs, ss
    # The ceiling for streaming this many bytes at all: the HBM read probe on
    # buffers of the M = 1 call's size, rotated like the heads (so none is
    # served from the MALL): the best fraction of the roofline any kernel
    # that reads the head once can reach at this size.
    nb = (bytes_nvfp4(1, w.H, w.V) + 15) // 16 * 16
    bufs = [torch.empty(nb // 2, dtype=torch.bfloat16, device=dev).normal_() for _ in range(copies)]
    _, _, pp = timed_calls(torch, [rotating([(lambda b=b: L.probe_hbm_read(b)) for b in bufs])],
                           warmup * copies, steps * copies)
    probe_us = 1e3 * float(np.mean(pp))
    res["hbm_read_probe_same_bytes"] = {"bytes": nb, "us_avg": round(probe_us, 2),
                                        "GBps": round(nb / probe_us / 1e3, 1),
                                        "frac_of_m1_roofline": round(res["1"]["roofline_us"] / probe_us, 4)}
    del bufs
    # Side by side: the bf16 entry point on a bf16 head of the same shape
    # (the same logits type), at the row count the tiled kernel serves.
    Wb = (0.02 * torch.randn(w.V, w.H, device=dev)).to(torch.bfloat16)
    for M in [m for m in w.Ms if m > 64]:
        out = torch.empty((M, w.V), dtype=torch.bfloat16, device=dev)
        _, _, per = timed_calls(torch, [lambda: L.logits(hd[:M], Wb, 1.0, None, torch.bfloat16,
                                                         out=out)], warmup, steps)
        res[str(M)]["bf16_head_same_shape_us"] = round(1e3 * float(np.mean(per[0])), 2)
    return res


def bench_f16(torch, L, wl, dev, warmup, steps):
    """fp16 hidden and weight, fp32 logits: decode rows (HBM-bound) and one
    prefill batch (MFMA-bound) over the same [V, H] head."""
    w = wl.F16
    log("f16: generating inputs")
    h, W = wl.hidden(w), wl.weight(w)
    hd = torch.from_numpy(h.view(np.int16)).view(torch.float16).to(dev)
    Wd = torch.from_numpy(W.view(np.int16)).view(torch.float16).to(dev)
    alpha = w.alphas[0]
    res = {}
    for M in w.Ms:
        out = torch.empty((M, w.V), dtype=torch.float32, device=dev)
        n = steps if M <= 64 else max(5, steps // 5)
        _, _, per = timed_calls(torch, [lambda: L.logits(hd[:M], Wd, alpha, None, out=out)],
                                warmup, n)
        us = 1e3 * float(np.mean(per[0]))
        by = bytes_bf16(M, w.H, w.V, 4, False)       # fp16 elements are 2 bytes, as bf16
        f = flops(M, w.H, w.V)
        r = {"us_avg": round(us, 2), "GBps": round(by / us / 1e3, 1),
             "TFLOPs": round(f / us / 1e6, 1)}
        if M <= 64:
            r["frac_hbm"] = round(by / us / 1e3 / HBM_PEAK_GBPS, 4)
        else:
            r["frac_mfma"] = round(f / us / 1e6 / BF16_PEAK_TFLOPS, 4)   # fp16 peak = bf16 peak
        res[str(M)] = r
        del out
    del hd, Wd
    return res


def bench_rowreduce(torch, L, wl, dev, warmup, steps):
    """The row-reduction epilogue (max, argmax, sum of exp) with no logits
    written, against the plain call that writes fp32 logits: decode M = 64
    and the spec-decode target M = 128 (with bias)."""
    res = {}
    for w, M, alpha, tag in ((wl.DECODE, 64, wl.DECODE.alphas[1], "decode_M64"),
                             (wl.SPEC, 128, wl.SPEC.alphas[0], "spec_M128")):
        log(f"rowreduce: {tag}")
        h, W, b = wl.hidden(w, M), wl.weight(w), wl.bias(w)
        hd, Wd = to_dev_bf16(torch, h, dev), to_dev_bf16(torch, W, dev)
        bd = torch.from_numpy(b).to(dev) if b is not None else None
        out = torch.empty((M, w.V), dtype=torch.float32, device=dev)
        ws = torch.empty(L.rowreduce_workspace_bytes(M, w.V), dtype=torch.uint8, device=dev)
        fns = [lambda: L.logits(hd, Wd, alpha, bd, out=out),
               lambda: L.logits_rowreduce(hd, Wd, alpha, bd, workspace=ws)]
        _, _, per = timed_calls(torch, fns, warmup, steps)
        plain_us, red_us = (1e3 * float(np.mean(p)) for p in per)
        by_red = bytes_bf16(M, w.H, w.V, 0, b is not None) + 2 * ws.numel() + 12 * M
        res[tag] = {"plain_us": round(plain_us, 2), "rowreduce_us": round(red_us, 2),
                    "rowreduce_GBps": round(by_red / red_us / 1e3, 1),
                    "rowreduce_frac_hbm": round(by_red / red_us / 1e3 / HBM_PEAK_GBPS, 4)}
        del hd, Wd, out, ws
        torch.cuda.empty_cache()
    return res


def bench_quantize(torch, L, wl, dev, warmup, steps):
    """BF16 -> NVFP4 quantisation of the NVFP4 workload's head (V = 151936,
    H = 2048, 622 MB of bf16): the absmax pass reads the weight once, the
    quantiser reads it again and writes 9/16 byte per element."""
    w = wl.NVFP4
    log("quantize: generating inputs")
    Wd = to_dev_bf16(torch, wl.bf16_head(w), dev)
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    _, _, per = timed_calls(torch, [lambda: L.quantize_nvfp4(Wd, workspace=ws)], warmup, steps)
    us = 1e3 * float(np.mean(per[0]))
    n = w.V * w.H
    by = 2 * n * 2 + n // 2 + n // 16
    del Wd
    return {"V": w.V, "H": w.H, "us_avg": round(us, 1), "GBps": round(by / us / 1e3, 1),
            "frac_hbm": round(by / us / 1e3 / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes": by, "roofline_us": round(by / HBM_PEAK_GBPS / 1e3, 1)}


def bench_copy(torch, dev, warmup, steps, nbytes=1 << 30):
    """A plain device-to-device copy of `nbytes` (torch's copy kernel): reads
    and writes exactly nbytes, so the HBM counters read on it give the scale
    factor from counter units to bytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    _, _, per = timed_calls(torch, [lambda: dst.copy_(src)], warmup, steps)
    us = 1e3 * float(np.mean(per[0]))
    return {"bytes_read": nbytes, "bytes_written": nbytes, "us_avg": round(us, 1),
            "GBps": round(2 * nbytes / us / 1e3, 1)}


def bench_libgemm(torch, dev, warmup, steps, M=2048, H=4096, V=151936):
    """Context, not part of the path: the vendor GEMM (hipBLASLt through
    torch.mm) at the prefill shape, with fp32 output (out_dtype, the call the
    sglang digest's fp32 head makes) and with bf16 output. Inputs are device
    normals of the prefill workload's scales (the GEMM's speed does not
    depend on the exact values)."""
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    a = torch.randn(M, H, generator=g, device=dev).to(torch.bfloat16)
    w = (0.02 * torch.randn(V, H, generator=g, device=dev)).to(torch.bfloat16)
    wt = w.t()
    f = flops(M, H, V)
    res = {"M": M, "H": H, "V": V}
    legs = {"bf16_out": lambda: torch.mm(a, wt)}
    try:
        torch.mm(a[:16], wt, out_dtype=torch.float32)
        legs["f32_out"] = lambda: torch.mm(a, wt, out_dtype=torch.float32)
    except (TypeError, RuntimeError):
        pass
    for name, fn in legs.items():
        _, _, per = timed_calls(torch, [fn], warmup, steps)
        us = 1e3 * float(np.mean(per[0]))
        res[name] = {"us_avg": round(us, 1), "TFLOPs": round(f / us / 1e6, 1),
                     "frac_mfma": round(f / us / 1e6 / BF16_PEAK_TFLOPS, 4)}
    return res


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the decode workload.
# ----------------------------------------------------------------------------

def cpu_baseline(wl, h, W, budget_s=12.0):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    w = wl.DECODE
    M = 64
    # grow the vocabulary slice until one oracle call takes a few seconds
    nv = 1024
    while True:
        t0 = time.perf_counter()
        oracle.lmhead_logits(h[:M], W[:nv], w.alphas[1], None, "f32")
        dt = time.perf_counter() - t0
        if dt > budget_s / 4 or nv >= w.V:
            break
        nv = min(w.V, nv * 4)
    # repeat until about budget_s seconds of oracle work have been timed
    reps, t_total = 0, 0.0
    while t_total < budget_s and reps < 100:
        t0 = time.perf_counter()
        oracle.lmhead_logits(h[:M], W[:nv], w.alphas[1], None, "f32")
        t_total += time.perf_counter() - t0
        reps += 1
    per_call = t_total / reps
    # one thread, on a smaller slice: ns per multiply-add of the fp64 oracle
    ns_mac = None
    try:
        from threadpoolctl import threadpool_limits
        nv1 = max(256, nv // 16)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.lmhead_logits(h[:M], W[:nv1], w.alphas[1], None, "f32")
            ns_mac = (time.perf_counter() - t0) / (M * nv1 * w.H) * 1e9
    except Exception:
        pass
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    b = nv * w.H * 2 + M * w.H * 2 + M * nv * 4
    return {"value": round(b / per_call / 1e9, 3), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"decode head M=64, first {nv} of {w.V} vocabulary rows, H={w.H}, fp32 out; "
                      f"{reps} calls, {per_call:.2f} s each (numpy fp64 oracle)",
            "us_per_call_full_vocab_est": round(per_call * w.V / nv * 1e6, 0),
            "cpu_model": cpu_model, "host_cpus": os.cpu_count(),
            "ns_per_mac_1thread": None if ns_mac is None else round(ns_mac, 3)}


def cpu_per_config(wl):
    """The oracle timed on each workload of the pages' configurations (the
    tiny head, the spec-decode target, the NVFP4 head at M = 256 and the
    prefill batch), on a stated sample where the whole call would take long:
    wall time, multiply-adds and ns per multiply-add of each timed call."""
    import oracle
    res = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    w = wl.TINY
    h, W = wl.hidden(w), wl.weight(w)
    dt = timed(lambda: oracle.lmhead_logits(h, W, w.alphas[0], None, "f32"))
    macs = w.M * w.H * w.V
    res["tiny"] = {"sample": "whole call (M=4, H=256, V=4096)", "s": round(dt, 4), "macs": macs,
                   "ns_per_mac": round(dt / macs * 1e9, 4)}

    w = wl.SPEC
    h, W, b = wl.hidden(w), wl.weight(w), wl.bias(w)
    dt = timed(lambda: oracle.lmhead_logits(h, W, w.alphas[0], b, "f32"))
    macs = w.M * w.H * w.V
    res["spec_M128"] = {"sample": "whole call (M=128, H=2048, V=151936, bias)", "s": round(dt, 3),
                        "macs": macs, "ns_per_mac": round(dt / macs * 1e9, 4)}
    del W

    w = wl.NVFP4
    nv = 16384
    h, c, sc = wl.hidden(w, 256), wl.codes(w, 0, nv), wl.scales(w, 0, nv)
    dt = timed(lambda: oracle.lmhead_logits_nvfp4(h, c, sc, w.g))
    macs = 256 * w.H * nv
    res["nvfp4_M256"] = {"sample": f"M=256, first {nv} of {w.V} vocabulary rows, H={w.H}",
                         "s": round(dt, 3), "macs": macs, "ns_per_mac": round(dt / macs * 1e9, 4),
                         "s_full_vocab_est": round(dt * w.V / nv, 2)}

    w = wl.PREFILL
    rows = sorted(set(range(0, w.M, 16)) | {w.M - 1})
    h, W = wl.hidden_rows(w, rows), wl.weight(w)
    dt = timed(lambda: oracle.lmhead_logits(h, W, w.alphas[0], None, "f32"))
    macs = len(rows) * w.H * w.V
    res["prefill_M2048"] = {"sample": f"{len(rows)} of {w.M} rows (every 16th and the last), "
                                      f"all {w.V} vocabulary rows, H={w.H}",
                            "s": round(dt, 3), "macs": macs, "ns_per_mac": round(dt / macs * 1e9, 4),
                            "s_all_rows_est": round(dt * w.M / len(rows), 2)}
    del W
    return res


def main():
    global WARM_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["decode", "tiny", "prefill", "spec", "nvfp4", "f16", "rowreduce",
                                       "quantize", "copy", "probes", "libgemm", "all"],
                    default="all",
                    help="run one workload only (for profiling; 'copy' is the HBM counter "
                         "calibration); the headline line needs decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm-ms", type=float, default=WARM_MS,
                    help="untimed work before each timed region, at least (ms)")
    args = ap.parse_args()
    WARM_MS = max(0.0, args.warm_ms)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library shards by vocabulary with no exchange, "
              "and multi-GPU runs are not part of this build. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import lm_head_logits_amd as L
    import synth.workloads as wl

    dev = "cuda:0"
    torch.cuda.set_device(0)
    run = (lambda name: args.only in (name, "all"))
    extra = {}
    if args.only != "all" and args.only != "decode":
        # a single non-headline workload, for profiling: print its numbers only
        fn = {"tiny": lambda: bench_tiny(torch, L, wl, dev, args.warmup, args.steps),
              "prefill": lambda: bench_prefill(torch, L, wl, dev, args.warmup, args.steps),
              "spec": lambda: bench_spec(torch, L, wl, dev, args.warmup, args.steps),
              "nvfp4": lambda: bench_nvfp4(torch, L, wl, dev, args.warmup, args.steps),
              "f16": lambda: bench_f16(torch, L, wl, dev, args.warmup, args.steps),
              "rowreduce": lambda: bench_rowreduce(torch, L, wl, dev, args.warmup, args.steps),
              "quantize": lambda: bench_quantize(torch, L, wl, dev, args.warmup, args.steps),
              "copy": lambda: bench_copy(torch, dev, args.warmup, args.steps),
              "probes": lambda: bench_probes(torch, L, dev, args.warmup, args.steps),
              "libgemm": lambda: bench_libgemm(torch, dev, args.warmup, max(5, args.steps // 5))}[args.only]
        print(json.dumps({"workload": args.only, "result": fn()}), flush=True)
        return
    dec = bench_decode(torch, L, wl, dev, args.warmup, args.steps)
    if run("shard"):
        extra["decode_shard_v8"] = bench_shard(torch, L, dec["w"], dec["hd"], dec["Wd"],
                                               args.warmup, args.steps)
    del dec["hd"], dec["Wd"]
    torch.cuda.empty_cache()
    if run("tiny"):
        extra["tiny"] = bench_tiny(torch, L, wl, dev, args.warmup, args.steps)
    if run("prefill"):
        extra["prefill"] = bench_prefill(torch, L, wl, dev, args.warmup, max(5, args.steps // 5))
        torch.cuda.empty_cache()
    if run("spec"):
        extra["spec_decode"] = bench_spec(torch, L, wl, dev, args.warmup, args.steps)
        torch.cuda.empty_cache()
    if run("nvfp4"):
        extra["nvfp4"] = bench_nvfp4(torch, L, wl, dev, args.warmup, args.steps)
        torch.cuda.empty_cache()
    if run("f16"):
        extra["f16_inputs"] = bench_f16(torch, L, wl, dev, args.warmup, args.steps)
        torch.cuda.empty_cache()
    if run("rowreduce"):
        extra["rowreduce"] = bench_rowreduce(torch, L, wl, dev, args.warmup, args.steps)
        torch.cuda.empty_cache()
    if run("quantize"):
        extra["quantize_nvfp4"] = bench_quantize(torch, L, wl, dev, args.warmup, args.steps)
        torch.cuda.empty_cache()
    if run("probes"):
        extra["probes"] = bench_probes(torch, L, dev, args.warmup, args.steps)
        torch.cuda.empty_cache()
    if run("libgemm"):
        extra["library_gemm_prefill_context"] = bench_libgemm(torch, dev, args.warmup,
                                                              max(5, args.steps // 5))
        torch.cuda.empty_cache()

    w = dec["w"]
    step_ms = dec["step_ms"]
    value = dec["bytes_per_step"] / (step_ms * 1e-3) / 1e9
    launches = len(w.Ms)
    achieved = dec["bytes_per_step"] / launches / (dec["launch_ms_sum"] / launches * 1e-3) / 1e9
    traffic = committed_traffic("skinny_decode")
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "warmup_min_ms": WARM_MS,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller inputs of the workload's shapes)",
        "config": {"workload": "decode head: H=4096, V=128256, bf16 W ~N(0,0.02), bf16 hidden "
                               "~N(0,1), alpha=1/16, fp32 out; one step = one call at each M in "
                               "{1,2,8,32,64}",
                   "H": w.H, "V": w.V, "Ms": list(w.Ms), "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": "skinny_kernel (decode, M<=64)"},
        "decode_per_M": dec["per_m"],
        **extra,
    }
    if "probes" in extra:
        # fractions of what this part sustains in practice (context; the
        # roofline fractions above use the published peaks)
        pr = extra["probes"]
        ctx = {"decode_achieved_over_read_probe": round(achieved / pr["hbm_read_GBps"], 4)}
        if "prefill" in extra:
            ctx["prefill_over_mfma_probe"] = round(extra["prefill"]["TFLOPs"] / pr["mfma_bf16_TFLOPs"], 4)
        line["vs_probes"] = ctx
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, dec["h"], dec["W"])
        del dec["W"]
        line["cpu_baseline"]["per_config"] = cpu_per_config(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
