#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = the whole path on one batch: fa2_forward (O, LSE) then the two backward kernels that
fa2_backward runs (dQ with the preprocess folded in, then dK/dV), on the causal prefill workload
B=2, H=32, N=8192, d=128, bf16 inputs drawn from the seeded generator and resident in HBM before
timing starts.

Prints ONE JSON line on stdout. FLOPs follow the counting rule 4*B*H*N^2*d for a forward,
halved when causal, and 2.5x that for the backward; the value is fwd+bwd TFLOP/s. Per-kernel
durations come from HIP events recorded on the launch stream between the kernels of every
timed step; the roofline object describes the longest-running kernel.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (fwd, fwd+bwd) bf16 causal d=128 N=8192; % MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
WORKLOAD = dict(B=2, Hq=32, Hkv=32, N=8192, d=128, causal=True)
SEED = 0x5EED0006

# The pages' own figures, all measured on NVIDIA hardware. Printed beside the MI355X numbers as
# context only: none is quoted for this workload, precision or chip, so none is a target.
PAGES_CONTEXT = [
    {"figure": "FlashAttention-1 utilisation of the theoretical peak FLOP/s", "value": "25-40 %",
     "hardware": "NVIDIA A100", "source": "FlashAttention-2 (wiki), section \"Разработка и цели\""},
    {"figure": "FlashAttention-2 utilisation of the theoretical peak FLOP/s", "value": "50-73 %",
     "hardware": "NVIDIA A100", "source": "FlashAttention-2 (wiki), section \"Производительность и эффективность\""},
    {"figure": "FlashAttention-2 speed-up over FlashAttention-1", "value": "about 2x", "hardware": "not stated",
     "source": "FlashAttention-2 (wiki), section \"Производительность и эффективность\""},
    {"figure": "FlashAttention-2 throughput", "value": "335 TFLOP/s", "hardware": "NVIDIA H100",
     "source": "FlashAttention-2 (wiki), section \"Производительность и эффективность\""},
    {"figure": "FlashAttention-3 throughput", "value": "up to 740 TFLOP/s, about 75 % of peak", "hardware": "NVIDIA H100",
     "source": "Flash Attention spiegata: una guida completa, section \"Flash Attention 3\""},
]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(kernel):
    """HBM bytes per launch of ``kernel`` from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE scaled by a plain copy's readings), or None when there is no entry or the kernel's
    source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            entry = json.load(f)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for name in (entry["source"], "fa2_device.h"):
        with open(os.path.join(ROOT, "exact_tiled_attention_fa2_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return entry["hbm_bytes"] if h.hexdigest() == entry["source_sha256"] else None


def counted_fwd_flops(B, Hq, N, d, causal):
    f = 4.0 * B * Hq * N * N * d
    return f / 2 if causal else f


def visible_pairs(N, causal, window=None):
    """(query, key) pairs per head that the mask leaves visible."""
    if not causal:
        return N * N
    if window is None or window >= N - 1:
        return N * (N + 1) // 2
    W = window
    return W * (W + 1) // 2 + (N - W) * (W + 1)


def time_sequence(calls, steps, warmup, stream, spread=None):
    """Median (over steps) of each call's duration and of the whole sequence, in ms, from HIP
    events recorded on ``stream`` between the calls. ``spread``, if a dict, receives the min and
    max of each call's duration ("min", "max": lists like the medians)."""
    import numpy as np
    import torch
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    for s in range(steps):
        for i, c in enumerate(calls):
            ev[s][i].record(stream)
            c()
        ev[s][len(calls)].record(stream)
    torch.cuda.synchronize()
    durs = [[ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)] for i in range(len(calls))]
    per = [float(np.median(d)) for d in durs]
    if spread is not None:
        spread["min"] = [float(np.min(d)) for d in durs]
        spread["max"] = [float(np.max(d)) for d in durs]
    total = float(np.median([ev[s][0].elapsed_time(ev[s][len(calls)]) for s in range(steps)]))
    return per, total


def time_back_to_back(call, reps, rounds, stream):
    """Median over ``rounds`` of the mean duration, in ms, of ``reps`` calls issued back to back
    between two HIP events on ``stream`` (no event between the calls). For launches of a few
    tens of microseconds the events recorded around every call in time_sequence add several
    microseconds each; this is the steady rate of repeated calls."""
    import numpy as np
    import torch
    for _ in range(3):
        call()
    ts = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / reps)
    return float(np.median(ts))


def extra_workloads(fa2, seedgen, dev, stream, steps, only=None):
    """Non-headline measurements: the sliding-window path at the headline shape, and the other
    workload shapes (forward-only prefill shapes, a training shape). Values are TFLOP/s of the
    counted FLOPs over the visible (query, key) pairs: 4d per pair forward, 10d fwd+bwd; forwards
    also report GB/s of their compulsory HBM bytes (Q, K, V read once, O and LSE written once).
    ``only``: names (substrings) of the workloads to run, or None for all."""
    import numpy as np
    import torch

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    def check(st, what):
        if st != 0:
            raise fa2.Fa2Error(st, what)

    def wanted(name):
        return only is None or any(p in name for p in only)

    out = {}
    cases = [("window_W1024_B2_H32_N8192_d128", 2, 32, 32, 8192, 128, True, 1024, True, 0x5EED0006),
             ("fwd_B1_H2_N256_d64", 1, 2, 2, 256, 64, False, None, False, 0x5EED0001),
             ("fwd_B4_H16_N2048_d64", 4, 16, 16, 2048, 64, False, None, False, 0x5EED0002),
             ("fwd_B1_Hq32_Hkv8_N32768_d128_causal", 1, 32, 8, 32768, 128, True, None, False, 0x5EED0004),
             ("fwdbwd_B4_H16_N4096_d128_causal", 4, 16, 16, 4096, 128, True, None, True, 0x5EED0005),
             ("fwdbwd_B2_H16_N8192_d256_causal", 2, 16, 16, 8192, 256, True, None, True, 0x5EED0008)]
    for name, B, Hq, Hkv, N, d, causal, W, with_bwd, seed in cases:
        if not wanted(name):
            continue
        if with_bwd:
            q, k, v, dO = seedgen.attention_inputs(seed, B, Hq, Hkv, N, d, with_do=True)
        else:
            (q, k, v), dO = seedgen.attention_inputs(seed, B, Hq, Hkv, N, d), None
        qd, kd, vd = up(q), up(k), up(v)
        dod = up(dO) if with_bwd else None
        o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
        dq = torch.empty_like(o)
        dk = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev)
        dv = torch.empty_like(dk)
        wsb = fa2.fa2_backward_workspace_size(B, Hq, N)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        scale = 1.0 / math.sqrt(d)
        if W is None:
            fcall = lambda: check(fa2.fa2_forward(qd, kd, vd, o, lse, B, Hq, Hkv, N, d, causal, scale, stream), name)
            bcall = lambda: check(fa2.fa2_backward(qd, kd, vd, o, lse, dod, dq, dk, dv, B, Hq, Hkv, N, d, causal,
                                                   scale, ws, wsb, stream), name)
        else:
            fcall = lambda: check(fa2.fa2_forward_window(qd, kd, vd, o, lse, B, Hq, Hkv, N, d, W, scale, stream), name)
            bcall = lambda: check(fa2.fa2_backward_window(qd, kd, vd, o, lse, dod, dq, dk, dv, B, Hq, Hkv, N, d, W,
                                                          scale, ws, wsb, stream), name)
        calls = [fcall, bcall] if with_bwd else [fcall]
        spread, runs = {}, steps
        per, total = time_sequence(calls, runs, 2, stream, spread)
        if per[0] < 0.5:  # short launches: many more samples (at least 200)
            runs = max(200, steps)
            per, total = time_sequence(calls, runs, 5, stream, spread)
        pairs = B * Hq * visible_pairs(N, causal, W)
        fwd_bytes = (B * Hq + 2 * B * Hkv) * N * d * 2 + B * Hq * N * (d + 1) * 4
        r = {"B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "d": d, "causal": causal, "window": W,
             "fwd_ms": round(per[0], 4), "fwd_ms_min": round(spread["min"][0], 4),
             "fwd_ms_max": round(spread["max"][0], 4), "timed_runs": runs,
             "fwd_tflops": round(pairs * 4 * d / (per[0] * 1e-3) / 1e12, 1),
             "fwd_algorithmic_bytes": fwd_bytes, "fwd_GBps": round(fwd_bytes / (per[0] * 1e-3) / 1e9, 1)}
        if per[0] < 0.5:
            b2b = time_back_to_back(fcall, 50, 7, stream)
            r["fwd_ms_back_to_back"] = round(b2b, 4)
            r["fwd_tflops_back_to_back"] = round(pairs * 4 * d / (b2b * 1e-3) / 1e12, 1)
        if with_bwd:
            r["bwd_ms"] = round(per[1], 4)
            # forward 4 FLOP per visible pair and head-dim element, backward 2.5 times that
            r["fwd_bwd_tflops"] = round(pairs * 14 * d / (total * 1e-3) / 1e12, 1)
        out[name] = r
        log("  extra %-38s %s" % (name, r))
        del q, k, v, dO, qd, kd, vd, dod, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    if wanted("hbm_sweep_d64_noncausal"):
        hbm_sweep(fa2, seedgen, dev, stream, steps, out)
    if wanted("fp8_fwd_B2_H32_N8192_d128_causal"):
        fp8_forward(fa2, seedgen, dev, stream, steps, out)
    if wanted("decode_B8_Hq32_Hkv8_Nq1_Nk32768_d128"):
        decode(fa2, seedgen, dev, stream, steps, out)
    return out


def hbm_sweep(fa2, seedgen, dev, stream, steps, out):
    """Forward on short sequences with many heads (d=64, non-causal). Per (b, h) the pass does
    4*N^2*d FLOP over N*(3*2d + 4d + 4) compulsory bytes, about 0.4*N FLOP per byte: below the
    chip's ridge point (~315) for N <= 512, so these shapes are bound by HBM and are reported in
    GB/s of the compulsory bytes (Q, K, V read once; O and LSE written once)."""
    import numpy as np
    import torch

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    d, res = 64, {}
    for N in (128, 256, 512):
        for B, H in ((4, 256), (16, 256)):
            q, k, v = seedgen.attention_inputs(0x5EED0010 + N, B, H, H, N, d)
            qd, kd, vd = up(q), up(k), up(v)
            o = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

            def call():
                st = fa2.fa2_forward(qd, kd, vd, o, lse, B, H, H, N, d, False, 0.125, stream)
                if st != 0:
                    raise fa2.Fa2Error(st, "fa2_forward")

            per, total = time_sequence([call], max(20, steps), 3, stream)
            b2b = time_back_to_back(call, 50, 7, stream)
            nbytes = 3 * B * H * N * d * 2 + B * H * N * (d + 1) * 4
            flops = 4.0 * B * H * N * N * d
            res["BH%d_N%d" % (B * H, N)] = {
                "B": B, "H": H, "N": N, "d": d, "ms": round(total, 4), "algorithmic_bytes": nbytes,
                "GBps": round(nbytes / (total * 1e-3) / 1e9, 1),
                "hbm_frac": round(nbytes / (total * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "flop_per_byte": round(flops / nbytes, 1), "tflops": round(flops / (total * 1e-3) / 1e12, 1),
                "ms_back_to_back": round(b2b, 4), "GBps_back_to_back": round(nbytes / (b2b * 1e-3) / 1e9, 1)}
            del q, k, v, qd, kd, vd, o, lse
    out["hbm_sweep_d64_noncausal"] = res
    log("  extra %-38s %s" % ("hbm_sweep_d64_noncausal", {k: v["GBps"] for k, v in res.items()}))
    torch.cuda.empty_cache()


def peak_from_device(props):
    """Dense bf16 MFMA peak recomputed from the device: CUs x 4096 FLOP/clk x peak clock, with the
    clock read by hipDeviceGetAttribute(hipDeviceAttributeClockRate) from the HIP runtime this
    process has loaded. None if that runtime cannot be found."""
    import ctypes
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                path = line.split()[-1]
                break
    if path is None:
        return None
    hip = ctypes.CDLL(path)
    khz = ctypes.c_int(0)
    hip_device_attribute_clock_rate = 5  # peak clock in kHz
    if hip.hipDeviceGetAttribute(ctypes.byref(khz), hip_device_attribute_clock_rate, 0) != 0:
        return None
    return {"cus": props.multi_processor_count, "clock_mhz": khz.value / 1e3,
            "bf16_tflops": round(props.multi_processor_count * 4096 * khz.value * 1e3 / 1e12, 1)}


def fp8_forward(fa2, seedgen, dev, stream, steps, out):
    """FP8 forward at the headline shape (Q, K, V as E4M3FN codes, per-tensor scale 1/32)."""
    import torch

    def check(st, what):
        if st != 0:
            raise fa2.Fa2Error(st, what)

    B, Hq, Hkv, N, d = 2, 32, 32, 8192, 128
    q8, k8, v8 = (torch.from_numpy(x).to(dev) for x in seedgen.fp8_attention_inputs(0x5EED0006, B, Hq, Hkv, N, d))
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    wsb = fa2.fa2_forward_fp8_workspace_size(B, Hkv, N, d)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    sc = 1.0 / math.sqrt(d)
    call = lambda: check(fa2.fa2_forward_fp8(q8, k8, v8, 1 / 32, 1 / 32, 1 / 32, o, lse, B, Hq, Hkv, N, d, True, sc,
                                             ws, wsb, stream), "fa2_forward_fp8")
    per, total = time_sequence([call], steps, 2, stream)
    pairs = B * Hq * visible_pairs(N, True)
    r = {"B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "d": d, "causal": True, "fwd_ms": round(total, 4),
         "fwd_tflops": round(pairs * 4 * d / (total * 1e-3) / 1e12, 1),
         "note": "S = Q K^T on FP8 MFMA, P V in bf16 (V widened exactly); time includes the widening pass"}
    out["fp8_fwd_B2_H32_N8192_d128_causal"] = r
    log("  extra %-38s %s" % ("fp8_fwd_B2_H32_N8192_d128_causal", r))
    del q8, k8, v8, o, lse, ws


def decode(fa2, seedgen, dev, stream, steps, out):
    """Decode: one new token per sequence against a 32K-token cache (grouped-query heads). The
    pass streams K and V once, so it is reported against HBM bandwidth."""
    import numpy as np
    import torch

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    def check(st, what):
        if st != 0:
            raise fa2.Fa2Error(st, what)

    B, Hq, Hkv, Nq, Nk, d = 8, 32, 8, 1, 32768, 128
    q = seedgen.normal_bf16(0x5EED0007, seedgen.TENSOR_IDS["q"], (B, Hq, Nq, d))
    kc = seedgen.normal_bf16(0x5EED0007, seedgen.TENSOR_IDS["k"], (B, Hkv, Nk, d))
    vc = seedgen.normal_bf16(0x5EED0007, seedgen.TENSOR_IDS["v"], (B, Hkv, Nk, d))
    qd, kd, vd = up(q), up(kc), up(vc)
    o = torch.empty((B, Hq, Nq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    wsb = fa2.fa2_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(d)
    call = lambda: check(fa2.fa2_decode(qd, kd, vd, o, lse, B, Hq, Hkv, Nq, Nk, d, True, scale, ws, wsb, stream),
                         "fa2_decode")
    per, total = time_sequence([call], max(20, steps), 3, stream)
    nbytes = 2 * B * Hkv * Nk * d * 2 + B * Hq * Nq * d * (2 + 4) + B * Hq * Nq * 4
    b2b = time_back_to_back(call, 50, 7, stream)
    r = {"B": B, "Hq": Hq, "Hkv": Hkv, "Nq": Nq, "Nk": Nk, "d": d, "causal": True, "ms": round(total, 4),
         "algorithmic_bytes": nbytes, "GBps": round(nbytes / (total * 1e-3) / 1e9, 1),
         "hbm_frac": round(nbytes / (total * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
         "ms_back_to_back": round(b2b, 4), "GBps_back_to_back": round(nbytes / (b2b * 1e-3) / 1e9, 1)}
    out["decode_B8_Hq32_Hkv8_Nq1_Nk32768_d128"] = r
    log("  extra %-38s %s" % ("decode_B8_Hq32_Hkv8_Nq1_Nk32768_d128", r))


def clock_under_load(call, seconds=2.0, settle=0.8):
    """Median graphics clock (MHz) while ``call`` (one kernel launch) runs back to back for about
    ``seconds``, sampled every few ms from the driver's GPU metrics (amdsmi); samples from the
    first ``settle`` seconds are dropped (the metrics lag the load and the clock settles under
    the power limit). None when the metrics cannot be read. Runs outside every timed region."""
    import threading
    import numpy as np
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        handle = None
        props = torch.cuda.get_device_properties(torch.cuda.current_device())
        try:  # the handle of the device the kernels run on, by PCI address
            bdf = "%04x:%02x:%02x.0" % (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
            handle = amdsmi.amdsmi_get_processor_handle_from_bdf(bdf)
        except Exception:  # noqa: BLE001
            if len(handles) == 1:
                handle = handles[0]
        if handle is None:
            raise RuntimeError("cannot tell which of %d GPUs runs the kernels" % len(handles))
    except Exception as e:  # noqa: BLE001 - no metrics on this machine: report none
        log("clock sampling unavailable: %s" % e)
        return None

    def read():
        m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
        xs = m.get("current_gfxclks")
        if isinstance(xs, (list, tuple)):
            xs = [x for x in xs if isinstance(x, (int, float)) and 0 < x < 10000]
            if xs:
                return float(np.mean(xs))
        x = m.get("current_gfxclk")
        return float(x) if isinstance(x, (int, float)) and 0 < x < 10000 else None

    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                v = read()
            except Exception:  # noqa: BLE001
                v = None
            if v is not None and time.perf_counter() - t0 >= settle:
                samples.append(v)
            time.sleep(0.004)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            call()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:  # noqa: BLE001
        pass
    if len(samples) < 5:
        return None
    return {"median_mhz": round(float(np.median(samples)), 1), "p10_mhz": round(float(np.percentile(samples, 10)), 1),
            "p90_mhz": round(float(np.percentile(samples, 90)), 1), "samples": len(samples)}


# The five workloads (B, Hq, Hkv, N, d, causal, with backward, seed) and how the oracle covers each.
CONFIGS = [
    ("C1", 1, 2, 2, 256, 64, False, False, 0x5EED0001),
    ("C2", 4, 16, 16, 2048, 64, False, False, 0x5EED0002),
    ("C3", 2, 32, 32, 8192, 128, True, False, 0x5EED0003),
    ("C4", 1, 32, 8, 32768, 128, True, False, 0x5EED0004),
    ("C5", 4, 16, 16, 4096, 128, True, True, 0x5EED0005),
]


def oracle_per_config(gpu_ms):
    """The fp64 oracle timed on each workload, outside every GPU timing: C1 and C2 in full; C3 and C4
    on 256 sampled query rows of four heads; C5 (forward + backward) with the full-row statistics
    of two heads, 256 sampled query rows (dQ) and key rows (dK, dV) of those heads. Work is counted
    like the GPU's (4d FLOP per visible query/key pair forward; 10d fwd+bwd); sampled configs give
    an extrapolated full time at the sample's rate. ``gpu_ms``: config name -> GPU time of the same
    pass (forward, or forward + backward for C5), or absent."""
    import numpy as np

    import oracle
    import seedgen
    cores = oracle.default_threads()
    f64 = seedgen.bf16_bits_to_f64
    out = {}
    for name, B, Hq, Hkv, N, d, causal, bwd, seed in CONFIGS:
        scale = 1.0 / math.sqrt(d)
        full_flop = counted_fwd_flops(B, Hq, N, d, causal) * (3.5 if bwd else 1.0)
        r = {"B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "d": d, "causal": causal,
             "pass": "fwd+bwd" if bwd else "fwd", "counted_gflop_full": round(full_flop / 1e9, 2)}
        if name in ("C1", "C2"):
            q, k, v = (f64(x) for x in seedgen.attention_inputs(seed, B, Hq, Hkv, N, d))
            t0 = time.perf_counter()
            oracle.forward(q, k, v, causal, scale, threads=cores)
            el = time.perf_counter() - t0
            r.update({"mode": "full", "oracle_s": round(el, 4), "rows": B * Hq * N,
                      "rows_per_s": round(B * Hq * N / el, 1), "fp64_gflops": round(full_flop / el / 1e9, 2),
                      "full_s": round(el, 4), "full_s_kind": "measured"})
        else:
            heads = [0, Hq - 1] if name == "C5" else [0, Hq // 4, Hq // 2, Hq - 1]
            nrows = 256
            group = Hq // Hkv
            bits = seedgen.attention_inputs(seed, 1, Hq, Hkv, N, d, with_do=bwd)  # batch 0 only
            q, k, v = bits[:3]
            dO = bits[3] if bwd else None
            rows = seedgen.sample_rows_all(seed, len(heads), N, nrows)
            el, work, nr = 0.0, 0.0, 0
            for i, h in enumerate(heads):
                g = h // group
                qs, ks, vs = f64(q[:, h:h + 1]), f64(k[:, g:g + 1]), f64(v[:, g:g + 1])
                rr = rows[i:i + 1]
                if not bwd:
                    t0 = time.perf_counter()
                    oracle.forward(qs, ks, vs, causal, scale, rows=rr, threads=cores)
                    el += time.perf_counter() - t0
                    work += sum(4 * d * ((int(x) + 1) if causal else N) for x in rr[0])
                    nr += rr.shape[1]
                else:
                    ds = f64(dO[:, h:h + 1])
                    t0 = time.perf_counter()
                    stats = oracle.row_stats(qs, ks, vs, ds, causal, scale, threads=cores)
                    oracle.backward(qs, ks, vs, ds, causal, scale, qrows=rr, krows=rr, stats=stats, threads=cores)
                    el += time.perf_counter() - t0
                    # statistics: 4d per visible pair of the head; dQ rows 6d, dK/dV keys 8d per pair
                    work += 4 * d * visible_pairs(N, causal)
                    work += sum(6 * d * ((int(x) + 1) if causal else N) for x in rr[0])
                    work += sum(8 * d * ((N - int(x)) if causal else N) for x in rr[0])
                    nr += 2 * rr.shape[1]
            rate = work / el
            r.update({"mode": "sampled", "sample": "%d rows in each of %d heads (batch 0)%s" % (
                nrows, len(heads), "; full-row statistics of those heads, then dQ at the rows and dK/dV at the same key indices" if bwd else ""),
                "oracle_s": round(el, 4), "rows": nr, "rows_per_s": round(nr / el, 1),
                "fp64_gflops": round(rate / 1e9, 2), "full_s": round(full_flop / rate, 2),
                "full_s_kind": "extrapolated"})
        r["cores"] = cores
        if gpu_ms.get(name):
            r["gpu_ms"] = round(gpu_ms[name], 4)
            r["speedup_gpu_over_oracle"] = round(r["full_s"] / (gpu_ms[name] * 1e-3), 1)
        out[name] = r
        log("  oracle %s %s" % (name, r))
    return out


def cpu_baseline(q, k, v, dO, w, budget_s):
    """The fp64 oracle on a bounded sample: whole (b, h) heads of the workload, forward and
    backward in full, one head at a time until ``budget_s`` seconds have been spent."""
    import numpy as np

    import oracle
    import seedgen
    N, d, causal = w["N"], w["d"], w["causal"]
    scale = 1.0 / math.sqrt(d)
    cores = oracle.default_threads()
    f64 = seedgen.bf16_bits_to_f64
    done_heads, flops, elapsed = 0, 0.0, 0.0
    for h in range(w["B"] * w["Hq"]):
        b, hq = divmod(h, w["Hq"])
        g = hq // (w["Hq"] // w["Hkv"])
        qs, ks, vs, ds = (f64(x[b:b + 1, hh:hh + 1]) for x, hh in ((q, hq), (k, g), (v, g), (dO, hq)))
        t0 = time.perf_counter()
        oracle.forward(qs, ks, vs, causal, scale, threads=cores)
        oracle.backward(qs, ks, vs, ds, causal, scale, threads=cores)
        elapsed += time.perf_counter() - t0
        done_heads += 1
        flops += 3.5 * counted_fwd_flops(1, 1, N, d, causal)
        if elapsed >= budget_s:
            break
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d of %d (batch, head) slices of the workload, full fp64 forward + backward per slice "
                  "(%.1f s; input generation not timed)" % (done_heads, w["B"] * w["Hq"], elapsed),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the non-headline workloads")
    ap.add_argument("--only-extras", default=None, metavar="NAMES",
                    help="run only the non-headline workloads whose names contain one of these "
                         "comma-separated strings (no headline step); prints them as one JSON line")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-oracle-configs", action="store_true",
                    help="skip timing the oracle on each of the five workloads")
    ap.add_argument("--no-clock", action="store_true", help="skip sampling the GPU clock under load")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (5 times), for scaling "
                         "HBM byte counters; prints nothing")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the benchmark runs on exactly one GPU (heads would shard across GPUs with no exchange, not implemented here); --gpus %d (WORLD_SIZE=%d) is not supported"
              % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        return

    import exact_tiled_attention_fa2_amd as fa2
    import seedgen

    if not os.path.exists(fa2.LIB_PATH):
        from exact_tiled_attention_fa2_amd import build as hipbuild
        hipbuild.build()
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    if args.only_extras:
        only = [p for p in args.only_extras.split(",") if p]
        extras = extra_workloads(fa2, seedgen, dev, torch.cuda.current_stream(), max(5, args.steps), only)
        print(json.dumps({"extras": extras, "steps": max(5, args.steps)}), flush=True)
        return
    w = WORKLOAD
    B, Hq, Hkv, N, d, causal = w["B"], w["Hq"], w["Hkv"], w["N"], w["d"], w["causal"]
    scale = 1.0 / math.sqrt(d)

    q, k, v, dO = seedgen.attention_inputs(SEED, B, Hq, Hkv, N, d, with_do=True)

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    qd, kd, vd, dod = up(q), up(k), up(v), up(dO)
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    dq = torch.empty_like(o)
    dk = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    ws_bytes = fa2.fa2_backward_workspace_size(B, Hq, N)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    # The calls fa2_backward makes, one by one so that each kernel is timed: dQ with the
    # preprocess folded in (it leaves -D and LSE*log2(e) in the workspace), then dK/dV.
    names = ["fwd", "bwd_dq", "bwd_dkdv"]

    def step(events=None):
        calls = [
            lambda: fa2.fa2_forward(qd, kd, vd, o, lse, B, Hq, Hkv, N, d, causal, scale, stream),
            lambda: fa2.fa2_backward_dq_preprocess(qd, kd, vd, o, lse, dod, ws, ws_bytes, dq, B, Hq, Hkv, N, d,
                                                   causal, scale, stream),
            lambda: fa2.fa2_backward_dkdv(qd, kd, vd, dod, ws, ws_bytes, dk, dv, B, Hq, Hkv, N, d, causal, scale,
                                          stream),
        ]
        for i, call in enumerate(calls):
            if events is not None:
                events[i].record(stream)
            st = call()
            if st != 0:
                raise fa2.Fa2Error(st, names[i])
        if events is not None:
            events[len(calls)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    per_kernel = {n: [] for n in names}
    steps_ms = []
    for s in range(args.steps):
        for i, n in enumerate(names):
            per_kernel[n].append(ev[s][i].elapsed_time(ev[s][i + 1]))
        steps_ms.append(ev[s][0].elapsed_time(ev[s][len(names)]))
    avg = {n: float(np.mean(per_kernel[n])) for n in names}
    ms_step = float(np.mean(steps_ms))

    F = counted_fwd_flops(B, Hq, N, d, causal)
    total = 3.5 * F
    fwd_tflops = F / (avg["fwd"] * 1e-3) / 1e12
    bwd_ms = avg["bwd_dq"] + avg["bwd_dkdv"]
    value = total / (ms_step * 1e-3) / 1e12
    # Algorithmic work per launch: MFMA FLOPs over the visible (query, key) pairs counted as
    # B*H*N^2/2 when causal: forward 4d per pair, dK/dV 8d, dQ 6d (the preprocess folded into
    # the dQ kernel, D = rowsum(dO * O), adds 2d per row, not counted).
    pairs = B * Hq * N * N / (2 if causal else 1)
    algo = {"fwd": ("mfma", pairs * 4 * d / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS),
            "bwd_dkdv": ("mfma", pairs * 8 * d / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS),
            "bwd_dq": ("mfma", pairs * 6 * d / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS)}
    kernels = {}
    for n in names:
        bound, work, unit, peak = algo[n]
        ach = work / (avg[n] * 1e-3)
        kernels[n] = {"avg_ms": round(avg[n], 4), "median_ms": round(float(np.median(per_kernel[n])), 4),
                      "min_ms": round(float(np.min(per_kernel[n])), 4),
                      "max_ms": round(float(np.max(per_kernel[n])), 4),
                      "achieved": round(ach, 1), "unit": unit, "frac": round(ach / peak, 4)}
    dom = max(names, key=lambda n: avg[n])
    bound, work, unit, peak = algo[dom]
    achieved = work / (avg[dom] * 1e-3)
    roofline = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(dom), "kernel": dom}

    extras = None
    if not args.no_extras:
        extras = extra_workloads(fa2, seedgen, dev, stream, max(5, args.steps))

    # The graphics clock while each MFMA kernel runs alone back to back (after the timed region):
    # the MFMA fraction at that clock says how much of the gap to the nominal peak is clock.
    clocks = None
    if not args.no_clock:
        ck = {"fwd": lambda: fa2.fa2_forward(qd, kd, vd, o, lse, B, Hq, Hkv, N, d, causal, scale, stream),
              "bwd_dkdv": lambda: fa2.fa2_backward_dkdv(qd, kd, vd, dod, ws, ws_bytes, dk, dv, B, Hq, Hkv, N, d,
                                                        causal, scale, stream),
              "bwd_dq": lambda: fa2.fa2_backward_dq_preprocess(qd, kd, vd, o, lse, dod, ws, ws_bytes, dq, B, Hq,
                                                               Hkv, N, d, causal, scale, stream)}
        clocks = {}
        for n, call in ck.items():
            c = clock_under_load(call)
            if c is not None:
                c["mfma_frac_at_this_clock"] = round(kernels[n]["frac"] * 2400.0 / c["median_mhz"], 4)
                kernels[n]["clock_under_load"] = c
            clocks[n] = c
        log("clock under load (MHz): %s" % {n: (c or {}).get("median_mhz") for n, c in clocks.items()})

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(q, k, v, dO, w, args.cpu_seconds)

    oracle_configs = None
    if not args.no_oracle_configs:
        gms = {"C3": avg["fwd"]}
        if extras:
            for cname, key, field in (("C1", "fwd_B1_H2_N256_d64", "fwd_ms"), ("C2", "fwd_B4_H16_N2048_d64", "fwd_ms"),
                                      ("C4", "fwd_B1_Hq32_Hkv8_N32768_d128_causal", "fwd_ms")):
                if key in extras:
                    gms[cname] = extras[key][field]
            e5 = extras.get("fwdbwd_B4_H16_N4096_d128_causal")
            if e5:
                gms["C5"] = e5["fwd_ms"] + e5["bwd_ms"]
        oracle_configs = oracle_per_config(gms)

    props = torch.cuda.get_device_properties(0)
    peak_dev = peak_from_device(props)
    if peak_dev is not None:
        log("peak recomputed from the device: %d CUs x 4096 FLOP/clk x %.0f MHz = %.1f TFLOP/s bf16"
            % (peak_dev["cus"], peak_dev["clock_mhz"], peak_dev["bf16_tflops"]))
    log("device %s, %d CUs; step %.3f ms (wall %.3f ms); fwd %.3f ms = %.1f TFLOP/s (%.1f%% peak); "
        "bwd %.3f ms; fwd+bwd %.1f TFLOP/s (%.1f%%)" % (props.name, props.multi_processor_count, ms_step, wall_ms,
                                                     avg["fwd"], fwd_tflops, 100 * fwd_tflops / PEAK_BF16_TFLOPS,
                                                     bwd_ms, value, 100 * value / PEAK_BF16_TFLOPS))
    for n in names:
        log("  %-15s %8.3f ms  %9.1f %s  (%.1f%% of peak)" % (n, avg[n], kernels[n]["achieved"], kernels[n]["unit"],
                                                             100 * kernels[n]["frac"]))
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. N(0,1) rounded to bf16)",
        "config": {"workload": "causal prefill attention forward+backward, B=2 H=32 N=8192 d=128",
                   "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "d": d, "causal": causal,
                   "global_batch": B, "seq_len": N, "parallelism": "single GPU"},
        "fwd": {"ms": round(avg["fwd"], 4), "tflops": round(fwd_tflops, 1),
                "frac_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4)},
        "fwd_bwd": {"ms": round(ms_step, 4), "tflops": round(value, 1),
                    "frac_peak": round(value / PEAK_BF16_TFLOPS, 4)},
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "oracle_per_config": oracle_configs,
        "pages_context": PAGES_CONTEXT,
        "extras": extras,
        "peak_tflops": PEAK_BF16_TFLOPS,
        "peak_from_device": peak_dev,
        "device": props.name,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
