#!/usr/bin/env python3
"""Benchmark of the I2_S W2A8 decode matmul on one MI355X.

Workload: the 2B-class decode stack -- 30 layers x {q, k, v, o, gate, up,
down} ternary projections (q/o 2560x2560, k/v 640x2560, gate/up 6912x2560,
down 2560x6912; 521,011,200 packed bytes), one token (N=1) of bf16
activations per dependency group: q/k/v share one token, gate/up share one,
o and down each have their own, as in a decoder layer.  One step = for every
layer and group, one fused launch that quantises the bf16 token per token
(absmax int8) and runs the I2_S GEMV of every projection fed by it, writing
int32 dots and fp32 outputs (4 launches per layer, 120 per step, in
dependency order).  The packed weights (2x the 256 MB last-level cache) are
re-read from HBM every step.  The step is captured once in a HIP graph and
replayed.

Prints ONE JSON line.  ``value`` = algorithmic bytes per step / step time
(GB/s): packed weights + bf16 tokens + int32 and fp32 outputs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
# HBM bytes per launch of the fused GEMV, from rocprofv3 FETCH_SIZE (x2.0) and
# WRITE_SIZE (x1.0) scaled by a 256 MiB copy (profiles/gemv_b2_decode_hbm_traffic.md);
# valid only for the kernel sources with this sha256.
TRAFFIC = {"sources": ("ternary_weight_i2_amd/csrc/gemv_valu.h", "ternary_weight_i2_amd/csrc/gemv.hip",
                       "ternary_weight_i2_amd/csrc/common.h"),
           "sha256": "57260f25eb1e0a22878b80bb5c867736de8007d8e1f421c8ab142d8ccaad54ed",
           "bytes_per_launch": 4552192}
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, vendor figure
# MFMA busy fraction of the prefill GEMM launches (y only), from rocprofv3
# SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/8 x 1024 SIMDs)
# (profiles/gemm_e06_prefill_counters.md); valid only for these sources.  At
# N = 128 the dispatch length under counter collection is mostly the
# profiler's own per-dispatch cost, so those fractions are lower bounds.
GEMM_COUNTERS = {"sources": ("ternary_weight_i2_amd/csrc/gemm.hip", "ternary_weight_i2_amd/csrc/gemm_tiles.h",
                             "ternary_weight_i2_amd/csrc/common.h"),
                 "sha256": "d7fb04af8d7923951791ef3388bf461e7a49b5b5766616e45e8210ddc5a14c7b",
                 "mfma_busy": {4096: {"q/k/v": 0.238, "o": 0.157, "gate/up": 0.284, "down": 0.203},
                               128: {"q/k/v": 0.016, "o": 0.008, "gate/up": 0.024, "down": 0.012}}}
GROUPS = (("attn", ("q", "k", "v")), ("o", ("o",)), ("ffn", ("gate", "up")),
          ("down", ("down",)))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the secondary per-row measurements")
    ap.add_argument("--only", choices=("pack", "convert", "quant", "decode", "large", "prefill",
                                       "ffn", "lut"),
                    help="run only this group of secondary rows and print them (profiling aid)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy three times "
                         "(calibrates HBM byte counters) and exit")
    return ap.parse_args()


COPY_PROBE_BYTES = 256 << 20


def measured_traffic():
    """The recorded per-launch HBM bytes, or None once the kernel changed."""
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return TRAFFIC["bytes_per_launch"] if h.hexdigest() == TRAFFIC["sha256"] else None


def measured_mfma_busy(n_tokens=4096):
    """The recorded MFMA busy fractions of the prefill launches at this token
    count, or None once the GEMM sources changed."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_COUNTERS["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != GEMM_COUNTERS["sha256"]:
        return None
    return dict(GEMM_COUNTERS["mfma_busy"][n_tokens])


def copy_probe():
    """A plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for it
    calibrates the counters taken on the library kernels."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "repeats": 3}), flush=True)


def build_stack(bn, synth, torch, layers):
    stack = []
    for l in range(layers):
        layer = {"groups": []}
        for gname, projs in GROUPS:
            K = synth.SHAPES["b2"][projs[0]][1]
            x = synth.tokens_bf16_torch(1, K, synth.stack_seed("b2", l, projs[0], "act"))
            xq = torch.empty((1, K), dtype=torch.int8, device="cuda")
            xs = torch.empty((1,), dtype=torch.float32, device="cuda")
            xsum = torch.empty((1,), dtype=torch.int32, device="cuda")
            mats = []
            for p in projs:
                M, Kp = synth.SHAPES["b2"][p]
                assert Kp == K
                W = synth.ternary_torch(M, K, synth.stack_seed("b2", l, p, "weights"))
                P = bn.pack(W)
                del W
                alpha = synth.weight_scale(synth.rng_for("b2", l, p, "scale"))
                dot = torch.empty((1, M), dtype=torch.int32, device="cuda")
                y = torch.empty((1, M), dtype=torch.float32, device="cuda")
                mats.append((P, alpha, dot, y, M, K))
            layer["groups"].append((x, xq, xs, xsum, mats))
        stack.append(layer)
    return stack


def step_bytes(stack):
    """Algorithmic bytes of one step: every packed weight byte once, each bf16
    token once per group, int32 dot + fp32 y per output."""
    b = 0
    for layer in stack:
        for x, xq, xs, xsum, mats in layer["groups"]:
            N, K = x.shape
            b += N * K * 2
            for P, alpha, dot, y, M, K in mats:
                b += M * K // 4 + N * M * 8
    return b


def run_step(bn, stack):
    """The timed step: one fused quantise+GEMV launch per dependency group."""
    for layer in stack:
        for x, xq, xs, xsum, mats in layer["groups"]:
            bn.linear(x, [(m[0], m[1]) for m in mats], out=[(m[2], m[3]) for m in mats])


def run_step_unfused(bn, stack):
    """Same work through the separate calls (quantiser, then one GEMV per matrix)."""
    for layer in stack:
        for x, xq, xs, xsum, mats in layer["groups"]:
            bn.quant_act(x, out=(xq, xs, xsum))
            for P, alpha, dot, y, M, K in mats:
                bn.gemv(P, alpha, xq, xs, xsum, out=(dot, y))


def kernel_only(bn, torch, stack, step_bytes_total, launches, replays=5):
    """Each launch's own duration -- its first workgroup's start to its last
    wave's end, s_memrealtime stamps (100 MHz) recorded by the instrumented
    build of the same sources (libbitnet_i2s_stamps.so) -- over a few replays
    of the same captured step: no tracer serialises the launches and the
    gaps between them are left out.  None if that build is missing."""
    try:
        bn.use_library("stamps")
    except RuntimeError:
        return None
    try:
        bn.stamps_reset(rewind=True)
        g = capture(torch, lambda: run_step(bn, stack))   # warm call + capture take 2 x launches slots
        for _ in range(5):
            g.replay()
        dur, spans = [], []
        for _ in range(replays):
            bn.stamps_reset(rewind=False)
            g.replay()
            pairs = bn.stamps_read(2 * launches)[-launches:]
            dur += [(e - s) * 0.01 for s, e in pairs]
            spans.append((max(e for _, e in pairs) - min(s for s, _ in pairs)) * 0.01)
        del g
    finally:
        bn.use_library("main")
    dur.sort()
    mean = sum(dur) / len(dur)
    return {"mean_us": round(mean, 3), "p10_us": round(dur[len(dur) // 10], 2),
            "p50_us": round(dur[len(dur) // 2], 2), "p90_us": round(dur[len(dur) * 9 // 10], 2),
            "achieved_GBs": round(step_bytes_total / launches / (mean * 1e-6) / 1e9, 1),
            "step_span_us": round(sum(spans) / len(spans), 2), "launches": launches,
            "replays": replays,
            "method": "first-workgroup start to last-wave end per launch, s_memrealtime stamps "
                      "(10 ns ticks) from libbitnet_i2s_stamps.so, the same sources built with "
                      "-DBITNET_STAMPS; graph replays of the same step"}


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                       # warm the launch path outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps, warmup, min_warm_s=0.0):
    """Seconds for ``reps`` replays of ``g`` after ``warmup`` untimed ones
    (and, for the secondary rows, untimed replays until ``min_warm_s`` of
    wall time has passed, so a short graph after host-side set-up is not
    timed while the clocks ramp)."""
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_warm_s:
        for _ in range(10):
            g.replay()
        torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3      # seconds


def device_clock_mhz():
    """Peak shader clock the HIP runtime reports for device 0
    (hipDeviceGetAttribute with hipDeviceAttributeClockRate, entry 5 of the
    attribute enum, in kHz), or None where the runtime cannot be asked."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return None
    v = ctypes.c_int(0)
    return v.value / 1000.0 if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0 else None


def device_context(torch):
    """The device, and the read rate torch's own sum reaches on 1 GiB of fp32:
    a library read stream for context, not a ceiling (the large-layer GEMV
    row reads faster)."""
    props = torch.cuda.get_device_properties(0)
    clock_mhz = device_clock_mhz()
    x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    for _ in range(3):
        x.sum()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(10):
        x.sum()
    e1.record(st)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / 10
    del x
    return {"device": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "peak_clock_MHz": clock_mhz,
            "torch_sum_read_GBs": round((1 << 30) / t / 1e9, 1),
            "torch_sum_read_method": "torch sum over 1 GiB fp32, 10 reps"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(seconds):
    """The CPU oracle (as written) on a bounded sample: layer 0 of the same
    stack, drawn on the host, quantised and multiplied -- once with one
    thread per usable core (at most 16: the CPU share a one-GPU job gets on
    the GPU hosts), once with a single thread."""
    import numpy as np

    import oracle
    from ternary_weight_i2_amd import synth
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = max(1, min(16, usable))
    mats, toks = [], {}
    for gname, projs in GROUPS:
        K = synth.SHAPES["b2"][projs[0]][1]
        toks[gname] = synth.tokens_bf16(synth.rng_for("b2", 0, projs[0], "act"), 1, K)
        for p in projs:
            W, alpha = synth.matrix("b2", p, 0)
            P, _ = oracle.pack_i2s(W)
            mats.append((gname, P, alpha, W.shape[0], W.shape[1]))
    layer_bytes = sum(M * K // 4 + M * 8 for _, _, _, M, K in mats) + \
        sum(t.shape[1] * 2 + 8 for t in toks.values())

    def timed(nthreads, budget):
        done, t0 = 0, time.perf_counter()
        while True:
            qs = {g: oracle.quant_act(t) for g, t in toks.items()}
            for gname, P, alpha, M, K in mats:
                q, s, _ = qs[gname]
                oracle.linear_i2s(P, K, q, s, alpha, nthreads=nthreads)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return done, el

    done, el = timed(threads, seconds * 0.6)
    done1, el1 = timed(1, seconds * 0.4)
    per_layer_s = el / done
    return {"value": round(layer_bytes * done / el / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "value_1core": round(layer_bytes * done1 / el1 / 1e9, 4),
            "tokens_per_s": round(1.0 / (30 * per_layer_s), 3),
            "host_cores": os.cpu_count(), "usable_cores": usable, "cpu_model": cpu_model(),
            "sample": f"{done} pass(es) with {threads} threads and {done1} with 1 thread over "
                      f"layer 0 of the stack (7 projections, {layer_bytes} algorithmic bytes "
                      f"each): quantisation + unpack + definition dot + epilogue, "
                      f"{el:.1f} s + {el1:.1f} s; tokens_per_s scales one layer to 30"}


def _events_time(torch, fn, reps, warmup=3):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def secondary_rows(bn, synth, torch, stack, only=None):
    """One figure per other hot-path row, each timed with HIP events on the
    launch stream.  Shapes are the workloads' own; weights reuse the decode
    stack where the shapes match (so they stream from HBM), else are drawn
    fresh on the device.  ``only`` picks one group of rows."""
    rows = {}
    parts = {"pack": row_pack, "convert": row_convert, "quant": row_quant,
             "decode": row_decode, "large": row_large, "prefill": row_prefill,
             "ffn": row_ffn, "lut": row_lut}
    for name, fn in parts.items():
        if only is None or only == name:
            rows.update(fn(bn, synth, torch, stack))
    return rows


def row_pack(bn, synth, torch, stack):
    rows = {}
    # a1: pack (one-time step) -- 6912x2560 int8 -> I2_S
    M, K = synth.SHAPES["b2"]["gate"]
    W = synth.ternary_torch(M, K, 11)
    out = torch.empty((M, K // 4), dtype=torch.uint8, device="cuda")
    lib = bn.load()
    st = torch.cuda.current_stream().cuda_stream

    def do_pack():
        lib.bitnet_pack_i2s(W.data_ptr(), M, K, out.data_ptr(), st)
    t = _events_time(torch, do_pack, 10)
    rows["pack"] = {"shape": f"{M}x{K}", "us": round(t * 1e6, 2),
                    "GB/s": round((M * K + M * K // 4) / t / 1e9, 1),
                    "note": "includes the stream sync that reads the bad-value count"}
    del W, out
    return rows


def row_convert(bn, synth, torch, stack):
    """NEXT f2: one-time conversion of a 6912x2560 bf16 weight (2B-class gate)
    with the AbsMean ternariser, and of fp32 already-ternary weights with the
    sign/threshold packer.  Both synchronise (they return the scale on the
    host); the AbsMean call reads the weights twice (sum, then pack)."""
    rows = {}
    M, K = synth.SHAPES["b2"]["gate"]
    W = synth.tokens_bf16_torch(M, K, 21) * 0.02          # N(0, 0.02^2) bf16 weights
    t = _events_time(torch, lambda: bn.absmean_pack(W), 10)
    rows["absmean_pack"] = {"shape": f"{M}x{K} bf16", "us": round(t * 1e6, 2),
                            "GB/s": round((M * K * 2 + M * K // 4) / t / 1e9, 1),
                            "note": "two passes over the weights; includes the stream sync"}
    Wf = synth.ternary_torch(M, K, 22).float() * 0.05
    t = _events_time(torch, lambda: bn.pack_f32(Wf), 10)
    rows["pack_f32"] = {"shape": f"{M}x{K} fp32", "us": round(t * 1e6, 2),
                        "GB/s": round((M * K * 4 + M * K // 4) / t / 1e9, 1),
                        "note": "includes the stream sync"}
    return rows


def row_ffn(bn, synth, torch, stack):
    """NEXT f3: the 2B-class squared-ReLU gated FFN block per layer -- fused
    gate/up launch, the activation + sub-norm + quantise kernel, then down --
    over 30 layers (weights from HBM), N = 1 and 128 tokens."""
    rows = {}
    F, H = synth.SHAPES["b2"]["gate"]
    layers = []
    for l in range(30):
        mats = {}
        for p in ("gate", "up", "down"):
            M, K = synth.SHAPES["b2"][p]
            mats[p] = (bn.pack(synth.ternary_torch(M, K, synth.stack_seed("b2", l, p, "weights"))),
                       synth.weight_scale(synth.rng_for("b2", l, p, "scale")))
        gamma = torch.rand(F, device="cuda") + 0.5
        layers.append((mats, gamma))
    for N in (1, 128):
        x = synth.tokens_bf16_torch(N, H, 23 + N)
        bufs = []
        for mats, gamma in layers:
            gu = [(None, torch.empty((N, F), dtype=torch.float32, device="cuda")) for _ in range(2)]
            q = (torch.empty((N, F), dtype=torch.int8, device="cuda"),
                 torch.empty((N,), dtype=torch.float32, device="cuda"),
                 torch.empty((N,), dtype=torch.int32, device="cuda"))
            qx = (torch.empty((N, H), dtype=torch.int8, device="cuda"),
                  torch.empty((N,), dtype=torch.float32, device="cuda"),
                  torch.empty((N,), dtype=torch.int32, device="cuda"))
            out = (torch.empty((N, H), dtype=torch.int32, device="cuda"),
                   torch.empty((N, H), dtype=torch.float32, device="cuda"))
            bufs.append((mats, gamma, gu, q, qx, out))

        def run(bufs=bufs, N=N):
            for mats, gamma, gu, q, qx, out in bufs:
                bn.linear(x, [mats["gate"], mats["up"]], out=gu, qout=qx if N > 2 else None)
                bn.ffn_act_quant(gu[0][1], gu[1][1], gamma, 1e-5, out=q)
                P, a = mats["down"]
                if N <= 64:
                    bn.gemv(P, a, q[0], q[1], q[2], out=out)
                else:
                    bn.gemm(P, a, q[0], q[1], q[2], out=out)
        g = capture(torch, run)
        t = time_graph(torch, g, 10, 3, 0.02) / 10
        del g
        wbytes = sum(m[p][0].numel() for m, _ in layers for p in ("gate", "up", "down"))
        byts = wbytes + 30 * N * (2 * H + 2 * F * 4 + F * 4 + 2 * F + H * 8)
        rows[f"ffn_N{N}"] = {"workload": "2B-class FFN block (gate/up, sqrelu + sub-norm + quantise, down) x 30 layers",
                             "launches_per_step": 90, "us_per_step": round(t * 1e6, 1),
                             "GB/s": round(byts / t / 1e9, 1),
                             "hbm_frac": round(byts / t / 1e9 / HBM_PEAK_GBS, 4)}
        del bufs
    return rows


def row_quant(bn, synth, torch, stack):
    rows = {}
    # a2: quantisation of a 4096x1024 bf16 prefill block.  One launch moves
    # 12 MB, well under the launch overhead of an eager ctypes call, so the
    # launches are captured in a graph over 32 distinct input/output sets
    # (384 MB, more than the last-level cache holds) and the replays timed.
    N, K, sets = 4096, 1024, 32
    xs = [synth.tokens_bf16_torch(N, K, 12 + i) for i in range(sets)]
    outs = [(torch.empty((N, K), dtype=torch.int8, device="cuda"),
             torch.empty((N,), dtype=torch.float32, device="cuda"),
             torch.empty((N,), dtype=torch.int32, device="cuda")) for _ in range(sets)]

    def run():
        for x, o in zip(xs, outs):
            bn.quant_act(x, out=o)
    g = capture(torch, run)
    t = time_graph(torch, g, 20, 3, 0.05) / 20 / sets
    del g
    rows["quant"] = {"shape": f"{N}x{K} bf16", "launches": f"{sets} per graph replay",
                     "us": round(t * 1e6, 2),
                     "GB/s": round((N * K * 3 + N * 8) / t / 1e9, 1)}
    return rows


def row_decode(bn, synth, torch, stack):
    rows = {}
    # a4: batched decode on the 2B stack shapes, N = 4, 16, 64 (weights from HBM):
    # one launch per matrix, then one grouped launch per dependency group
    for N in (4, 16, 64):
        bufs = []
        for layer in stack:
            for xg, xq, xs, xsum, mats in layer["groups"]:
                K = xg.shape[1]
                xb = synth.tokens_bf16_torch(N, K, 13 + N)
                q = bn.quant_act(xb)
                for P, alpha, dot, y, M, _ in mats:
                    d = torch.empty((N, M), dtype=torch.int32, device="cuda")
                    yy = torch.empty((N, M), dtype=torch.float32, device="cuda")
                    bufs.append((P, alpha, q, d, yy, M, K))

        def run(bufs=bufs):
            for P, alpha, q, d, yy, M, K in bufs:
                bn.gemv(P, alpha, q[0], q[1], q[2], out=(d, yy))
        g = capture(torch, run)
        t = time_graph(torch, g, 10, 3, 0.02) / 10
        byts = sum(M * K // 4 + N * K + N * M * 8 for P, a, q, d, yy, M, K in bufs)
        ops = sum(2 * M * K * N for P, a, q, d, yy, M, K in bufs)
        rows[f"decode_N{N}"] = {"workload": "2B-class stack, 30 layers x 7 GEMVs",
                                "us_per_step": round(t * 1e6, 1),
                                "GB/s": round(byts / t / 1e9, 1),
                                "TOPS": round(ops / t / 1e12, 3),
                                "hbm_frac": round(byts / t / 1e9 / HBM_PEAK_GBS, 4)}
        del bufs, g
        groups = []
        for layer in stack:
            for xg, xq, xs, xsum, mats in layer["groups"]:
                K = xg.shape[1]
                q = bn.quant_act(synth.tokens_bf16_torch(N, K, 13 + N))
                ms = [(P, alpha) for P, alpha, dot, y, M, _ in mats]
                outs = [(torch.empty((N, M), dtype=torch.int32, device="cuda"),
                         torch.empty((N, M), dtype=torch.float32, device="cuda"))
                        for P, alpha, dot, y, M, _ in mats]
                groups.append((ms, q, outs, K))

        def run_g(groups=groups):
            for ms, q, outs, K in groups:
                bn.gemv_group(ms, q[0], q[1], q[2], out=outs)
        g = capture(torch, run_g)
        t = time_graph(torch, g, 10, 3, 0.02) / 10
        rows[f"decode_N{N}_grouped"] = {
            "workload": "2B-class stack, 30 layers x 4 grouped launches (q/k/v, o, gate/up, down)",
            "us_per_step": round(t * 1e6, 1), "GB/s": round(byts / t / 1e9, 1),
            "TOPS": round(ops / t / 1e12, 3),
            "hbm_frac": round(byts / t / 1e9 / HBM_PEAK_GBS, 4)}
        del groups, g
        # the same through bitnet_linear_i2s on bf16 tokens (the quantiser
        # included: fused into the GEMV for N <= 2, its own launch above)
        lin = []
        for layer in stack:
            for xg, xq, xs, xsum, mats in layer["groups"]:
                K = xg.shape[1]
                xb = synth.tokens_bf16_torch(N, K, 13 + N)
                q = bn.quant_act(xb)
                ms = [(P, alpha) for P, alpha, dot, y, M, _ in mats]
                outs = [(torch.empty((N, M), dtype=torch.int32, device="cuda"),
                         torch.empty((N, M), dtype=torch.float32, device="cuda"))
                        for P, alpha, dot, y, M, _ in mats]
                lin.append((xb, ms, outs, q))

        def run_l(lin=lin):
            for xb, ms, outs, q in lin:
                bn.linear(xb, ms, out=outs, qout=q if N > 2 else None)
        g = capture(torch, run_l)
        t = time_graph(torch, g, 10, 3, 0.02) / 10
        lbytes = byts + sum(N * xb.shape[1] for xb, ms, outs, q in lin)   # bf16 tokens: one more byte each
        rows[f"decode_N{N}_linear"] = {
            "workload": "2B-class stack, bf16 tokens, bitnet_linear_i2s per dependency group",
            "us_per_step": round(t * 1e6, 1), "GB/s": round(lbytes / t / 1e9, 1),
            "hbm_frac": round(lbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
        del lin, g
    return rows


def row_lut(bn, synth, torch, stack):
    """NEXT f4: the table-lookup decode matmul against the unpack GEMV on the
    same launches (one per matrix, int8 tokens, N = 1, weights from HBM): the
    2B-class stack (30 layers x 7 matrices) and eight 28672x8192 matrices of
    the large layer's gate shape (470 MB packed)."""
    rows = {}
    cases = []
    bufs = []
    for layer in stack:
        for xg, xq, xs, xsum, mats in layer["groups"]:
            K = xg.shape[1]
            q = bn.quant_act(synth.tokens_bf16_torch(1, K, 19 + K))
            for P, alpha, dot, y, M, _ in mats:
                bufs.append((P, alpha, q, dot, y, M, K))
    cases.append(("b2", "2B-class stack, 30 layers x 7 matrices, one launch each", bufs))
    M, K = synth.SHAPES["large"]["gate"]
    big = []
    q = bn.quant_act(synth.tokens_bf16_torch(1, K, 23))
    for l in range(8):
        W = synth.ternary_torch(M, K, synth.stack_seed("large", l, "gate", "weights"))
        P = bn.pack(W)
        del W
        big.append((P, 0.02, q, torch.empty((1, M), dtype=torch.int32, device="cuda"),
                    torch.empty((1, M), dtype=torch.float32, device="cuda"), M, K))
    cases.append(("large_gate", "8 x 28672x8192 matrices, one launch each", big))
    for tag, what, bufs in cases:
        byts = sum(M * K // 4 + K + M * 8 for P, a, q, d, yy, M, K in bufs)
        for how in ("lut", "unpack"):
            fn = bn.gemv_lut if how == "lut" else bn.gemv

            def run(bufs=bufs, fn=fn):
                for P, alpha, q, d, yy, M, K in bufs:
                    fn(P, alpha, q[0], q[1], q[2], out=(d, yy))
            g = capture(torch, run)
            t = time_graph(torch, g, 10, 3, 0.02) / 10
            del g
            rows[f"lut_{tag}_N1_{how}"] = {"workload": what, "us_per_step": round(t * 1e6, 1),
                                           "us_per_launch": round(t * 1e6 / len(bufs), 2),
                                           "GB/s": round(byts / t / 1e9, 1),
                                           "hbm_frac": round(byts / t / 1e9 / HBM_PEAK_GBS, 4)}
    del big
    return rows

def row_large(bn, synth, torch, stack):
    """a3 at streaming sizes: the large-layer stack (8 layers x 7 projections,
    1.71 GB packed, streamed from HBM every step).  N = 1: one grouped GEMV
    launch per dependency group (q/k/v, o, gate/up, down) on int8 tokens;
    also the fused quantise + GEMV on bf16 tokens and the per-matrix GEMV.
    N = 16: quantiser + batched decode per group (bitnet_linear_i2s)."""
    rows = {}
    layers = []
    for l in range(8):
        groups = []
        for _, projs in GROUPS:
            K = synth.SHAPES["large"][projs[0]][1]
            mats = []
            for p in projs:
                M, Kp = synth.SHAPES["large"][p]
                W = synth.ternary_torch(M, Kp, synth.stack_seed("large", l, p, "weights"))
                mats.append((bn.pack(W), synth.weight_scale(synth.rng_for("large", l, p, "scale"))))
                del W
            groups.append((K, mats))
        layers.append(groups)
    packed = sum(P.numel() for groups in layers for K, mats in groups for P, _ in mats)
    for N, how in ((1, "group"), (1, "linear"), (1, "gemv"), (16, "linear")):
        bufs = []
        for groups in layers:
            for K, mats in groups:
                x = synth.tokens_bf16_torch(N, K, 17 + K)
                q = bn.quant_act(x)
                outs = [(torch.empty((N, P.shape[0]), dtype=torch.int32, device="cuda"),
                         torch.empty((N, P.shape[0]), dtype=torch.float32, device="cuda"))
                        for P, _ in mats]
                qout = q if N > 2 else None
                bufs.append((x, q, mats, outs, qout))

        def run(bufs=bufs, how=how):
            for x, q, mats, outs, qout in bufs:
                if how == "linear":
                    bn.linear(x, mats, out=outs, qout=qout)
                elif how == "group":
                    bn.gemv_group(mats, q[0], q[1], q[2], out=outs)
                else:
                    for (P, a), o in zip(mats, outs):
                        bn.gemv(P, a, q[0], q[1], q[2], out=o)
        g = capture(torch, run)
        t = time_graph(torch, g, 5, 2, 0.02) / 5
        del g
        K_tok = sum(x.shape[1] for x, q, mats, outs, qout in bufs)
        M_out = sum(P.shape[0] for x, q, mats, outs, qout in bufs for P, _ in mats)
        tok_bytes = N * K_tok * (2 if how == "linear" else 1)
        byts = packed + tok_bytes + N * M_out * 8
        tag = f"large_N{N}" + ("" if how == "group" or N > 2 else
                               {"linear": "_fused_bf16", "gemv": "_per_matrix"}[how])
        rows[tag] = {"workload": "large layer stack, 8 layers x 7 projections, 1.71 GB packed",
                     "launches": {"group": "32 grouped GEMV, int8 tokens",
                                  "linear": ("32 fused quantise + GEMV, bf16 tokens" if N <= 2 else
                                             "32 x (quantiser + batched-decode GEMV), bf16 tokens"),
                                  "gemv": "56 GEMV, int8 tokens"}[how],
                     "us_per_step": round(t * 1e6, 1), "GB/s": round(byts / t / 1e9, 1),
                     "hbm_frac": round(byts / t / 1e9 / HBM_PEAK_GBS, 4),
                     "tokens_per_s": round(N / t, 1)}
        del bufs
    del layers
    return rows


def row_prefill(bn, synth, torch, stack):
    """a5: prefill GEMM on the 0.6B-class layer, N = 128 and 4096 tokens: one
    grouped launch per group of projections sharing their input (q/k/v, o,
    gate/up, down), tokens already quantised; plus the whole layer step through
    bitnet_linear_i2s (quantiser + grouped GEMM) and the per-matrix launches."""
    rows = {}
    groups = []
    for _, projs in GROUPS:
        K = synth.SHAPES["e06"][projs[0]][1]
        mats = []
        for p in projs:
            M, Kp = synth.SHAPES["e06"][p]
            W = synth.ternary_torch(M, Kp, synth.stack_seed("e06", 0, p, "weights"))
            mats.append((bn.pack(W), synth.weight_scale(synth.rng_for("e06", 0, p, "scale"))))
            del W
        groups.append((K, mats))
    for N in (128, 4096):
        xs = [synth.tokens_bf16_torch(N, K, 19 + K) for K, _ in groups]
        qs = [bn.quant_act(x) for x in xs]
        ops = sum(2 * P.shape[0] * K * N for K, mats in groups for P, _ in mats)
        variants = [("y", False, "group"), ("dot+y", True, "group"), ("y_linear", False, "linear")]
        if N == 4096:
            variants.append(("y_per_matrix", False, "single"))
        for tag, want_dot, how in variants:
            outs = [[(torch.empty((N, P.shape[0]), dtype=torch.int32, device="cuda") if want_dot else None,
                      torch.empty((N, P.shape[0]), dtype=torch.float32, device="cuda"))
                     for P, _ in mats] for K, mats in groups]

            def run(how=how, outs=outs):
                for (K, mats), x, q, o in zip(groups, xs, qs, outs):
                    if how == "group":
                        bn.gemm_group(mats, q[0], q[1], q[2], out=o)
                    elif how == "linear":
                        bn.linear(x, mats, out=o, qout=q)
                    else:
                        for (P, a), (d, y) in zip(mats, o):
                            bn.gemm(P, a, q[0], q[1], q[2], want_dot=d is not None, out=(d, y))
            g = capture(torch, run)
            t = time_graph(torch, g, 50, 10, 0.02) / 50   # short graphs: more replays
            del g
            rows[f"prefill_N{N}_{tag}"] = {
                "workload": "0.6B-class layer q/k/v/o/gate/up/down",
                "launches": {"group": "4 grouped GEMM", "linear": "4 x (quantise + grouped GEMM)",
                             "single": "7 GEMM"}[how],
                "us": round(t * 1e6, 1), "TOPS": round(ops / t / 1e12, 2),
                "mfma_frac": round(ops / t / 1e12 / INT8_PEAK_TOPS, 4)}
            if tag == "y" and how == "group":
                rows[f"prefill_N{N}_{tag}"]["mfma_busy_counters"] = measured_mfma_busy(N)
            del outs
    return rows


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
              "splitting the matrices across GPUs (by rows, or by K with an int32 "
              "all-reduce before the epilogue) is not implemented.", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_probe:
        torch.cuda.set_device(0)
        copy_probe()
        return

    import ternary_weight_i2_amd as bn
    from ternary_weight_i2_amd import synth
    bn.load()
    torch.cuda.set_device(0)

    if args.only:
        # one group of secondary rows alone (for profiling); not the bench line
        stack = build_stack(bn, synth, torch, args.layers) if args.only in ("decode", "lut") else None
        rows = secondary_rows(bn, synth, torch, stack, only=args.only)
        print(json.dumps({"only": args.only, "rows": rows}), flush=True)
        return

    stack = build_stack(bn, synth, torch, args.layers)
    torch.cuda.synchronize()
    sbytes = step_bytes(stack)

    g_step = capture(torch, lambda: run_step(bn, stack))
    el = time_graph(torch, g_step, args.steps, args.warmup)
    ms = el / args.steps * 1e3
    value = sbytes / (el / args.steps) / 1e9
    launches = len(stack) * len(GROUPS)
    # the dominant (and only) kernel of the step is the fused GEMV: its average
    # launch duration is the step time over its launches (HIP events on the
    # stream the graph runs on)
    per_launch_s = el / (args.steps * launches)
    achieved = sbytes / launches / per_launch_s / 1e9

    # spread: the same graph replayed one step at a time (each figure also
    # holds the graph's own launch latency)
    st = torch.cuda.current_stream()
    single = []
    for _ in range(max(20, min(args.steps, 100))):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        g_step.replay()
        e1.record(st)
        e1.synchronize()
        single.append(e0.elapsed_time(e1))
    single.sort()
    pct = {f"p{q}": round(single[int(q / 100 * (len(single) - 1))], 4) for q in (10, 50, 90)}
    context = device_context(torch)
    konly = kernel_only(bn, torch, stack, sbytes, launches)

    # context: the same work through the unfused calls, in a graph, and eager
    g_unf = capture(torch, lambda: run_step_unfused(bn, stack))
    unfused_ms = time_graph(torch, g_unf, args.steps, args.warmup) / args.steps * 1e3
    del g_unf
    run_step(bn, stack)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        run_step(bn, stack)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) / 5 * 1e3

    rows = None if args.no_rows else secondary_rows(bn, synth, torch, stack)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)

    out = {
        "metric": "I2_S W2A8 GEMV GB/s (% HBM peak) at bs1",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"2B-class decode stack: {args.layers} layers x "
                               "q/k/v/o/gate/up/down I2_S GEMVs, N=1, bf16 tokens",
                   "packed_bytes_per_step": sum(m[0].numel() for layer in stack
                                                for g in layer["groups"] for m in g[4]),
                   "algorithmic_bytes_per_step": sbytes,
                   "launches_per_step": launches,
                   "graph": True,
                   "eager_ms_per_step": round(eager_ms, 3),
                   "unfused_graph_ms_per_step": round(unfused_ms, 4)},
        "tokens_per_s": round(args.steps / el, 1),
        "roofline": {"bound": "hbm", "kernel": "gemv_valu_kernel<1,LPR,2,JM> (fused bf16 quantise + GEMV)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "avg_launch_us": round(per_launch_s * 1e6, 3),
                     "avg_launch_method": "step time / launches per step (HIP events on the "
                                          "replay stream; includes the gaps between launches)",
                     "kernel_only": konly},
        "cpu_baseline": cpu,
        "single_step_ms": pct,
        "context": context,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
