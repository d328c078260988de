"""Benchmark of the FP8 paged KV-cache path on one MI355X.

Headline workload: one decode step of a Llama-3-8B-shaped attention layer
(B=32 sequences, Hq=32, Hkv=8, dh=128, context lengths ~ U{512..8192}, cache
blocks of 16 tokens, per-tensor E4M3 scales = amax/448).  A step is what the
library does for that layer per generated token: quantize-write the new
token's K/V into the paged cache (kvq_cache_write) and run split-K paged
decode attention over the whole cached history (kvq_decode_attn).  The scales
are calibrated once over the prompt's K/V (kvq_calibrate_scales) before the
timed region, as a serving engine would.

Inputs are synthetic (seeded, see workloads.py) and already resident in HBM
when timing starts.  Each timed step reads a different one of several
identical cache copies, so the working set (> 1 GB) exceeds the 256 MB
Infinity Cache and the HBM figure is honest.

Printed: one JSON line with the headline metric, a roofline object for the
decode kernel (algorithmic KV bytes / average kernel time from HIP events on
the launch stream), the CPU oracle's throughput on a bounded sample, and the
other hot-path rows (calibration, full-context write, FP8 prefill) measured
on their own workloads after the timed loop.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense FP8 matrix peak


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--copies", type=int, default=4, help="cache copies rotated per step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-cpu-rows", action="store_true",
                   help="time only the headline decode sample on the CPU")
    p.add_argument("--no-rows", action="store_true", help="skip the extra per-row measurements")
    p.add_argument("--no-ragged", action="store_true",
                   help="skip the ragged prefill row (so a profile's prefill dispatches are "
                        "the equal-chunk batch only)")
    p.add_argument("--cpu-sample-rows", type=int, default=0,
                   help="(b, hq) rows in the CPU oracle sample (0 = all rows)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time of the oracle baseline (the sample is repeated)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="after the run, copy this many MiB device-to-device three times (a "
                        "plain copy kernel of known size, to calibrate HBM byte counters)")
    return p.parse_args()


# HBM bytes per decode call from rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by the
# counters' reading for a plain copy of known size; valid only for the decode
# source it was measured on.
TRAFFIC_SUMMARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "decode_llama3_8b_layer_hbm_traffic.md")
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quantized_kv_cache_fp8_amd",
                    "csrc")
# the sources the headline decode kernels are compiled from
DECODE_SRCS = ("decode.hip", "attn_common.hpp", "codec.hpp")


def decode_source_digest() -> str:
    """sha256 over the decode kernels' sources, in DECODE_SRCS order."""
    import hashlib
    h = hashlib.sha256()
    for name in DECODE_SRCS:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """traffic_bytes_per_call from the committed counter summary, or None when
    the summary is missing or was taken on a different decode source."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- `") and "`: " in line:
            k, v = line[3:].split("`: ", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("decode_source_sha256") != decode_source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    import quantized_kv_cache_fp8_amd as K
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def dt(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ------------------------------------------------------------ setup (untimed)
    wl = W.llama_layer_decode()
    B, Hq, Hkv, dh, bs = wl.B, wl.Hq, wl.Hkv, wl.dh, wl.bs
    cl = wl.paging.context_lens
    sum_ctx = int(cl.sum())
    max_ctx = int(cl.max())
    k_all, v_all = dt(wl.kv.k), dt(wl.kv.v)
    slots_all = dt(wl.kv.slot_mapping)
    q = dt(wl.q)
    bt = dt(wl.paging.block_tables)
    ctx = dt(cl)
    ks = torch.empty(1, device=dev)
    vs = torch.empty(1, device=dev)
    amax = torch.empty(1, device=dev)
    K.kvq_calibrate_scales(k_all, "fp8_e4m3", "tensor", amax, ks)
    K.kvq_calibrate_scales(v_all, "fp8_e4m3", "tensor", amax, vs)
    caches = []
    for _ in range(args.copies):
        # K tiles: 16-channel chunks, token-major inside a chunk
        kc = torch.empty((wl.paging.num_blocks, Hkv, dh // 16, bs, 16), dtype=torch.uint8,
                         device=dev)
        vc = torch.empty((wl.paging.num_blocks, Hkv, dh, bs), dtype=torch.uint8, device=dev)
        K.kvq_cache_write(k_all, v_all, slots_all, kc, vc, ks, vs, "fp8_e4m3", "tensor")
        caches.append((kc, vc))
    # the step's new token of every sequence: its last position (already in the
    # caches from the setup write; the step writes it again, as a decode step does)
    last = wl.kv.seq_offsets[1:] - 1
    k_new, v_new = k_all[torch.from_numpy(last).to(dev)], v_all[torch.from_numpy(last).to(dev)]
    k_new, v_new = k_new.contiguous(), v_new.contiguous()
    slot_new = slots_all[torch.from_numpy(last).to(dev)]
    out = torch.empty((B, Hq, dh), dtype=torch.float32, device=dev)
    ws_bytes = K.kvq_decode_workspace_size(B, Hq, dh, max_ctx, bs)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    # the setup's Python objects are collected now and frozen out of later
    # collections, so no full garbage-collector pass (tens of ms) lands inside
    # a timed loop of host launches
    gc.collect()
    gc.freeze()

    sh = stream.cuda_stream

    def step(i):
        # one decode step: quantize-write the new token and attend, in one kernel
        # launch (plus the split combine)
        kc, vc = caches[i % len(caches)]
        K.kvq_decode_attn_append(out, q, k_new, v_new, kc, vc, bt, ctx, max_ctx, ks, vs,
                                 "fp8_e4m3", "tensor", workspace=ws, stream=sh)

    kv_bytes = sum_ctx * Hkv * dh * 2  # FP8 K + V history read by one decode step

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # kernel time from HIP events on the launch stream around the timed region
    # (the step is the one append call: split kernel + combine), averaged per step
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    dec_ms = ev0.elapsed_time(ev1) / args.steps
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes / (dec_ms * 1e-3) / 1e9

    result = {
        "metric": "decode-attn KV GB/s & % of HBM peak (Llama-3-8B-shaped layer); prefill TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 cache, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "Hq": Hq, "Hkv": Hkv, "dh": dh,
                   "block_size": bs, "sum_context": sum_ctx, "max_context": max_ctx,
                   "kv_format": "e4m3", "scale": "per-tensor amax/448",
                   "step": "decode_attn_append (new token quantize-write + decode, one kernel)",
                   "cache_copies": args.copies,
                   "kv_bytes_per_step": kv_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "kvq_decode_attn_append (split + combine)",
                     "avg_ms": round(dec_ms, 5)},
    }

    # ------------------------------------------------------------ other rows (untimed loop)
    if not args.no_rows:
        result["rows"] = measure_rows(K, W, torch, dev, stream, k_all, v_all, slots_all, caches,
                                      ks, vs, wl, (q, bt, ctx, max_ctx, ws, out),
                                      ragged=not args.no_ragged)

        # the rows above left other formats in some cache copies: every copy
        # holds the E4M3 cache again, and the calls rotate over them so that
        # each decode reads from HBM (one copy alone would sit largely in the
        # 256 MB Infinity Cache)
        for kc, vc in caches:
            K.kvq_cache_write(k_all, v_all, slots_all, kc, vc, ks, vs, "fp8_e4m3", "tensor")

        def two_calls(i):
            kc, vc = caches[i % len(caches)]
            K.kvq_cache_write(k_new, v_new, slot_new, kc, vc, ks, vs, "fp8_e4m3", "tensor")
            K.kvq_decode_attn(out, q, kc, vc, bt, ctx, max_ctx, ks, vs, "fp8_e4m3", "tensor",
                              workspace=ws)
        ms = time_rotating(torch, stream, two_calls, 50)
        result["rows"]["step_write_then_decode"] = {
            "workload": wl.name + " (kvq_cache_write of the new tokens, then kvq_decode_attn)",
            "ms": round(ms, 5), "GB/s": round(kv_bytes / ms / 1e6, 1)}

    # ------------------------------------------------------------ copy probe (untimed)
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.full((n,), 7, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = n
        del src, dst

    # ------------------------------------------------------------ CPU oracle baseline
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample_rows, args.cpu_seconds,
                                              W=None if args.no_cpu_rows else W)

    print(json.dumps(result), flush=True)


def time_rotating(torch, stream, fn, reps, warm=5):
    """Mean time per call of fn(i), i = 0 .. reps - 1, between one pair of
    events on the launch stream (per-call event pairs would also count any host
    delay between an event and the launch that follows it)."""
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(reps):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def time_call(torch, stream, fn, reps, warmup=1):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def decode_row(K, torch, dev, stream, k_all, v_all, slots_all, caches, wl, dec, fmt, reps=50):
    """Decode attention of the headline layer with the cache in another format
    (the caches are rewritten); KV bytes per call / mean event time."""
    q, bt, ctx, max_ctx, ws, out = dec
    ks = torch.empty(1, device=dev)
    vs = torch.empty(1, device=dev)
    amax = torch.empty(1, device=dev)
    K.kvq_calibrate_scales(k_all, fmt, "tensor", amax, ks)
    K.kvq_calibrate_scales(v_all, fmt, "tensor", amax, vs)
    for kc, vc in caches:
        K.kvq_cache_write(k_all, v_all, slots_all, kc, vc, ks, vs, fmt, "tensor")
    def call(i):
        kc, vc = caches[i % len(caches)]
        K.kvq_decode_attn(out, q, kc, vc, bt, ctx, max_ctx, ks, vs, fmt, "tensor", workspace=ws)
    ms = time_rotating(torch, stream, call, reps)
    kv_bytes = int(wl.paging.context_lens.sum()) * wl.Hkv * wl.dh * 2
    gbs = kv_bytes / ms / 1e6
    return {"workload": wl.name + f" ({fmt} cache, per-tensor scale)", "ms": round(ms, 5),
            "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def token_scale_rows(K, torch, dev, stream, k_all, v_all, slots_all, caches, wl, dec, reps=50):
    """Per-token-head fp16 scales (textbook 10.4.3): the full-context write that
    derives them, and decode of the headline layer over that cache; bytes count
    codes plus the 2-byte scales."""
    q, bt, ctx, max_ctx, ws, out = dec
    T = k_all.shape[0]
    nb = caches[0][0].shape[0]
    scs = [(torch.empty((nb, wl.Hkv, wl.bs), dtype=torch.int16, device=dev),
            torch.empty((nb, wl.Hkv, wl.bs), dtype=torch.int16, device=dev)) for _ in caches]
    rows = {}
    kc, vc = caches[0]
    ksc, vsc = scs[0]

    def write():
        K.kvq_cache_write_token_scales(k_all, v_all, slots_all, kc, vc, ksc, vsc, "fp8_e4m3")
    ms = time_call(torch, stream, write, 10)
    nbytes = T * (wl.Hkv * wl.dh * 2 * 2 + wl.Hkv * wl.dh * 2 + wl.Hkv * 4 + 8)
    rows["cache_write_token_scales"] = {"workload": wl.name + " full context, e4m3",
                                        "ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1)}
    for (kc, vc), (ksc, vsc) in zip(caches, scs):
        K.kvq_cache_write_token_scales(k_all, v_all, slots_all, kc, vc, ksc, vsc, "fp8_e4m3")
    def call(i):
        (kc, vc), (ksc, vsc) = caches[i % len(caches)], scs[i % len(caches)]
        K.kvq_decode_attn_token_scales(out, q, kc, vc, ksc, vsc, bt, ctx, max_ctx, "fp8_e4m3",
                                       workspace=ws)
    ms = time_rotating(torch, stream, call, reps)
    kv_bytes = int(wl.paging.context_lens.sum()) * wl.Hkv * (wl.dh * 2 + 4)
    gbs = kv_bytes / ms / 1e6
    rows["decode_token_scales"] = {"workload": wl.name + " (e4m3 cache, fp16 per-token-head "
                                   "scales)", "ms": round(ms, 5), "GB/s": round(gbs, 1),
                                   "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    return rows


def kivi_rows(K, W, torch, dev, stream, reps=50):
    """KIVI-style 2-bit cache (textbook 10.4.4): quantize of every full group and
    decode over it plus the bf16 residual, on B=8, Hq=32, Hkv=8, S=16384."""
    kw = W.kivi_2bit_decode()

    def dt(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    k, v, gb = dt(kw.k), dt(kw.v), dt(kw.group_blocks)
    nb = kw.paging.num_blocks
    # copies of the cache in rotation so no call reads another's data from L2 / MALL
    # (6 x 104 MB: well past the 256 MB MALL, so every call reads from HBM)
    caches = [torch.empty((nb, kw.Hkv, K.KIVI_TILE), dtype=torch.uint8, device=dev)
              for _ in range(6)]
    rows = {}

    def quant():
        K.kvq_kivi_quantize(k, v, gb, caches[0])
    ms = time_call(torch, stream, quant, 10)
    ng = len(kw.group_blocks)
    nbytes = ng * 32 * kw.Hkv * 128 * 2 * 2 + ng * kw.Hkv * K.KIVI_TILE + ng * 4
    rows["kivi_quantize"] = {"workload": kw.name + " all full groups", "ms": round(ms, 4),
                             "GB/s": round(nbytes / ms / 1e6, 1)}
    for c in caches[1:]:
        K.kvq_kivi_quantize(k, v, gb, c)
    q, bt, qg, rk, rv, rl = (dt(kw.q), dt(kw.paging.block_tables), dt(kw.quant_groups),
                             dt(kw.res_k), dt(kw.res_v), dt(kw.res_lens))
    mg = int(kw.quant_groups.max())
    out = torch.empty((kw.B, kw.Hq, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(K.kvq_kivi_decode_workspace_size(kw.B, kw.Hq, kw.Hkv, mg), dtype=torch.uint8,
                     device=dev)
    def call(i):
        K.kvq_kivi_decode_attn(out, q, caches[i % len(caches)], bt, qg, mg, rk, rv, rl,
                               workspace=ws)
    ms = time_rotating(torch, stream, call, 2 * reps, warm=20)
    # algorithmic bytes: every quantized tile once, the residual once
    nbytes = (int(kw.quant_groups.sum()) * kw.Hkv * K.KIVI_TILE +
              int(kw.res_lens.sum()) * kw.Hkv * 128 * 2 * 2)
    gbs = nbytes / ms / 1e6
    rows["kivi_decode"] = {"workload": kw.name, "ms": round(ms, 5), "bytes": nbytes,
                           "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    return rows


def long_context_rows(K, W, torch, dev, stream, steps=200, copies=4):
    """Long-context decode with per-head scales: B=4, S=32768, Hq=32, Hkv=8,
    dh=128, k/v scales [8] from per-head amax; the append step (new token's
    quantize-write + attention) as for the headline layer, once with an E4M3
    and once with an E5M2 cache.  Bytes per step: the FP8 K+V history,
    4 x 32768 x 8 x 128 x 2 = 268,435,456."""
    import dataclasses
    base = W.long_context_decode("e4m3")

    def dt(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    k_all, v_all, slots = dt(base.kv.k), dt(base.kv.v), dt(base.kv.slot_mapping)
    q, bt, ctx = dt(base.q), dt(base.paging.block_tables), dt(base.paging.context_lens)
    B, Hq, Hkv, dh, bs = base.B, base.Hq, base.Hkv, base.dh, base.bs
    max_ctx = int(base.paging.context_lens.max())
    last = torch.from_numpy(base.kv.seq_offsets[1:] - 1).to(dev)
    k_new, v_new = k_all[last].contiguous(), v_all[last].contiguous()
    nb = base.paging.num_blocks
    kcs = [torch.empty((nb, Hkv, dh // 16, bs, 16), dtype=torch.uint8, device=dev)
           for _ in range(copies)]
    vcs = [torch.empty((nb, Hkv, dh, bs), dtype=torch.uint8, device=dev) for _ in range(copies)]
    out = torch.empty((B, Hq, dh), dtype=torch.float32, device=dev)
    ws = torch.empty(max(K.kvq_decode_workspace_size(B, Hq, dh, max_ctx, bs), 16),
                     dtype=torch.uint8, device=dev)
    kv_bytes = int(base.paging.context_lens.sum()) * Hkv * dh * 2
    rows = {}
    for fmt in ("e4m3", "e5m2"):
        wl = dataclasses.replace(base, name=f"long-context-decode-b{B}-s{max_ctx}-{fmt}", fmt=fmt)
        ks = torch.empty(Hkv, device=dev)
        vs = torch.empty(Hkv, device=dev)
        am = torch.empty(Hkv, device=dev)
        K.kvq_calibrate_scales(k_all, fmt, "head", am, ks)
        K.kvq_calibrate_scales(v_all, fmt, "head", am, vs)
        for kc, vc in zip(kcs, vcs):
            K.kvq_cache_write(k_all, v_all, slots, kc, vc, ks, vs, fmt, "head")

        def call(i):
            K.kvq_decode_attn_append(out, q, k_new, v_new, kcs[i % copies], vcs[i % copies], bt,
                                     ctx, max_ctx, ks, vs, fmt, "head", workspace=ws)
        ms = time_rotating(torch, stream, call, steps, warm=10)
        gbs = kv_bytes / ms / 1e6
        rows[f"decode_long_{fmt}"] = {
            "workload": wl.name + " (per-head k/v scales [8], append step)",
            "ms": round(ms, 5), "bytes": kv_bytes, "GB/s": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    del kcs, vcs
    return rows


def tiny_row(K, W, torch, dev, stream, reps=200):
    """The tiny decode configuration (B=1, Hq=4, Hkv=2, dh=64, context 256 in 16
    shuffled blocks, scale 1.0, E4M3): quantize-write of the 256 tokens then one
    decode step, per call; latency-bound (64 KiB of cache)."""
    wl = W.tiny_decode()

    def dt(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    k, v, slots = dt(wl.kv.k), dt(wl.kv.v), dt(wl.kv.slot_mapping)
    q, bt, ctx = dt(wl.q), dt(wl.paging.block_tables), dt(wl.paging.context_lens)
    nb = wl.paging.num_blocks
    kc = torch.empty((nb, wl.Hkv, wl.dh // 16, wl.bs, 16), dtype=torch.uint8, device=dev)
    vc = torch.empty((nb, wl.Hkv, wl.dh, wl.bs), dtype=torch.uint8, device=dev)
    one = torch.ones(1, device=dev)
    out = torch.empty((wl.B, wl.Hq, wl.dh), device=dev)
    mc = int(wl.paging.context_lens.max())
    ws = torch.empty(max(K.kvq_decode_workspace_size(wl.B, wl.Hq, wl.dh, mc, wl.bs), 16),
                     dtype=torch.uint8, device=dev)

    def call():
        K.kvq_cache_write(k, v, slots, kc, vc, one, one, "fp8_e4m3", "tensor")
        K.kvq_decode_attn(out, q, kc, vc, bt, ctx, mc, one, one, "fp8_e4m3", "tensor",
                          workspace=ws)
    ms = time_call(torch, stream, call, reps)
    # the same two calls captured once in a HIP graph and replayed: the
    # kernels' own latency, without the binding's per-call host work
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    out.fill_(float("nan"))
    ms_graph = time_call(torch, stream, g.replay, reps)
    return {"workload": wl.name + " (kvq_cache_write of 256 tokens, then kvq_decode_attn)",
            "us": round(ms * 1e3, 2), "us_graph_replay": round(ms_graph * 1e3, 2),
            "graph_replay_matches_eager": bool(torch.equal(out, eager))}


def measure_rows(K, W, torch, dev, stream, k_all, v_all, slots_all, caches, ks, vs, wl, dec,
                 ragged=True):
    rows = {}
    rows["tiny_write_then_decode"] = tiny_row(K, W, torch, dev, stream)
    rows.update(long_context_rows(K, W, torch, dev, stream))
    rows.update(kivi_rows(K, W, torch, dev, stream))
    rows.update(token_scale_rows(K, torch, dev, stream, k_all, v_all, slots_all, caches, wl,
                                 dec))
    # the same decode with a symmetric INT8 cache (textbook 10.4.2 write rule)
    rows["decode_int8"] = decode_row(K, torch, dev, stream, k_all, v_all, slots_all, caches, wl,
                                     dec, "int8")
    T = k_all.shape[0]
    amax = torch.empty(1, device=dev)
    sc = torch.empty(1, device=dev)

    amax2 = torch.empty(1, device=dev)
    sc2 = torch.empty(1, device=dev)

    def calib():  # K and V together: three launches
        K.kvq_calibrate_scales_kv(k_all, v_all, "fp8_e4m3", "tensor", amax, amax2, sc, sc2)
    ms = time_call(torch, stream, calib, 10)
    nbytes = 2 * T * wl.Hkv * wl.dh * 2
    rows["calibrate"] = {"workload": wl.name + " K+V per-tensor (one kvq_calibrate_scales_kv call)",
                         "ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                         "frac_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}

    def calib_one():  # one tensor per call: three launches each
        K.kvq_calibrate_scales(k_all, "fp8_e4m3", "tensor", amax, sc)
    ms = time_call(torch, stream, calib_one, 10)
    rows["calibrate_single"] = {"workload": wl.name + " K per-tensor (one kvq_calibrate_scales call)",
                                "ms": round(ms, 4), "GB/s": round(nbytes / 2 / ms / 1e6, 1)}
    kc, vc = caches[0]

    def write():
        K.kvq_cache_write(k_all, v_all, slots_all, kc, vc, ks, vs, "fp8_e4m3", "tensor")
    ms = time_call(torch, stream, write, 10)
    nbytes = T * (wl.Hkv * wl.dh * 2 * 2 + wl.Hkv * wl.dh * 2 + 8)
    rows["cache_write"] = {"workload": wl.name + " full context", "ms": round(ms, 4),
                           "GB/s": round(nbytes / ms / 1e6, 1)}
    del kc, vc
    # FP8-domain causal chunked prefill: 8 x (4096 cached + 4096 new), per-head
    # scales; and a ragged batch of the same head shape (chunk = prefix, 256 to
    # 4096 tokens), where work per sequence differs 16-fold
    def dt(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def prefill_case(pw):
        q = dt(pw.q)
        pk, pv = dt(pw.kv.k), dt(pw.kv.v)
        qs = torch.empty(pw.Hq, device=dev)
        pks = torch.empty(pw.Hkv, device=dev)
        pvs = torch.empty(pw.Hkv, device=dev)
        am = torch.empty(pw.Hq, device=dev)
        K.kvq_calibrate_scales(q, "fp8_e4m3", "head", am, qs)
        K.kvq_calibrate_scales(pk, "fp8_e4m3", "head", am[:pw.Hkv], pks)
        K.kvq_calibrate_scales(pv, "fp8_e4m3", "head", am[:pw.Hkv], pvs)
        pkc = torch.empty((pw.paging.num_blocks, pw.Hkv, pw.dh // 16, pw.bs, 16),
                          dtype=torch.uint8, device=dev)
        pvc = torch.empty((pw.paging.num_blocks, pw.Hkv, pw.dh, pw.bs), dtype=torch.uint8,
                          device=dev)
        K.kvq_cache_write(pk, pv, dt(pw.kv.slot_mapping), pkc, pvc, pks, pvs, "fp8_e4m3", "head")
        out = torch.empty((q.shape[0], pw.Hq, pw.dh), dtype=torch.float32, device=dev)
        cu, bt, cl = dt(pw.cu_seqlens), dt(pw.paging.block_tables), dt(pw.paging.context_lens)
        max_q = int(np.diff(pw.cu_seqlens).max())

        def prefill():
            K.kvq_prefill_attn(out, q, cu, max_q, qs, "head", pkc, pvc, bt, cl, pks, pvs,
                               "fp8_e4m3", "head")
        # the first few calls of a fresh 3 ms kernel run measurably slower
        # (about 15 %); the row reports the steady state
        ms = time_call(torch, stream, prefill, 10, warmup=5)
        flops = 0
        for b in range(len(pw.prefix_lens)):
            P, C = int(pw.prefix_lens[b]), int(pw.cu_seqlens[b + 1] - pw.cu_seqlens[b])
            flops += 4 * pw.dh * pw.Hq * (C * P + C * (C + 1) // 2)
        tf = flops / (ms * 1e-3) / 1e12
        return {"workload": pw.name, "ms": round(ms, 4),
                "algorithmic_TFLOP": round(flops / 1e12, 4), "TFLOP/s": round(tf, 1),
                "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)}

    rows["prefill"] = prefill_case(W.fp8_chunked_prefill())
    if ragged:
        rows["prefill_ragged"] = prefill_case(W.ragged_chunked_prefill())
    return rows


def host_info():
    """Threads the oracle runs with, the host's logical CPUs and its CPU model."""
    import oracle
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return oracle.num_threads(), nproc, model


def timed(fn, min_seconds=0.0):
    """(seconds per call, calls): fn repeated until min_seconds have passed (once at least)."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        t = time.perf_counter() - t0
        if t >= min_seconds:
            return t / n, n


def cpu_baseline(wl, sample_rows, min_seconds, W=None):
    """The fp64 oracle on the host.  The headline figure: decode attention of
    the Llama-shaped layer over a bounded sample of (sequence, head) rows,
    repeated until at least min_seconds of work have been timed.  `rows`: the
    oracle's calibrate, write and decode of the tiny and long-context
    workloads and of the same layer, and FP8 prefill on a seeded subset of
    (sequence, head) pairs scaled by pair count, each with the algorithmic
    bytes or flops of the GPU rows."""
    import oracle
    fmt, gran = oracle.FMT_E4M3, oracle.GRAN_TENSOR
    threads, nproc, model = host_info()
    ks = oracle.calibrate(wl.kv.k, fmt, gran)[1]
    vs = oracle.calibrate(wl.kv.v, fmt, gran)[1]
    kc = np.zeros(oracle.k_cache_shape(wl.paging.num_blocks, wl.Hkv, wl.bs, wl.dh), np.uint8)
    vc = np.zeros((wl.paging.num_blocks, wl.Hkv, wl.dh, wl.bs), np.uint8)
    oracle.cache_write(wl.kv.k, wl.kv.v, wl.kv.slot_mapping, kc, vc, ks, vs, fmt, gran)
    rows = np.array([(b, h) for b in range(wl.B) for h in range(wl.Hq)], np.int32)
    if sample_rows:
        rows = rows[np.random.Generator(np.random.PCG64(5)).permutation(len(rows))[:sample_rows]]
    cl = wl.paging.context_lens
    t, reps = timed(lambda: oracle.decode_rows(rows, wl.q, kc, vc, wl.paging.block_tables, cl,
                                               ks, vs, fmt, gran), min_seconds)
    # bytes of the FP8 history the sampled rows read (each row reads its sequence's K and V)
    G = wl.Hq // wl.Hkv
    kv_bytes = float(sum(int(cl[b]) for b, _ in rows)) * wl.dh * 2 / G
    res = {"value": round(kv_bytes / t / 1e9, 4), "unit": "GB/s", "cores": threads,
           "kind": "oracle", "nproc": nproc, "cpu_model": model,
           "seconds": round(t * reps, 3), "repeats": reps,
           "sample": f"decode attention of {len(rows)} of {wl.B * wl.Hq} (sequence, head) rows "
                     f"of the same layer, repeated {reps} times; fp64, OpenMP over rows with "
                     f"{threads} threads; bytes counted as the FP8 K+V history those rows read "
                     f"(shared by the {G} heads of a group)"}
    if W is not None:
        res["rows"] = cpu_rows(oracle, W, wl, kc, vc, ks, vs)
    return res


def cpu_rows(oracle, W, wl, kc, vc, ks, vs):
    """Oracle timings of calibrate, write and decode per workload (one pass
    each, at the GPU rows' algorithmic bytes) and of prefill on a subset."""
    out = {}

    def rec(name, secs, nbytes=None, flops=None, note=None):
        r = {"seconds": round(secs, 4)}
        if nbytes is not None:
            r["GB/s"] = round(nbytes / secs / 1e9, 4)
        if flops is not None:
            r["TFLOP/s"] = round(flops / secs / 1e12, 6)
        if note:
            r["sample"] = note
        out[name] = r

    # the tiny decode (scale 1.0): write of 256 tokens, one decode step
    tw = W.tiny_decode()
    s1 = np.ones(1, np.float32)
    tkc = np.zeros(oracle.k_cache_shape(tw.paging.num_blocks, tw.Hkv, tw.bs, tw.dh), np.uint8)
    tvc = np.zeros((tw.paging.num_blocks, tw.Hkv, tw.dh, tw.bs), np.uint8)
    t, n = timed(lambda: (oracle.cache_write(tw.kv.k, tw.kv.v, tw.kv.slot_mapping, tkc, tvc, s1,
                                             s1, 0, 0),
                          oracle.decode_attn(tw.q, tkc, tvc, tw.paging.block_tables,
                                             tw.paging.context_lens, s1, s1, 0, 0)), 1.0)
    out["tiny_write_then_decode"] = {"us": round(t * 1e6, 2), "repeats": n}
    # the Llama-shaped layer: calibrate K+V, full-context write, one decode step (every row)
    T = wl.kv.k.shape[0]
    fmt, gran = oracle.FMT_E4M3, oracle.GRAN_TENSOR
    t, _ = timed(lambda: (oracle.calibrate(wl.kv.k, fmt, gran), oracle.calibrate(wl.kv.v, fmt, gran)))
    rec("calibrate", t, 2 * T * wl.Hkv * wl.dh * 2)
    t, _ = timed(lambda: oracle.cache_write(wl.kv.k, wl.kv.v, wl.kv.slot_mapping, kc, vc, ks, vs,
                                            fmt, gran))
    rec("cache_write", t, T * (wl.Hkv * wl.dh * 2 * 2 + wl.Hkv * wl.dh * 2 + 8))
    t, _ = timed(lambda: oracle.decode_attn(wl.q, kc, vc, wl.paging.block_tables,
                                            wl.paging.context_lens, ks, vs, fmt, gran))
    rec("decode", t, T * wl.Hkv * wl.dh * 2)
    # long context, per-head scales, E4M3: calibrate, write, decode
    lw = W.long_context_decode("e4m3")
    gh = oracle.GRAN_HEAD
    LT = lw.kv.k.shape[0]
    t, _ = timed(lambda: (oracle.calibrate(lw.kv.k, fmt, gh), oracle.calibrate(lw.kv.v, fmt, gh)))
    rec("calibrate_long_e4m3", t, 2 * LT * lw.Hkv * lw.dh * 2)
    lks = oracle.calibrate(lw.kv.k, fmt, gh)[1]
    lvs = oracle.calibrate(lw.kv.v, fmt, gh)[1]
    lkc = np.zeros(oracle.k_cache_shape(lw.paging.num_blocks, lw.Hkv, lw.bs, lw.dh), np.uint8)
    lvc = np.zeros((lw.paging.num_blocks, lw.Hkv, lw.dh, lw.bs), np.uint8)
    t, _ = timed(lambda: oracle.cache_write(lw.kv.k, lw.kv.v, lw.kv.slot_mapping, lkc, lvc, lks,
                                            lvs, fmt, gh))
    rec("cache_write_long_e4m3", t, LT * (lw.Hkv * lw.dh * 2 * 2 + lw.Hkv * lw.dh * 2 + 8))
    t, _ = timed(lambda: oracle.decode_attn(lw.q, lkc, lvc, lw.paging.block_tables,
                                            lw.paging.context_lens, lks, lvs, fmt, gh))
    rec("decode_long_e4m3", t, LT * lw.Hkv * lw.dh * 2)
    del lw, lkc, lvc
    # FP8 prefill: every query row of one seeded (sequence, head) pair of the
    # 8 x (4096 + 4096) workload, scaled to all 256 pairs by pair count (every pair
    # does the same causal work)
    pw = W.fp8_chunked_prefill()
    qs = oracle.calibrate(pw.q, fmt, gh)[1]
    pks = oracle.calibrate(pw.kv.k, fmt, gh)[1]
    pvs = oracle.calibrate(pw.kv.v, fmt, gh)[1]
    pkc = np.zeros(oracle.k_cache_shape(pw.paging.num_blocks, pw.Hkv, pw.bs, pw.dh), np.uint8)
    pvc = np.zeros((pw.paging.num_blocks, pw.Hkv, pw.dh, pw.bs), np.uint8)
    oracle.cache_write(pw.kv.k, pw.kv.v, pw.kv.slot_mapping, pkc, pvc, pks, pvs, fmt, gh)
    g = np.random.Generator(np.random.PCG64(11))
    nseq, npairs = len(pw.prefix_lens), 1
    pairs = [(int(g.integers(nseq)), int(g.integers(pw.Hq))) for _ in range(npairs)]
    cu = pw.cu_seqlens
    rws = np.array([(r, h) for b, h in pairs for r in range(cu[b], cu[b + 1])], np.int64)
    t, _ = timed(lambda: oracle.prefill_rows(rws, pw.q, pw.cu_seqlens, qs, gh, pkc, pvc,
                                             pw.paging.block_tables, pw.paging.context_lens,
                                             pks, pvs, fmt, gh))
    total_pairs = nseq * pw.Hq
    flops = 0
    for b in range(nseq):
        P, C = int(pw.prefix_lens[b]), int(cu[b + 1] - cu[b])
        flops += 4 * pw.dh * pw.Hq * (C * P + C * (C + 1) // 2)
    rec("prefill", t * total_pairs / npairs, flops=flops,
        note=f"all {len(rws)} query rows of {npairs} seeded (sequence, head) pairs, timed "
             f"{t:.2f} s, scaled by {total_pairs}/{npairs} pairs")
    return out


if __name__ == "__main__":
    main()
