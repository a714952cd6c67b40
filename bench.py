"""Benchmark of the GQA forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--only NAME]

A step is one call of the hot path over one batch of synthetic input, with
inputs already resident in HBM.  The default workload is the split-KV decode
(B=16, Hq=32, Hkv=8, Skv=8192, d=128, TILE_S_KV=1024: partial kernel + merge
kernel); `value` is its K/V-stream throughput in GB/s of algorithmic bytes
(Q + K + V read once, O written once).  The same JSON line also carries:

* roofline: the dominant kernel (the split-KV partial kernel) timed alone
  with HIP events on its own stream, algorithmic bytes per launch over its
  mean duration, against MI355X's 8 TB/s HBM peak; `traffic` is the HBM
  bytes per launch from the committed counter summary
  (profiles/decode_partial_hbm_traffic.txt), null once the kernel sources
  differ from the ones it was measured on;
* secondary: the other named workloads (short-q/long-kv prefill, causal
  prefill, ragged paged, causal chunked prefill, the other head dims, paged
  decode with and without the fused append, the in-kernel merge, tiny
  prefill), each timed the same way with its own roofline fraction;
* cold_cache: the decode, short-q and causal workloads again, one call per
  HIP-event pair with a 512 MiB buffer read before each (outside the events)
  so the L2 caches and the MALL start cold; median and min;
* cpu_baseline: the fp64 oracle timed on this host's cores on a bounded
  sample of the decode workload.

One GPU only: --gpus above 1 exits with a message.
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
METRIC = "GQA attn prefill TFLOP/s & decode KV GB/s at 1 GPU, % of MI355X peak"


def gqa():
    import gqa_attention_forward_amd as m
    return m


# ---------------------------------------------------------------- algorithmic work

def dense_bytes(c, kv_len=None):
    """Q + true K/V rows + O, each once (bf16)."""
    n = c.Skv if kv_len is None else kv_len
    q = c.B * c.Hq * c.Sq * c.d * 2
    kv = 2 * c.B * c.Hkv * n * c.d * 2
    return q + kv + q, q + kv


def dense_flops(c):
    """4 d flops per visible (query, key) pair; causal counts j <= i only."""
    if c.causal:
        pairs = c.B * c.Hq * sum(min(c.Skv, c.Skv - c.Sq + i + 1) for i in range(c.Sq))
    else:
        pairs = c.B * c.Hq * c.Sq * c.Skv
    return 4 * c.d * pairs


def paged_work(w, causal=False):
    """Algorithmic bytes (Q, O, K, V once) and flops (4 d per visible pair)."""
    ql = w["q_len"].numpy().astype(np.int64)
    kl = w["kv_len"].numpy().astype(np.int64)
    Hq, Hkv, d = w["Hq"], w["Hkv"], w["d"]
    bytes_ = int((2 * ql * Hq * d * 2).sum() + (2 * kl * Hkv * d * 2).sum())
    if causal:  # bottom-right: row i sees kv_len - q_len + i + 1 keys
        pairs = ql * (kl - ql) + ql * (ql + 1) // 2
    else:
        pairs = ql * kl
    flops = int((4 * d * Hq * pairs).sum())
    return bytes_, flops


# ---------------------------------------------------------------- timing

def time_loop(fn, steps, warmup, stream):
    """Mean ms per call of `fn` over `steps` calls on `stream` (HIP events)."""
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            fn()
        stop.record(stream)
        torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def warm_steps(fn, stream, seconds=0.15):
    """Warm-up count for a secondary workload: enough calls for about
    `seconds` of GPU work.  Compute-bound kernels speed up by ~20% over their
    first tens of milliseconds of sustained load (clocks ramp); timing
    before that measures the ramp."""
    ms = time_loop(fn, 1, 1, stream)
    return int(min(2000, max(2, seconds * 1e3 / max(ms, 1e-3))))


def time_graph(fn, reps, replays, stream):
    """Mean ms per call of `fn` with `reps` calls captured in one HIP graph
    (for kernels too short for per-call launches to keep the GPU busy)."""
    with torch.cuda.stream(stream):
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for _ in range(reps):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(replays):
            graph.replay()
        stop.record(stream)
        torch.cuda.synchronize()
    return start.elapsed_time(stop) / (reps * replays)


def time_cold(fn, stream, flush, min_iters=50, min_ms=200.0):
    """(median, min) ms of single calls of `fn`, each timed with its own HIP
    events after all of `flush` (>= 512 MiB) is read, outside the events, so
    that the L2 caches and the 256 MB MALL hold none of the inputs.  The
    flush reads rather than writes: rewritten lines would sit dirty in the
    caches and be written back during the timed call (+55% on the decode).
    At least `min_iters` calls or `min_ms` of timed work, whichever is more."""
    words = flush.view(torch.int32)
    total = torch.empty((), dtype=torch.int64, device=flush.device)
    with torch.cuda.stream(stream):
        for _ in range(5):
            torch.sum(words, dim=(0,), dtype=torch.int64, out=total)
            fn()
        torch.cuda.synchronize()
        per = time_loop(fn, 3, 0, stream)
        iters = int(max(min_iters, min_ms / max(per, 1e-3)))
        marks = []
        for _ in range(iters):
            torch.sum(words, dim=(0,), dtype=torch.int64, out=total)
            start = torch.cuda.Event(enable_timing=True)
            stop = torch.cuda.Event(enable_timing=True)
            start.record(stream)
            fn()
            stop.record(stream)
            marks.append((start, stop))
        torch.cuda.synchronize()
    times = sorted(a.elapsed_time(b) for a, b in marks)
    return times[len(times) // 2], times[0], iters


# Kernel sources behind the split-KV partial kernel; the committed counter
# summary records their hash.
PARTIAL_SOURCES = ("attn_stream.hpp", "common.hpp", "launch.hpp", "gqa_api.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_partial_hbm_traffic.txt")


def measured_traffic():
    """HBM bytes per partial launch from the committed FETCH_SIZE/WRITE_SIZE
    summary (copy-calibrated), or None once the kernel sources differ from
    the ones the counters were taken on."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    nbytes = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    digest = re.search(r"^source_sha256: ([0-9a-f]{64})$", text, re.M)
    if not nbytes or not digest:
        return None
    h = hashlib.sha256()
    for name in PARTIAL_SOURCES:
        with open(os.path.join(ROOT, "gqa_attention_forward_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return int(nbytes.group(1)) if h.hexdigest() == digest.group(1) else None


def roof(bound, achieved, peak, unit, traffic=None):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


# ---------------------------------------------------------------- workloads

def setup_dense(name, device):
    c = workloads.CASES[name] if name in workloads.CASES else workloads.HEAD_DIM_CASES[name]
    inp = workloads.make_case(c)
    g = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    return c, inp, g


def decode_step_fns(g, c):
    m = gqa()
    out = torch.empty_like(g["q"])
    ns = m.n_splits(c.Skv, c.tile_s_kv)
    ws = torch.empty(m.workspace_size(c.B, c.Hq, 1, c.Skv, c.d, c.tile_s_kv), dtype=torch.uint8,
                     device=g["q"].device)

    def step():
        m.decode_splitkv(g["q"], g["k"], g["v"], kv_len=g["kv_len"], scale=g["scale"],
                         tile_s_kv=c.tile_s_kv, out=out, workspace=ws)

    def partial():
        m.splitkv_partial(g["q"], g["k"], g["v"], tile_s_kv=c.tile_s_kv, kv_len=g["kv_len"],
                          scale=g["scale"], workspace=ws)

    def merge():
        m.splitkv_merge(ws, B=c.B, Hq=c.Hq, Sq=1, d=c.d, n_split=ns, out=out)

    return step, partial, merge, out


def prefill_step_fn(g, c, tile=0):
    m = gqa()
    out = torch.empty_like(g["q"])
    ws = None
    if tile:
        ws = torch.empty(m.workspace_size(c.B, c.Hq, c.Sq, c.Skv, c.d, tile), dtype=torch.uint8,
                         device=g["q"].device)

    def step():
        m.prefill(g["q"], g["k"], g["v"], kv_len=g["kv_len"], scale=g["scale"], causal=c.causal,
                  tile_s_kv=tile, out=out, workspace=ws)

    return step, out


def bench_decode(args, device, stream):
    c, inp, g = setup_dense("decode_splitkv", device)
    step, partial, merge, out = decode_step_fns(g, c)
    ms = time_loop(step, args.steps, args.warmup, stream)
    total_bytes, read_bytes = dense_bytes(c)
    gbs = total_bytes / (ms * 1e-3) / 1e9
    # dominant kernel alone: the split-KV partial kernel (reads Q, K, V once)
    ms_p = time_loop(partial, args.steps, max(1, args.warmup // 2), stream)
    # the merge kernel runs a few microseconds: time it from a captured graph
    ms_m = time_graph(merge, 20, 5, stream)
    assert torch.isfinite(out.float()).all()
    rf = roof("hbm", read_bytes / (ms_p * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", measured_traffic())
    # the dominant kernel's fraction is `frac`; the whole step's (partial +
    # merge kernels, the headline value) is reported beside it
    rf["step_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    return c, inp, {
        "ms_per_step": ms, "value": gbs, "total_bytes": total_bytes,
        "roofline": rf,
        "kernel_ms": {"partial": round(ms_p, 5), "merge": round(ms_m, 5)},
        "kernel_bytes_per_launch": {"partial": read_bytes},
    }


def paged_head_major(w, device):
    """The paged decode workload's tensors on `device`, with its K/V pools
    stored head-major ([n_pages, Hkv, 64, d], laid out on the host) and
    returned as the same logical [n_pages, 64, Hkv, d] views."""
    gw = {k: (v.to(device) if isinstance(v, torch.Tensor) and k not in ("k_cache", "v_cache")
              else v) for k, v in w.items()}
    khm = w["k_cache"].permute(0, 2, 1, 3).contiguous().to(device).permute(0, 2, 1, 3)
    vhm = w["v_cache"].permute(0, 2, 1, 3).contiguous().to(device).permute(0, 2, 1, 3)
    return gw, khm, vhm


def fresh_allocations():
    """Release the blocks the caching allocator kept from earlier workloads,
    so that the next workload's tensors are new device allocations, as in a
    process of its own.  Carved from reused blocks, the paged decode's pools
    read 98.7 us per step against 92.6 us when freshly allocated (91.5 us
    alone in a process); a serving process allocates its pools up front."""
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def bench_cold(device, stream):
    """The decode, short-q and causal workloads with cold caches before every
    call: median and min over single timed calls."""
    fresh_allocations()
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device=device)
    res = {}
    c, _, g = setup_dense("decode_splitkv", device)
    step, _, _, _ = decode_step_fns(g, c)
    med, mn, it = time_cold(step, stream, flush)
    tb, _ = dense_bytes(c)
    res["decode_splitkv"] = {"median_ms": round(med, 5), "min_ms": round(mn, 5), "calls": it,
                             "GB/s": round(tb / (med * 1e-3) / 1e9, 1),
                             "roofline_frac": round(tb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del g
    c, _, g = setup_dense("shortq_longkv", device)
    for tile in (2048, 4096):
        step, _ = prefill_step_fn(g, c, tile)
        med, mn, it = time_cold(step, stream, flush)
        tb, _ = dense_bytes(c)
        res[f"shortq_longkv_tile{tile}"] = {
            "median_ms": round(med, 5), "min_ms": round(mn, 5), "calls": it,
            "GB/s": round(tb / (med * 1e-3) / 1e9, 1),
            "roofline_frac": round(tb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del g
    c, _, g = setup_dense("causal_prefill", device)
    step, _ = prefill_step_fn(g, c, 0)
    warm_steps(step, stream)  # let the clock ramp first
    med, mn, it = time_cold(step, stream, flush)
    fl = dense_flops(c)
    res["causal_prefill"] = {"median_ms": round(med, 5), "min_ms": round(mn, 5), "calls": it,
                             "TFLOP/s": round(fl / (med * 1e-3) / 1e12, 2),
                             "roofline_frac": round(fl / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    del g, flush
    return res


def bench_secondary(args, device, stream):
    res = {}
    steps = max(3, min(args.steps, 20))
    fresh_allocations()
    # short-q / long-kv prefill (HBM-bound): one pass, and split-KV with 8
    # splits of 2048 keys (4-wave form, two workgroups per CU) or 4 of 4096
    # (two key groups per 8-wave workgroup, one per CU)
    c, _, g = setup_dense("shortq_longkv", device)
    for tile in (0, 2048, 4096):
        step, out = prefill_step_fn(g, c, tile)
        ms = time_loop(step, steps, warm_steps(step, stream), stream)
        tb, _ = dense_bytes(c)
        fl = dense_flops(c)
        res[f"shortq_longkv_tile{tile}"] = {
            "ms": round(ms, 5), "GB/s": round(tb / (ms * 1e-3) / 1e9, 1),
            "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2),
            "roofline": roof("hbm", tb / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")}
    del g, out
    fresh_allocations()
    # causal prefill (MFMA-bound)
    c, _, g = setup_dense("causal_prefill", device)
    step, out = prefill_step_fn(g, c, 0)
    ms = time_loop(step, steps, warm_steps(step, stream), stream)
    fl = dense_flops(c)
    res["causal_prefill"] = {
        "ms": round(ms, 5), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2), "flops": fl,
        "roofline": roof("mfma", fl / (ms * 1e-3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s")}
    del g, out
    fresh_allocations()
    # the same decode with the in-kernel merge (one launch; tickets zeroed once)
    c, _, g = setup_dense("decode_splitkv", device)
    m = gqa()
    outf = torch.empty_like(g["q"])
    wsf = torch.empty(m.workspace_size(c.B, c.Hq, 1, c.Skv, c.d, c.tile_s_kv), dtype=torch.uint8,
                      device=device)
    tk = torch.zeros(c.B * c.Hq, dtype=torch.int32, device=device)

    def fstep():
        m.decode_splitkv(g["q"], g["k"], g["v"], kv_len=g["kv_len"], scale=g["scale"],
                         tile_s_kv=c.tile_s_kv, out=outf, workspace=wsf, fused=True, tickets=tk)
    ms = time_loop(fstep, steps, warm_steps(fstep, stream), stream)
    tb, _ = dense_bytes(c)
    res["decode_splitkv_fused_merge"] = {
        "ms": round(ms, 5), "GB/s": round(tb / (ms * 1e-3) / 1e9, 1),
        "roofline": roof("hbm", tb / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")}
    del g, outf, wsf, tk
    fresh_allocations()
    # the other head dims: decode at d = 256 and 512, causal prefill at d = 32,
    # 256 and 512
    for name in ("decode_splitkv_d256", "decode_splitkv_d512"):
        c, _, g = setup_dense(name, device)
        step, _, _, _ = decode_step_fns(g, c)
        ms = time_loop(step, steps, warm_steps(step, stream), stream)
        tb, _ = dense_bytes(c)
        res[name] = {
            "ms": round(ms, 5), "GB/s": round(tb / (ms * 1e-3) / 1e9, 1),
            "roofline": roof("hbm", tb / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")}
        del g
        fresh_allocations()
    for name in ("causal_prefill_d32", "causal_prefill_d256", "causal_prefill_d512"):
        c, _, g = setup_dense(name, device)
        step, out = prefill_step_fn(g, c, 0)
        ms = time_loop(step, steps, warm_steps(step, stream), stream)
        fl = dense_flops(c)
        res[name] = {
            "ms": round(ms, 5), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2), "flops": fl,
            "roofline": roof("mfma", fl / (ms * 1e-3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s")}
        del g, out
    fresh_allocations()
    # ragged paged with sink: one pass and split-KV (tiles of 1024 keys)
    w = workloads.make_paged()
    gw = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}
    m = gqa()
    outp = torch.empty_like(gw["q"])
    pb, pf = paged_work(w)
    t_roof = max(pb / (HBM_PEAK_GBS * 1e9), pf / (BF16_PEAK_TFLOPS * 1e12))
    for tile in (0, 1024):
        ws = None
        if tile:
            ws = torch.empty(m.workspace_size(1, w["Hq"], w["total_q"],
                                              gw["page_table"].shape[1] * 64, w["d"], tile),
                             dtype=torch.uint8, device=device)

        def pstep(tile=tile, ws=ws):
            m.paged(gw["q"], gw["cu_seqlens_q"], gw["k_cache"], gw["v_cache"], gw["page_table"],
                    gw["kv_len"], max_q_len=w["max_q_len"], scale=w["scale"], sink=gw["sink"],
                    tile_s_kv=tile, out=outp, workspace=ws)
        ms = time_loop(pstep, steps, warm_steps(pstep, stream), stream)
        res[f"ragged_paged_tile{tile}"] = {"ms": round(ms, 5), "bytes": pb, "flops": pf,
                                           "roofline_frac": round(t_roof / (ms * 1e-3), 4)}
    fresh_allocations()
    # causal chunked prefill over a cached prefix (paged, bottom-right causal)
    w = workloads.make_paged_chunked()
    gw = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}
    outc = torch.empty_like(gw["q"])
    cb, cf = paged_work(w, causal=True)
    t_roof = max(cb / (HBM_PEAK_GBS * 1e9), cf / (BF16_PEAK_TFLOPS * 1e12))
    for tile in (0, 1024):
        ws = None
        if tile:
            ws = torch.empty(m.workspace_size(1, w["Hq"], w["total_q"],
                                              gw["page_table"].shape[1] * 64, w["d"], tile),
                             dtype=torch.uint8, device=device)

        def cstep(tile=tile, ws=ws):
            m.paged(gw["q"], gw["cu_seqlens_q"], gw["k_cache"], gw["v_cache"], gw["page_table"],
                    gw["kv_len"], max_q_len=w["max_q_len"], scale=w["scale"], sink=gw["sink"],
                    causal=True, tile_s_kv=tile, out=outc, workspace=ws)
        ms = time_loop(cstep, steps, warm_steps(cstep, stream), stream)
        res[f"paged_causal_chunked_tile{tile}"] = {
            "ms": round(ms, 5), "bytes": cb, "flops": cf,
            "tflops": round(cf / (ms * 1e-3) / 1e12, 2),
            "roofline_frac": round(t_roof / (ms * 1e-3), 4)}
    fresh_allocations()
    # paged decode at the split-KV decode shape, plain and with the fused append
    # of each token's K/V (the token's key row comes from k_new and is written
    # into its page by the same launch)
    w = workloads.make_paged_decode()
    kn, vn, _, _ = workloads.take_new_kv(w)
    gw = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}
    kn, vn = kn.to(device), vn.to(device)
    outd = torch.empty_like(gw["q"])
    db, _ = paged_work(w)
    tile = 1024
    ws = torch.empty(m.workspace_size(1, w["Hq"], w["total_q"], gw["page_table"].shape[1] * 64,
                                      w["d"], tile), dtype=torch.uint8, device=device)
    for name, append, kc, vc in (
            ("paged_decode_tile1024", False, gw["k_cache"], gw["v_cache"]),
            ("paged_decode_append_tile1024", True, gw["k_cache"], gw["v_cache"])):
        def dstep(append=append, kc=kc, vc=vc):
            if append:
                m.paged_append(gw["q"], gw["cu_seqlens_q"], kc, vc,
                               gw["page_table"], gw["kv_len"], kn, vn, max_q_len=1,
                               scale=w["scale"], tile_s_kv=tile, out=outd, workspace=ws)
            else:
                m.paged(gw["q"], gw["cu_seqlens_q"], kc, vc,
                        gw["page_table"], gw["kv_len"], max_q_len=1, scale=w["scale"],
                        tile_s_kv=tile, out=outd, workspace=ws)
        ms = time_loop(dstep, steps, warm_steps(dstep, stream), stream)
        res[name] = {"ms": round(ms, 5), "GB/s": round(db / (ms * 1e-3) / 1e9, 1),
                     "roofline": roof("hbm", db / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")}
    del gw, kn, vn, ws
    fresh_allocations()
    # the same pool stored head-major ([n_pages, Hkv, 64, d]) and passed by
    # strides as the same logical view (one head's rows of a page contiguous),
    # in fresh allocations of its own
    gw, khm, vhm = paged_head_major(w, device)
    ws = torch.empty(m.workspace_size(1, w["Hq"], w["total_q"], gw["page_table"].shape[1] * 64,
                                      w["d"], tile), dtype=torch.uint8, device=device)
    outd = torch.empty_like(gw["q"])

    def hstep():
        m.paged(gw["q"], gw["cu_seqlens_q"], khm, vhm, gw["page_table"], gw["kv_len"],
                max_q_len=1, scale=w["scale"], tile_s_kv=tile, out=outd, workspace=ws)
    ms = time_loop(hstep, steps, warm_steps(hstep, stream), stream)
    res["paged_decode_head_major_tile1024"] = {
        "ms": round(ms, 5), "GB/s": round(db / (ms * 1e-3) / 1e9, 1),
        "roofline": roof("hbm", db / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")}
    del gw, khm, vhm, ws, outd
    fresh_allocations()
    # B = 1 decode over 1K-32K keys (Hq 32, Hkv 8, d 128) with the library's
    # split size for the shape (gqa_attention_decode_tile) and with splits of
    # 1024; latency-bound, so timed from captured graphs (GPU time per call)
    # and eagerly (host and launch included)
    for skv in (1024, 4096, 16384, 32768):
        c = workloads.DenseCase(f"decode_b1_{skv}", 1, 32, 8, 1, skv, 128, tile_s_kv=1024,
                                decode=True, seed=1014)
        inp = workloads.make_case(c)
        g = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        outb = torch.empty_like(g["q"])
        tb, _ = dense_bytes(c)
        row = {}
        for label, tile in (("auto", m.decode_tile(1, 8, skv)), ("tile1024", 1024)):
            wsb = torch.empty(m.workspace_size(1, 32, 1, skv, 128, tile), dtype=torch.uint8,
                              device=device)

            def bstep(tile=tile, wsb=wsb):
                m.decode_splitkv(g["q"], g["k"], g["v"], kv_len=g["kv_len"], scale=g["scale"],
                                 tile_s_kv=tile, out=outb, workspace=wsb)
            gms = time_graph(bstep, 20, 10, stream)
            row[label] = {"tile_s_kv": tile, "us": round(gms * 1e3, 2),
                          "eager_us": round(time_loop(bstep, 50, 20, stream) * 1e3, 2),
                          "GB/s": round(tb / (gms * 1e-3) / 1e9, 1),
                          "roofline_frac": round(tb / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        res[f"decode_b1_{skv}"] = row
        del g, inp
    fresh_allocations()
    # tiny prefill (launch-bound)
    c, _, g = setup_dense("tiny_prefill", device)
    step, out = prefill_step_fn(g, c, 0)
    ms = time_loop(step, steps, warm_steps(step, stream), stream)
    # eager calls are bound by the host side of each call; a captured graph of
    # 20 calls shows the GPU time
    res["tiny_prefill"] = {"ms": round(ms, 5), "graph_ms": round(time_graph(step, 20, 5, stream), 5)}
    return res


def run_only(args, device, stream):
    """One workload's kernels alone (for counter collection under rocprofv3)."""
    name = args.only
    if name == "copy":
        # calibration for HBM byte counters: a plain 256 MiB device copy
        x = torch.empty(128 << 20, dtype=torch.bfloat16, device=device).fill_(1.0)
        y = torch.empty_like(x)
        ms = time_loop(lambda: y.copy_(x), args.steps, args.warmup, stream)
        return {"workload": name, "ms": ms, "bytes_read": x.numel() * 2, "bytes_written": y.numel() * 2}
    if name == "decode_partial":
        c, _, g = setup_dense("decode_splitkv", device)
        _, partial, _, _ = decode_step_fns(g, c)
        ms = time_loop(partial, args.steps, args.warmup, stream)
        return {"workload": name, "ms": ms, "GB/s": dense_bytes(c)[1] / (ms * 1e-3) / 1e9}
    if name in ("ragged_paged", "ragged_paged_onepass"):
        w = workloads.make_paged()
        gw = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}
        m = gqa()
        tile = 1024 if name == "ragged_paged" else 0
        fn = lambda: m.paged(gw["q"], gw["cu_seqlens_q"], gw["k_cache"], gw["v_cache"],  # noqa: E731
                             gw["page_table"], gw["kv_len"], max_q_len=w["max_q_len"],
                             scale=w["scale"], sink=gw["sink"], tile_s_kv=tile)
        return {"workload": name, "ms": time_loop(fn, args.steps, args.warmup, stream)}
    if name == "paged_decode_head_major":
        w = workloads.make_paged_decode()
        gw, khm, vhm = paged_head_major(w, device)
        m = gqa()
        fn = lambda: m.paged(gw["q"], gw["cu_seqlens_q"], khm, vhm,  # noqa: E731
                             gw["page_table"], gw["kv_len"], max_q_len=1, scale=w["scale"],
                             tile_s_kv=1024)
        ms = time_loop(fn, args.steps, args.warmup, stream)
        return {"workload": name, "ms": ms, "GB/s": paged_work(w)[0] / (ms * 1e-3) / 1e9}
    if name in ("paged_decode", "paged_decode_append"):
        w = workloads.make_paged_decode()
        kn, vn, _, _ = workloads.take_new_kv(w)
        gw = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}
        kn, vn = kn.to(device), vn.to(device)
        m = gqa()
        if name == "paged_decode":
            fn = lambda: m.paged(gw["q"], gw["cu_seqlens_q"], gw["k_cache"],  # noqa: E731
                                 gw["v_cache"], gw["page_table"], gw["kv_len"], max_q_len=1,
                                 scale=w["scale"], tile_s_kv=1024)
        else:
            fn = lambda: m.paged_append(gw["q"], gw["cu_seqlens_q"], gw["k_cache"],  # noqa: E731
                                        gw["v_cache"], gw["page_table"], gw["kv_len"], kn, vn,
                                        max_q_len=1, scale=w["scale"], tile_s_kv=1024)
        ms = time_loop(fn, args.steps, args.warmup, stream)
        return {"workload": name, "ms": ms, "GB/s": paged_work(w)[0] / (ms * 1e-3) / 1e9}
    if name == "paged_causal_chunked":
        w = workloads.make_paged_chunked()
        gw = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}
        m = gqa()
        fn = lambda: m.paged(gw["q"], gw["cu_seqlens_q"], gw["k_cache"], gw["v_cache"],  # noqa: E731
                             gw["page_table"], gw["kv_len"], max_q_len=w["max_q_len"],
                             scale=w["scale"], sink=gw["sink"], causal=True)
        ms = time_loop(fn, args.steps, args.warmup, stream)
        return {"workload": name, "ms": ms,
                "TFLOP/s": paged_work(w, causal=True)[1] / (ms * 1e-3) / 1e12}
    c, _, g = setup_dense(name, device)
    if c.decode:
        step, _, _, _ = decode_step_fns(g, c)
    else:
        step, _ = prefill_step_fn(g, c, 4096 if name == "shortq_longkv" else 0)
    ms = time_loop(step, args.steps, args.warmup, stream)
    return {"workload": name, "ms": ms, "TFLOP/s": dense_flops(c) / (ms * 1e-3) / 1e12,
            "GB/s": dense_bytes(c)[0] / (ms * 1e-3) / 1e9}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        return len(os.sched_getaffinity(0))


def _timed(fn):
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def cpu_baseline(inp, c, budget_s):
    """The oracle on this host's cores (never tuned for this), input conversion
    outside the timed regions.  The headline figure cycles over whole decode
    sequences (all heads and keys of one sequence per call) for about half the
    budget; the other configs get the rest:
      tiny prefill and ragged paged: one full evaluation each;
      short-q/long-kv: whole (b, kv head) groups (all G heads x 16 rows x 16384
        keys), cycling, for about a sixth of the budget;
      causal prefill: rows spread over the sequence (each over its visible
        keys), cycling, for about a sixth of the budget.
    Each entry reports the throughput in the workload's own unit and the
    sample it was measured on."""
    import oracle
    threads = _oracle_threads()
    per = {}
    # decode (headline): whole sequences
    elapsed, done = 0.0, 0
    cache = {}
    while elapsed < budget_s / 2:
        b = done % c.B
        if b not in cache:
            cache[b] = tuple(t[b:b + 1].to(torch.float64).numpy()
                             for t in (inp["q"], inp["k"], inp["v"]))
        qb, kb, vb = cache[b]
        elapsed += _timed(lambda: oracle.attention_fp64(qb, kb, vb, scale=inp["scale"]))
        done += 1
    per_seq = (2 * c.Hq * c.d * 2) + 2 * c.Hkv * c.Skv * c.d * 2
    dec_gbs = done * per_seq / elapsed / 1e9
    per["decode_splitkv"] = {"value": round(dec_gbs, 4), "unit": "GB/s",
                             "sample": f"{done} whole sequences (of {c.B}), {elapsed:.1f} s"}
    # tiny prefill: in full
    ct = workloads.CASES["tiny_prefill"]
    t = workloads.make_case(ct)
    f64 = [x.to(torch.float64).numpy() for x in (t["q"], t["k"], t["v"])]
    sec = min(_timed(lambda: oracle.attention_fp64(*f64, scale=t["scale"])) for _ in range(5))
    per["tiny_prefill"] = {"value": round(sec * 1e3, 4), "unit": "ms per call",
                           "sample": "the whole workload (best of 5 calls)"}
    # short-q / long-kv: whole (b, kv head) groups
    cs = workloads.CASES["shortq_longkv"]
    t = workloads.make_case(cs)
    q64, k64, v64 = (x.to(torch.float64).numpy() for x in (t["q"], t["k"], t["v"]))
    G = cs.Hq // cs.Hkv
    elapsed, done = 0.0, 0
    while elapsed < budget_s / 6:
        b, g = (done // cs.Hkv) % cs.B, done % cs.Hkv
        qs = q64[b:b + 1, g * G:(g + 1) * G]
        ks, vs = k64[b:b + 1, g:g + 1], v64[b:b + 1, g:g + 1]
        elapsed += _timed(lambda: oracle.attention_fp64(qs, ks, vs, scale=t["scale"]))
        done += 1
    grp_flops = 4 * cs.d * G * cs.Sq * cs.Skv
    grp_bytes = (2 * G * cs.Sq + 2 * cs.Skv) * cs.d * 2
    per["shortq_longkv"] = {"value": round(done * grp_bytes / elapsed / 1e9, 4), "unit": "GB/s",
                            "TFLOP/s": round(done * grp_flops / elapsed / 1e12, 6),
                            "sample": f"{done} (b, kv head) groups of {cs.B * cs.Hkv}, "
                                      f"{elapsed:.1f} s"}
    del q64, k64, v64, t
    # causal prefill: rows spread over the sequence
    cc = workloads.CASES["causal_prefill"]
    t = workloads.make_case(cc)
    q64, k64, v64 = (x.to(torch.float64).numpy() for x in (t["q"], t["k"], t["v"]))
    rng = np.random.default_rng(0)
    elapsed, rows, flops = 0.0, 0, 0
    while elapsed < budget_s / 6:
        n = 64
        bi = rng.integers(0, cc.B, n)
        hi = rng.integers(0, cc.Hq, n)
        ii = rng.integers(0, cc.Sq, n)
        elapsed += _timed(lambda: oracle.attention_rows_fp64(q64, k64, v64, bi, hi, ii,
                                                             scale=t["scale"], causal=True))
        rows += n
        flops += int((4 * cc.d * (ii + 1)).sum())
    per["causal_prefill"] = {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s",
                             "sample": f"{rows} rows drawn over the sequence (of "
                                       f"{cc.B * cc.Hq * cc.Sq}), {elapsed:.1f} s"}
    del q64, k64, v64, t
    # ragged paged: in full
    w = workloads.make_paged()
    args = [workloads.to_f64(w["q"]), w["cu_seqlens_q"].numpy(), workloads.to_f64(w["k_cache"]),
            workloads.to_f64(w["v_cache"]), w["page_table"].numpy(), w["kv_len"].numpy()]
    sec = _timed(lambda: oracle.paged_attention_fp64(*args, scale=w["scale"], page_size=64,
                                                      sink=workloads.to_f64(w["sink"])))
    pb, pf = paged_work(w)
    per["ragged_paged"] = {"value": round(sec * 1e3, 3), "unit": "ms per call",
                           "TFLOP/s": round(pf / sec / 1e12, 6),
                           "sample": "the whole workload (one call)"}
    return {"value": round(dec_gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": per["decode_splitkv"]["sample"] + " of the decode_splitkv workload (each "
                      f"all {c.Hq} heads x {c.Skv} keys)",
            "per_config": per}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 200 untimed steps (about 17 ms of decode): after 20 the decode step still
    # read 85 us, after 200 or 1000 it reads 81.3-81.7 us
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=18.0,
                    help="seconds of oracle time for the CPU baseline (0 = skip)")
    ap.add_argument("--only", choices=["decode_partial", "shortq_longkv", "causal_prefill",
                                       "ragged_paged", "ragged_paged_onepass",
                                       "paged_causal_chunked", "paged_decode",
                                       "paged_decode_head_major", "paged_decode_append", "copy",
                                       *workloads.HEAD_DIM_CASES],
                    help="profiling aid: time only this workload's kernels and print its line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    stream = torch.cuda.Stream(device)
    torch.cuda.synchronize()
    if args.only:
        print(json.dumps(run_only(args, device, stream)), flush=True)
        return

    c, inp, dec = bench_decode(args, device, stream)
    secondary = None if args.no_secondary else bench_secondary(args, device, stream)
    cold = None if args.no_secondary else bench_cold(device, stream)
    cpu = cpu_baseline(inp, c, args.cpu_budget) if args.cpu_budget > 0 else None

    line = {
        "metric": METRIC,
        "value": round(dec["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_splitkv", "B": c.B, "Hq": c.Hq, "Hkv": c.Hkv, "Sq": 1,
                   "Skv": c.Skv, "d": c.d, "tile_s_kv": c.tile_s_kv,
                   "seq_len": c.Skv, "global_batch": c.B, "parallelism": "none (1 GPU)"},
        "roofline": dec["roofline"],
        "kernel_ms": dec["kernel_ms"],
        "kernel_bytes_per_launch": dec["kernel_bytes_per_launch"],
        "cpu_baseline": cpu,
        "secondary": secondary,
        "cold_cache": cold,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
