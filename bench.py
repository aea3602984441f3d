#!/usr/bin/env python3
"""Benchmark of the KVarN hot path on one MI355X: tile quantization + paged decode attention.

Default workload (prefill burst: 64 sequences x 16384 tokens, 8 KV heads, head_dim 128, even KV
heads N(0,1), odd KV heads Student-t(2.5), k4v2_g128, 8 normalization iterations): one step =
quantize all 131072 K and V tiles of the burst into a page pool (one launch), then one batched
decode step of the 64 query heads of all 64 sequences. Two page-pool copies alternate: step s
quantizes into copy s mod 2 and decodes copy (s + 1) mod 2, whose pages were written one step
earlier; the 5.2 GB the quantize moves in between evict them from the 256 MB Infinity Cache, so
the decode reads cold pages (the warm decode, right after the quantize of the same pages, is
reported apart). Synthetic data; inputs resident in HBM before timing.

Prints one JSON line. Numbers:
  value / ms_per_step: whole step (quantize + decode), algorithmic bytes / step time.
  roofline: the dominant kernel (the quantizer) against the HBM peak; its fractions of the
    fp32 vector peaks ride along. roofline_other: the cold decode against the HBM peak.
  quantize_by_iters: the quantize launch at 2, 4 and 8 normalization iterations.
  hbm_read_probe: a streaming-read kernel's GB/s; decodes also report their fraction of it.
  decode_workloads: the decode-bound workloads (batched paged, long context) run briefly in the
    same process, their decode's HBM fraction and launch-time percentiles.
  cpu_baseline: the float64 CPU oracle on a bounded sample of the same step.

Other workloads (--workload): one_layer_16k (batch 1, 16384 tokens, 64 layer copies cycled),
batched_paged / long_context (append + decode steps), chunked_prefill (chunk write +
multi-query read).

Profiling recipe (--print-profile-commands) and the reductions of its rocprofv3 output into
profiles/ (--reduce-profiles DIR): kernel-trace statistics, HBM traffic per launch
(FETCH_SIZE / WRITE_SIZE scaled by a device copy of known size) and SQ instruction / busy /
LDS counters per kernel.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Algorithmic work units (what the method must move / compute, not what the kernels do)
Q_READ = 128 * 128 * 2                 # float16 tile in
HBM_PEAK_GBPS = 8000.0                 # MI355X HBM3E
# published fp32 vector figure: 256 CU x 4 SIMD x 64 lanes x 2 FLOP per 2 cycles x 2.4 GHz. A
# wave64 v_fma_f32 (no packed forms) holds a SIMD about 2 cycles: the VALU calibration probe
# (kvarn_probe_valu_fma) measures it, so this is the peak of the quantizer's plain fp32 code.
FP32_VECTOR_PEAK_TFLOPS = 157.3
MFMA_F16_PEAK_TFLOPS = 2500.0          # MI355X dense float16 matrix cores
N_SIMD = 256 * 4
N_XCC = 8
VALU_ISSUE_CYCLES = 2                  # cycles per wave64 fp32 VALU instruction and SIMD
MIN_WARM_S = [0.3]      # warm-up GPU time before a timed region (--min-warm-s)

WORKLOADS = ("prefill_burst", "one_layer_16k", "chunked_prefill", "batched_paged", "long_context")
METRIC = "decode-attn KV GB/s (% HBM roofline) + tiles quantized/s, k4v2_g128"


def quant_flop_per_tile(n_iters: int) -> int:
    """FWHT-128 (7 x 16384 add/sub) + per iteration two moment passes in each direction
    (4 x 16384 FMA = 131072 FLOP) + RTN (~131072: min/max, scale, round)."""
    return 7 * 16384 + n_iters * 131072 + 131072


def source_hash() -> str:
    """Hash of the HIP sources (every file under csrc, recursively, in path order)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_quantization_tile_amd", "csrc")
    files = []
    for d, _, names in os.walk(csrc):
        files += [os.path.join(d, n) for n in names]
    for path in sorted(files, key=lambda p: os.path.relpath(p, csrc)):
        with open(path, "rb") as f:
            h.update(os.path.relpath(path, csrc).encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, src_hash: str, workload: str):
    """HBM bytes per launch of `kernel` in `workload` measured by rocprofv3 counters
    (profiles/traffic.json), or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    kernels = t.get("workloads", {}).get(workload, {}).get("kernels", {})
    if t.get("source_hash") != src_hash or kernel not in kernels:
        return None
    return kernels[kernel].get("bytes_per_launch")


def percentiles(xs) -> dict:
    """mean, p10, p50, p90 (linear interpolation) of a list of floats, rounded."""
    s = sorted(xs)
    if not s:
        return {}

    def q(p):
        x = p * (len(s) - 1)
        i = int(math.floor(x))
        j = min(i + 1, len(s) - 1)
        return s[i] + (s[j] - s[i]) * (x - i)
    return {"mean": round(sum(s) / len(s), 5), "p10": round(q(0.1), 5),
            "p50": round(q(0.5), 5), "p90": round(q(0.9), 5), "n": len(s)}


def host_threads():
    """(BLAS threads, os.cpu_count())."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    return blas, os.cpu_count()


# ----------------------------------------------------------------------------- CPU oracle legs


def cpu_baseline(w, n_iters: int, budget_s: float, k_bits: int = 4, v_bits: int = 2):
    """The float64 oracle on a time-bounded sample of one step, scaled to the whole step: tiles
    of the step quantized in batches of 16 (one KV head and kind per batch, in step order)
    for about budget_s / 2 seconds or until every tile of the step is done, then the decode
    (dequantize the pages, attention of every query head of the group) of chunks of pages for
    about budget_s / 2 seconds or until every (page, KV head) pair of the step is done."""
    import numpy as np
    from oracle import kvarn_oracle as O
    blas_threads, _ = host_threads()
    k = w.k_src.cpu().numpy()
    v = w.v_src.cpu().numpy()
    q = w.step_inputs(0, device="cpu")[0].numpy()
    n_pages = sum(L // 128 for L in w.prompt_lens)
    n_tiles_step = 2 * n_pages * w.hkv
    nb = min(16, n_pages)
    batches = [(h, kind, t0) for h in range(w.hkv) for kind in (O.KIND_K, O.KIND_V)
               for t0 in range(0, n_pages - nb + 1, nb)]
    recs = {}
    n_q, t_q = 0, 0.0
    for h, kind, t0 in batches:
        src = k if kind == O.KIND_K else v
        tiles = np.stack([src[128 * (t0 + i):128 * (t0 + i + 1), h, :].T for i in range(nb)])
        start = time.perf_counter()
        r = O.quantize_tiles(tiles, kind, n_iters, k_bits=k_bits, v_bits=v_bits)
        t_q += time.perf_counter() - start
        n_q += nb
        recs.setdefault(kind, r)
        if t_q >= budget_s / 2 and O.KIND_V in recs:
            break
    tq = t_q / n_q                                            # seconds per tile
    G = w.hq // w.hkv
    rk, rv = recs[O.KIND_K], recs[O.KIND_V]
    # decode: chunks of at most 256 pages of one KV head (every query head of the group);
    # the attention cost is linear in the pages, so the time per page scales to the step
    chunk = min(256, n_pages)
    n_d, t_d = 0, 0.0
    while n_d < n_pages * w.hkv:
        g = (n_d // n_pages) % w.hkv
        start = time.perf_counter()
        kd = np.concatenate([O.dequantize_tiles(rk["codes"][i % nb], rk["r"][i % nb], rk["s"][i % nb],
                                                rk["scale"][i % nb], rk["zero"][i % nb], O.KIND_K).T
                             for i in range(chunk)])
        vd = np.concatenate([O.dequantize_tiles(rv["codes"][i % nb], rv["r"][i % nb], rv["s"][i % nb],
                                                rv["scale"][i % nb], rv["zero"][i % nb], O.KIND_V).T
                             for i in range(chunk)])
        for h in range(G):
            O.attention(q[0, g * G + h].astype(np.float64), kd, vd, 1 / math.sqrt(128))
        t_d += time.perf_counter() - start
        n_d += chunk
        if t_d >= budget_s / 2:
            break
    td = t_d / n_d * n_pages * w.hkv                          # whole decode step
    t_step = tq * n_tiles_step + td
    return t_step, blas_threads, (f"{n_q} of the step's {n_tiles_step} tiles quantized and "
                                  f"{n_d} of its {n_pages * w.hkv} (page, KV head) pairs decoded "
                                  f"({G} query heads, chunks of {chunk} pages), "
                                  f"{t_q + t_d:.1f} s, scaled to the step")


def cpu_baseline_decode(w, n_iters: int, budget_s: float, tail: int, k_bits: int = 4,
                        v_bits: int = 2):
    """The float64 oracle's decode (dequantize each K and V page, then attention of the G query
    heads of a KV head) on a bounded number of pages of sequence 0, KV head 0, scaled to the
    step's pages over all sequences and KV heads."""
    import numpy as np
    from oracle import kvarn_oracle as O
    blas_threads, _ = host_threads()
    nq = 4
    k = w.k_src[:128 * nq].cpu().numpy()
    v = w.v_src[:128 * nq].cpu().numpy()
    tiles_k = np.stack([k[128 * i:128 * (i + 1), 0, :].T for i in range(nq)])
    tiles_v = np.stack([v[128 * i:128 * (i + 1), 0, :].T for i in range(nq)])
    rk = O.quantize_tiles(tiles_k, O.KIND_K, n_iters, k_bits=k_bits)
    rv = O.quantize_tiles(tiles_v, O.KIND_V, n_iters, v_bits=v_bits)
    q = w.step_inputs(0, device="cpu")[0].numpy()
    G = w.hq // w.hkv
    kt = np.asarray(k[:tail, 0, :], np.float64)
    vt = np.asarray(v[:tail, 0, :], np.float64)

    def run(pages):
        kd = np.concatenate([O.dequantize_tiles(rk["codes"][i % nq], rk["r"][i % nq],
                                                rk["s"][i % nq], rk["scale"][i % nq],
                                                rk["zero"][i % nq], O.KIND_K).T
                             for i in range(pages)] + [kt])
        vd = np.concatenate([O.dequantize_tiles(rv["codes"][i % nq], rv["r"][i % nq],
                                                rv["s"][i % nq], rv["scale"][i % nq],
                                                rv["zero"][i % nq], O.KIND_V).T
                             for i in range(pages)] + [vt])
        for h in range(G):
            O.attention(q[0, h].astype(np.float64), kd, vd, 1 / math.sqrt(128))

    # chunks of 256 pages (+ the staged tokens) for about budget_s seconds, or every page of
    # the step once
    total_pages = sum(L // 128 for L in w.prompt_lens) * w.hkv
    done, spent = 0, 0.0
    while done < total_pages and spent < budget_s:
        t0 = time.perf_counter()
        run(256)
        spent += time.perf_counter() - t0
        done += 256
    per_page = spent / done
    return per_page * total_pages, blas_threads, (
        f"oracle decode of {G} query heads over {done} pages in chunks of 256 (+{tail} staged "
        f"tokens each), {spent:.1f} s, scaled to the {total_pages} (sequence, KV head) pages of "
        f"one step")


def cpu_baseline_entry(bytes_step, t_step, threads, sample):
    return {"value": round(bytes_step / t_step / 1e9, 5), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "sample": sample, "seconds_per_step": round(t_step, 3),
            "blas_threads": threads, "host_cpu_count": os.cpu_count(),
            "cores_note": "cores = BLAS threads the oracle's matrix products use; its "
                          "elementwise NumPy work runs on one thread"}


# ----------------------------------------------------------------------------- GPU helpers


def calibration_copy(args, dev):
    """One device copy of --calibration-copy-mb MiB (its HBM counters scale the kernels')."""
    if not args.calibration_copy_mb:
        return
    import torch
    a = torch.empty(args.calibration_copy_mb << 20, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def hbm_read_probe(dev, gib: int = 4, reps: int = 6):
    """GB/s of the streaming-read probe (libkvarn_probe.so) over a gib-GiB buffer, far beyond
    the Infinity Cache: median and best of `reps` launches timed with HIP events on the launch
    stream."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "kv_cache_quantization_tile_amd", "libkvarn_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m kv_cache_quantization_tile_amd.build`")
    lib = ctypes.CDLL(path)
    fn = lib.kvarn_probe_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                   ctypes.c_void_p]
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    grid = 16384
    sink = torch.empty(grid, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = [(ev(), ev()) for _ in range(reps + 1)]
    for e0, e1 in marks:
        e0.record()
        st = fn(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), grid,
                ctypes.c_void_p(stream.cuda_stream))
        e1.record()
        if st != 0:
            raise RuntimeError(f"kvarn_probe_stream_read failed ({st})")
    torch.cuda.synchronize()
    gbps = sorted(nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9 for e0, e1 in marks[1:])
    del buf, sink
    torch.cuda.empty_cache()
    return {"kernel": f"stream_read_kernel (16-byte nontemporal loads, {grid} workgroups x 256 "
                      "lanes, a contiguous block each)",
            "bytes": nbytes, "gbps_median": round(gbps[len(gbps) // 2], 1),
            "gbps_best": round(gbps[-1], 1),
            "frac_of_peak": round(gbps[len(gbps) // 2] / HBM_PEAK_GBPS, 4)}


def valu_calibration(dev, rounds: int = 20000, grid: int = 2048):
    """Cycles one wave64 v_fma_f32 holds a SIMD, from the VALU probe (libkvarn_probe.so): grid
    workgroups of 4 waves (8 waves per SIMD), rounds x 32 FMAs each, best of 4 launches, at
    the nominal 2.4 GHz (a lower clock under load shows as more cycles)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "kv_cache_quantization_tile_amd", "libkvarn_probe.so"))
    fn = lib.kvarn_probe_valu_fma
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    out = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    marks = [(_ev(), _ev()) for _ in range(5)]
    for e0, e1 in marks:
        e0.record()
        if fn(ctypes.c_void_p(out.data_ptr()), grid, rounds, ctypes.c_void_p(stream.cuda_stream)):
            raise RuntimeError("kvarn_probe_valu_fma failed")
        e1.record()
    torch.cuda.synchronize()
    ms = min(e0.elapsed_time(e1) for e0, e1 in marks[1:])
    per_simd = grid * 4 * 32 * rounds / N_SIMD
    tflops = grid * 256 * 32 * rounds * 2 / (ms * 1e-3) / 1e12
    return {"kernel": "valu_fma_kernel (8 independent v_fma_f32 chains per lane, 8 waves per SIMD)",
            "ms": round(ms, 4), "cycles_per_wave64_fma_at_2400MHz": round(ms * 1e-3 * 2.4e9 / per_simd, 3),
            "tflops": round(tflops, 1), "frac_of_fp32_vector_peak": round(tflops / FP32_VECTOR_PEAK_TFLOPS, 4)}


def _ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def timed_steps(step_fns, steps, warmup, first=None):
    """Warm-up (steps 0 .. warmup - 1), then exactly `steps` steps (first .., by default
    following the warm-up) with nothing recorded between launches (an event between two
    kernels keeps the second from dispatching under the first's tail), bracketed by
    synchronizations. step_fns(s) returns the launch groups of step s (callables).
    Returns (ms per step, wall seconds)."""
    import torch
    first = warmup if first is None else first
    # warm-up: the given steps, repeated until at least min_warm_s of GPU work has run (short
    # steps alone leave the clocks ramping when the timed region starts)
    t0 = time.perf_counter()
    while True:
        for s in range(warmup):
            for f in step_fns(s):
                f()
        torch.cuda.synchronize()
        if warmup == 0 or time.perf_counter() - t0 >= MIN_WARM_S[0]:
            break
    start, stop = _ev(), _ev()
    t_wall = time.perf_counter()
    start.record()
    for s in range(steps):
        for f in step_fns(first + s):
            f()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps, time.perf_counter() - t_wall


def evented_steps(step_fns, steps, first):
    """The same steps again with HIP events (on torch's current stream, the launch stream)
    around each launch group; returns per-group lists of ms and per-step totals."""
    import torch
    marks = []
    for s in range(steps):
        groups = step_fns(first + s)
        es = [_ev() for _ in range(len(groups) + 1)]
        es[0].record()
        for f, e in zip(groups, es[1:]):
            f()
            e.record()
        marks.append(es)
    torch.cuda.synchronize()
    n = len(marks[0]) - 1
    per = [[m[i].elapsed_time(m[i + 1]) for m in marks] for i in range(n)]
    tot = [m[0].elapsed_time(m[-1]) for m in marks]
    return per, tot


# ----------------------------------------------------------------------------- workloads


def quantize_and_decode(args, K, synth, params, dev, probe):
    """prefill_burst and one_layer_16k: one K+V quantize launch over every tile of the workload
    plus one decode step over the pages of a copy written earlier (cold), copies cycled."""
    import torch
    n_iters = params.sinkhorn_iters
    k_rec = K.page_bytes(params, K.KIND_K)
    v_rec = K.page_bytes(params, K.KIND_V)
    one_layer = args.workload == "one_layer_16k"
    L = max(2, args.layers or (64 if one_layer else 2))
    print(f"[bench] generating {args.workload} (context {args.context}), {L} page-pool copies",
          file=sys.stderr, flush=True)
    copies = []
    if one_layer:
        # a 64-layer model's per-layer calls: each copy has its own keys and values
        for i in range(L):
            w = synth.one_layer(device=dev, seed=1 + i, context=args.context)
            copies.append(w)
    else:
        w = synth.prefill_burst(device=dev, seed=4, context=args.context, n_iters=n_iters)
        copies = [w] * L
    w0 = copies[0]
    B, hq, hkv, T = w0.batch, w0.hq, w0.hkv, args.context
    seq_lens = torch.tensor(w0.prompt_lens, dtype=torch.int32, device=dev)
    ws = K.new_workspace(params, B, hq, hkv, T)
    out = torch.empty((B, hq, 128), dtype=torch.float16, device=dev)
    calls = []
    for i, w in enumerate(copies):
        q = w.step_inputs(0)[0]
        kp = K.new_pool(w.num_pages, hkv, K.KIND_K, params=params)
        vp = K.new_pool(w.num_pages, hkv, K.KIND_V, params=params)
        qkv = K.prepare_quantize_kv(params, w.k_src, w.v_src, w.tile_src_token,
                                    w.tile_dst_page, kp, vp)
        dc = K.prepare_decode(params, q, kp, vp, w.block_table, seq_lens, T, ws, out)
        calls.append((qkv, dc, kp, vp, q))
    for c in calls:                  # every copy holds valid pages before the first decode
        c[0]()
    torch.cuda.synchronize()
    n_tiles = w0.tile_src_token.numel() * hkv          # per kind
    calibration_copy(args, dev)

    # step s quantizes copy s mod L and decodes copy (s + L/2) mod L, written L/2 steps before
    # (one step before for two copies): the traffic in between evicts its pages
    half = L // 2

    def cold(s):
        return [calls[s % L][0], calls[(s + half) % L][1]]

    def warm(s):
        return [calls[s % L][0], calls[s % L][1]]

    ms_step, t_wall = timed_steps(cold, args.steps, args.warmup)
    (q_list, d_list), tot = evented_steps(cold, args.steps, args.warmup)
    n_warm = min(args.steps, 8)
    (_, dw_list), _ = evented_steps(warm, n_warm, args.warmup)
    q_ms = sum(q_list) / len(q_list)
    d_ms = sum(d_list) / len(d_list)
    dw_ms = sum(dw_list) / len(dw_list)

    # quantize launch at other iteration counts (same tiles, the first pool copy)
    by_iters = {}
    flop_tile = quant_flop_per_tile(n_iters)
    q_bytes = n_tiles * (Q_READ + k_rec) + n_tiles * (Q_READ + v_rec)
    for n in sorted(set(args.sweep_iters) | {n_iters}):
        if n == n_iters:
            t = q_ms
        else:
            p_n = K.params_from_dtype(args.preset, n, format=params.format)
            f = K.prepare_quantize_kv(p_n, w0.k_src, w0.v_src, w0.tile_src_token,
                                      w0.tile_dst_page, calls[0][2], calls[0][3])
            (ts,), _ = evented_steps(lambda s: [f], 4, 0)
            t = sum(ts[1:]) / len(ts[1:])
        fl = 2 * n_tiles * quant_flop_per_tile(n) / (t * 1e-3) / 1e12
        by_iters[str(n)] = {"ms": round(t, 5), "tiles_per_s": round(2 * n_tiles / (t * 1e-3), 1),
                            "hbm_frac": round(q_bytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                            "tflops": round(fl, 2),
                            "frac_of_fp32_vector_peak": round(fl / FP32_VECTOR_PEAK_TFLOPS, 4)}

    # algorithmic bytes
    full_pages = T // 128
    d_bytes = B * hkv * full_pages * (k_rec + v_rec) + 2 * B * hq * 128 * 2
    step_bytes = q_bytes + d_bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    decode_gbps = d_bytes / (d_ms * 1e-3) / 1e9
    decode_warm_gbps = d_bytes / (dw_ms * 1e-3) / 1e9
    src_hash = source_hash()
    q_gbps = q_bytes / (q_ms * 1e-3) / 1e9
    q_tflops = 2 * n_tiles * flop_tile / (q_ms * 1e-3) / 1e12
    quant_roof = {"kernel": "quantize_kv_kernel", "bound": "hbm",
                  "achieved": round(q_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                  "frac": round(q_gbps / HBM_PEAK_GBPS, 4),
                  "traffic": load_traffic("quantize_kv_kernel", src_hash, args.workload),
                  "per_launch": f"{2 * n_tiles} K+V tiles x (32768 B in + {k_rec} / {v_rec} B "
                                f"record out) = {q_bytes} B",
                  "launch_ms": round(q_ms, 5), "launch_ms_pct": percentiles(q_list),
                  "tflops": round(q_tflops, 2),
                  "flop_per_launch": f"{2 * n_tiles} tiles x {flop_tile} FLOP",
                  "frac_of_fp32_vector_peak_157_3": round(q_tflops / FP32_VECTOR_PEAK_TFLOPS, 4)}
    dec_roof = {"kernel": "decode (decode_pages_kernel + decode_merge_kernel), cold pages",
                "bound": "hbm", "achieved": round(decode_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(decode_gbps / HBM_PEAK_GBPS, 4),
                "traffic": load_traffic("decode_pages_kernel", src_hash, args.workload),
                "per_launch": f"{B * hkv * full_pages} K+V page pairs x {k_rec + v_rec} B + q/out "
                              f"= {d_bytes} B",
                "launch_ms": round(d_ms, 5), "launch_ms_pct": percentiles(d_list),
                "frac_of_read_probe": round(decode_gbps / probe["gbps_median"], 4)}
    dominant, other = (quant_roof, dec_roof) if q_ms >= d_ms else (dec_roof, quant_roof)
    if one_layer:
        wl = (f"one_layer_16k: batch 1, 64 q / 8 KV heads, {T} tokens; quantize {2 * n_tiles} "
              f"K+V tiles + 1 decode step, {L} layer copies cycled")
    else:
        wl = (f"prefill_burst: 64 sequences x {T} tokens, 8 KV heads, even heads N(0,1), odd "
              f"Student-t(2.5); quantize {2 * n_tiles} K+V tiles + 1 batched decode step over "
              f"pages written one step earlier (cold)")
    res = {
        "metric": METRIC,
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16 in/out, f32 compute",
        "data": "synthetic",
        "config": {"workload": wl, "batch": B, "num_q_heads": hq, "num_kv_heads": hkv,
                   "head_dim": 128, "context": T, "kv_cache_dtype": args.preset,
                   "sinkhorn_iters": n_iters, "record_format": params.format,
                   "page_pool_copies": L,
                   "parallelism": "single GPU"},
        "timing": "ms_per_step over the timed steps with nothing recorded between launches; "
                  "launch_ms and the percentiles (mean/p10/p50/p90 over the steps) from the same "
                  "steps run again with HIP events around each launch group on the launch stream",
        "value_definition": "algorithmic bytes of one step (quantize: tile in + record out; "
                            "decode: K+V records + q + out) / step time",
        "step_ms_pct": percentiles(tot),
        "quantize_tiles_per_s": round(2 * n_tiles / (q_ms * 1e-3), 1),
        "quantize_ms": round(q_ms, 5),
        "quantize_by_iters": by_iters,
        "decode_kv_gbps": round(decode_gbps, 1),
        "decode_hbm_frac": round(decode_gbps / HBM_PEAK_GBPS, 4),
        "decode_ms": round(d_ms, 5),
        "decode_warm": {"ms": round(dw_ms, 5), "kv_gbps": round(decode_warm_gbps, 1),
                        "hbm_frac": round(decode_warm_gbps / HBM_PEAK_GBPS, 4),
                        "note": "decode of the pages the same step's quantize has just written "
                                "(partly served by the Infinity Cache)"},
        "roofline": dominant,
        "roofline_other": other,
        "hbm_read_probe": probe,
        "wall_s_timed": round(t_wall, 4),
        "source_hash": src_hash,
    }
    if not args.no_cpu_baseline:
        t_step, threads, sample = cpu_baseline(w0, n_iters, args.cpu_budget, params.k_bits,
                                               params.v_bits)
        res["cpu_baseline"] = cpu_baseline_entry(step_bytes, t_step, threads, sample)
    return res


def chunked_prefill(args, K, synth, params, dev, probe):
    """Chunk write (kvarn_write_tokens) + multi-query read (kvarn_chunk_attention), steady state:
    every step rewrites the same 128 positions after the 16384 cached tokens of each of 8
    sequences, so the cache does not grow between steps."""
    import torch
    B, ctx, n = 8, args.context, 128
    w = synth.prefill_burst(device=dev, seed=11, batch=B, context=ctx + n, n_iters=params.sinkhorn_iters)
    hq, hkv = w.hq, w.hkv
    kp = K.new_pool(w.num_pages, hkv, K.KIND_K, params=params)
    vp = K.new_pool(w.num_pages, hkv, K.KIND_V, params=params)
    k_rec = K.page_bytes(params, K.KIND_K)
    v_rec = K.page_bytes(params, K.KIND_V)
    # the prompt: every tile but the last of each sequence; the last is the chunk
    keep = torch.tensor([i for i in range(w.tile_src_token.numel()) if (i + 1) % ((ctx + n) // 128) != 0],
                        dtype=torch.long, device=dev)
    K.quantize_kv_tiles(params, w.k_src, w.v_src, w.tile_src_token[keep].contiguous(),
                        w.tile_dst_page[keep].contiguous(), kp, vp)
    rows = torch.cat([torch.arange(w.seq_start[b] + ctx, w.seq_start[b] + ctx + n, device=dev)
                      for b in range(B)])
    kn, vn = w.k_src[rows].contiguous(), w.v_src[rows].contiguous()
    cu = torch.arange(0, (B + 1) * n, n, dtype=torch.int32, device=dev)
    sl0 = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    sl1 = sl0 + n
    kt = torch.zeros((B, hkv, 128, 128), dtype=torch.float16, device=dev)
    vt = torch.zeros_like(kt)
    q = torch.randn((B * n, hq, 128), generator=torch.Generator(device=dev).manual_seed(12),
                    device=dev).to(torch.float16)
    ws = K.new_chunk_workspace(params, B * n, hq, hkv, ctx + n)
    out = torch.empty_like(q)
    write = lambda: K.write_tokens(params, kn, vn, cu, sl0, kt, vt, w.block_table, kp, vp, n)
    attend = lambda: K.chunk_attention(params, q, cu, kp, vp, w.block_table, sl1, ctx + n, kt,
                                       vt, workspace=ws, out=out)
    calibration_copy(args, dev)
    steps = lambda s: [write, attend]
    ms_step, t_wall = timed_steps(steps, args.steps, args.warmup, first=0)
    (w_list, a_list), tot = evented_steps(steps, args.steps, 0)
    w_ms = sum(w_list) / len(w_list)
    a_ms = sum(a_list) / len(a_list)
    pages = (ctx + n) // 128
    write_bytes = B * hkv * (2 * Q_READ + k_rec + v_rec)                 # chunk in, records out
    unique_kv = B * hkv * pages * (k_rec + v_rec)                      # each page once
    per_row_kv = sum(B * hkv * ((ctx + i + 1) // 128) * (k_rec + v_rec) for i in range(n))
    qo = 2 * B * n * hq * 128 * 2
    attn_flops = sum(B * hq * 4 * 128 * (ctx + i + 1) for i in range(n))   # QK + PV, 2 FLOP/MAC
    value = (write_bytes + unique_kv + qo) / (ms_step * 1e-3) / 1e9
    src_hash = source_hash()
    return {
        "metric": METRIC,
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16 in/out, f32 compute",
        "data": "synthetic",
        "config": {"workload": f"chunked_prefill: {B} sequences x {ctx} cached tokens, "
                               f"{n}-token chunk written and attended per step",
                   "batch": B, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": 128,
                   "context": ctx, "chunk": n, "kv_cache_dtype": args.preset,
                   "sinkhorn_iters": params.sinkhorn_iters, "parallelism": "single GPU"},
        "timing": "ms_per_step over the timed steps with nothing recorded between calls; "
                  "write_ms / attention_ms and percentiles from the same steps run again with "
                  "HIP events around each call",
        "value_definition": "unique algorithmic bytes of one step (chunk in + records out, every "
                            "page read once, q + out) / step time",
        "step_ms_pct": percentiles(tot),
        "chunk_tokens_per_s": round(B * n / (ms_step * 1e-3), 1),
        "write_ms": round(w_ms, 5), "attention_ms": round(a_ms, 5),
        "attention_ms_pct": percentiles(a_list),
        # many query rows per page: attention is a dense contraction, so the bound is the
        # float16 matrix-core peak, priced on the attention's own FLOPs (QK and PV over each
        # row's causal prefix); the page stream per row is reported beside it
        "roofline": {"kernel": "mq_pages_kernel (16 query vectors per wave)", "bound": "mfma",
                     "achieved": round(attn_flops / (a_ms * 1e-3) / 1e12, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_flops / (a_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": load_traffic("mq_pages_kernel", src_hash, "chunked_prefill"),
                     "per_launch": f"{B * n} query rows x {hq} heads x 4 x 128 FLOP per causal "
                                   f"key = {attn_flops / 1e9:.1f} GFLOP",
                     "launch_ms": round(a_ms, 5),
                     "row_page_stream_gbps": round(per_row_kv / (a_ms * 1e-3) / 1e9, 1)},
        "hbm_read_probe": probe,
        "wall_s_timed": round(t_wall, 4),
        "source_hash": src_hash,
    }


def decode_steps(args, K, synth, params, dev, probe, workload=None, steps=None, warmup=None,
                 cpu=True):
    """Decode with appends over a paged cache, the decode-bound workloads. One step appends
    one K/V token per sequence into its float16 staging tile (kvarn_append_tokens; a tile
    that fills is quantized into its page) and then runs decode attention of all query heads
    over the pages and the staging tile (kvarn_decode_attention).
      batched_paged: 32 sequences, lengths U[4096, 32768] rounded to 128, pages placed by a
        random permutation, K/V Student-t(3); ~530 MB of pages per step, larger than the
        256 MB Infinity Cache;
      long_context: one 131072-token sequence (117.5 MB of pages), so `--layers` distinct
        copies (8 by default, as layers of a model) are cycled step by step.
    Every step s starts from prompt length + s: re-running a step (warm-up, the timed pass,
    the pass with events) rewrites the same staging position with the same token. The pages
    a step decodes were written before the timed region (cold)."""
    import torch
    workload = workload or args.workload
    S = steps or args.steps
    W = warmup if warmup is not None else args.warmup
    L = args.layers if (args.layers and workload == args.workload) else (
        8 if workload == "long_context" else 1)
    print(f"[bench] generating {L} copies of {workload}", file=sys.stderr, flush=True)
    k_rec = K.page_bytes(params, K.KIND_K)
    v_rec = K.page_bytes(params, K.KIND_V)
    n_steps = -(-max(S, W) // L)      # steps per copy
    copies = []
    q_launch = None
    for c in range(L):
        if workload == "batched_paged":
            w = synth.batched_paged(device=dev, seed=2 + c, steps=n_steps)
        else:
            w = synth.long_context(device=dev, seed=3 + c, steps=n_steps)
        B, hq, hkv = w.batch, w.hq, w.hkv
        kp = K.new_pool(w.num_pages, hkv, K.KIND_K, params=params)
        vp = K.new_pool(w.num_pages, hkv, K.KIND_V, params=params)
        qkv = K.prepare_quantize_kv(params, w.k_src, w.v_src, w.tile_src_token,
                                    w.tile_dst_page, kp, vp)
        qkv()
        if c == 0:                      # the prompt quantize launch, timed once per rep
            q_launch = (qkv, w.tile_src_token.numel() * hkv)
        bt = w.block_table.clone()
        spare = n_steps // 128 + 1
        for b, Lb in enumerate(w.prompt_lens):      # pages that staging tiles fill into
            for j in range(spare):
                bt[b, Lb // 128 + j] = int(w.free_pages[b + j * B])
        kt = torch.zeros((B, hkv, 128, 128), dtype=torch.float16, device=dev)
        vt = torch.zeros_like(kt)
        base = torch.tensor(w.prompt_lens, dtype=torch.int32, device=dev)
        lens = [base + s for s in range(n_steps + 1)]
        max_len = max(w.prompt_lens) + n_steps
        ws = K.new_workspace(params, B, hq, hkv, max_len)
        out = torch.empty((B, hq, 128), dtype=torch.float16, device=dev)
        steps_c = []
        for s in range(n_steps):
            q, kn, vn = w.step_inputs(s)
            app = K.prepare_append(params, kn, vn, lens[s], kt, vt, bt, kp, vp)
            dec = K.prepare_decode(params, q, kp, vp, bt, lens[s + 1], max_len, ws, out,
                                   k_tail=kt, v_tail=vt)
            steps_c.append((app, dec, q, kn, vn))
        # every buffer the prepared calls point to stays referenced here
        copies.append((w, steps_c, kp, vp, kt, vt, lens, ws, out, bt))
        if c == 0:
            w0 = w
        if c > 0:                       # the prompt sources are no longer needed
            w.k_src = w.k_src[:0]
            w.v_src = w.v_src[:0]
    torch.cuda.synchronize()
    calibration_copy(args, dev)
    B, hq, hkv = w0.batch, w0.hq, w0.hkv

    def step_index(s):
        return (s % L, (s // L) if L > 1 else s)

    def groups(s):
        c, i = step_index(s)
        return list(copies[c][1][i][:2])

    ms_step, t_wall = timed_steps(groups, S, W, first=0)
    (a_list, d_list), tot = evented_steps(groups, S, 0)
    a_ms = sum(a_list) / S
    d_ms = sum(d_list) / S
    # the prompt quantize launch of copy 0 (rewrites the same pages)
    qkv, n_q_tiles = q_launch
    (pq,), _ = evented_steps(lambda s: [qkv], 4, 0)
    pq_ms = min(pq)

    # algorithmic bytes of a step, averaged over the timed steps: K+V records of the full
    # pages, the staged float16 tokens, q and out; the append's token in and staging write
    def dec_bytes(c, i):
        w = copies[c][0]
        tot_b = 0
        for Lb in w.prompt_lens:
            n = Lb + i + 1
            tot_b += hkv * ((n // 128) * (k_rec + v_rec) + 2 * (n % 128) * 256)
        return tot_b + 2 * B * hq * 256
    d_bytes = sum(dec_bytes(*step_index(s)) for s in range(S)) / S
    a_bytes = 2 * 2 * B * hkv * 256
    value = (d_bytes + a_bytes) / (ms_step * 1e-3) / 1e9
    decode_gbps = d_bytes / (d_ms * 1e-3) / 1e9
    src_hash = source_hash()
    pages_step = sum(Lb // 128 for Lb in w0.prompt_lens) * hkv
    res = {
        "metric": METRIC,
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": S,
        "warmup": W, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16 in/out, f32 compute",
        "data": "synthetic",
        "config": {"workload": f"{workload}: append 1 token per sequence + 1 decode step",
                   "batch": B, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": 128,
                   "prompt_tokens": sum(w0.prompt_lens), "kv_cache_dtype": args.preset,
                   "sinkhorn_iters": params.sinkhorn_iters, "record_format": params.format,
                   "copies_cycled": L,
                   "parallelism": "single GPU"},
        "timing": "ms_per_step over the timed steps with nothing recorded between launches; "
                  "append_ms / decode_ms and percentiles from the same steps run again with HIP "
                  "events around each call on the launch stream",
        "value_definition": "algorithmic bytes of one step (decode: K+V records of the full "
                            "pages + staged float16 tokens + q + out; append: token in + "
                            "staging write) / step time",
        "step_ms_pct": percentiles(tot),
        "decode_kv_gbps": round(decode_gbps, 1),
        "decode_hbm_frac": round(decode_gbps / HBM_PEAK_GBPS, 4),
        "decode_frac_of_read_probe": round(decode_gbps / probe["gbps_median"], 4),
        "decode_ms": round(d_ms, 5), "decode_ms_pct": percentiles(d_list),
        "append_ms": round(a_ms, 5),
        "prompt_quantize": {"tiles": 2 * n_q_tiles, "ms": round(pq_ms, 4),
                            "tiles_per_s": round(2 * n_q_tiles / (pq_ms * 1e-3), 1)},
        "roofline": {"kernel": "decode (decode_pages_kernel + decode_merge_kernel)", "bound": "hbm",
                     "achieved": round(decode_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(decode_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic("decode_pages_kernel", src_hash, workload),
                     "per_launch": f"{pages_step} K+V page pairs x {k_rec + v_rec} B + staged "
                                   "tokens + q/out (mean over the timed steps)",
                     "launch_ms": round(d_ms, 5)},
        "hbm_read_probe": probe,
        "wall_s_timed": round(t_wall, 4),
        "source_hash": src_hash,
    }
    if cpu and not args.no_cpu_baseline:
        t_step, threads, sample = cpu_baseline_decode(w0, params.sinkhorn_iters, args.cpu_budget,
                                                      tail=1 + S // 2, k_bits=params.k_bits,
                                                      v_bits=params.v_bits)
        res["cpu_baseline"] = cpu_baseline_entry(d_bytes, t_step, threads, sample)
    return res


def decode_workload_summary(r: dict) -> dict:
    """The keys of a decode-bound workload's line carried on the headline line."""
    return {"workload": r["config"]["workload"], "batch": r["config"]["batch"],
            "prompt_tokens": r["config"]["prompt_tokens"], "steps": r["steps"],
            "copies_cycled": r["config"]["copies_cycled"],
            "decode_ms": r["decode_ms"], "decode_ms_pct": r["decode_ms_pct"],
            "decode_kv_gbps": r["decode_kv_gbps"], "decode_hbm_frac": r["decode_hbm_frac"],
            "decode_frac_of_read_probe": r["decode_frac_of_read_probe"],
            "append_ms": r["append_ms"], "ms_per_step": r["ms_per_step"],
            "traffic": r["roofline"]["traffic"]}


# ----------------------------------------------------------------------------- profiling

# rocprofv3 counter passes: each stays within one pass's hardware limits (at most 8 SQ and 2
# GRBM counters; FETCH_SIZE and WRITE_SIZE in passes of their own)
PMC_PASSES = {
    "f": ["FETCH_SIZE"],
    "w": ["WRITE_SIZE"],
    "i": ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD",
          "SQ_INSTS_VMEM_WR", "SQ_WAVES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
    "a": ["SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_LDS",
          "SQ_LDS_BANK_CONFLICT", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
          "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"],
    "l": ["TCC_HIT_sum", "TCC_MISS_sum"],     # L2 hits and misses, summed over the channels
}
PROFILE_KERNELS = {
    "prefill_burst": ["quantize_kv_kernel", "decode_pages_kernel", "decode_merge_kernel"],
    "one_layer_16k": ["quantize_kv_kernel", "decode_pages_kernel", "decode_merge_kernel"],
    "batched_paged": ["decode_pages_kernel", "decode_merge_kernel", "append_tokens_kernel"],
    "long_context": ["decode_pages_kernel", "decode_merge_kernel", "append_tokens_kernel"],
    "chunked_prefill": ["mq_pages_kernel", "decode_merge_kernel", "write_tiles_kernel",
                        "write_staging_kernel"],
}
PROFILE_FILES = {
    "prefill_burst": "quantize_kv_and_decode_prefill_burst",
    "one_layer_16k": "quantize_kv_and_decode_one_layer_16k",
    "batched_paged": "append_and_decode_batched_paged",
    "long_context": "append_and_decode_long_context",
    "chunked_prefill": "write_tokens_and_mq_read_chunked_prefill",
}
CALIB_MB = 256


def profile_commands(outdir: str = "gpurun_out/prof"):
    """The rocprofv3 commands whose output --reduce-profiles reads (run from the repository
    root on one MI355X with TMPDIR=/tmp; counter passes under a 60 s kill timer)."""
    cmds = []
    bench = "python bench.py --no-cpu-baseline --no-extras --min-warm-s 0 --sweep-iters"
    for wl in WORKLOADS:
        st = "--decode-steps" if wl in ("batched_paged", "long_context") else "--steps"
        cmds.append(f"rocprofv3 --kernel-trace --stats --output-format csv -d {outdir}/t_{wl} "
                    f"-o run -- {bench} --workload {wl} {st} 12 --warmup 4")
        for p, counters in PMC_PASSES.items():
            calib = f" --calibration-copy-mb {CALIB_MB}" if p in ("f", "w") else ""
            cmds.append(f"rocprofv3 --pmc {' '.join(counters)} --output-format csv -d "
                        f"{outdir}/{p}_{wl} -o run -- {bench} --workload {wl} {st} 3 "
                        f"--warmup 1{calib}")
    return cmds


def _short(name: str):
    m = re.search(r"::(\w+)(<|\()", name.replace("(anonymous namespace)", "anon"))
    return m.group(1) if m else None


def _read_counters(d: str):
    """{kernel short name: {counter: [per-dispatch values]}} and the calibration copy's
    {counter: value} from a rocprofv3 --pmc output directory."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    calib = {}
    for r in csv.DictReader(open(files[0])):
        n, c, v = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
        if "kvarn" in n:
            per[_short(n)][c].append(v)
        elif "copy" in n.lower() and v > 50000 and ("rocclr" in n.lower() or "unsigned char" in n):
            calib.setdefault(c, []).append(v)
    return per, calib


def _bench_line(path: str):
    try:
        lines = [l for l in open(path) if l.startswith('{"metric"')]
    except OSError:
        return None
    return json.loads(lines[-1]) if lines else None


def _alg_bytes(wl: str, d: dict):
    """Algorithmic bytes per launch of the kernels a bench line prices."""
    alg = {}
    if d is None:
        return alg
    if wl in ("one_layer_16k", "prefill_burst"):
        for r in (d["roofline"], d["roofline_other"]):
            key = "quantize_kv_kernel" if r["kernel"].startswith("quantize") else "decode_pages_kernel"
            alg[key] = r["achieved"] * 1e9 * r["launch_ms"] * 1e-3
    elif wl in ("batched_paged", "long_context"):
        alg["decode_pages_kernel"] = d["decode_kv_gbps"] * 1e9 * d["decode_ms"] * 1e-3
    return alg


def reduce_profiles(d: str, out_dir: str):
    """Summaries of the rocprofv3 runs of profile_commands() under d into out_dir: one text
    file per workload (trace statistics, HBM traffic, counters), traffic.json (bytes per launch
    for the bench line's roofline.traffic) and counters.json."""
    src = source_hash()
    traffic = {"source_hash": src,
               "note": "HBM bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, "
                       f"separate rocprofv3 --pmc runs) scaled by what the same counters read "
                       f"for a {CALIB_MB} MiB device copy in the same run",
               "workloads": {}}
    counters = {"source_hash": src, "workloads": {}}
    cmds = profile_commands()
    for wl in WORKLOADS:
        tdir = os.path.join(d, f"t_{wl}")
        if not os.path.isdir(tdir):
            continue
        lines = [f"# rocprofv3 summary: {wl} ({PROFILE_FILES[wl]})",
                 f"# source_hash {src}; commands, run from the repository root on one MI355X "
                 "(cd to the root, TMPDIR=/tmp):"]
        lines += [f"#   {c}" for c in cmds if f"_{wl} " in c]
        lines.append(f"#   python bench.py --reduce-profiles {d}")
        stats = glob.glob(os.path.join(tdir, "**", "*kernel_stats.csv"), recursive=True)
        durations = {}
        lines.append(f"{'kernel':28s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}")
        for r in csv.DictReader(open(stats[0])):
            if "kvarn" in r["Name"] and "probe" not in r["Name"]:
                k = _short(r["Name"])
                durations[k] = float(r["AverageNs"]) / 1e3
                lines.append(f"{k:28s} {r['Calls']:>6s} {float(r['AverageNs']) / 1e3:9.2f} "
                             f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}")
        line = _bench_line(os.path.join(tdir + ".log"))
        if line:
            lines.append(f"# bench line of the traced run (times under the tracer): ms_per_step "
                         f"{line['ms_per_step']}")
        # traffic
        fdir, wdir = os.path.join(d, f"f_{wl}"), os.path.join(d, f"w_{wl}")
        if os.path.isdir(fdir) and os.path.isdir(wdir):
            fetch, fcal = _read_counters(fdir)
            write, wcal = _read_counters(wdir)
            copy = CALIB_MB << 20
            if len(fcal.get("FETCH_SIZE", [])) != 1 or len(wcal.get("WRITE_SIZE", [])) != 1:
                raise RuntimeError(f"{wl}: expected one calibration copy, got {fcal} {wcal}")
            ff = copy / (fcal["FETCH_SIZE"][0] * 1024)
            wf = copy / (wcal["WRITE_SIZE"][0] * 1024)
            alg = _alg_bytes(wl, _bench_line(fdir + ".log"))
            ks = {}
            for k in sorted(set(fetch) | set(write)):
                fv = fetch.get(k, {}).get("FETCH_SIZE", [0.0])
                wv = write.get(k, {}).get("WRITE_SIZE", [0.0])
                rb = sum(fv) / len(fv) * 1024 * ff
                wb = sum(wv) / len(wv) * 1024 * wf
                e = {"fetch_kib_raw": round(sum(fv) / len(fv), 2),
                     "write_kib_raw": round(sum(wv) / len(wv), 2),
                     "read_bytes": int(rb), "write_bytes": int(wb), "bytes_per_launch": int(rb + wb)}
                if k in alg:
                    e["algorithmic_bytes"] = int(alg[k])
                    e["ratio_to_algorithmic"] = round((rb + wb) / alg[k], 4)
                ks[k] = e
            traffic["workloads"][wl] = {
                "calibration": {"copy_bytes_each_way": copy,
                                "fetch_kib_raw": fcal["FETCH_SIZE"][0],
                                "write_kib_raw": wcal["WRITE_SIZE"][0],
                                "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
                "kernels": ks}
            lines.append(f"# HBM traffic per launch, FETCH_SIZE x {ff:.4f} + WRITE_SIZE x {wf:.4f} "
                         f"(a {CALIB_MB} MiB device copy in the same run read FETCH "
                         f"{fcal['FETCH_SIZE'][0]:.0f} KiB and WRITE {wcal['WRITE_SIZE'][0]:.0f} KiB):")
            for k, e in ks.items():
                extra = (f"  = {e['ratio_to_algorithmic']:.3f} x algorithmic "
                         f"{e['algorithmic_bytes'] / 1e6:.3f} MB") if "algorithmic_bytes" in e else ""
                lines.append(f"#   {k:24s} read {e['read_bytes'] / 1e6:10.3f} MB  write "
                             f"{e['write_bytes'] / 1e6:9.3f} MB{extra}")
        # SQ counters
        idir, adir = os.path.join(d, f"i_{wl}"), os.path.join(d, f"a_{wl}")
        if os.path.isdir(idir) and os.path.isdir(adir):
            ci, _ = _read_counters(idir)
            ca, _ = _read_counters(adir)
            cw = {}
            lines.append("# SQ counters per dispatch (mean over dispatches; summed over shader "
                         "engines and XCDs). cycles = GRBM_GUI_ACTIVE / 8 XCDs;")
            lines.append(f"#   valu_issue = SQ_INSTS_VALU x {VALU_ISSUE_CYCLES} / (1024 SIMDs x "
                         "cycles): share of the SIMDs' VALU issue slots used, at one wave64 VALU "
                         f"instruction per {VALU_ISSUE_CYCLES} cycles (the rate the VALU probe "
                         "measures for v_fma_f32; MFMA instructions are counted as VALU);")
            lines.append(f"#   valu_busy = SQ_ACTIVE_INST_VALU x {VALU_ISSUE_CYCLES} / (1024 x "
                         "cycles) (SQ_ACTIVE_INST_VALU equals SQ_INSTS_VALU on the probe: one "
                         "count per single-issue instruction, more for multi-cycle ones);")
            lines.append("#   mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 x cycles); "
                         "lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS / 4 (stall "
                         "cycles per LDS-active cycle)")
            for k in PROFILE_KERNELS[wl]:
                if k not in ci or k not in ca:
                    continue
                m = {c: sum(v) / len(v) for c, v in ci[k].items()}
                m.update({c + ("_a" if c == "GRBM_GUI_ACTIVE" else ""): sum(v) / len(v)
                          for c, v in ca[k].items()})
                cyc = m["GRBM_GUI_ACTIVE"] / N_XCC
                cyc_a = m["GRBM_GUI_ACTIVE_a"] / N_XCC
                waves = max(m["SQ_WAVES"], 1.0)
                derived = {
                    "cycles": round(cyc, 1),
                    "clock_mhz_from_trace": round(cyc / durations[k], 1) if k in durations else None,
                    "waves": int(m["SQ_WAVES"]),
                    "valu_per_wave": round(m["SQ_INSTS_VALU"] / waves, 1),
                    "mfma_per_wave": round(m["SQ_INSTS_MFMA"] / waves, 1),
                    "lds_per_wave": round(m["SQ_INSTS_LDS"] / waves, 1),
                    "salu_per_wave": round(m["SQ_INSTS_SALU"] / waves, 1),
                    "vmem_rd_per_wave": round(m["SQ_INSTS_VMEM_RD"] / waves, 1),
                    "vmem_wr_per_wave": round(m["SQ_INSTS_VMEM_WR"] / waves, 1),
                    "valu_issue": round(m["SQ_INSTS_VALU"] * VALU_ISSUE_CYCLES / (N_SIMD * cyc), 4),
                    "valu_busy": round(m["SQ_ACTIVE_INST_VALU"] * VALU_ISSUE_CYCLES / (N_SIMD * cyc_a), 4),
                    "mfma_busy": round(m["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * cyc_a), 4),
                    "lds_conflict": round(m["SQ_LDS_BANK_CONFLICT"] /
                                          max(m["SQ_ACTIVE_INST_LDS"] * 4, 1.0), 4),
                    "lds_conflict_cycles_per_cu": round(m["SQ_LDS_BANK_CONFLICT"] / 256, 1),
                    "raw": {c: round(v, 1) for c, v in m.items()},
                }
                cw[k] = derived
                lines.append(f"#   {k:24s} waves {derived['waves']:8d}  VALU/wave "
                             f"{derived['valu_per_wave']:8.1f}  MFMA/wave {derived['mfma_per_wave']:6.1f}"
                             f"  LDS/wave {derived['lds_per_wave']:6.1f}  valu_issue "
                             f"{derived['valu_issue']:.3f}  valu_busy {derived['valu_busy']:.3f}  "
                             f"mfma_busy {derived['mfma_busy']:.3f}  lds_conflict "
                             f"{derived['lds_conflict']:.4f}")
            # L2 (TCC) hit rate per kernel, from its own pass
            ldir = os.path.join(d, f"l_{wl}")
            if os.path.isdir(ldir):
                cl, _ = _read_counters(ldir)
                lines.append("#   L2: hit_rate = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum) "
                             "per dispatch (requests of 128 bytes)")
                for k in PROFILE_KERNELS[wl]:
                    if k not in cl or k not in cw:
                        continue
                    hit = sum(cl[k]["TCC_HIT_sum"]) / len(cl[k]["TCC_HIT_sum"])
                    miss = sum(cl[k]["TCC_MISS_sum"]) / len(cl[k]["TCC_MISS_sum"])
                    cw[k]["l2_hit_rate"] = round(hit / max(hit + miss, 1.0), 4)
                    cw[k]["raw"].update({"TCC_HIT_sum": round(hit, 1), "TCC_MISS_sum": round(miss, 1)})
                    lines.append(f"#   {k:24s} L2 hits {hit:14.0f}  misses {miss:14.0f}  "
                                 f"hit_rate {cw[k]['l2_hit_rate']:.3f}")
            counters["workloads"][wl] = cw
        path = os.path.join(out_dir, PROFILE_FILES[wl] + ".txt")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))
    with open(os.path.join(out_dir, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    with open(os.path.join(out_dir, "counters.json"), "w") as f:
        json.dump(counters, f, indent=1)


# ----------------------------------------------------------------------------- main


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=None,
                    help="distinct page-pool copies cycled across steps (defeats the 256 MB "
                         "Infinity Cache): 2 for prefill_burst, 64 for one_layer_16k, 8 for "
                         "long_context")
    ap.add_argument("--sinkhorn-iters", type=int, default=8)
    ap.add_argument("--sweep-iters", type=int, nargs="*", default=[2, 4],
                    help="other iteration counts at which the quantize launch is timed")
    ap.add_argument("--preset", default="kvarn_k4v2_g128",
                    choices=[f"kvarn_{w}_g{g}" for g in (128, 64) for w in ("k4v2", "k2v2", "k4v4")],
                    help="kv_cache_dtype preset (the released k4v2_g128 by default)")
    ap.add_argument("--format", type=int, default=1, choices=[1, 2],
                    help="page record format: 1 separate normalizers and scales (default), "
                         "2 folded (each group's normalizer folded into its scale and zero)")
    ap.add_argument("--context", type=int, default=16384)
    ap.add_argument("--workload", choices=WORKLOADS, default="prefill_burst",
                    help="prefill_burst (default, the headline line): 64 sequences x 16384 "
                         "tokens (131072 tiles) + one cold batched decode; one_layer_16k: batch 1 "
                         "one decoder layer; chunked_prefill: 128-token chunks written and "
                         "attended; batched_paged / long_context: append + decode steps")
    ap.add_argument("--decode-steps", type=int, default=128,
                    help="timed steps of the decode-bound workloads (batched_paged, long_context), "
                         "standalone and on the headline line")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the decode-bound workloads on the prefill_burst line")
    ap.add_argument("--min-warm-s", type=float, default=MIN_WARM_S[0],
                    help="repeat the warm-up steps until this much time has passed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="also run one device copy of this size (HBM counter calibration)")
    ap.add_argument("--print-profile-commands", action="store_true",
                    help="print the rocprofv3 commands of the profiling recipe and exit")
    ap.add_argument("--reduce-profiles", metavar="DIR",
                    help="summarize the recipe's rocprofv3 output under DIR into profiles/")
    ap.add_argument("--profiles-out", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()
    MIN_WARM_S[0] = args.min_warm_s
    if args.print_profile_commands:
        print("\n".join(profile_commands()))
        return
    if args.reduce_profiles:
        return reduce_profiles(args.reduce_profiles, args.profiles_out)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path needs no cross-GPU exchange; see the sharding notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from kv_cache_quantization_tile_amd import kvarn as K
    from kv_cache_quantization_tile_amd import synth

    dev = torch.device("cuda:0")
    params = K.params_from_dtype(args.preset, args.sinkhorn_iters, format=args.format)
    probe = hbm_read_probe(dev)
    print(f"[bench] read probe {probe['gbps_median']} GB/s", file=sys.stderr, flush=True)
    valu = valu_calibration(dev)
    if args.workload == "chunked_prefill":
        res = chunked_prefill(args, K, synth, params, dev, probe)
    elif args.workload in ("batched_paged", "long_context"):
        res = decode_steps(args, K, synth, params, dev, probe, steps=args.decode_steps)
    else:
        res = quantize_and_decode(args, K, synth, params, dev, probe)
        if args.workload == "prefill_burst" and not args.no_extras:
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            extra = {}
            for wl in ("batched_paged", "long_context"):
                r = decode_steps(args, K, synth, params, dev, probe, workload=wl,
                                 steps=args.decode_steps, warmup=16, cpu=False)
                extra[wl] = decode_workload_summary(r)
                torch.cuda.synchronize()
                torch.cuda.empty_cache()
            res["decode_workloads"] = extra
    res["valu_fma_probe"] = valu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
