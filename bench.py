#!/usr/bin/env python3
"""Benchmark of the KVarN hot path on one MI355X: tile quantization + paged decode attention.

Workload (one decoder layer of a Qwen3-32B-like model, the pages' measurement shape): batch 1,
64 query / 8 KV heads, head_dim 128, 16384 tokens of float16 K/V (channel magnitudes
lognormal(0,1), 3 outlier channels x10, times N(0,1)); one step = quantize all 2048 K and V
tiles (k4v2_g128, 8 Sinkhorn iterations) into pages, then one decode-attention step of all
64 query heads over those pages. Synthetic data; inputs resident in HBM before timing.

Distinct layer copies (64 by default, as in a 64-layer model) are cycled step by step, so
each step's ~82 MB of inputs and pages are not resident in the 256 MB Infinity Cache.

Prints one JSON line. Numbers:
  value / ms_per_step: whole step (quantize + decode), algorithmic bytes / step time.
  decode_kv_gbps, quantize_tiles_per_s: the two halves, from HIP events around each launch.
  roofline: the dominant kernel (by time) against its bound; roofline_other: the other one.
  cpu_baseline: the float64 CPU oracle on a bounded sample of the same step.

--workload chunked_prefill measures the chunk write and multi-query read path instead: 8
sequences holding 16384 tokens each; one step writes a 128-token chunk per sequence (one tile
completed and quantized per sequence and head) and runs causal attention for its 1024 query
rows over the quantized cache.

--workload batched_paged (32 sequences, lengths U[4096, 32768] in permuted pages) and
--workload long_context (one 131072-token sequence, 8 copies cycled) measure the decode-bound
steps: append one token per sequence into staging (quantize-on-fill), then decode attention
over the pages and the staging tile; the roofline is the decode's HBM fraction.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Algorithmic work units (what the method must move / compute, not what the kernels do)
Q_READ = 128 * 128 * 2                 # float16 tile in
HBM_PEAK_GBPS = 8000.0                 # MI355X HBM3E
# fp32 FMA on the vector ALUs without packed-FP32 forms: 256 CU x 4 SIMD x 16 lanes x 2 x 2.4 GHz
ALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
MFMA_F16_PEAK_TFLOPS = 2500.0          # MI355X dense float16 matrix cores


def quant_flop_per_tile(n_iters: int) -> int:
    """FWHT-128 (7 x 16384 add/sub) + per iteration two moment passes in each direction
    (4 x 16384 FMA = 131072 FLOP) + RTN (~131072: min/max, scale, round)."""
    return 7 * 16384 + n_iters * 131072 + 131072


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_quantization_tile_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
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


def cpu_baseline(w, n_iters: int, budget_s: float, k_bits: int = 4, v_bits: int = 2):
    """The float64 oracle on a time-bounded sample of one step, scaled to the whole step: tiles
    of the step quantized in batches of 16 (one KV head and kind per batch, in step order)
    for about budget_s / 2 seconds or until every tile of the step is done, then the decode
    (dequantize the pages, attention of every query head of the group) of chunks of pages for
    about budget_s / 2 seconds or until every (page, KV head) pair of the step is done."""
    import numpy as np
    from oracle import kvarn_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    k = w.k_src.cpu().numpy()
    v = w.v_src.cpu().numpy()
    q = w.step_inputs(0, device="cpu")[0].numpy()
    T = k.shape[0]
    n_pages = T // 128
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=None,
                    help="distinct layer copies cycled across steps (defeats the 256 MB MALL); "
                         "64 for one_layer_16k, 8 for long_context")
    ap.add_argument("--sinkhorn-iters", type=int, default=8)
    ap.add_argument("--preset", default="kvarn_k4v2_g128", choices=["kvarn_k4v2_g128", "kvarn_k2v2_g128", "kvarn_k4v4_g128"],
                    help="kv_cache_dtype preset (the released k4v2_g128 by default)")
    ap.add_argument("--context", type=int, default=16384)
    ap.add_argument("--workload", choices=["one_layer_16k", "prefill_burst", "chunked_prefill",
                                           "batched_paged", "long_context"],
                    default="one_layer_16k",
                    help="one_layer_16k: batch 1 one decoder layer (default, the headline line); "
                         "prefill_burst: 64 sequences x 16384 tokens (131072 tiles) + one batched "
                         "decode; chunked_prefill: 128-token chunks written and attended; "
                         "batched_paged / long_context: append + decode steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="also run one device copy of this size (HBM counter calibration)")
    args = ap.parse_args()
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
    n_iters = args.sinkhorn_iters
    params = K.params_from_dtype(args.preset, n_iters)
    if args.workload == "chunked_prefill":
        return chunked_prefill(args, K, synth, params, dev)
    if args.workload in ("batched_paged", "long_context"):
        return decode_steps(args, K, synth, params, dev)
    k_rec = K.page_bytes(params, K.KIND_K)
    v_rec = K.page_bytes(params, K.KIND_V)
    L = max(1, args.layers or 64) if args.workload == "one_layer_16k" else 1
    print(f"[bench] generating {L} copies of {args.workload} (context {args.context})",
          file=sys.stderr, flush=True)
    layers = []
    for i in range(L):
        if args.workload == "one_layer_16k":
            w = synth.one_layer(device=dev, seed=1 + i, context=args.context)
        else:
            w = synth.prefill_burst(device=dev, seed=4 + i, context=args.context, n_iters=n_iters)
        q = w.step_inputs(0)[0]
        n_pages = w.num_pages
        kp = K.new_pool(n_pages, w.hkv, K.KIND_K, params=params)
        vp = K.new_pool(n_pages, w.hkv, K.KIND_V, params=params)
        layers.append((w, q, kp, vp))
    w0 = layers[0][0]
    B, hq, hkv, T = w0.batch, w0.hq, w0.hkv, args.context
    seq_lens = torch.tensor(w0.prompt_lens, dtype=torch.int32, device=dev)
    ws = K.new_workspace(params, B, hq, hkv, T)
    out = torch.empty((B, hq, 128), dtype=torch.float16, device=dev)
    calls = []
    for (w, q, kp, vp) in layers:
        qkv = K.prepare_quantize_kv(params, w.k_src, w.v_src, w.tile_src_token, w.tile_dst_page,
                                    kp, vp)
        dc = K.prepare_decode(params, q, kp, vp, w.block_table, seq_lens, T, ws, out)
        calls.append((qkv, dc))
    n_tiles = w0.tile_src_token.numel() * hkv          # per kind
    torch.cuda.synchronize()

    calibration_copy(args, dev)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    # warmup
    for s in range(args.warmup):
        qkv, dc = calls[s % L]
        qkv(); dc()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, nothing recorded between the launches (an event
    # between two kernels keeps the second from dispatching under the first's tail)
    start, stop = ev(), ev()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for s in range(args.steps):
        qkv, dc = calls[(args.warmup + s) % L]
        qkv(); dc()
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / args.steps
    # the same steps again with events around each launch group: the per-kernel launch times
    marks = [(ev(), ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        qkv, dc = calls[(args.warmup + s) % L]
        e0, e1, e2 = marks[s]
        e0.record(); qkv(); e1.record(); dc(); e2.record()
    torch.cuda.synchronize()
    q_ms = sum(m[0].elapsed_time(m[1]) for m in marks) / args.steps      # 1 K+V quantize launch
    d_ms = sum(m[1].elapsed_time(m[2]) for m in marks) / args.steps      # decode launches

    # algorithmic bytes
    q_bytes = n_tiles * (Q_READ + k_rec) + n_tiles * (Q_READ + v_rec)
    full_pages = T // 128
    d_bytes = B * hkv * full_pages * (k_rec + v_rec) + 2 * B * hq * 128 * 2
    step_bytes = q_bytes + d_bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    tiles_per_s = 2 * n_tiles / (q_ms * 1e-3)
    decode_gbps = d_bytes / (d_ms * 1e-3) / 1e9

    src_hash = source_hash()
    flop_tile = quant_flop_per_tile(n_iters)
    q_launch_ms = q_ms
    q_achieved = 2 * n_tiles * flop_tile / (q_launch_ms * 1e-3) / 1e12
    quant_roof = {"kernel": "quantize_kv_kernel", "bound": "alu",
                  "achieved": round(q_achieved, 2), "peak": round(ALU_PEAK_TFLOPS, 1),
                  "unit": "TFLOP/s", "frac": round(q_achieved / ALU_PEAK_TFLOPS, 4),
                  "traffic": load_traffic("quantize_kv_kernel", src_hash, args.workload),
                  "hbm_gbps": round(q_bytes / (q_launch_ms * 1e-3) / 1e9, 1),
                  # the published fp32 vector figure counts packed-FP32 forms, kept out of the
                  # library's code: the fraction of it, for reference
                  "frac_of_packed_fp32_peak": round(q_achieved / (2 * ALU_PEAK_TFLOPS), 4),
                  "per_launch": f"{2 * n_tiles} K+V tiles x {flop_tile} FLOP",
                  "launch_ms": round(q_launch_ms, 5)}
    dec_roof = {"kernel": "decode (pages + merge)", "bound": "hbm",
                "achieved": round(decode_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(decode_gbps / HBM_PEAK_GBPS, 4),
                "traffic": load_traffic("decode_pages_kernel", src_hash, args.workload),
                "per_launch": f"{B * hkv * full_pages} K+V page pairs x {k_rec + v_rec} B + q/out",
                "launch_ms": round(d_ms, 5)}
    dominant, other = (quant_roof, dec_roof) if q_ms >= d_ms else (dec_roof, quant_roof)

    res = {
        "metric": "decode-attn KV GB/s (% HBM roofline) + tiles quantized/s, k4v2_g128",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16 in/out, f32 compute",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: quantize {2 * n_tiles} K+V tiles + 1 decode step",
                   "batch": B, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": 128,
                   "context": T, "kv_cache_dtype": args.preset, "sinkhorn_iters": n_iters,
                   "layer_copies_cycled": L, "parallelism": "single GPU"},
        "timing": "ms_per_step over the timed steps with nothing recorded between launches; "
                  "launch_ms (roofline) from the same steps run again with HIP events around "
                  "each launch group on the launch stream",
        "value_definition": "algorithmic bytes of one step (quantize: tile in + record out; "
                            "decode: K+V records + q + out) / step time",
        "decode_kv_gbps": round(decode_gbps, 1),
        "decode_hbm_frac": round(decode_gbps / HBM_PEAK_GBPS, 4),
        "decode_ms": round(d_ms, 5),
        "quantize_tiles_per_s": round(tiles_per_s, 1),
        "quantize_ms": round(q_ms, 5),
        "roofline": dominant,
        "roofline_other": other,
        "wall_s_timed": round(t_wall, 4),
        "source_hash": src_hash,
    }
    if not args.no_cpu_baseline:
        t_step, cores, sample = cpu_baseline(w0, n_iters, args.cpu_budget, params.k_bits, params.v_bits)
        res["cpu_baseline"] = {"value": round(step_bytes / t_step / 1e9, 5), "unit": "GB/s",
                               "cores": cores, "kind": "oracle", "sample": sample,
                               "seconds_per_step": round(t_step, 3)}
    print(json.dumps(res), flush=True)


def chunked_prefill(args, K, synth, params, dev):
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
    step = lambda: (K.write_tokens(params, kn, vn, cu, sl0, kt, vt, w.block_table, kp, vp, n),
                    K.chunk_attention(params, q, cu, kp, vp, w.block_table, sl1, ctx + n, kt, vt,
                                      workspace=ws, out=out))
    calibration_copy(args, dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: the steps alone; then the same steps with events around each call
    start, stop = ev(), ev()
    t_wall = time.perf_counter()
    start.record()
    for s in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / args.steps
    marks = [(ev(), ev(), ev()) for _ in range(args.steps)]
    for s in range(args.steps):
        e0, e1, e2 = marks[s]
        e0.record()
        K.write_tokens(params, kn, vn, cu, sl0, kt, vt, w.block_table, kp, vp, n)
        e1.record()
        K.chunk_attention(params, q, cu, kp, vp, w.block_table, sl1, ctx + n, kt, vt,
                          workspace=ws, out=out)
        e2.record()
    torch.cuda.synchronize()
    w_ms = sum(m[0].elapsed_time(m[1]) for m in marks) / args.steps
    a_ms = sum(m[1].elapsed_time(m[2]) for m in marks) / args.steps
    pages = (ctx + n) // 128
    write_bytes = B * hkv * (2 * Q_READ + k_rec + v_rec)                 # chunk in, records out
    unique_kv = B * hkv * pages * (k_rec + v_rec)                      # each page once
    per_row_kv = sum(B * hkv * ((ctx + i + 1) // 128) * (k_rec + v_rec) for i in range(n))
    qo = 2 * B * n * hq * 128 * 2
    attn_flops = sum(B * hq * 4 * 128 * (ctx + i + 1) for i in range(n))   # QK + PV, 2 FLOP/MAC
    value = (write_bytes + unique_kv + qo) / (ms_step * 1e-3) / 1e9
    res = {
        "metric": "decode-attn KV GB/s (% HBM roofline) + tiles quantized/s, k4v2_g128",
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
                  "write_ms / attention_ms from the same steps run again with HIP events around "
                  "each call",
        "value_definition": "unique algorithmic bytes of one step (chunk in + records out, every "
                            "page read once, q + out) / step time",
        "chunk_tokens_per_s": round(B * n / (ms_step * 1e-3), 1),
        "write_ms": round(w_ms, 5), "attention_ms": round(a_ms, 5),
        # many query rows per page: attention is a dense contraction, so the bound is the
        # float16 matrix-core peak, priced on the attention's own FLOPs (QK and PV over each
        # row's causal prefix); the page stream per row is reported beside it
        "roofline": {"kernel": "mq_pages_kernel (16 query vectors per wave)", "bound": "mfma",
                     "achieved": round(attn_flops / (a_ms * 1e-3) / 1e12, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_flops / (a_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": load_traffic("mq_pages_kernel", source_hash(), "chunked_prefill"),
                     "per_launch": f"{B * n} query rows x {hq} heads x 4 x 128 FLOP per causal "
                                   f"key = {attn_flops / 1e9:.1f} GFLOP",
                     "launch_ms": round(a_ms, 5),
                     "row_page_stream_gbps": round(per_row_kv / (a_ms * 1e-3) / 1e9, 1)},
        "wall_s_timed": round(t_wall, 4),
        "source_hash": source_hash(),
    }
    print(json.dumps(res), flush=True)


def cpu_baseline_decode(w, n_iters: int, budget_s: float, tail: int, k_bits: int = 4,
                        v_bits: int = 2):
    """The float64 oracle's decode (dequantize each K and V page, then attention of the G query
    heads of a KV head) on a bounded number of pages of sequence 0, KV head 0, scaled to the
    step's pages over all sequences and KV heads."""
    import numpy as np
    from oracle import kvarn_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
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


def decode_steps(args, K, synth, params, dev):
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
    the pass with events) rewrites the same staging position with the same token."""
    import torch
    S = args.steps
    L = args.layers if args.layers else (8 if args.workload == "long_context" else 1)
    print(f"[bench] generating {L} copies of {args.workload}", file=sys.stderr, flush=True)
    k_rec = K.page_bytes(params, K.KIND_K)
    v_rec = K.page_bytes(params, K.KIND_V)
    n_steps = -(-max(S, args.warmup) // L)      # steps per copy
    copies = []
    q_launch = None
    for c in range(L):
        if args.workload == "batched_paged":
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
        steps = []
        for s in range(n_steps):
            q, kn, vn = w.step_inputs(s)
            app = K.prepare_append(params, kn, vn, lens[s], kt, vt, bt, kp, vp)
            dec = K.prepare_decode(params, q, kp, vp, bt, lens[s + 1], max_len, ws, out,
                                   k_tail=kt, v_tail=vt)
            steps.append((app, dec, q, kn, vn))
        # every buffer the prepared calls point to stays referenced here
        copies.append((w, steps, kp, vp, kt, vt, lens, ws, out, bt))
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

    ev = lambda: torch.cuda.Event(enable_timing=True)
    for s in range(args.warmup):
        c, i = step_index(s)
        app, dec = copies[c][1][i][:2]
        app(); dec()
    torch.cuda.synchronize()
    start, stop = ev(), ev()
    t_wall = time.perf_counter()
    start.record()
    for s in range(S):
        c, i = step_index(s)
        app, dec = copies[c][1][i][:2]
        app(); dec()
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / S
    marks = [(ev(), ev(), ev()) for _ in range(S)]
    torch.cuda.synchronize()
    for s in range(S):
        c, i = step_index(s)
        app, dec = copies[c][1][i][:2]
        e0, e1, e2 = marks[s]
        e0.record(); app(); e1.record(); dec(); e2.record()
    torch.cuda.synchronize()
    a_ms = sum(m[0].elapsed_time(m[1]) for m in marks) / S
    d_ms = sum(m[1].elapsed_time(m[2]) for m in marks) / S
    # the prompt quantize launch of copy 0 (rewrites the same pages)
    qkv, n_q_tiles = q_launch
    qe = [(ev(), ev()) for _ in range(4)]
    for e0, e1 in qe:
        e0.record(); qkv(); e1.record()
    torch.cuda.synchronize()
    pq_ms = min(e0.elapsed_time(e1) for e0, e1 in qe)

    # algorithmic bytes of a step, averaged over the timed steps: K+V records of the full
    # pages, the staged float16 tokens, q and out; the append's token in and staging write
    def dec_bytes(c, i):
        w = copies[c][0]
        tot = 0
        for Lb in w.prompt_lens:
            n = Lb + i + 1
            tot += hkv * ((n // 128) * (k_rec + v_rec) + 2 * (n % 128) * 256)
        return tot + 2 * B * hq * 256
    d_bytes = sum(dec_bytes(*step_index(s)) for s in range(S)) / S
    a_bytes = 2 * 2 * B * hkv * 256
    value = (d_bytes + a_bytes) / (ms_step * 1e-3) / 1e9
    decode_gbps = d_bytes / (d_ms * 1e-3) / 1e9
    src_hash = source_hash()
    pages_step = sum(Lb // 128 for Lb in w0.prompt_lens) * hkv
    res = {
        "metric": "decode-attn KV GB/s (% HBM roofline) + tiles quantized/s, k4v2_g128",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": S,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16 in/out, f32 compute",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: append 1 token per sequence + 1 decode step",
                   "batch": B, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": 128,
                   "prompt_tokens": sum(w0.prompt_lens), "kv_cache_dtype": args.preset,
                   "sinkhorn_iters": params.sinkhorn_iters, "copies_cycled": L,
                   "parallelism": "single GPU"},
        "timing": "ms_per_step over the timed steps with nothing recorded between launches; "
                  "append_ms / decode_ms from the same steps run again with HIP events around "
                  "each call on the launch stream",
        "value_definition": "algorithmic bytes of one step (decode: K+V records of the full "
                            "pages + staged float16 tokens + q + out; append: token in + "
                            "staging write) / step time",
        "decode_kv_gbps": round(decode_gbps, 1),
        "decode_hbm_frac": round(decode_gbps / HBM_PEAK_GBPS, 4),
        "decode_ms": round(d_ms, 5), "append_ms": round(a_ms, 5),
        "prompt_quantize": {"tiles": 2 * n_q_tiles, "ms": round(pq_ms, 4),
                            "tiles_per_s": round(2 * n_q_tiles / (pq_ms * 1e-3), 1)},
        "roofline": {"kernel": "decode (pages + merge)", "bound": "hbm",
                     "achieved": round(decode_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(decode_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic("decode_pages_kernel", src_hash, args.workload),
                     "per_launch": f"{pages_step} K+V page pairs x {k_rec + v_rec} B + staged "
                                   "tokens + q/out (mean over the timed steps)",
                     "launch_ms": round(d_ms, 5)},
        "wall_s_timed": round(t_wall, 4),
        "source_hash": src_hash,
    }
    if not args.no_cpu_baseline:
        t_step, cores, sample = cpu_baseline_decode(w0, params.sinkhorn_iters, args.cpu_budget,
                                                    tail=1 + S // 2, k_bits=params.k_bits,
                                                    v_bits=params.v_bits)
        res["cpu_baseline"] = {"value": round(d_bytes / t_step / 1e9, 5), "unit": "GB/s",
                               "cores": cores, "kind": "oracle", "sample": sample,
                               "seconds_per_step": round(t_step, 3)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
