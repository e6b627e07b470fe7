#!/usr/bin/env python3
"""Throughput of the DSA lightning indexer forward pass on one MI355X.

Default workload (the headline): one full indexer layer over one causal sequence of
T = 65,536 tokens -- q/k/w projections from x [T,7168] and c_q [T,1536], then causal scores
I = sum_h w_h ReLU(q_h . k) over the whole prefix and the top 2,048 keys per query, with no
T x T score matrix stored.  One step = dsa_idx_project + dsa_idx_score_topk on resident
inputs.  `value` is queries/s.

Also reported on the same line (each with median and min over its timed iterations):
  * roofline of the dominant kernel (the score-and-filter pass of dsa_idx_score_topk) against
    the bf16 MFMA peak: its duration from HIP events the library records around it on the
    stream it runs on (diagnostic phase timing), and the phases of the call;
  * the other workloads: scores + top-k only at T = 2,560; the full layer at T = 8,192; 24
    indexer layers (own weights each) over 16 ragged sequences of log-uniform length in
    [2,048, 32,768];
  * the decode leg: 64 sequences with cached bf16 keys of U[32768, 131072] tokens, one new
    query each (project + decode), as HBM GB/s of the decode kernels; the FP8-cache and
    64-head decodes and the sparse-MLA consumer beside it;
  * the chunked-prefill leg and the 64-head (DeepSeek-V3.2-shaped) layer;
  * a measured device-copy rate (the HBM rate a plain read+write reaches on this machine);
  * cpu_baseline: the fp64 CPU oracle on a bounded sample of the same workload, with the
    extrapolation to the full layer.

Inputs are seeded synthetic tensors with the shapes and distributions of the workloads
(x, c_q ~ N(0,1); W_q ~ N(0,1/1536); W_k, W_w ~ N(0,1/7168); LayerNorm gain 1 + N(0,0.02),
bias N(0,0.02), eps 1e-6; q, k ~ N(0,1) and w ~ N(0,0.1) for the score-only case; all bf16).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (published)
# HBM bytes per launch of the score-and-filter pass at T=65536, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE scaled by a 1 GiB device-copy calibration; reported only while the kernel
# source is the one the counters were taken on (None: not measured for this source)
TRAFFIC_FILTER_T65536 = {"source_sha256_prefix": "bb1dc1f08911e03b", "bytes": 3229462775}
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E (published)
H, D, QLAT, HIDDEN = 32, 128, 1536, 7168
MLA_HEADS, MLA_KV, MLA_V = 96, 576, 512          # the sparse MLA consumer (gated-MLA row)
V32_H = 64                                        # the DeepSeek-V3.2-shaped indexer
PROJ_FLOP_PER_TOKEN = 2 * (QLAT * 4096 + HIDDEN * D + HIDDEN * H)   # 14,876,672
SCORE_FLOP_PER_PAIR = 2 * H * D                                     # 8,192


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--T", type=int, default=65536)
    p.add_argument("--topk", type=int, default=2048)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--decode-batch", type=int, default=64)
    p.add_argument("--no-chunk", action="store_true")
    p.add_argument("--no-mla", action="store_true")
    p.add_argument("--no-v32", action="store_true")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the score-only T=2560, layer T=8192 and 24-layer ragged legs")
    p.add_argument("--chunk", type=int, default=4096)
    p.add_argument("--window", type=int, default=1048576)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    return p.parse_args()


def dev_bf16(a):
    import torch
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def filter_traffic(args):
    src = os.path.join(ROOT, "sparse_attention_token_idx_amd", "csrc", "prefill.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if args.T == 65536 and args.topk == 2048 and h == TRAFFIC_FILTER_T65536["source_sha256_prefix"]:
        return TRAFFIC_FILTER_T65536["bytes"]
    return None


def stats(v):
    v = np.asarray(v, np.float64)
    return dict(median=round(float(np.median(v)), 4), min=round(float(np.min(v)), 4),
                mean=round(float(np.mean(v)), 4))


def timed(step, n, stream, nev):
    """Runs step(events) n times with nev events each; returns the per-interval times [n][nev-1]."""
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(n)]
    for i in range(n):
        step(evs[i])
    torch.cuda.synchronize()
    return [[e[j].elapsed_time(e[j + 1]) for j in range(nev - 1)] for e in evs]


def phase_split(dsa, steps):
    """Per-call milliseconds of the phases recorded since phase_timing(True)."""
    t = dsa.phase_times()
    return {k: round(ms / steps, 4) for k, (ms, n) in t.items() if n > 0}


def bench_layer(dsa, args, T, steps, warmup, label):
    """One indexer layer (project + score_topk) over one causal sequence of T tokens."""
    import torch
    from synth import workloads as wl
    topk = args.topk
    t0 = time.time()
    Wt = wl.layer_weights(layer=0, seed=0)
    act = wl.layer_activations(T, seed=0)
    log(f"{label}: generated inputs T={T} in {time.time() - t0:.1f}s")
    W = {k: dev_bf16(v) for k, v in Wt.items() if k != "eps"}
    W["eps"] = Wt["eps"]
    x, cq = dev_bf16(act["x"]), dev_bf16(act["c_q"])
    del act
    q = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((T, topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((T, topk), dtype=torch.float32, device="cuda")
    ws = torch.empty(dsa.workspace_size(dsa.OP_SCORE_TOPK, T, topk=topk), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dsa.project(x, cq, W, q=q, k_out=k, w=w)
        if ev is not None:
            ev[1].record(stream)
        dsa.score_topk(q, k, w, topk=topk, ws=ws, out=(idx, sc))
        if ev is not None:
            ev[2].record(stream)

    for i in range(warmup):
        step()
        torch.cuda.synchronize()
    log(f"{label}: {warmup} warmup steps done")
    dsa.phase_timing(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    times = timed(step, steps, stream, 3)
    wall = time.perf_counter() - t0
    phases = phase_split(dsa, steps)
    dsa.phase_timing(False)
    dsa.workspace_status(ws)
    proj = [t[0] for t in times]
    st = [t[1] for t in times]
    step_ms = [a + b for a, b in times]
    pairs = T * (T + 1) // 2
    log(f"{label}: {steps} steps in {wall:.3f}s; project {np.median(proj):.3f} ms, "
        f"score_topk {np.median(st):.3f} ms (median); phases {phases}")
    del ws, x, cq
    return dict(T=T, wall=wall, proj=stats(proj), score_topk=stats(st), step=stats(step_ms), phases=phases,
                pairs=pairs, score_flop=pairs * SCORE_FLOP_PER_PAIR, proj_flop=T * PROJ_FLOP_PER_TOKEN)


def bench_score_only(dsa, args, T=2560, steps=50):
    """Scores + top-k only over one causal sequence (q, k ~ N(0,1), w ~ N(0,0.1), seed 0)."""
    import torch
    from synth import workloads as wl
    topk = args.topk
    s = wl.score_inputs(T, seed=0)
    q, k, w = dev_bf16(s["q"]), dev_bf16(s["k"]), dev_bf16(s["w"])
    idx = torch.empty((T, topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((T, topk), dtype=torch.float32, device="cuda")
    ws = torch.empty(dsa.workspace_size(dsa.OP_SCORE_TOPK, T, topk=topk), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dsa.score_topk(q, k, w, topk=topk, ws=ws, out=(idx, sc))
        if ev is not None:
            ev[1].record(stream)

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)   # the calls queue up ahead of the GPU: events time the GPU
    times = [t[0] for t in timed(step, steps, stream, 2)]
    pairs = T * (T + 1) // 2
    log(f"score only T={T}: {np.median(times):.4f} ms median, {np.min(times):.4f} ms min")
    return dict(T=T, ms=stats(times), pairs=pairs, score_flop=pairs * SCORE_FLOP_PER_PAIR)


def bench_varlen_layers(dsa, args, layers=24, steps=3):
    """24 indexer layers, each with its own weights, over 16 ragged sequences (lengths
    log-uniform in [2048, 32768]): per layer project + score_topk_varlen."""
    import torch
    from synth import workloads as wl
    topk = args.topk
    B = 16
    lens = wl.varlen_lengths(B, seed=0)
    cu = wl.cu_seqlens(lens)
    total = int(cu[-1])
    t0 = time.time()
    act = wl.layer_activations(total, seed=0)
    x, cq = dev_bf16(act["x"]), dev_bf16(act["c_q"])
    del act
    Ws = []
    for layer in range(layers):
        Wt = wl.layer_weights(layer=layer, seed=0)
        W = {k: dev_bf16(v) for k, v in Wt.items() if k != "eps"}
        W["eps"] = Wt["eps"]
        Ws.append(W)
    log(f"varlen: {layers} layers, {B} sequences, {total} tokens: inputs in {time.time() - t0:.1f}s")
    cu_d = torch.from_numpy(cu).cuda()
    maxL = int(lens.max())
    q = torch.empty((total, H, D), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((total, D), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((total, H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((total, topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((total, topk), dtype=torch.float32, device="cuda")
    ws = torch.empty(dsa.workspace_size(dsa.OP_SCORE_TOPK_VARLEN, total, B, maxL, topk), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        for W in Ws:
            dsa.project(x, cq, W, q=q, k_out=k, w=w)
            dsa.score_topk_varlen(q, k, w, cu_d, maxL, topk=topk, ws=ws, out=(idx, sc))
        if ev is not None:
            ev[1].record(stream)

    step()
    torch.cuda.synchronize()
    times = [t[0] for t in timed(step, steps, stream, 2)]
    dsa.workspace_status(ws)
    pairs = int(sum(L * (L + 1) // 2 for L in lens.tolist()))
    flop = layers * (pairs * SCORE_FLOP_PER_PAIR + total * PROJ_FLOP_PER_TOKEN)
    log(f"varlen: {layers} layers in {np.median(times):.2f} ms median "
        f"({flop / (np.median(times) * 1e-3) / 1e12:.1f} TFLOP/s)")
    del ws, x, cq
    return dict(layers=layers, B=B, total=total, ms=stats(times), pairs_per_layer=pairs, flop=flop)


def copy_rate(n_bytes=1 << 30, steps=10):
    """GB/s of a plain device-to-device copy (bytes read + bytes written per second)."""
    import torch
    src = torch.empty(n_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del src, dst
    return round(2 * n_bytes / (ms * 1e-3) / 1e9, 1)


def mfma_rate(dsa, iters=6000, steps=5):
    """Sustained bf16 MFMA rate of this device (TFLOP/s): the library's calibration kernel, 16
    independent products per wave on register operands, zero and random bf16 operands (the
    matrix cores' power, hence the clock, depends on the data); median of `steps` launches."""
    import torch
    out = {}
    stream = torch.cuda.current_stream()
    for name, rnd in (("random_operands", True), ("zero_operands", False)):
        flop, sink = dsa.mfma_calibrate(iters, random_operands=rnd)
        torch.cuda.synchronize()
        t = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dsa.mfma_calibrate(iters, random_operands=rnd, sink=sink)
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1))
        out[name] = round(flop / (float(np.median(t)) * 1e-3) / 1e12, 1)
    return out


def vendor_q_gemm(T, steps=10):
    """A yardstick, not part of the path: torch.matmul (the vendor BLAS) on the q projection's
    shape, [T, 1536] x [1536, 4096] bf16 with the weights K-contiguous as the library keeps
    them, random normal operands; median and min of `steps` calls, ms."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(T, QLAT, device="cuda", generator=g).to(torch.bfloat16)
    bt = (torch.randn(4096, QLAT, device="cuda", generator=g) / QLAT ** 0.5).to(torch.bfloat16)
    for _ in range(3):
        a @ bt.t()
    torch.cuda.synchronize()
    t = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        a @ bt.t()
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1))
    del a, bt
    return stats(t)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def bench_decode(dsa, args):
    import torch
    from synth import workloads as wl
    B, topk = args.decode_batch, args.topk
    lens = wl.decode_lengths(B, seed=0)
    t0 = time.time()
    cache, start = wl.decode_cache(lens, seed=0)
    Wt = wl.layer_weights(layer=0, seed=1)
    act = wl.layer_activations(B, seed=1)
    log(f"decode: generated {cache.shape[0]} cached keys in {time.time() - t0:.1f}s")
    W = {k: dev_bf16(v) for k, v in Wt.items() if k != "eps"}
    W["eps"] = Wt["eps"]
    cache_d = dev_bf16(cache)
    del cache
    x, cq = dev_bf16(act["x"]), dev_bf16(act["c_q"])
    start_d = torch.from_numpy(start).cuda()
    lens_d = torch.from_numpy(lens.astype(np.int32)).cuda()
    slots = torch.from_numpy((start + lens - 1).astype(np.int64)).cuda()
    maxL = int(lens.max())
    q = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((B, topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, topk), dtype=torch.float32, device="cuda")
    ws = torch.empty(dsa.workspace_size(dsa.OP_DECODE, 0, B, maxL, topk), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dsa.project(x, cq, W, q=q, k_out=cache_d, k_slot=slots, w=w)
        if ev is not None:
            ev[1].record(stream)
        dsa.decode(q, w, cache_d, start_d, lens_d, maxL, topk=topk, ws=ws, out=(idx, sc))
        if ev is not None:
            ev[2].record(stream)

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    n = max(args.steps, 10)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    # The host side of one decode step (Python binding, launches) takes longer than the GPU
    # work of its small kernels, so timed back to back the events would measure the host.
    # A GPU-side spin of about 50 ms ahead of the steps lets all of them queue up first; the
    # events then bracket GPU execution only.
    host_t0 = time.perf_counter()
    for i in range(n):
        step()
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - host_t0) * 1e3 / n
    torch.cuda._sleep(100_000_000)
    for i in range(n):
        step(evs[i])
    torch.cuda.synchronize()
    proj_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))

    # FP8 key cache: the cache quantised once (not timed: it is written as the keys arrive);
    # a step quantises the new tokens' keys into it and decodes against it
    k8, k8s = dsa.quantize_keys(cache_d)
    ws8 = torch.empty(dsa.workspace_size(dsa.OP_DECODE_FP8, 0, B, maxL, topk), dtype=torch.uint8,
                      device="cuda")

    def step8(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dsa.quantize_keys(cache_d[slots], k8, k8s, slot=slots)
        if ev is not None:
            ev[1].record(stream)
        dsa.decode_fp8(q, w, k8, k8s, start_d, lens_d, maxL, topk=topk, ws=ws8, out=(idx, sc))
        if ev is not None:
            ev[2].record(stream)

    for _ in range(max(args.warmup, 1)):
        step8()
    torch.cuda.synchronize()
    evs8 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    torch.cuda._sleep(100_000_000)
    for i in range(n):
        step8(evs8[i])
    torch.cuda.synchronize()
    q8_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs8]))
    dec8_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs8]))
    sumL = int(lens.sum())
    # algorithmic bytes of the decode kernels: every cached key once, q and w of the new
    # tokens, the selected indices and scores
    dec_bytes = 256 * sumL + B * (H * D * 2 + H * 2) + B * topk * 8
    proj_bytes = 2 * (QLAT * 4096 + HIDDEN * D + HIDDEN * H + 2 * D) + B * 2 * (HIDDEN + QLAT) \
        + B * 2 * (H * D + D + H)
    gbps = dec_bytes / (dec_ms * 1e-3) / 1e9
    # FP8: 128 code bytes and a 4-byte scale per cached key
    dec8_bytes = 132 * sumL + B * (H * D * 2 + H * 2) + B * topk * 8
    gbps8 = dec8_bytes / (dec8_ms * 1e-3) / 1e9
    log(f"decode: B={B} sum L={sumL}: project {proj_ms:.3f} ms, decode {dec_ms:.3f} ms "
        f"({gbps:.0f} GB/s); one step issued from Python, host-bound: {host_ms:.3f} ms")
    log(f"decode fp8: quantise new keys {q8_ms:.3f} ms, decode {dec8_ms:.3f} ms ({gbps8:.0f} GB/s)")
    mla = None if args.no_mla else bench_mla(dsa, args, idx, start_d, sumL, n)

    # the 64-head indexer's decode against the same cache (its queries and weights from the
    # 64-head projection of the same activations)
    W64t = wl.layer_weights_v32(layer=0, seed=1)
    W64 = {k: dev_bf16(v) for k, v in W64t.items() if k != "eps"}
    W64["eps"] = W64t["eps"]
    q64, _, w64 = dsa.v32_project(x, cq, W64)
    for _ in range(max(args.warmup, 1)):
        dsa.decode(q64, w64, cache_d, start_d, lens_d, maxL, topk=topk, ws=ws, out=(idx, sc))
    torch.cuda.synchronize()
    ev64 = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda._sleep(100_000_000)
    ev64[0].record(stream)
    for i in range(n):
        dsa.decode(q64, w64, cache_d, start_d, lens_d, maxL, topk=topk, ws=ws, out=(idx, sc))
        ev64[i + 1].record(stream)
    torch.cuda.synchronize()
    dec64_ms = float(np.mean([ev64[i].elapsed_time(ev64[i + 1]) for i in range(n)]))
    dec64_bytes = 256 * sumL + B * (64 * D * 2 + 64 * 2) + B * topk * 8
    log(f"decode, 64 heads: {dec64_ms:.3f} ms ({dec64_bytes / (dec64_ms * 1e-3) / 1e9:.0f} GB/s)")
    for _ in range(max(args.warmup, 1)):
        dsa.decode_fp8(q64, w64, k8, k8s, start_d, lens_d, maxL, topk=topk, ws=ws8, out=(idx, sc))
    torch.cuda.synchronize()
    torch.cuda._sleep(100_000_000)
    ev64[0].record(stream)
    for i in range(n):
        dsa.decode_fp8(q64, w64, k8, k8s, start_d, lens_d, maxL, topk=topk, ws=ws8, out=(idx, sc))
        ev64[i + 1].record(stream)
    torch.cuda.synchronize()
    dec64f_ms = float(np.mean([ev64[i].elapsed_time(ev64[i + 1]) for i in range(n)]))
    dec64f_bytes = 132 * sumL + B * (64 * D * 2 + 64 * 2) + B * topk * 8
    log(f"decode fp8, 64 heads: {dec64f_ms:.3f} ms ({dec64f_bytes / (dec64f_ms * 1e-3) / 1e9:.0f} GB/s)")
    return dict(mla=mla, v32=dict(decode_ms=dec64_ms, bytes=dec64_bytes,
                                  GBps=dec64_bytes / (dec64_ms * 1e-3) / 1e9,
                                  fp8_decode_ms=dec64f_ms, fp8_bytes=dec64f_bytes,
                                  fp8_GBps=dec64f_bytes / (dec64f_ms * 1e-3) / 1e9), batch=B, sum_keys=sumL, project_ms=proj_ms, decode_ms=dec_ms, host_step_ms=host_ms,
                fp8=dict(quantize_ms=q8_ms, decode_ms=dec8_ms, bytes=dec8_bytes, GBps=gbps8),
                decode_bytes=dec_bytes, decode_GBps=gbps, decode_hbm_frac=gbps / PEAK_HBM_GBPS,
                step_GBps=(dec_bytes + proj_bytes) / ((dec_ms + proj_ms) * 1e-3) / 1e9)


def bench_mla(dsa, args, idx, start_d, sum_keys, n):
    """The consumer step of the decode: each sequence's new query attends, with all 96 heads,
    to the latent-cache rows its indexer selection names (idx relative to the sequence start)."""
    import torch
    B, topk = idx.shape
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    t0 = time.time()
    # latent cache rows laid out like the key cache (one row per cached token), and absorbed
    # queries; seeded, generated on the device (about 6 GB)
    latent = torch.randn((sum_keys, MLA_KV), generator=g, device="cuda", dtype=torch.float32
                         ).to(torch.bfloat16) if sum_keys * MLA_KV < (1 << 31) else None
    if latent is None:
        latent = torch.empty((sum_keys, MLA_KV), dtype=torch.bfloat16, device="cuda")
        for r0 in range(0, sum_keys, 1 << 20):
            r1 = min(sum_keys, r0 + (1 << 20))
            latent[r0:r1] = torch.randn((r1 - r0, MLA_KV), generator=g, device="cuda").to(torch.bfloat16)
    qm = (torch.randn((B, MLA_HEADS, MLA_KV), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    torch.cuda.synchronize()
    log(f"mla: latent cache of {sum_keys} rows generated in {time.time() - t0:.1f}s")
    o = torch.empty((B, MLA_HEADS, MLA_V), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, MLA_HEADS), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(dsa.workspace_size(dsa.OP_SPARSE_MLA, B, 0, 0, topk), 1), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(max(args.warmup, 1)):
        dsa.sparse_mla(qm, latent, idx, row0=start_d, ws=ws, out=(o, lse))
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda._sleep(100_000_000)   # as for the decode: the calls queue up ahead of the GPU
    evs[0].record(stream)
    for i in range(n):
        dsa.sparse_mla(qm, latent, idx, row0=start_d, ws=ws, out=(o, lse))
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([evs[i].elapsed_time(evs[i + 1]) for i in range(n)]))
    # algorithmic bytes: each selected latent row once, the queries, indices, outputs and lse
    nbytes = B * topk * MLA_KV * 2 + B * MLA_HEADS * MLA_KV * 2 + B * topk * 4 + B * MLA_HEADS * (MLA_V * 2 + 4)
    flop = B * MLA_HEADS * topk * (MLA_KV + MLA_V) * 2
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"mla: B={B} top-{topk}: {ms * 1e3:.1f} us per call, {gbps:.0f} GB/s, "
        f"{flop / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
    del latent, ws
    return dict(ms=ms, bytes=nbytes, flop=flop, GBps=gbps)


def bench_v32(dsa, args):
    """The 64-head (DeepSeek-V3.2-shaped) indexer layer at the same T: projections with the
    rotary step, then scores (all 64 heads in one pass) and top-k."""
    import torch
    from synth import workloads as wl
    T, topk = args.T, args.topk
    t0 = time.time()
    Wt = wl.layer_weights_v32(layer=0, seed=0)
    act = wl.layer_activations(T, seed=0)
    W = {k: dev_bf16(v) for k, v in Wt.items() if k != "eps"}
    W["eps"] = Wt["eps"]
    x, cq = dev_bf16(act["x"]), dev_bf16(act["c_q"])
    del act
    log(f"v32: inputs T={T} in {time.time() - t0:.1f}s")
    q = torch.empty((T, V32_H, D), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((T, V32_H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((T, topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((T, topk), dtype=torch.float32, device="cuda")
    ws = torch.empty(dsa.workspace_size(dsa.OP_V32_SCORE_TOPK, T, topk=topk), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dsa.v32_project(x, cq, W, q=q, k=k, w=w)
        if ev is not None:
            ev[1].record(stream)
        dsa.v32_score_topk(q, k, w, topk=topk, ws=ws, out=(idx, sc))
        if ev is not None:
            ev[2].record(stream)

    step()
    torch.cuda.synchronize()
    n = max(2, min(args.steps, 5))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    for i in range(n):
        step(evs[i])
    torch.cuda.synchronize()
    proj_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    st_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    pairs = T * (T + 1) // 2
    score_flop = pairs * 2 * V32_H * D
    log(f"v32: project {proj_ms:.3f} ms, scores + select {st_ms:.3f} ms "
        f"({score_flop / (st_ms * 1e-3) / 1e12:.1f} TFLOP/s of scoring over the call)")
    del ws
    return dict(proj_ms=proj_ms, score_topk_ms=st_ms, pairs=pairs, score_flop=score_flop,
                qps=T / ((proj_ms + st_ms) * 1e-3))


def bench_chunk(dsa, args):
    """The last `chunk` queries of a `window`-token sequence against its whole prefix."""
    import torch
    from synth import workloads as wl
    C, topk = args.chunk, args.topk
    prefix = args.window - C
    t0 = time.time()
    inp = wl.chunk_inputs(prefix, C, seed=2)
    q, k, w = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["w"])
    del inp
    log(f"chunk: prefix {prefix}, C {C}: inputs in {time.time() - t0:.1f}s")
    idx = torch.empty((C, topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((C, topk), dtype=torch.float32, device="cuda")
    ws = torch.empty(dsa.workspace_size(dsa.OP_PREFILL_CHUNK, C, 0, prefix, topk), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    dsa.prefill_chunk(q, k, w, prefix, topk=topk, ws=ws, out=(idx, sc))
    torch.cuda.synchronize()
    n = max(3, min(args.steps, 5))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    evs[0].record(stream)
    for i in range(n):
        dsa.prefill_chunk(q, k, w, prefix, topk=topk, ws=ws, out=(idx, sc))
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([evs[i].elapsed_time(evs[i + 1]) for i in range(n)]))
    pairs = C * prefix + C * (C + 1) // 2
    tflops = pairs * SCORE_FLOP_PER_PAIR / (ms * 1e-3) / 1e12
    log(f"chunk: {ms:.3f} ms per call, {C / (ms * 1e-3):.0f} queries/s, {tflops:.1f} TFLOP/s of scoring")
    del ws
    return dict(C=C, prefix=prefix, ms=ms, qps=C / (ms * 1e-3), tflops=tflops, pairs=pairs)


def cpu_baseline(args):
    """The oracle on a bounded sample of the T-token layer, extrapolated per its cost model.

    Keys are projected for every token the sampled rows need; then batches of sampled rows
    (q and w projected, each row scored over its whole causal prefix and fully sorted), each
    batch twice the last, until about 10 s of oracle work has been measured."""
    import oracle
    from synth import workloads as wl
    T, topk = args.T, args.topk
    cores = oracle.num_threads()
    rng = np.random.default_rng(0)
    Wt = wl.layer_weights(layer=0, seed=0)
    act = wl.layer_activations(T, seed=0)
    t0 = time.perf_counter()
    _, k_all, _ = oracle.project(act["x"], None, Wt, want=("k",))   # every key
    t_k = time.perf_counter() - t0
    t_qw = t_rows = 0.0
    n_rows = pairs = 0
    batch = np.array([0, T - 1] + rng.integers(0, T, 62).tolist())
    while True:
        t0 = time.perf_counter()
        q_s, _, w_s = oracle.project(act["x"][batch], act["c_q"][batch], Wt, want=("q", "w"))
        t_qw += time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.rows(q_s, w_s, k_all, np.zeros(len(batch), np.int64), batch, topk=topk)
        t_rows += time.perf_counter() - t0
        n_rows += len(batch)
        pairs += int((batch + 1).sum())
        if t_k + t_qw + t_rows >= 10.0 or n_rows >= 8192:
            break
        batch = rng.integers(0, T, 2 * len(batch))
    total = t_k + t_qw * T / n_rows + t_rows * (T * (T + 1) / 2) / float(pairs)
    return dict(value=round(T / total, 2), unit="queries/s", cores=cores, cpu_model=cpu_model(), kind="oracle",
                sample=(f"fp64 oracle, OpenMP over {cores} host threads: keys projected for all {T} "
                        f"tokens, q and w for {n_rows} sampled rows, those rows scored over their whole "
                        f"causal prefix and fully sorted; extrapolated to all {T} rows by tokens "
                        f"(projections) and causal pairs (scores)"),
                measured_s=round(t_k + t_qw + t_rows, 2), extrapolated_s=round(total, 1))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is described in the design notes but not built.",
              file=sys.stderr, flush=True)
        sys.exit(2)
    import torch
    import sparse_attention_token_idx_amd as dsa
    assert torch.cuda.is_available(), "no GPU visible"
    log(f"{dsa.version()} on {torch.cuda.get_device_name(0)}")
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration: copied 1073741824 bytes device to device")
        del src, dst
    copy_gbps = copy_rate()
    log(f"device copy: {copy_gbps} GB/s (read + write)")
    pre = bench_layer(dsa, args, args.T, args.steps, args.warmup, "prefill")
    cfg1 = cfg2 = cfg5 = None
    if not args.no_configs:
        cfg1 = bench_score_only(dsa, args)
        cfg2 = bench_layer(dsa, args, 8192, 30, 3, "layer T=8192")
        cfg5 = bench_varlen_layers(dsa, args)
    dec = None if args.no_decode else bench_decode(dsa, args)
    chk = None if args.no_chunk else bench_chunk(dsa, args)
    v32 = None if args.no_v32 else bench_v32(dsa, args)
    vgemm = vendor_q_gemm(args.T)
    log(f"yardstick: torch.matmul on the q projection's shape {vgemm} ms")
    # last, so that its full matrix-core load (and the heat) comes after every timed leg
    mfma_meas = mfma_rate(dsa)
    log(f"sustained bf16 MFMA (calibration kernel): {mfma_meas} TFLOP/s")
    ms_wall = pre["wall"] * 1e3 / args.steps
    qps = args.T / (ms_wall * 1e-3)
    tflops = (pre["score_flop"] + pre["proj_flop"]) / (ms_wall * 1e-3) / 1e12
    filt_ms = pre["phases"].get("filter")
    achieved = pre["score_flop"] / (filt_ms * 1e-3) / 1e12 if filt_ms else None
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: running the oracle on a bounded sample")
        cpu = cpu_baseline(args)
        log(f"cpu baseline: {cpu['value']:.1f} queries/s ({cpu['measured_s']} s measured)")

    def frac(flop, ms):
        return round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)

    configs = None
    if cfg1 is not None:
        configs = {
            "score_only_T2560": {
                "workload": "scores + top-2048 of one causal sequence, T=2560, q/k ~ N(0,1), w ~ N(0,0.1)",
                "ms": cfg1["ms"], "queries_per_s_median": round(cfg1["T"] / (cfg1["ms"]["median"] * 1e-3), 1),
                "score_tflops_median": round(cfg1["score_flop"] / (cfg1["ms"]["median"] * 1e-3) / 1e12, 1),
                "frac_of_bf16_peak_median": frac(cfg1["score_flop"], cfg1["ms"]["median"]),
                "frac_of_bf16_peak_best": frac(cfg1["score_flop"], cfg1["ms"]["min"])},
            "layer_T8192": {
                "workload": "one indexer layer, causal prefill T=8192: project + scores + top-2048",
                "step_ms": cfg2["step"], "project_ms": cfg2["proj"], "score_topk_ms": cfg2["score_topk"],
                "queries_per_s_median": round(cfg2["T"] / (cfg2["step"]["median"] * 1e-3), 1),
                "tflops_median": round((cfg2["score_flop"] + cfg2["proj_flop"]) / (cfg2["step"]["median"] * 1e-3) / 1e12, 1),
                "frac_of_bf16_peak_median": frac(cfg2["score_flop"] + cfg2["proj_flop"], cfg2["step"]["median"]),
                "phases_ms": cfg2["phases"]},
            "varlen_24_layers": {
                "workload": f"24 indexer layers (own weights each), {cfg5['B']} ragged sequences, "
                            f"{cfg5['total']} tokens, lengths log-uniform in [2048, 32768]: per layer "
                            "project + scores + top-2048",
                "ms": cfg5["ms"],
                "queries_per_s_median": round(cfg5["layers"] * cfg5["total"] / (cfg5["ms"]["median"] * 1e-3), 1),
                "tflops_median": round(cfg5["flop"] / (cfg5["ms"]["median"] * 1e-3) / 1e12, 1),
                "frac_of_bf16_peak_median": frac(cfg5["flop"], cfg5["ms"]["median"])},
        }
    line = {
        "metric": "DSA indexer queries/s + TFLOP/s (T=64K prefill, top-2048); decode HBM GB/s",
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_wall, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"one indexer layer, causal prefill T={args.T}, top-{args.topk}: "
                               "project + scores + select, no T x T score matrix stored",
                   "seq_len": args.T, "topk": args.topk, "heads": H, "head_dim": D,
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 1),
        "step_ms": pre["step"],
        "split_ms": {"project": pre["proj"], "score_topk": pre["score_topk"], "phases": pre["phases"]},
        "yardstick": {"what": f"torch.matmul (vendor BLAS) on the q projection's shape [{args.T},1536] x "
                              f"[1536,4096] bf16, not part of the path",
                      "ms": vgemm,
                      "frac_of_bf16_peak_median": frac(2 * args.T * QLAT * 4096, vgemm["median"])},
        "roofline": {"kernel": "score_kernel<32, filter> (score-and-filter pass)", "bound": "mfma",
                     "achieved": None if achieved is None else round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": None if achieved is None else round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": filter_traffic(args), "algorithmic_flop_per_launch": pre["score_flop"],
                     "measured_peak": mfma_meas["random_operands"],
                     "frac_of_measured_peak": None if achieved is None
                     else round(achieved / mfma_meas["random_operands"], 4)},
        "device_copy_GBps": copy_gbps,
        "mfma_sustained_TFLOPs": mfma_meas,
        "configs": configs,
        "decode": None if dec is None else {
            "workload": f"{dec['batch']} sequences, one new query each, cached bf16 keys "
                        f"U[32768,131072] (sum {dec['sum_keys']}), top-{args.topk}",
            "decode_ms": round(dec["decode_ms"], 4), "project_ms": round(dec["project_ms"], 4),
            "GBps": round(dec["decode_GBps"], 1), "hbm_frac": round(dec["decode_hbm_frac"], 4),
            "frac_of_copy_rate": round(dec["decode_GBps"] / copy_gbps, 4),
            "step_GBps_incl_project": round(dec["step_GBps"], 1),
            "host_step_ms": round(dec["host_step_ms"], 4),
            "algorithmic_bytes": dec["decode_bytes"],
            "fp8_cache": {"decode_ms": round(dec["fp8"]["decode_ms"], 4),
                          "quantize_new_keys_ms": round(dec["fp8"]["quantize_ms"], 4),
                          "GBps": round(dec["fp8"]["GBps"], 1),
                          "hbm_frac": round(dec["fp8"]["GBps"] / PEAK_HBM_GBPS, 4),
                          "algorithmic_bytes": dec["fp8"]["bytes"]},
            "v32_64_heads": {"decode_ms": round(dec["v32"]["decode_ms"], 4),
                             "GBps": round(dec["v32"]["GBps"], 1),
                             "hbm_frac": round(dec["v32"]["GBps"] / PEAK_HBM_GBPS, 4),
                             "algorithmic_bytes": dec["v32"]["bytes"],
                             "fp8_cache": {"decode_ms": round(dec["v32"]["fp8_decode_ms"], 4),
                                           "GBps": round(dec["v32"]["fp8_GBps"], 1),
                                           "hbm_frac": round(dec["v32"]["fp8_GBps"] / PEAK_HBM_GBPS, 4),
                                           "algorithmic_bytes": dec["v32"]["fp8_bytes"]}},
            "sparse_mla": None if dec["mla"] is None else {
                "workload": f"the decode's consumer: {dec['batch']} queries x {MLA_HEADS} heads over "
                            f"the {args.topk} latent-cache rows (576 values) each selection names",
                "us": round(dec["mla"]["ms"] * 1e3, 2), "GBps": round(dec["mla"]["GBps"], 1),
                "bound": "hbm", "hbm_frac": round(dec["mla"]["GBps"] / PEAK_HBM_GBPS, 4),
                "tflops": round(dec["mla"]["flop"] / (dec["mla"]["ms"] * 1e-3) / 1e12, 2),
                "algorithmic_bytes": dec["mla"]["bytes"]}},
        "chunked_prefill": None if chk is None else {
            "workload": f"last {chk['C']} queries of a {chk['prefix'] + chk['C']}-token window "
                        f"against the whole prefix, top-{args.topk}",
            "ms": round(chk["ms"], 3), "queries_per_s": round(chk["qps"], 1),
            "score_tflops_over_call": round(chk["tflops"], 1),
            "frac_of_bf16_peak": round(chk["tflops"] / PEAK_BF16_TFLOPS, 4),
            "causal_pairs": chk["pairs"]},
        "v32_indexer": None if v32 is None else {
            "workload": f"the 64-head (DeepSeek-V3.2-shaped) indexer layer, causal prefill T={args.T}, "
                        f"top-{args.topk}: project + rotary step, scores (64 heads in one pass) + select",
            "ms_per_step": round(v32["proj_ms"] + v32["score_topk_ms"], 3),
            "queries_per_s": round(v32["qps"], 1), "project_ms": round(v32["proj_ms"], 3),
            "score_topk_ms": round(v32["score_topk_ms"], 3),
            "score_tflops_over_call": round(v32["score_flop"] / (v32["score_topk_ms"] * 1e-3) / 1e12, 1)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
