"""Benchmark of the HGA routed-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-prefill] [--no-secondary]
                    [--offload-only]

A step is one decode step of the 32K-context workload (B=8, 32 query / 8 KV
heads, d=128, C=64, G=16, sink 1, local 4, top-k 16, top-g 32, bf16): the
library's hga_decode, one kernel launch that routes (summary scan + chunk
top-k + group scoring + group top-g), attends over the union of the routed
groups and the always-visible chunks, and writes the summaries of the chunk
the query completes.  Inputs are resident in HBM.

Timing protocol.  Consecutive steps rotate over 12 independent copies of the
cache (as consecutive layers of a model would), so between two uses of one
copy more than 512 MB of other copies pass through the 256 MB Infinity Cache.
The K timed steps are one HIP graph of exactly K launches; the headline value
is B * K / (host time of one replay, bracketed by device synchronisations).
The same graph is then replayed 50 times with HIP events on the launch stream
around each replay: median, p10 and p90 of the per-step time over those
replays.  A warm-cache figure (every step on one copy) is reported apart.

Printed: one JSON line with the throughput (query tokens/s), the roofline of
the decode step (its one launch; achieved = the algorithmic bytes of the step
/ the median per-step time), the CPU oracle timed on a bounded sample, and the
32K prefill, 64K decode, route-reuse, streaming-head and cold-tier figures.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "routed-attention query tokens/s + % HBM/MFMA roofline, 32K decode & prefill"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_fingerprint():
    """sha256 over the library's kernel and API sources (file names and contents)."""
    import hashlib
    h = hashlib.sha256()
    base = os.path.join(ROOT, "hierarchical_sparse_attention_build_amd", "csrc")
    files = sorted(os.path.join(base, f) for f in os.listdir(base) if f.endswith((".hip", ".hpp", ".cpp")))
    files.append(os.path.join(ROOT, "include", "hga.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the calibrated rocprofv3 counter
    summaries under profiles/ (a line `traffic <kernel> <bytes> sources <sha256>`),
    or None when no summary was taken on the current sources."""
    d = os.path.join(ROOT, "profiles")
    fp = source_fingerprint()
    want = kernel.replace(" ", "")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f)) as fh:
            for line in fh:
                # kernel names may hold spaces ("k<bf16, 128, 4>"): read the
                # fields from the right
                t = line.strip().strip("`").split()
                if len(t) >= 5 and t[0] == "traffic" and t[-2] == "sources":
                    if "".join(t[1:-3]) == want and t[-1] == fp:
                        return int(t[-3])
    return None


def decode_bytes(s):
    """Algorithmic HBM bytes of one decode step, by part: what the method must
    touch per (b, KV head) unit, times the units.

    routing: the candidate chunk summaries and the group summaries of the
        routed chunks (fp32);
    attention: the forced (sink + local + current) and routed K and V rows;
    q_o: Q read and O (fp32) written.
    Returns (bytes by part, total bytes, attended tokens per unit).  Work that
    is not the method's own (partial softmax results exchanged between the
    workgroups of a unit, the index lists, the summary of the chunk a query
    completes, once every C steps) is left out.
    """
    C, G, d = s.chunk_size, s.group_size, s.head_dim
    L = s.n_tokens
    j = (L - 1) // C
    n_forced = len(set(range(min(s.n_sink, j + 1))) | set(range(max(0, j - s.n_local), j + 1)))
    m = C // G
    n_cand = max(0, j - s.n_local - s.n_sink)
    n_routed_chunks = min(s.top_k, n_cand)
    n_groups = min(s.top_g, n_routed_chunks * m)
    gq = s.n_q_heads // s.n_kv_heads
    units = s.batch * s.n_kv_heads
    e = 2 if s.dtype == "bf16" else 4
    forced_tok = n_forced * C
    routed_tok = n_groups * G
    parts = {
        "routing": units * (n_cand + n_routed_chunks * m) * d * 4,
        "attention": units * (forced_tok + routed_tok) * d * e * 2,
        "q_o": units * gq * d * (e + 4),
    }
    return parts, sum(parts.values()), forced_tok + routed_tok


def graph_of(fn, n):
    """A HIP graph of n calls fn(0..n-1), captured after one eager pass."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def replay_stats(g, steps_per_replay, n_replays):
    """Per-step microseconds of each of n_replays replays of g, from HIP events on
    the launch stream around each replay: (median, p10, p90, mean)."""
    import torch
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_replays + 1)]
    ev[0].record(st)
    for i in range(n_replays):
        g.replay()
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 / steps_per_replay for i in range(n_replays)])
    return float(np.median(per)), float(np.percentile(per, 10)), float(np.percentile(per, 90)), float(per.mean())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=12)
    ap.add_argument("--stat-replays", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the 64K decode and the 128K cold-tier decode figures")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy, a known-size reference for HBM counters")
    ap.add_argument("--offload-only", action="store_true",
                    help="only the 128K host-offload decode (cold and warm tiers), for a kernel trace of it")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the routed-attention path "
                                   "shards by (batch, KV head) with no communication, so N GPUs "
                                   "run N independent copies of this measurement"}))
        sys.exit(2)

    import torch
    from hierarchical_sparse_attention_build_amd import hga
    from hierarchical_sparse_attention_build_amd import workloads as W

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    hga.lib()
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copy calibration: 3 x 1 GiB device-to-device copies done")
    if args.offload_only:
        print(json.dumps({"offload_decode_128k": bench_offload(args, dev)}), flush=True)
        return

    s = W.spec("decode_32k")
    log(f"[bench] generating {s.name} (seed {s.seed})")
    w = W.make(s)
    B, Hq, H, d, L, C, G = s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.n_tokens, s.chunk_size, s.group_size
    m = C // G
    p = hga.params(B, Hq, H, d, C, G, s.n_sink, s.n_local, s.top_k, s.top_g, s.rope_base,
                   s.hf_threshold, qkv_dtype=hga.HGA_BF16, out_dtype=hga.HGA_F32)
    Q0 = W.to_torch(w.Q, s.dtype).to(dev)
    K0 = W.to_torch(w.K, s.dtype).to(dev)
    V0 = W.to_torch(w.V, s.dtype).to(dev)
    nC = L // C
    jq = (L - 1) // C
    R = max(1, args.replicas)
    reps = []
    for r in range(R):
        K = K0 if r == 0 else K0.clone()
        V = V0 if r == 0 else V0.clone()
        cs = torch.zeros((B, H, nC, d), device=dev)
        gs = torch.zeros((B, H, nC * m, d), device=dev)
        hga.build_summaries(p, K, L, 0, jq, cs, gs)
        reps.append(dict(K=K, V=V, Q=Q0.clone(), cs=cs, gs=gs,
                         O=torch.empty((B, Hq, 1, d), device=dev),
                         gi=torch.empty((B, H, 1, s.top_g), dtype=torch.int32, device=dev),
                         ci=torch.empty((B, H, 1, s.top_k), dtype=torch.int32, device=dev),
                         ws=hga.workspace(p, hga.OP_DECODE, 1, L, device=dev)))
    seq = torch.from_numpy(w.seq_len.astype(np.int32)).to(dev)
    torch.cuda.synchronize()
    log(f"[bench] {R} cache replicas resident; warmup {args.warmup}, steps {args.steps}")

    def step(i):
        r = reps[i % R]
        hga.decode(p, r["Q"], r["K"], r["V"], L, seq, r["cs"], r["gs"], r["O"], r["ws"],
                   chunk_idx=r["ci"], group_idx=r["gi"])

    # exactly K steps per graph: one replay is the timed region
    steps = max(1, args.steps)
    g_cold = graph_of(step, steps)
    g_warm = graph_of(lambda i: step(0), steps)
    n_warm_replays = max(1, -(-args.warmup // steps))
    for _ in range(n_warm_replays):
        g_cold.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_cold.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec_per_step = (t1 - t0) / steps
    value = B / sec_per_step
    log(f"[bench] decode step {sec_per_step * 1e6:.2f} us (host clock, {steps} steps) -> {value:.0f} query tokens/s")

    # statistics over replays, HIP events on the launch stream
    med, p10, p90, mean = replay_stats(g_cold, steps, max(1, args.stat_replays))
    wmed, _, _, _ = replay_stats(g_warm, steps, max(1, args.stat_replays // 5))
    parts, step_bytes, tokens = decode_bytes(s)
    step_gbs = step_bytes / (med * 1e-6) / 1e9
    log(f"[bench] decode step (HIP events, {args.stat_replays} replays of {steps} steps) median {med:.2f} us "
        f"(p10 {p10:.2f}, p90 {p90:.2f}): {step_bytes / 1e6:.2f} MB -> {step_gbs:.0f} GB/s; warm cache {wmed:.2f} us")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": n_warm_replays * steps,
        "ms_per_step": round(sec_per_step * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_32k", "batch": B, "context": L, "q_heads": Hq, "kv_heads": H,
                   "head_dim": d, "chunk": C, "group": G, "sink": s.n_sink, "local": s.n_local,
                   "top_k": s.top_k, "top_g": s.top_g, "rope_base": s.rope_base,
                   "tokens_attended": tokens, "cache_replicas": R},
        "step_us": {"median": round(med, 3), "p10": round(p10, 3), "p90": round(p90, 3), "mean": round(mean, 3),
                    "replays": args.stat_replays, "steps_per_replay": steps, "clock": "HIP events"},
        "roofline": {"kernel": "decode_step_kernel<bf16,128,4>",
                     "bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decode_step_kernel<bf16,128,4>"),
                     "bytes_per_launch": step_bytes, "avg_us": round(med, 3), "avg_us_is": "median per step",
                     "bytes_by_part": parts},
        "warm_cache": {"us_per_step": round(wmed, 3), "value": round(B / (wmed * 1e-6), 1)},
    }

    del reps, g_cold, g_warm
    torch.cuda.empty_cache()
    if not args.no_prefill:
        out["prefill"] = bench_prefill(args, dev)
    if not args.no_secondary:
        out["decode_64k"] = bench_decode_64k(args, dev)
        out.update(bench_reuse_and_streaming(args, dev))
        out["offload_decode_128k"] = bench_offload(args, dev)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(s, w, prefill=not args.no_prefill)

    print(json.dumps(out), flush=True)


def prefill_flops(s):
    """Algorithmic attention FLOPs of a full prefill: 4*d per (query row, visible key)."""
    C, G = s.chunk_size, s.group_size
    m = C // G
    pairs = 0
    for j in range(s.n_tokens // C):
        n_forced_full = len(set(range(min(s.n_sink, j + 1))) | set(range(max(0, j - s.n_local), j)))
        n_cand = max(0, j - s.n_local - s.n_sink)
        routed = min(s.top_g, min(s.top_k, n_cand) * m) * G
        pairs += C * (n_forced_full * C + routed) + C * (C + 1) // 2
    return pairs * s.n_q_heads * s.batch * 4 * s.head_dim


def routing_flops(s):
    """Algorithmic routing FLOPs: 2*d per (query row, scored summary), chunks and groups."""
    C, G = s.chunk_size, s.group_size
    m = C // G
    gq = s.n_q_heads // s.n_kv_heads
    tot = 0
    for j in range(s.n_tokens // C):
        n_cand = max(0, j - s.n_local - s.n_sink)
        tot += n_cand + min(s.top_k, n_cand) * m
    return tot * gq * C * s.n_kv_heads * s.batch * 2 * s.head_dim


def bench_prefill(args, dev):
    """hga_prefill on the 32K workload: the whole call, and each of its three
    kernels launched alone (same launch configurations) timed with HIP events."""
    import torch
    from hierarchical_sparse_attention_build_amd import hga
    from hierarchical_sparse_attention_build_amd import workloads as W
    s = W.spec("prefill_32k")
    log(f"[bench] generating {s.name} (seed {s.seed})")
    w = W.make(s)
    B, Hq, H, d, n, C, G = s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.n_tokens, s.chunk_size, s.group_size
    p = hga.params(B, Hq, H, d, C, G, s.n_sink, s.n_local, s.top_k, s.top_g, s.rope_base,
                   s.hf_threshold, qkv_dtype=hga.HGA_BF16, out_dtype=hga.HGA_F32)
    Q = W.to_torch(w.Q, s.dtype).to(dev)
    K = W.to_torch(w.K, s.dtype).to(dev)
    V = W.to_torch(w.V, s.dtype).to(dev)
    nC = n // C
    cs = torch.empty((B, H, nC, d), device=dev)
    gs = torch.empty((B, H, nC * (C // G), d), device=dev)
    O = torch.empty((B, Hq, n, d), device=dev)
    ci = torch.empty((B, H, nC, s.top_k), dtype=torch.int32, device=dev)
    gi = torch.empty((B, H, nC, s.top_g), dtype=torch.int32, device=dev)
    ws = hga.workspace(p, hga.OP_PREFILL, n, n, device=dev)
    wsr = hga.workspace(p, hga.OP_ROUTE, n, n, device=dev)
    wsa = hga.workspace(p, hga.OP_ATTEND, n, n, device=dev)
    qpos = torch.zeros(B, dtype=torch.int32, device=dev)

    def timed(fn, reps):
        for _ in range(3):  # warm-up: clocks and caches settle
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3  # us

    reps = max(1, args.prefill_steps)
    t_all = timed(lambda: hga.prefill(p, Q, K, V, n, cs, gs, O, ws, chunk_idx=ci, group_idx=gi), reps)
    t_sum = timed(lambda: hga.build_summaries(p, K, n, 0, nC, cs, gs), reps)
    t_route = timed(lambda: hga.route(p, Q, n, qpos, cs, gs, n, ci, gi, wsr), reps)
    t_att = timed(lambda: hga.attend(p, Q, n, qpos, K, V, n, gi, O, wsa), reps)
    fl_att = prefill_flops(s)
    fl_route = routing_flops(s)
    tf_att = fl_att / (t_att * 1e-6) / 1e12
    tf_route = fl_route / (t_route * 1e-6) / 1e12
    summ_bytes = B * H * n * d * 2 + B * H * (nC + n // G) * d * 4
    log(f"[bench] prefill {t_all:.1f} us: summaries {t_sum:.1f}, route {t_route:.1f}, attend {t_att:.1f} us "
        f"({tf_att:.1f} TFLOP/s = {tf_att / MFMA_BF16_PEAK_TFLOPS:.3f} of bf16 peak)")
    return {"workload": "prefill_32k", "ms_per_call": round(t_all / 1e3, 4),
            "query_tokens_per_s": round(B * n / (t_all * 1e-6), 1),
            # avg_us and achieved cover the whole hga_attend call: the V pre-pass
            # (v16_blocks_kernel) and the attention kernel; traffic likewise
            "roofline": {"kernel": "attend_prefill_pipe_kernel<128,8>", "bound": "mfma",
                         "achieved": round(tf_att, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf_att / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("hga_attend_prefill"),
                         "flops_per_launch": fl_att, "avg_us": round(t_att, 2),
                         "includes": ["v16_blocks_kernel<128>", "attend_prefill_pipe_kernel<128,8>"]},
            "route": {"kernel": "route_prefill_mfma_kernel<128,8,true>", "avg_us": round(t_route, 2),
                      "includes": ["summary_split_kernel<128> (x2)", "route_prefill_mfma_kernel<128,8,true>"],
                      "flops_per_launch": fl_route, "achieved_tflops": round(tf_route, 1),
                      "frac": round(tf_route / MFMA_BF16_PEAK_TFLOPS, 4),
                      "traffic_mfma_kernel": measured_traffic("route_prefill_mfma_kernel<128,8,true>")},
            "summaries": {"kernel": "summaries_fast_kernel<128,4>", "avg_us": round(t_sum, 2),
                          "bytes_per_launch": summ_bytes,
                          "traffic": measured_traffic("summaries_fast_kernel<128,4>"),
                          "achieved_gbs": round(summ_bytes / (t_sum * 1e-6) / 1e9, 1),
                          "frac": round(summ_bytes / (t_sum * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
            "backward": bench_backward(s, p, Q, K, V, gi, dev)}


def bench_backward(s, p, Q, K, V, gi, dev):
    """hga_prefill_backward on the 32K prefill with its own routing: dQ, dK, dV
    for a random dO.  Algorithmic work: 10*d FLOPs per (query row, visible key)
    (scores recomputed, dP, dQ, dK, dV).  The contractions run on the bf16
    matrix cores; dO, P and dS enter as two bf16 parts each, so the MFMA work
    issued is a multiple of the algorithmic figure that the roofline uses."""
    import torch
    from hierarchical_sparse_attention_build_amd import hga
    B, Hq, H, d, n = s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.n_tokens
    g = torch.Generator(device=dev).manual_seed(s.seed + 5)
    dO = torch.randn((B, Hq, n, d), device=dev, generator=g)
    dQ = torch.empty((B, Hq, n, d), device=dev)
    dK = torch.empty((B, H, n, d), device=dev)
    dV = torch.empty_like(dK)
    ws = hga.workspace(p, hga.OP_PREFILL_BACKWARD, n, n, device=dev)
    run = lambda: hga.prefill_backward(p, Q, K, V, n, gi, dO, dQ, dK, dV, ws)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        run()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 3 * 1e3
    fl = prefill_flops(s) // 4 * 10
    tf = fl / (us * 1e-6) / 1e12
    log(f"[bench] prefill backward {us / 1e3:.2f} ms: {tf:.1f} TFLOP/s = {tf / MFMA_BF16_PEAK_TFLOPS:.3f} of the "
        f"bf16 MFMA peak")
    del dO, dQ, dK, dV
    return {"workload": "prefill_32k", "ms_per_call": round(us / 1e3, 4),
            "roofline": {"kernel": "bwd_dq_mfma_kernel<128,8> + bwd_dkv_mfma_kernel<128>", "bound": "mfma",
                         "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "flops_per_call": fl,
                         "includes": ["bwd_split_do_kernel", "bwd_vis_kernel", "bwd_count_kernel",
                                      "bwd_dq_mfma_kernel<128,8>", "bwd_dkv_mfma_kernel<128>"]}}


def bench_decode_64k(args, dev):
    """The 64K decode workload (B=16, 32/8 heads): hga_decode step time from HIP
    events around graph replays over 4 cache replicas, and its HBM roofline."""
    import torch
    from hierarchical_sparse_attention_build_amd import hga
    from hierarchical_sparse_attention_build_amd import workloads as W
    s = W.spec("decode_64k")
    log(f"[bench] generating {s.name} (seed {s.seed})")
    w = W.make(s)
    B, Hq, H, d, L, C, G = s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.n_tokens, s.chunk_size, s.group_size
    p = hga.params(B, Hq, H, d, C, G, s.n_sink, s.n_local, s.top_k, s.top_g, s.rope_base,
                   s.hf_threshold, qkv_dtype=hga.HGA_BF16, out_dtype=hga.HGA_F32)
    Q = W.to_torch(w.Q, s.dtype).to(dev)
    K0 = W.to_torch(w.K, s.dtype).to(dev)
    V0 = W.to_torch(w.V, s.dtype).to(dev)
    del w
    nC, m, jq = L // C, C // G, (L - 1) // C
    R = 4
    reps = []
    for r in range(R):
        K = K0 if r == 0 else K0.clone()
        V = V0 if r == 0 else V0.clone()
        cs = torch.zeros((B, H, nC, d), device=dev)
        gs = torch.zeros((B, H, nC * m, d), device=dev)
        hga.build_summaries(p, K, L, 0, jq, cs, gs)
        reps.append(dict(K=K, V=V, cs=cs, gs=gs, O=torch.empty((B, Hq, 1, d), device=dev),
                         ws=hga.workspace(p, hga.OP_DECODE, 1, L, device=dev)))
    seq = torch.full((B,), L, dtype=torch.int32, device=dev)

    def step(i):
        r = reps[i % R]
        hga.decode(p, Q, r["K"], r["V"], L, seq, r["cs"], r["gs"], r["O"], r["ws"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(R):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(R):
            step(i)
    for _ in range(4):
        g.replay()
    torch.cuda.synchronize()
    n_rep = max(1, args.steps // R)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(n_rep):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3 / (n_rep * R)
    _, step_bytes, tokens = decode_bytes(s)
    gbs = step_bytes / (step_us * 1e-6) / 1e9
    log(f"[bench] decode_64k step {step_us:.2f} us -> {B / (step_us * 1e-6):.0f} query tokens/s, {gbs:.0f} GB/s")
    del reps, g
    torch.cuda.empty_cache()
    return {"workload": "decode_64k", "batch": B, "context": L, "top_k": s.top_k, "top_g": s.top_g,
            "ms_per_step": round(step_us / 1e3, 6), "query_tokens_per_s": round(B / (step_us * 1e-6), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_step": step_bytes}}


def bench_reuse_and_streaming(args, dev):
    """Two variants of the decode_32k step, HIP events around graph replays over
    4 cache replicas:
    - route once, attend many: hga_attend over group lists routed by an earlier
      decode step (as a layer reusing another layer's routing would), against the
      full step; the difference is the routing share that reuse saves;
    - streaming heads: top_k = top_g = 0, only the sink, local and current
      chunks."""
    import torch
    from hierarchical_sparse_attention_build_amd import hga
    from hierarchical_sparse_attention_build_amd import workloads as W
    s = W.spec("decode_32k")
    log(f"[bench] generating {s.name} (seed {s.seed}) for route reuse and streaming heads")
    w = W.make(s)
    B, Hq, H, d, L, C, G = s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.n_tokens, s.chunk_size, s.group_size
    mk = lambda top_k, top_g: hga.params(B, Hq, H, d, C, G, s.n_sink, s.n_local, top_k, top_g, s.rope_base,
                                         s.hf_threshold, qkv_dtype=hga.HGA_BF16, out_dtype=hga.HGA_F32)
    p, p0 = mk(s.top_k, s.top_g), mk(0, 0)
    Q = W.to_torch(w.Q, s.dtype).to(dev)
    K0 = W.to_torch(w.K, s.dtype).to(dev)
    V0 = W.to_torch(w.V, s.dtype).to(dev)
    del w
    nC, m, jq = L // C, C // G, (L - 1) // C
    R = 4
    reps = []
    for r in range(R):
        K = K0 if r == 0 else K0.clone()
        V = V0 if r == 0 else V0.clone()
        cs = torch.zeros((B, H, nC, d), device=dev)
        gs = torch.zeros((B, H, nC * m, d), device=dev)
        hga.build_summaries(p, K, L, 0, jq, cs, gs)
        reps.append(dict(K=K, V=V, cs=cs, gs=gs, O=torch.empty((B, Hq, 1, d), device=dev),
                         gi=torch.empty((B, H, 1, s.top_g), dtype=torch.int32, device=dev),
                         ws=hga.workspace(p, hga.OP_DECODE, 1, L, device=dev),
                         wa=hga.workspace(p, hga.OP_ATTEND, 1, L, device=dev),
                         w0=hga.workspace(p0, hga.OP_DECODE, 1, L, device=dev)))
    seq = torch.full((B,), L, dtype=torch.int32, device=dev)
    qpos = seq - 1

    def full(i):
        r = reps[i % R]
        hga.decode(p, Q, r["K"], r["V"], L, seq, r["cs"], r["gs"], r["O"], r["ws"], group_idx=r["gi"])

    def reuse(i):
        r = reps[i % R]
        hga.attend(p, Q, 1, qpos, r["K"], r["V"], L, r["gi"], r["O"], r["wa"])

    def streaming(i):
        r = reps[i % R]
        hga.decode(p0, Q, r["K"], r["V"], L, seq, r["cs"], r["gs"], r["O"], r["w0"])

    def timed(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(R):
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(R):
                fn(i)
        for _ in range(4):
            g.replay()
        torch.cuda.synchronize()
        n_rep = max(1, args.steps // R)
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(n_rep):
            g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (n_rep * R)

    full_us = timed(full)     # also leaves every replica's group lists in place
    reuse_us = timed(reuse)
    stream_us = timed(streaming)
    log(f"[bench] decode_32k full step {full_us:.2f} us, attend over reused lists {reuse_us:.2f} us, "
        f"streaming heads {stream_us:.2f} us")
    del reps
    torch.cuda.empty_cache()
    return {"route_once_attend_many": {"workload": "decode_32k", "full_step_us": round(full_us, 3),
                                       "attend_reused_lists_us": round(reuse_us, 3),
                                       "share_saved": round(1 - reuse_us / full_us, 4)},
            "streaming_heads": {"workload": "decode_32k with top_k = top_g = 0", "step_us": round(stream_us, 3),
                                "query_tokens_per_s": round(B / (stream_us * 1e-6), 1)}}


def bench_offload(args, dev):
    """The 128K cold-tier decode workload: K/V in pinned host memory, summaries and
    the hot windows in HBM, the routed groups copied over PCIe on a side stream by
    hga_decode_offload.  Timed with HIP events on the launch stream; the rate of
    the routed-group copies is reported as PCIe GB/s (whole step, PCIe-inclusive)."""
    import torch
    from hierarchical_sparse_attention_build_amd import hga
    from hierarchical_sparse_attention_build_amd import workloads as W
    s = W.spec("offload_decode_128k")
    log(f"[bench] generating {s.name} (seed {s.seed})")
    w = W.make(s)
    B, Hq, H, d, L, C, G = s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.n_tokens, s.chunk_size, s.group_size
    p = hga.params(B, Hq, H, d, C, G, s.n_sink, s.n_local, s.top_k, s.top_g, s.rope_base,
                   s.hf_threshold, qkv_dtype=hga.HGA_BF16, out_dtype=hga.HGA_F32)
    K_host = W.to_torch(w.K, s.dtype, pin=True)
    V_host = W.to_torch(w.V, s.dtype, pin=True)
    Q = W.to_torch(w.Q, s.dtype).to(dev)
    nC, m, j = L // C, C // G, (L - 1) // C
    cs = torch.zeros((B, H, nC, d), device=dev)
    gs = torch.zeros((B, H, nC * m, d), device=dev)
    K_dev = K_host.to(dev)
    hga.build_summaries(p, K_dev, L, 0, j, cs, gs)
    hot = s.n_sink + s.n_local + 1
    K_hot = torch.zeros((B, H, hot * C, d), dtype=K_dev.dtype, device=dev)
    V_hot = torch.zeros_like(K_hot)
    V_dev = V_host.to(dev)
    for c in list(range(s.n_sink)) + list(range(j - s.n_local, j + 1)):
        sl = hga.hot_slot(c, s.n_sink, s.n_local)
        K_hot[:, :, sl * C:(sl + 1) * C] = K_dev[:, :, c * C:(c + 1) * C]
        V_hot[:, :, sl * C:(sl + 1) * C] = V_dev[:, :, c * C:(c + 1) * C]
    del K_dev, V_dev, w
    torch.cuda.empty_cache()
    seq = torch.full((B,), L, dtype=torch.int32, device=dev)
    O = torch.empty((B, Hq, 1, d), device=dev)
    copy_bytes = B * H * s.top_g * G * d * 2 * 2
    staging = torch.empty(copy_bytes, dtype=torch.uint8, device=dev)
    ws = hga.workspace(p, hga.OP_DECODE_OFFLOAD, 1, L, device=dev)
    copy_stream = torch.cuda.Stream()

    def step():
        hga.decode_offload(p, Q, K_host, V_host, K_hot, V_hot, L, seq, cs, gs, O, staging, ws,
                           copy_stream=copy_stream.cuda_stream)

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    n = max(5, args.steps // 10)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(n):
        step()
    e1.record(st)
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3 / n
    pcie = copy_bytes / (step_us * 1e-6) / 1e9
    log(f"[bench] offload_decode_128k step {step_us:.1f} us -> {B / (step_us * 1e-6):.0f} query tokens/s, "
        f"routed groups over PCIe at {pcie:.1f} GB/s (step-inclusive)")

    # warm tier: an LRU of 2 * top_g routed groups per (b, kv head) in HBM; only
    # missing groups cross the host link.  Two query sequences: the same query
    # every step (routed sets repeat), and a random walk of the query (each step
    # adds N(0, 0.25^2) to every component, so routed sets drift).  The steps go
    # in HIP graphs, as a serving loop would issue them: from a fresh cache, 5
    # warm-up steps, then n_w timed steps; the median over a few such runs.  The
    # same steps issued one by one from Python are logged for comparison.
    slots = 2 * s.top_g
    group_bytes = G * d * 2 * 2  # K and V rows of one group (bf16)
    rng = np.random.default_rng(s.seed + 17)
    q0 = Q.float().cpu().numpy()
    n_w, n_runs = 20, 5
    walk = [q0]
    for _ in range(5 + n_w - 1):
        walk.append(walk[-1] + 0.25 * rng.standard_normal(q0.shape).astype(np.float32))
    Q_walk = [W.to_torch(W.bf16_bits(q), "bf16").to(dev) for q in walk]
    warm_out = {"slots_per_kv_head": slots, "group_bytes": group_bytes, "timed_steps": n_w, "runs": n_runs,
                "timing": "HIP graphs of the steps, HIP events around the timed graph; median over runs"}
    for name, qs in (("repeat", [Q] * (5 + n_w)), ("drift", Q_walk)):
        warm = hga.warm_state(p, slots, device=dev)
        hits = torch.zeros((5 + n_w, B, H), dtype=torch.int32, device=dev)
        miss = torch.zeros_like(hits)
        wsw = hga.workspace(p, hga.OP_DECODE_OFFLOAD, 1, L, device=dev)

        def wstep(i):
            warm["hits"], warm["misses"] = hits[i], miss[i]
            hga.decode_offload_warm(p, qs[i], K_host, V_host, K_hot, V_hot, L, seq, cs, gs, O, warm, wsw)

        def reset():
            warm["tags"].fill_(-1)
            warm["stamps"].zero_()
            warm["clock"].zero_()

        # host-issued steps
        reset()
        for i in range(5):
            wstep(i)
        torch.cuda.synchronize()
        e0.record(st)
        for i in range(5, 5 + n_w):
            wstep(i)
        e1.record(st)
        torch.cuda.synchronize()
        host_us = e0.elapsed_time(e1) * 1e3 / n_w
        # graph replays
        g_pre = graph_of(wstep, 5)
        g_run = graph_of(lambda i: wstep(5 + i), n_w)
        runs = []
        for _ in range(n_runs):
            reset()
            g_pre.replay()
            e0.record(st)
            g_run.replay()
            e1.record(st)
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1) * 1e3 / n_w)
        w_us = float(np.median(runs))
        h, mi = hits[5:].sum().item(), miss[5:].sum().item()
        rate = h / max(1, h + mi)
        wbytes = mi * group_bytes / n_w
        log(f"[bench] offload_decode_128k warm tier ({name}): step {w_us:.1f} us (graph, median of {n_runs} runs of "
            f"{n_w} steps; {min(runs):.1f}-{max(runs):.1f}; issued from Python {host_us:.1f} us), hit rate {rate:.3f}, "
            f"{wbytes / 1e6:.2f} MB over the host link per step (vs {copy_bytes / 1e6:.2f} MB without)")
        warm_out[name] = {"ms_per_step": round(w_us / 1e3, 6), "ms_per_step_host_issued": round(host_us / 1e3, 6),
                          "hit_rate": round(rate, 4), "host_to_hbm_bytes_per_step": int(wbytes),
                          "pcie_gbs_step_inclusive": round(wbytes / (w_us * 1e-6) / 1e9, 2)}
        del g_pre, g_run
    return {"workload": "offload_decode_128k", "batch": B, "context": L, "top_k": s.top_k, "top_g": s.top_g,
            "ms_per_step": round(step_us / 1e3, 6), "query_tokens_per_s": round(B / (step_us * 1e-6), 1),
            "host_to_hbm_bytes_per_step": copy_bytes, "pcie_gbs_step_inclusive": round(pcie, 2),
            "bound": "host link (PCIe Gen5 x16, about 64 GB/s)", "warm_tier": warm_out}


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo ("unknown" if absent)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(s, w, prefill=True):
    """The oracle timed on this host's cores.

    Decode: full decode steps of all sequences (routing over prebuilt oracle
    summary tables + exact attention), repeated for about 12 s.
    Prefill (32K): the oracle's summary build over the whole sequence, then
    routing and attention of a sample of 64 units (8 query chunks spread over
    the sequence per KV head); the full call's time is estimated as the summary
    time + the sample's time scaled to all 4096 units."""
    from threadpoolctl import threadpool_limits

    import oracle as O
    from hierarchical_sparse_attention_build_amd import workloads as W
    log("[bench] cpu baseline: preparing oracle tables")
    cfg = O.HGAConfig(**W.hga_config_kwargs(s))
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        Kf = W.to_f64(w.K, s.dtype)
        Vf = W.to_f64(w.V, s.dtype)
        Qf = W.to_f64(w.Q, s.dtype)
        jq = (s.n_tokens - 1) // s.chunk_size
        cs, gs = O.build_summaries(Kf[:, :, : jq * s.chunk_size], cfg)
        cs = np.concatenate([cs, np.zeros((*cs.shape[:2], s.n_tokens // s.chunk_size - jq, s.head_dim))], 2)
        reps = 0
        t0 = time.perf_counter()
        while True:
            O.decode(Qf, Kf, Vf, w.seq_len, cs, gs, cfg, s.n_kv_heads)
            reps += 1
            el = time.perf_counter() - t0
            if el > 12.0:
                break
        del Kf, Vf, Qf, cs, gs
        rate = s.batch * reps / el
        log(f"[bench] cpu oracle decode: {reps} steps in {el:.1f} s -> {rate:.1f} query tokens/s")
        out = {"value": round(rate, 2), "unit": "query tokens/s", "cores": cores, "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": f"{reps} full decode steps of decode_32k (all {s.batch} sequences, 64 units; "
                         "routing over prebuilt oracle summary tables + exact attention), numpy float64, "
                         f"BLAS threads = {cores} (the host cores available to the process)"}
        if prefill:
            out["prefill"] = cpu_baseline_prefill(cores)
    return out


def cpu_baseline_prefill(cores):
    import oracle as O
    from hierarchical_sparse_attention_build_amd import workloads as W
    sp = W.spec("prefill_32k")
    log(f"[bench] cpu baseline prefill: generating {sp.name}")
    wp = W.make(sp)
    cfg = O.HGAConfig(**W.hga_config_kwargs(sp))
    H, n, C = sp.n_kv_heads, sp.n_tokens, sp.chunk_size
    nU = n // C
    Qf, Kf, Vf = W.to_f64(wp.Q, sp.dtype), W.to_f64(wp.K, sp.dtype), W.to_f64(wp.V, sp.dtype)
    del wp
    t0 = time.perf_counter()
    cs, gs = O.build_summaries(Kf, cfg)
    t_sum = time.perf_counter() - t0
    q_pos = np.zeros(1, dtype=np.int64)
    units = [(0, h, int(u)) for h in range(H) for u in np.linspace(nU // 16, nU - 1, 8).astype(int)]
    t1 = time.perf_counter()
    _, gi, _ = O.route(Qf, q_pos, cs, gs, cfg, H, units=units)
    for (b, h, u) in units:
        O.attend_unit_block(Qf, q_pos, Kf, Vf, gi, cfg, H, b, h, u)
    t_units = time.perf_counter() - t1
    frac = len(units) / (H * nU)
    est = t_sum + t_units / frac
    rate = n / est
    log(f"[bench] cpu oracle prefill: summaries {t_sum:.1f} s, {len(units)} units {t_units:.1f} s -> "
        f"full call about {est:.0f} s, {rate:.1f} query tokens/s")
    return {"value": round(rate, 2), "unit": "query tokens/s", "cores": cores, "kind": "oracle",
            "est_s_per_call": round(est, 2),
            "sample": f"prefill_32k: the oracle's summary build over all 32768 tokens ({t_sum:.1f} s), then "
                      f"routing + attention of {len(units)} of the {H * nU} units (8 query chunks per KV head, "
                      f"spread over the sequence; {t_units:.1f} s), scaled to all units"}


if __name__ == "__main__":
    main()
