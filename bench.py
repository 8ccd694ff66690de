"""Benchmark of the CSA2 decode hot path on one MI355X.

Default workload: one Full-mode CSA2 layer, decode, 32 sequences x 1 query token, 16384 FP4
entries of 512 channels per sequence (a 65536-token context at compression 4), 64 query heads,
8 x 64 bf16 indexer heads, Top-K 512. A step is one csa2_layer_step(FULL): indexer scores over
every entry -> Top-K -> sparse attention over the selected FP4 rows. Inputs are seeded and
synthetic and already resident in HBM; two copies of the per-step inputs alternate so the
256 MB last-level cache cannot hold one step's keys for the next.

Prints one JSON line: query-tokens/s, achieved HBM GB/s of the dominant kernel (the streaming
indexer) against the 8 TB/s peak, and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]
    python bench.py --calibrate-copy     # a plain 1 GiB copy, for rocprofv3 counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
COUNTERS = os.path.join(ROOT, "profiles", "index_stream_full_decode_b32_n16384.counters.json")
COUNTERS_WORKLOAD = "full_decode_b32_n16384"
INDEX_SOURCES = ["fp4_kv_cache_e2m1_amd/csrc/index_decode.hip", "fp4_kv_cache_e2m1_amd/csrc/common.h"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dev_bf16(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def build_inputs(wl, dev, copies):
    """Device inputs of the workload: FP4 cache (quantized on the GPU), indexer keys, queries."""
    import torch
    import fp4_kv_cache_e2m1_amd as P
    from fp4_kv_cache_e2m1_amd import workloads as W
    rows = torch.empty(wl.B, wl.N, P.row_bytes(wl.D), dtype=torch.uint8, device=dev)
    kidx = torch.empty(wl.B, wl.N, wl.Hk, wl.Di, dtype=torch.bfloat16, device=dev)
    for b in range(wl.B):
        P.quantize_kv_fp4(torch.from_numpy(W.kv_source(wl, b)).to(dev), out=rows[b])
        kidx[b] = dev_bf16(W.k_idx(wl, b), dev)
    nl = len(wl.modes)
    q = [torch.stack([dev_bf16(W.q_main(wl, b, l), dev) for b in range(wl.B)]) for l in range(nl)]
    qi = [torch.stack([dev_bf16(W.q_idx(wl, b, l), dev) for b in range(wl.B)]) for l in range(nl)]
    sets = [dict(rows=rows, kidx=kidx, q=q, qi=qi)]
    for _ in range(copies - 1):
        sets.append(dict(rows=rows.clone(), kidx=kidx.clone(), q=[t.clone() for t in q], qi=[t.clone() for t in qi]))
    return sets


def algorithmic_bytes(wl):
    """Bytes the method must move per step: for every index-producing layer the indexer keys it
    scores (all entries, or the pool), its indexer query, the pool it reads or writes and the
    Top-K it writes; for every layer the Top-K it reads, the 288-byte FP4 rows it gathers, its
    bf16 query and its fp32 output. Score arrays are intermediates and are not counted."""
    R = wl.B * wl.T
    kbytes = wl.Hk * wl.Di * 2
    row_b = wl.D // 2 + wl.D // 16
    P = wl.pool_blocks * wl.block
    total = 0
    for l, mode in enumerate(wl.modes):
        if mode == 0:                                   # Full: every entry
            total += wl.B * wl.N * kbytes + R * wl.Hi * wl.Di * 2 + R * wl.k * 4
            if P:
                total += R * P * 4                      # pool written
        elif mode == 1:                                 # Reindex: the pool, or every entry
            keys = R * P * kbytes + R * P * 4 if P else wl.B * wl.N * kbytes
            total += keys + R * wl.Hi * wl.Di * 2 + R * wl.k * 4
        total += R * wl.k * 4 + R * wl.k * row_b + R * wl.H * wl.D * 2 + R * wl.H * wl.D * 4
    return total


def index_kernel_bytes(wl):
    """Algorithmic bytes of one flat indexer launch: every key row once plus the queries."""
    return wl.B * wl.N * wl.Hk * wl.Di * 2 + wl.B * wl.T * wl.Hi * wl.Di * 2


def sources_sha():
    h = hashlib.sha256()
    for p in INDEX_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_counters(launch_bytes):
    """HBM bytes per indexer launch from committed rocprofv3 counters, if the kernel is unchanged."""
    if not os.path.exists(COUNTERS):
        return None
    c = json.load(open(COUNTERS))
    if c.get("sources_sha") != sources_sha():
        return None
    return float(c["fetch_bytes_per_launch"] + c["write_bytes_per_launch"])


def cpu_baseline(wl, n_seq, min_seconds):
    """The oracle's layer step on host cores, in query-tokens/s.

    n_seq sequences of the workload are generated and their caches quantized up front (untimed);
    the timed loop then runs full Full-layer steps over them, cycling, until at least min_seconds
    of CPU work have been done.
    """
    import threadpoolctl
    from fp4_kv_cache_e2m1_amd import workloads as W
    from oracle import csa2_oracle as O
    f64 = lambda b: W.bf16_bits_to_f32(b).astype(np.float64)
    prepared = []
    for b in range(n_seq):
        seq = W.sequence(wl, b)
        prepared.append((seq, O.quantize_kv_fp4(seq["kv_src"])))
    info = threadpoolctl.threadpool_info()
    threads = max(i.get("num_threads", 1) for i in info) if info else 1
    done = 0
    t0 = time.perf_counter()
    while True:
        seq, packed = prepared[done % n_seq]
        kv = O.dequant_kv_fp4(packed)
        O.layer_step(O.FULL, q=f64(seq["q"][0]), kv_deq=kv, k_idx=f64(seq["k_idx"]), q_idx=f64(seq["q_idx"][0]),
                     n_vis=[wl.N], k=wl.k, sm_scale=wl.sm_scale)
        done += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds and done >= n_seq:
            break
    return {"value": round(done * wl.T / dt, 3), "unit": "query-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} Full-layer steps over {n_seq} of the {wl.B} sequences (each: dequantize the "
                      f"{wl.N}-entry cache, score it, Top-{wl.k}, attention over {wl.H} heads); numpy fp64, "
                      f"{dt:.1f} s"}


def fp4_indexer_leg(wl, sets, steps, dev, stream):
    """csa2_index_scores_mxfp4 over the workload's B x N entries with their Hi x Di indexer
    channels stored as MXFP4 rows (seeded synthetic codes and scales), two alternating copies;
    achieved bytes per launch against the HBM peak. Then the whole Full layer step with those
    keys (indexer, Top-K, attention over the same FP4 main-KV rows), timed the same way."""
    import torch
    import fp4_kv_cache_e2m1_amd as P
    from fp4_kv_cache_e2m1_amd import workloads as W
    kc, qc = wl.Hk * wl.Di, wl.Hi * wl.Di          # channels of a key row and of a query row
    shared = wl.Hk == 1 and wl.Di == 128
    keys = [torch.from_numpy(np.stack([W.mxfp4_rows(wl, b, wl.N, kc, copy=c) for b in range(wl.B)])).to(dev)
            for c in range(2)]
    q = torch.from_numpy(np.stack([W.mxfp4_rows(wl, b, wl.T, qc, copy=2) for b in range(wl.B)])).to(dev)
    C, qh = (wl.Di, wl.Hi) if shared else (kc, 0)
    out = torch.empty(wl.B * wl.T, wl.N, dtype=torch.float32, device=dev)
    for i in range(3):
        P.index_scores_mxfp4(q, keys[i % 2], C, out=out, q_heads=qh)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        P.index_scores_mxfp4(q, keys[i % 2], C, out=out, q_heads=qh)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    rb, qrb = kc // 2 + kc // 32, qc // 2 + qc // 32
    nbytes = wl.B * wl.N * rb + wl.B * wl.T * qrb
    gbs = nbytes / (us * 1e-6) / 1e9
    # the Full layer step with FP4 indexer keys
    ws = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    layer = []
    for c in range(2):
        s = sets[c % len(sets)]
        kv = P.KVState(s["rows"], None, k_mx=keys[c], mx_heads=(wl.Hk, wl.Di))
        idx = P.IdxState.empty(wl.B * wl.T, wl.k, dev)
        o = torch.empty(wl.B, wl.T, wl.H, wl.D, dtype=torch.float32, device=dev)
        layer.append((s["q"][0], kv, idx, o))

    def full_step(i):
        qm, kv, idx, o = layer[i % 2]
        P.layer_step(P.FULL, qm, kv, idx, q_idx_mx=q, sm_scale=wl.sm_scale, with_lse=False, ws=ws, out=o)

    for i in range(3):
        full_step(i)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        full_step(i)
    b.record(stream)
    torch.cuda.synchronize()
    step_us = a.elapsed_time(b) / steps * 1e3
    row_b = wl.D // 2 + wl.D // 16
    R = wl.B * wl.T
    step_bytes = nbytes + R * wl.k * 4 * 2 + R * wl.k * row_b + R * wl.H * wl.D * 2 + R * wl.H * wl.D * 4
    extra = {}
    if len(wl.modes) > 1:
        # the workload's whole layer schedule with FP4 indexer keys (and its pool)
        use_pool = wl.pool_blocks > 0
        stacks = []
        for c in range(2):
            s = sets[c % len(sets)]
            kv = P.KVState(s["rows"], None, k_mx=keys[c], mx_heads=(wl.Hk, wl.Di))
            idx = P.IdxState.empty(R, wl.k, dev, pool_size=wl.pool_blocks * wl.block if use_pool else 0)
            outs = [torch.empty(wl.B, wl.T, wl.H, wl.D, dtype=torch.float32, device=dev) for _ in wl.modes]
            stacks.append((s, kv, idx, outs))

        def schedule(i):
            s, kv, idx, outs = stacks[i % 2]
            for l, mode in enumerate(wl.modes):
                P.layer_step(mode, s["q"][l], kv, idx, q_idx_mx=q if mode != 2 else None, sm_scale=wl.sm_scale,
                             use_pool=use_pool, pool_blocks=wl.pool_blocks if use_pool else 0, with_lse=False,
                             ws=ws, out=outs[l])

        for i in range(3):
            schedule(i)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(steps):
            schedule(i)
        b.record(stream)
        torch.cuda.synchronize()
        sched_us = a.elapsed_time(b) / steps * 1e3
        extra = {"schedule_us": round(sched_us, 2), "schedule_query_tokens_per_s": round(R / (sched_us * 1e-6), 1),
                 "schedule_pool": use_pool}
    return {**extra, "kernel": "index_mxfp4_kernel (MXFP4 indexer scores)", "bound": "hbm", "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": round(us, 2), "row_bytes": rb,
            "full_step_us": round(step_us, 2), "full_step_query_tokens_per_s": round(R / (step_us * 1e-6), 1),
            "full_step_algorithmic_bytes": step_bytes,
            "full_step_hbm_frac": round(step_bytes / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def window_leg(wl, sets, state, n_rows, steps, dev, stream):
    """Attention over the last step's Top-K joined with full windows of n_rows FP8 rows
    (csa2_sparse_attn_swa in decode, csa2_sparse_attn_swa_prefill for many query tokens, each
    token's window ending at its own), timed beside the same attention without the window."""
    import torch
    import fp4_kv_cache_e2m1_amd as P
    from fp4_kv_cache_e2m1_amd import _lib, workloads as W
    B, T = wl.B, wl.T
    buf_rows = n_rows if T == 1 else T + n_rows - 1
    wins = [W.swa_window(wl, b, buf_rows) for b in range(B)]
    codes = torch.from_numpy(np.stack([c for c, _ in wins])).to(dev)
    exps = torch.from_numpy(np.stack([e for _, e in wins])).to(dev)
    n_win = torch.full((B,) if T == 1 else (B, T), n_rows, dtype=torch.int32, device=dev)
    need = _lib.lib().csa2_sparse_attn_swa_prefill_workspace_size(B, T, wl.H, wl.D, wl.k) if T > 1 else 0
    ws = torch.empty(max(64 << 20, need), dtype=torch.uint8, device=dev)
    calls = []
    for s, kv, idx, _ in state:
        q = s["q"][0] if T > 1 else s["q"][0].view(B, wl.H, wl.D)
        calls.append((q, s["rows"], idx.topk.view(B, T, wl.k) if T > 1 else idx.topk.view(B, wl.k)))

    def timed(fn):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(steps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps * 1e3

    def with_window(i):
        q, rows, topk = calls[i % len(calls)]
        if T == 1:
            P.sparse_attn_swa(q, rows, topk, codes, exps, n_win, wl.sm_scale, with_lse=False, ws=ws)
        else:
            P.sparse_attn_swa_prefill(q, rows, topk, codes, exps, n_win, wl.sm_scale, with_lse=False, ws=ws)

    def without(i):
        q, rows, topk = calls[i % len(calls)]
        P.sparse_attn(q.view(B, T, wl.H, wl.D), rows, topk.view(B, T, wl.k), wl.sm_scale, with_lse=False, ws=ws)

    us_w, us_s = timed(with_window), timed(without)
    row_b = wl.D // 2 + wl.D // 16
    nbytes = B * (T * wl.k * (4 + row_b) + buf_rows * (wl.D + 1) + T * wl.H * wl.D * 2 + T * wl.H * wl.D * 4)
    return {"window_rows": n_rows, "us_per_call": round(us_w, 2), "sparse_only_us_per_call": round(us_s, 2),
            "algorithmic_bytes": nbytes, "hbm_gbs": round(nbytes / (us_w * 1e-6) / 1e9, 1)}


def calibrate_copy(dev):
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {n} bytes x 5")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--copies", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=2)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay each step from a captured HIP graph")
    ap.add_argument("--fp4-indexer", action="store_true",
                    help="also time the FP4 (MXFP4) indexer on the workload's keys, stored as MXFP4 rows")
    ap.add_argument("--window", type=int, default=0,
                    help="also time decode attention with each sequence's window of this many FP8 rows")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the hot path has no "
              "multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp4_kv_cache_e2m1_amd as P
    from fp4_kv_cache_e2m1_amd import _lib, workloads as W
    if not os.path.exists(_lib.LIB_PATH):
        from fp4_kv_cache_e2m1_amd import build_lib
        build_lib.build()
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(dev)
        return

    wl = W.CONFIGS[args.config]
    log(f"[bench] workload {wl.name}: generating inputs")
    sets = build_inputs(wl, dev, args.copies)
    stream = torch.cuda.current_stream(dev)
    R = wl.B * wl.T
    n_vis = None
    if wl.T > 1:
        n_vis = torch.clamp(P.prefill_n_vis(wl.p0, wl.T, wl.ratio, dev), max=wl.N).repeat(wl.B)
    # per-set shared state and buffers, allocated once
    state = []
    for s in sets:
        kv = P.KVState(s["rows"], s["kidx"], n_vis)
        idx = P.IdxState.empty(R, wl.k, dev, pool_size=wl.pool_blocks * wl.block)
        outs = [torch.empty(wl.B, wl.T, wl.H, wl.D, dtype=torch.float32, device=dev) for _ in wl.modes]
        state.append((s, kv, idx, outs))
    ws = torch.empty(256 << 20, dtype=torch.uint8, device=dev)

    def step(i):
        s, kv, idx, outs = state[i % len(state)]
        for l, mode in enumerate(wl.modes):
            P.layer_step(mode, s["q"][l], kv, idx, q_idx=s["qi"][l] if mode != 2 else None,
                         sm_scale=wl.sm_scale, use_pool=wl.pool_blocks > 0, pool_blocks=wl.pool_blocks,
                         with_lse=False, ws=ws, out=outs[l])

    log(f"[bench] warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.graph:
        # one graph per input set; replays alternate like the eager steps
        graphs = []
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for i in range(len(state)):
                step(i)
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        for i in range(len(state)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        torch.cuda.synchronize()
        eager_step = step

        def step(i):  # noqa: F811
            graphs[i % len(graphs)].replay()

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # dominant kernel: the flat streaming indexer, timed alone on the same stream
    sc = torch.empty(R, wl.N, dtype=torch.float32, device=dev)
    for i in range(3):
        s = sets[i % len(sets)]
        P.index_scores(s["qi"][0], s["kidx"], n_vis=n_vis, out=sc)
    torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for i in range(args.steps):
        s = sets[i % len(sets)]
        P.index_scores(s["qi"][0], s["kidx"], n_vis=n_vis, out=sc)
    k1.record(stream)
    torch.cuda.synchronize()
    kms = k0.elapsed_time(k1) / args.steps
    kbytes = index_kernel_bytes(wl)
    if wl.T > 1:
        # prefill: the indexer is a causal MFMA contraction; report it against the bf16 MFMA peak
        kflops = 2.0 * wl.Hi * wl.Di * float(n_vis.clamp(min=0, max=wl.N).sum().item())
        achieved = kflops / (kms * 1e-3) / 1e12
        roofline = {"kernel": "index_prefill_qs_kernel (causal indexer scores)", "bound": "mfma",
                    "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "algorithmic_flops_per_launch": kflops, "avg_launch_us": round(kms * 1e3, 2)}
    else:
        achieved = kbytes / (kms * 1e-3) / 1e9
        traffic = traffic_from_counters(kbytes) if wl.name == COUNTERS_WORKLOAD else None
        roofline = {"kernel": "index_stream_kernel (flat indexer scores)", "bound": "hbm",
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "algorithmic_bytes_per_launch": kbytes, "avg_launch_us": round(kms * 1e3, 2)}

    step_bytes = algorithmic_bytes(wl)
    value = R / (ms * 1e-3)
    line = {
        "metric": "CSA2 decode query-tokens/s + achieved HBM GB/s (% of peak) at 1 MI355X",
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "query_tokens": wl.T, "entries": wl.N,
                   "latent_dim": wl.D, "heads": wl.H, "index_heads": wl.Hi, "index_dim": wl.Di,
                   "topk": wl.k, "layers": [["FULL", "REINDEX", "REUSE"][m] for m in wl.modes],
                   "pool_blocks": wl.pool_blocks, "kv_format": "E2M1 + E4M3 per 16 channels (288 B/entry)"},
        "launch": "hip graph replay" if args.graph else "eager",
        "step_hbm_gbs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_algorithmic_bytes": step_bytes,
        "roofline": roofline,
    }
    fp4_shape = (wl.Hk == wl.Hi and wl.Hi * wl.Di in (256, 512)) or (wl.Hk == 1 and wl.Di == 128)
    if args.fp4_indexer and wl.T == 1 and fp4_shape:
        line["fp4_indexer"] = fp4_indexer_leg(wl, sets, args.steps, dev, stream)
    if args.window > 0:
        line["window_attention"] = window_leg(wl, sets, state, args.window, args.steps, dev, stream)
    if not args.no_cpu_baseline and args.config == 2:
        log(f"[bench] CPU oracle on {args.cpu_sample} sequences, >= {args.cpu_seconds} s")
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
