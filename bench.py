"""Benchmark of the CSA2 decode hot path on one MI355X.

Headline workload (the largest decode workload that fits one GPU): a three-layer CSA2 stack
Full -> Reindex -> Reuse over one shared FP4 main-KV cache and one indexer-key cache, decode, 16
sequences x 1 query token, 65536 FP4 entries of 512 channels per sequence (a 262144-token
context at compression 4), 64 query heads, 8 x 64 bf16 indexer heads, Top-K 512. A step is the
three csa2_layer_step calls: Full (indexer over every entry -> Top-K -> sparse attention),
Reindex (its own indexer query over every entry -> Top-K -> attention), Reuse (attention over
the Reindex layer's Top-K). Inputs are seeded and synthetic and already resident in HBM; two
copies of the per-step inputs alternate so the 256 MB last-level cache cannot hold one step's
keys for the next.

Prints one JSON line: query-tokens/s of the headline step, the achieved HBM GB/s of its dominant
kernel (the streaming indexer) against the 8 TB/s peak, the CPU oracle timed on a bounded sample,
and `legs`: the same measurement for the one-layer decode workload (32 x 16384), the
hierarchical-indexer decode workload (4 x 262144, pool of 8192) and the prefill chunk (4096
tokens over 33792 entries; its roofline is the MFMA indexer against the bf16 MFMA peak).

    python bench.py [--steps K] [--warmup W] [--config 3] [--legs 2,4,5|none] [--no-cpu-baseline]
    python bench.py --calibrate-copy     # a plain 1 GiB copy, for rocprofv3 counter scaling
    python bench.py --trace-summary DB   # per-kernel, per-grid table of a rocprofv3 results database
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
MFMA_FP4_PEAK_TFLOPS = 10100.0
PROFILES = os.path.join(ROOT, "profiles")
INDEX_SOURCES = ["fp4_kv_cache_e2m1_amd/csrc/index_decode.hip", "fp4_kv_cache_e2m1_amd/csrc/common.h"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dev_bf16(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def build_inputs(wl, dev, copies):
    """Device inputs of the workload: FP4 cache (quantized on the GPU), indexer keys, queries.
    The seeded host draws of the sequences run on a thread pool (numpy's generators release the
    interpreter lock), a few sequences at a time."""
    import concurrent.futures as cf
    import torch
    import fp4_kv_cache_e2m1_amd as P
    from fp4_kv_cache_e2m1_amd import workloads as W
    rows = torch.empty(wl.B, wl.N, P.row_bytes(wl.D), dtype=torch.uint8, device=dev)
    kidx = torch.empty(wl.B, wl.N, wl.Hk, wl.Di, dtype=torch.bfloat16, device=dev)
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(workers) as ex:
        for b0 in range(0, wl.B, workers):
            bs = range(b0, min(wl.B, b0 + workers))
            for b, (src, keys) in zip(bs, ex.map(lambda b: (W.kv_source(wl, b), W.k_idx(wl, b)), bs)):
                P.quantize_kv_fp4(torch.from_numpy(src).to(dev), out=rows[b])
                kidx[b] = dev_bf16(keys, dev)
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


def counters_path(workload):
    return os.path.join(PROFILES, f"index_stream_{workload}.counters.json")


def traffic_from_counters(workload):
    """HBM bytes per indexer launch from committed rocprofv3 counters of this workload, if the
    kernel's sources are unchanged since they were taken; else None."""
    path = counters_path(workload)
    if not os.path.exists(path):
        return None
    c = json.load(open(path))
    if c.get("sources_sha") != sources_sha():
        return None
    return float(c["fetch_bytes_per_launch"] + c["write_bytes_per_launch"])


def _pmc_by_kernel(db_path):
    """{(kernel, grid): [counter value per dispatch]} from a rocprofv3 --pmc results database."""
    import collections
    import sqlite3
    db = sqlite3.connect(db_path)
    names = {r[0]: r[1] or r[2] for r in db.execute("select id, display_name, kernel_name from rocpd_info_kernel_symbol")}
    vals = collections.defaultdict(float)
    for eid, v in db.execute("select event_id, value from rocpd_pmc_event"):
        vals[eid] += v
    out = collections.defaultdict(list)
    for kid, eid, gx, gy, gz in db.execute(
            "select kernel_id, event_id, grid_size_x, grid_size_y, grid_size_z from rocpd_kernel_dispatch"):
        out[(names.get(kid, "?").split("(")[0], f"{gx}x{gy}x{gz}")].append(vals[eid])
    return out


def counter_summary(config, fetch_db, write_db, copy_fetch_db, copy_write_db, commands):
    """Writes profiles/index_stream_<workload>.counters.json and a markdown table of HBM bytes per
    dispatch from two --pmc runs of `bench.py --config N --legs none` (FETCH_SIZE, then
    WRITE_SIZE) and two of `bench.py --calibrate-copy` (a 1 GiB copy), which give the factor that
    turns each counter into bytes."""
    from fp4_kv_cache_e2m1_amd import workloads as W
    wl = W.CONFIGS[config]
    F, Wr = _pmc_by_kernel(fetch_db), _pmc_by_kernel(write_db)
    CF, CW = _pmc_by_kernel(copy_fetch_db), _pmc_by_kernel(copy_write_db)
    cf = max(v for k, vs in CF.items() if "copyBuffer" in k[0] for v in vs)      # KiB of the 1 GiB copy
    cw = max(v for k, vs in CW.items() if "copyBuffer" in k[0] for v in vs)
    fs, ws = (1 << 30) / (cf * 1024), (1 << 30) / (cw * 1024)
    idx = max((k for k in F if "index_stream_kernel" in k[0]), key=lambda k: sum(F[k]))
    fk, wk = sum(F[idx]) / len(F[idx]), sum(Wr[idx]) / len(Wr[idx])
    alg = index_kernel_bytes(wl)
    out = {"kernel": idx[0], "grid": idx[1], "workload": wl.name, "sources_sha": sources_sha(),
           "fetch_size_kib_per_dispatch": fk, "write_size_kib_per_dispatch": wk,
           "copy_calibration": {"bytes_copied": 1 << 30, "fetch_size_kib": cf, "write_size_kib": cw,
                                "fetch_scale": fs, "write_scale": ws},
           "fetch_bytes_per_launch": fk * 1024 * fs, "write_bytes_per_launch": wk * 1024 * ws,
           "algorithmic_bytes_per_launch": alg, "commands": commands}
    json.dump(out, open(counters_path(wl.name), "w"), indent=1)
    lines = [f"# HBM bytes per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE), {wl.name}", "",
             f"Each counter was collected in its own pass. FETCH_SIZE reads {1 / fs:.4f} of the bytes a plain 1 GiB "
             f"copy moves (scale {fs:.4f}); WRITE_SIZE scale {ws:.4f}. Scaled values below.", "", "Commands:", "",
             "```", *commands, "```", "",
             "| kernel | grid | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB (scaled) | HBM write MB (scaled) |",
             "|---|---|---|---|---|---|---|"]
    rows = []
    for k in F:
        f = sum(F[k]) / len(F[k])
        w = sum(Wr.get(k, [0.0])) / max(1, len(Wr.get(k, [0.0])))
        rows.append((f * 1024 * fs / 1e6, k, len(F[k]), f, w))
    for mb, k, n, f, w in sorted(rows, reverse=True):
        lines.append(f"| `{k[0][:90]}` | {k[1]} | {n} | {f:.1f} | {w:.1f} | {f * 1024 * fs / 1e6:.2f} | "
                     f"{w * 1024 * ws / 1e6:.2f} |")
    lines += ["", f"Indexer: algorithmic {alg / 1e6:.2f} MB per launch (keys + queries); measured HBM read "
                  f"{fk * 1024 * fs / 1e6:.2f} MB ({fk * 1024 * fs / alg:.4f}x), write {wk * 1024 * ws / 1e6:.2f} MB "
                  "(the fp32 scores)."]
    print("\n".join(lines))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, n_seq, min_seconds):
    """The oracle's whole layer schedule of the workload on host cores, in query-tokens/s.

    n_seq sequences of the workload are generated and their caches quantized up front (untimed);
    the timed loop then runs the workload's layer schedule (e.g. Full -> Reindex -> Reuse) for one
    sequence at a time, cycling, until at least min_seconds of CPU work have been done. The
    oracle's BLAS calls may use every core this process may run on (len(os.sched_getaffinity(0))),
    which is the core count reported; its element-wise numpy work runs on one thread.
    """
    import threadpoolctl
    from fp4_kv_cache_e2m1_amd import workloads as W
    from oracle import csa2_oracle as O
    f64 = lambda b: W.bf16_bits_to_f32(b).astype(np.float64)
    cores = len(os.sched_getaffinity(0))
    prepared = []
    for b in range(n_seq):
        seq = W.sequence(wl, b)
        prepared.append((seq, O.quantize_kv_fp4(seq["kv_src"])))
    use_pool = wl.pool_blocks > 0
    done = 0
    with threadpoolctl.threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        while True:
            seq, packed = prepared[done % n_seq]
            kv = O.dequant_kv_fp4(packed)
            kf = f64(seq["k_idx"])
            topk, pool = None, None
            for l, mode in enumerate(wl.modes):
                r = O.layer_step(mode, q=f64(seq["q"][l]), kv_deq=kv, k_idx=kf,
                                 q_idx=f64(seq["q_idx"][l]) if mode != O.REUSE else None, n_vis=[wl.N], k=wl.k,
                                 shared_topk=topk, pool=pool, pool_blocks=wl.pool_blocks if use_pool else 0,
                                 sm_scale=wl.sm_scale)
                topk, pool = r["topk"], r["pool"]
            done += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds and done >= n_seq:
                break
    layers = " -> ".join(["Full", "Reindex", "Reuse"][m] for m in wl.modes)
    return {"value": round(done * wl.T / dt, 3), "unit": "query-tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} steps of the {layers} schedule, one sequence each, cycling over {n_seq} of the "
                      f"{wl.B} sequences (each: dequantize the {wl.N}-entry cache, then every layer: index scores, "
                      f"Top-{wl.k}, attention over {wl.H} heads); numpy fp64, {dt:.1f} s"}


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
    warm(lambda i: P.index_scores_mxfp4(q, keys[i % 2], C, out=out, q_heads=qh), 3, 60)
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

    warm(full_step, 3, 60)
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

        warm(schedule, 3, 60)
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


def fp4_prefill_leg(wl, n_vis, steps, dev, stream):
    """The prefill indexer over FP4 (MXFP4) query and key rows (seeded synthetic codes and scales,
    two alternating key copies): csa2_index_scores_mxfp4 on the scaled FP4 MFMA, causal, against
    the FP4 dense MFMA peak; the fp32 score writes are reported against the HBM peak too, since
    the contraction itself needs a quarter of the bf16 form's bytes and they dominate its traffic."""
    import torch
    import fp4_kv_cache_e2m1_amd as P
    from fp4_kv_cache_e2m1_amd import workloads as W
    C = wl.Hi * wl.Di
    keys = [torch.from_numpy(np.stack([W.mxfp4_rows(wl, b, wl.N, C, copy=c) for b in range(wl.B)])).to(dev)
            for c in range(2)]
    q = torch.from_numpy(np.stack([W.mxfp4_rows(wl, b, wl.T, C, copy=2) for b in range(wl.B)])).to(dev)
    out = torch.empty(wl.B * wl.T, wl.N, dtype=torch.float32, device=dev)

    def call(i):
        P.index_scores_mxfp4(q, keys[i % 2], C, n_vis=n_vis, out=out)

    warm(call, 3, 60)
    us = time_on_stream(call, steps, stream) * 1e3
    pairs = float(n_vis.clamp(min=0, max=wl.N).sum().item())
    flops = 2.0 * C * pairs
    wbytes = 4.0 * pairs
    tf = flops / (us * 1e-6) / 1e12
    return {"kernel": "index_mxfp4_prefill_kernel (causal indexer scores, FP4 x FP4 MFMA)", "bound": "mfma",
            "achieved": round(tf, 1), "peak": MFMA_FP4_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / MFMA_FP4_PEAK_TFLOPS, 4),
            "algorithmic_flops_per_launch": flops, "avg_launch_us": round(us, 2),
            "score_write_bytes": wbytes, "score_write_gbs": round(wbytes / (us * 1e-6) / 1e9, 1),
            "score_write_frac_of_hbm": round(wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def production_leg(wl, sets, state, n_vis, steps, dev, stream):
    """Producing the caches (csa2_compress_kv: compressor at 4 tokens per entry, FP4 packing and
    the indexer-K projection) for the workload's new tokens: 4 per sequence in decode (one new
    entry each, at the end of the cache), the whole chunk in prefill (T / 4 entries after the
    existing ones). Timed alone, and as part of the first layer (a Full layer that compresses its
    new tokens before scoring) beside the same layer without it, each from a replayed HIP graph of
    back-to-back calls (so the kernels' own time is measured, not the Python enqueue cost)."""
    import torch
    import fp4_kv_cache_e2m1_amd as P
    from fp4_kv_cache_e2m1_amd import workloads as W
    ratio = 4
    n_tok = 4 if wl.T == 1 else wl.T
    n_new = n_tok // ratio
    first = wl.N - n_new
    toks = [W.token_kv(wl, b, n_tok, first=ratio * first) for b in range(wl.B)]
    c = dev_bf16(np.stack([t[0] for t in toks]), dev)
    z = dev_bf16(np.stack([t[1] for t in toks]), dev)
    w = dev_bf16(W.w_index_k(wl), dev)
    e0 = torch.full((wl.B,), first, dtype=torch.int32, device=dev)
    rows = [s["rows"] for s in sets]
    keys = [s["kidx"] for s in sets]

    def compress(i):
        P.compress_kv(c, z, ratio, e0, rows[i % len(rows)], w_t=w, k_idx=keys[i % len(keys)])

    warm(compress, 3, 60)
    us = time_graph(compress, steps, stream) * 1e3
    kc = wl.Hk * wl.Di
    nbytes = wl.B * n_tok * wl.D * 2 * 2 + wl.B * n_new * (wl.D // 2 + wl.D // 16 + kc * 2) + kc * wl.D * 2
    ws = torch.empty(max(256, max(P.layer_workspace_size(0, P.layer_args(0, s_["q"][0], kv, idx, q_idx=s_["qi"][0]),
                                                         kv, idx) for s_, kv, idx, _ in state)),
                     dtype=torch.uint8, device=dev)

    def layer(i, produce):
        s_, kv, idx, outs = state[i % len(state)]
        P.layer_step(0, s_["q"][0], kv, idx, q_idx=s_["qi"][0], sm_scale=wl.sm_scale, with_lse=False, ws=ws,
                     out=outs[0], produce=(c, z, ratio, e0, w) if produce else None)

    warm(lambda i: layer(i, True), 3, 60)
    with_us = time_graph(lambda i: layer(i, True), steps, stream) * 1e3
    without_us = time_graph(lambda i: layer(i, False), steps, stream) * 1e3
    return {"kernel": "compress_kv_kernel (compressor + FP4 packing + indexer-K projection)", "bound": "hbm",
            "new_tokens_per_sequence": n_tok, "new_entries_per_sequence": n_new, "avg_launch_us": round(us, 2),
            "algorithmic_bytes_per_launch": nbytes, "achieved": round(nbytes / (us * 1e-6) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "full_layer_with_production_us": round(with_us, 2), "full_layer_without_us": round(without_us, 2)}


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
        warm(fn, 3, 60)
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


def trace_summary(db_path):
    """Markdown table of a rocprofv3 results database (`rocprofv3 --kernel-trace`): per kernel and
    grid size, the launch count and the average, minimum and maximum duration. Launches of one
    kernel on different workloads have different grids, so their averages stay apart."""
    import collections
    import sqlite3
    db = sqlite3.connect(db_path)
    names = {r[0]: r[1] or r[2] for r in db.execute("select id, display_name, kernel_name from rocpd_info_kernel_symbol")}
    groups = collections.defaultdict(list)
    for kid, st, en, gx, gy, gz, wx in db.execute(
            "select kernel_id, start, end, grid_size_x, grid_size_y, grid_size_z, workgroup_size_x "
            "from rocpd_kernel_dispatch"):
        groups[(names.get(kid, "?").split("(")[0], f"{gx}x{gy}x{gz}/{wx}")].append((en - st) / 1e3)
    total = sum(sum(v) for v in groups.values())
    print("| kernel | grid (threads) / workgroup | calls | total us | avg us | min us | max us | % |")
    print("|---|---|---|---|---|---|---|---|")
    for (name, grid), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{name[:100]}` | {grid} | {len(v)} | {sum(v):.1f} | {sum(v) / len(v):.2f} | {min(v):.2f} | "
              f"{max(v):.2f} | {100 * sum(v) / total:.1f} |")


def time_on_stream(fn, steps, stream):
    """Average milliseconds of fn(i) over `steps` calls, bracketed by HIP events on `stream`."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def warm(fn, min_calls, min_ms):
    """Untimed calls of fn(i): at least min_calls, and until min_ms of wall time have passed. The
    matrix-core kernels of the prefill workload reach their steady clock only after some tens of
    milliseconds of work (the prefill attention read 891, 815, 774, 755, 734 and 731 us in
    successive rounds of ten calls), so one-kernel timings and the further workloads of the line
    warm up by time."""
    import time
    import torch
    i, t0 = 0, time.perf_counter()
    while i < min_calls or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def time_graph(fn, steps, stream):
    """Average milliseconds of fn(i) when `steps` calls are captured into one HIP graph and
    replayed: the launches then run back to back without the Python enqueue cost between them,
    which would otherwise exceed a short kernel's own duration."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(2):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ms = time_on_stream(lambda i: g.replay(), 3, stream) / steps
    del g
    return ms


def measure_workload(wl, args, dev, extras):
    """Times the workload's whole layer schedule (eager launches or graph replay) and its dominant
    kernel, each on the launch stream with HIP events; returns the measurement as a dict."""
    import torch
    import fp4_kv_cache_e2m1_amd as P
    log(f"[bench] workload {wl.name}: generating inputs")
    sets = build_inputs(wl, dev, args.copies)
    stream = torch.cuda.current_stream(dev)
    R = wl.B * wl.T
    n_vis = None
    if wl.T > 1:
        n_vis = P.prefill_n_vis([wl.p0] * wl.B, wl.T, wl.ratio, dev, n_max=wl.N)
    # per-set shared state and buffers, allocated once
    state = []
    for s in sets:
        kv = P.KVState(s["rows"], s["kidx"], n_vis)
        idx = P.IdxState.empty(R, wl.k, dev, pool_size=wl.pool_blocks * wl.block)
        outs = [torch.empty(wl.B, wl.T, wl.H, wl.D, dtype=torch.float32, device=dev) for _ in wl.modes]
        state.append((s, kv, idx, outs))
    # one workspace sized for the largest layer of the schedule
    need = 0
    for l, mode in enumerate(wl.modes):
        s, kv, idx, outs = state[0]
        a = P.layer_args(mode, s["q"][l], kv, idx, q_idx=s["qi"][l] if mode != 2 else None,
                         use_pool=wl.pool_blocks > 0, pool_blocks=wl.pool_blocks)
        need = max(need, P.layer_workspace_size(mode, a, kv, idx))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def step(i):
        s, kv, idx, outs = state[i % len(state)]
        for l, mode in enumerate(wl.modes):
            P.layer_step(mode, s["q"][l], kv, idx, q_idx=s["qi"][l] if mode != 2 else None,
                         sm_scale=wl.sm_scale, use_pool=wl.pool_blocks > 0, pool_blocks=wl.pool_blocks,
                         with_lse=False, ws=ws, out=outs[l])

    log(f"[bench] {wl.name}: warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if not extras:
        # a further workload of the line (not its headline): warmed up by time as well
        warm(lambda i: step(args.warmup + i), 0, 150)
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

        def step(i):  # noqa: F811
            graphs[i % len(graphs)].replay()

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
    log(f"[bench] {wl.name}: timing {args.steps} steps")
    torch.cuda.synchronize()
    ms = time_on_stream(step, args.steps, stream)

    # dominant kernel, timed alone on the same stream: the indexer call of the workload's first
    # (Full) layer, with the block maxima when the layer builds the pool
    bm = wl.pool_blocks > 0
    sc = torch.empty(R, wl.N, dtype=torch.float32, device=dev)
    bmax = torch.empty(R, (wl.N + 7) // 8, dtype=torch.float32, device=dev) if bm else None

    def index_call(i):
        s = sets[i % len(sets)]
        P.index_scores(s["qi"][0], s["kidx"], n_vis=n_vis, out=sc, block_max_out=bmax)

    warm(index_call, 3, 60)
    kms = time_on_stream(index_call, args.steps, stream)
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
        traffic = None if bm else traffic_from_counters(wl.name)
        kname = "index_stream_kernel (flat indexer scores" + (" + 8-entry block max)" if bm else ")")
        roofline = {"kernel": kname, "bound": "hbm",
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "algorithmic_bytes_per_launch": kbytes, "avg_launch_us": round(kms * 1e3, 2)}
    step_bytes = algorithmic_bytes(wl)
    res = {
        "workload": wl.name,
        "value": round(R / (ms * 1e-3), 1),
        "unit": "query-tokens/s",
        "ms_per_step": round(ms, 5),
        "config": {"workload": wl.name, "batch": wl.B, "query_tokens": wl.T, "entries": wl.N,
                   "latent_dim": wl.D, "heads": wl.H, "index_heads": wl.Hi, "index_dim": wl.Di,
                   "topk": wl.k, "layers": [["FULL", "REINDEX", "REUSE"][m] for m in wl.modes],
                   "pool_blocks": wl.pool_blocks, "kv_format": "E2M1 + E4M3 per 16 channels (288 B/entry)"},
        "launch": "hip graph replay" if args.graph else "eager",
        "roofline": roofline,
    }
    if wl.T == 1:
        res.update(step_hbm_gbs=round(step_bytes / (ms * 1e-3) / 1e9, 1),
                   step_hbm_frac=round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   step_algorithmic_bytes=step_bytes)
    else:
        # prefill attention over the step's own Top-K, timed alone: f16 MFMA, 4 H D flops per
        # (query token, selected entry)
        s, kv, idx, outs = state[0]
        q = s["q"][0]
        aws = torch.empty(max(256, P.sparse_attn_workspace_size(wl.B, wl.T, wl.H, wl.D, wl.k)), dtype=torch.uint8,
                          device=dev)

        def attn_call(i):
            P.sparse_attn(q, s["rows"], idx.topk.view(wl.B, wl.T, wl.k), wl.sm_scale, with_lse=False, ws=aws,
                          out=outs[0])

        warm(attn_call, 1, 60)
        ams = time_on_stream(attn_call, args.steps, stream)
        n_sel = float((idx.topk >= 0).sum().item())
        aflops = 4.0 * wl.H * wl.D * n_sel
        res["attention_roofline"] = {
            "kernel": "sparse_attn_prefill_kernel", "bound": "mfma", "achieved": round(aflops / (ams * 1e-3) / 1e12, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s (f16)",
            "frac": round(aflops / (ams * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "algorithmic_flops_per_launch": aflops, "avg_launch_us": round(ams * 1e3, 2)}
    if wl.T > 1 and wl.Hk == wl.Hi and wl.Hi * wl.Di in (256, 512):
        res["fp4_indexer"] = fp4_prefill_leg(wl, n_vis, args.steps, dev, stream)
    if (wl.Hk * wl.Di) % 128 == 0:
        res["cache_production"] = production_leg(wl, sets, state, n_vis, args.steps, dev, stream)
    if extras:
        fp4_shape = (wl.Hk == wl.Hi and wl.Hi * wl.Di in (256, 512)) or (wl.Hk == 1 and wl.Di == 128)
        if args.fp4_indexer and wl.T == 1 and fp4_shape:
            res["fp4_indexer"] = fp4_indexer_leg(wl, sets, args.steps, dev, stream)
        if args.window > 0:
            res["window_attention"] = window_leg(wl, sets, state, args.window, args.steps, dev, stream)
    del state, sets, ws, sc, bmax
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--legs", default="2,4,5",
                    help="comma-separated further workloads measured after the headline one, or 'none'")
    ap.add_argument("--copies", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=2)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--trace-summary", metavar="DB", help="print a per-kernel table of a rocprofv3 results database")
    ap.add_argument("--counter-summary", nargs=4, metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB"),
                    help="write the indexer's HBM counters of --config from four rocprofv3 --pmc databases")
    ap.add_argument("--counter-commands", nargs="*", default=[], help="commands recorded with --counter-summary")
    ap.add_argument("--graph", action="store_true", help="replay each step from a captured HIP graph")
    ap.add_argument("--fp4-indexer", action="store_true",
                    help="also time the FP4 (MXFP4) indexer on the workload's keys, stored as MXFP4 rows")
    ap.add_argument("--window", type=int, default=0,
                    help="also time decode attention with each sequence's window of this many FP8 rows")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.counter_summary:
        counter_summary(args.config, *args.counter_summary, commands=args.counter_commands)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the hot path has no "
              "multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    from fp4_kv_cache_e2m1_amd import _lib, workloads as W
    if not os.path.exists(_lib.LIB_PATH):
        from fp4_kv_cache_e2m1_amd import build_lib
        build_lib.build()
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(dev)
        return

    wl = W.CONFIGS[args.config]
    head = measure_workload(wl, args, dev, extras=True)
    legs = [] if args.legs in ("", "none") else [int(c) for c in args.legs.split(",") if int(c) != args.config]
    line = {
        "metric": "CSA2 decode query-tokens/s + achieved HBM GB/s (% of peak) at 1 MI355X",
        "value": head["value"],
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
    }
    line.update({k: v for k, v in head.items() if k not in ("workload", "value", "unit", "ms_per_step", "config")})
    if legs:
        line["legs"] = {}
        for c in legs:
            r = measure_workload(W.CONFIGS[c], args, dev, extras=False)
            line["legs"][r.pop("workload")] = r
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle on {args.cpu_sample} sequences of {wl.name}, >= {args.cpu_seconds} s")
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
