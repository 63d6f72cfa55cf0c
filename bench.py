#!/usr/bin/env python3
"""Benchmark of the lightning-indexer hot path on one MI355X.

Headline (``value``): scored causal (query, key) pairs per second of the fused
indexer + top-k at L = 65536 (H_I = 64, d_I = 128, k = 2048, fp8 q/k, bf16 w),
one step = one Full layer routed through ``idx_cache_route`` (score, ReLU,
head-weighted sum, causal mask and per-row top-k in one kernel, T written).

Secondary (``secondary``): the 200K-context decode step (32 sequences, one query
each): Full layer = indexer + top-k + sparse MLA, Shared layer = sparse MLA
only, and a 4-layer F,S,S,S group against an all-Full group, in decode tokens
per second; plus the gather bandwidth of sparse MLA.

``roofline``: the fused indexer kernel against the fp8 MFMA peak; ``achieved``
is algorithmic flops (pairs x H x D x 2) over the average launch time measured
with HIP events on the launch stream.  ``traffic`` comes from rocprofv3 counter
runs committed under profiles/ (null when not measured for this kernel build).

``cpu_baseline``: the plain fp64 CPU oracle on a bounded seeded sample of query
rows of the same workload, in the same unit.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_prefill_64k_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the retention-ratio sweep")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle wall time")
    ap.add_argument("--profile-only", action="store_true", help="run warmup+steps of the headline only")
    ap.add_argument("--profile", choices=["prefill", "decode", "mla_prefill", "copy"],
                    help="run warmup+steps of one workload (for profiler runs) and exit")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="write the headline kernel's HBM traffic from rocprofv3 counter runs in DIR "
                         "(subdirectories fetch/, write/, copy_fetch/, copy_write/) and exit")
    return ap.parse_args()


def causal_pairs(Lq: int, Lk: int, B: int = 1) -> int:
    """sum over queries i of (position + 1), position = Lk - Lq + i."""
    return B * (Lq * (Lk - Lq + 1) + Lq * (Lq - 1) // 2)


def time_steps(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(s)
    for _ in range(steps):
        fn()
    ev1.record(s)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps  # ms per step


def headline(args, torch, sa, inputs):
    wl = inputs.WORKLOADS["prefill_64k"]
    dev = torch.device("cuda:0")
    q, k, w = inputs.indexer_inputs(wl, 0, dev)
    t_cache = torch.empty(wl.B, wl.Lq, wl.topk, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def step():
        sa.idx_cache_route("F", 0, q, k, w, t_cache)

    ms = time_steps(step, args.steps, args.warmup, torch)
    pairs = causal_pairs(wl.Lq, wl.Lk, wl.B)
    flops = pairs * wl.H * wl.D * 2
    return wl, ms, pairs, flops


def decode(args, torch, sa, inputs):
    wl = inputs.WORKLOADS["decode_200k"]
    dev = torch.device("cuda:0")
    q, k, w = inputs.indexer_inputs(wl, 0, dev)
    qa, kv = inputs.attention_inputs(wl, 0, dev)
    t = torch.empty(wl.B, wl.Lq, wl.topk, dtype=torch.int32, device=dev)
    out = torch.empty(wl.B, wl.Lq, wl.Hq, wl.Dv, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(sa.idx_score_topk_workspace(q, k, w, wl.topk), dtype=torch.uint8, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)   # evicts the 256 MB MALL
    scale = 1.0 / math.sqrt(wl.Dqk)
    sa.idx_cache_route("FSSS", 0, q, k, w, t, ws=ws)
    torch.cuda.synchronize()
    n = max(3, args.steps)

    def timed(fn):
        for _ in range(2):
            fn()
        tot = 0.0
        for _ in range(n):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1)
        return tot / n

    t_idx = timed(lambda: sa.idx_cache_route("FSSS", 0, q, k, w, t, ws=ws))
    t_att = timed(lambda: sa.sparse_mla_attn(qa, kv, t, scale, wl.Dv, out=out))
    t_f = t_idx + t_att

    # the same step as a serving batch: caches in pools of 64-row pages at
    # random slots (one shared block table), query rows packed
    bs = 64
    npg = (wl.Lk + bs - 1) // bs
    g = torch.Generator(device="cpu").manual_seed(11)
    perm = torch.randperm(wl.B * npg, generator=g).to(dev)
    table = perm.view(wl.B, npg).to(torch.int32)
    k_pool = torch.empty(wl.B * npg, bs, wl.D, dtype=k.dtype, device=dev)
    k_pool[perm.long()] = k.view(wl.B * npg, bs, wl.D)
    kv_pool = torch.empty(wl.B * npg, bs, wl.Dqk, dtype=kv.dtype, device=dev)
    kv_pool[perm.long()] = kv.view(wl.B * npg, bs, wl.Dqk)
    qs = torch.arange(wl.B + 1, dtype=torch.int32, device=dev)
    sl = torch.full((wl.B,), wl.Lk, dtype=torch.int32, device=dev)
    qp, wp, qap = q.view(wl.B, wl.H, wl.D), w.view(wl.B, wl.H), qa.view(wl.B, wl.Hq, wl.Dqk)
    tp = torch.empty(wl.B, wl.topk, dtype=torch.int32, device=dev)
    outp = torch.empty(wl.B, wl.Hq, wl.Dv, dtype=torch.bfloat16, device=dev)
    wsp = torch.empty(sa.idx_score_topk_paged_workspace(qp, k_pool, wp, table, qs, wl.topk, wl.Lk),
                      dtype=torch.uint8, device=dev)
    wsa = torch.empty(max(1, sa.sparse_mla_attn_paged_workspace(qap, kv_pool, table, qs, tp, wl.Dv)),
                      dtype=torch.uint8, device=dev)
    t_pidx = timed(lambda: sa.idx_score_topk_paged(qp, k_pool, table, qs, sl, wp, wl.topk, wl.Lk, t_out=tp, ws=wsp))
    t_patt = timed(lambda: sa.sparse_mla_attn_paged(qap, kv_pool, table, qs, sl, tp, scale, wl.Dv, out=outp,
                                                    ws=wsa))
    same_t = bool(torch.equal(tp, t.view(wl.B, wl.topk)))
    del k_pool, kv_pool
    gathered = wl.B * wl.Lq * wl.topk * wl.Dqk * 2
    key_bytes = wl.B * wl.Lk * wl.D
    tok = wl.B * wl.Lq
    return {
        "workload": "decode_200k", "batch": wl.B, "context": wl.Lk,
        "indexer_topk_ms": round(t_idx, 4), "sparse_mla_ms": round(t_att, 4),
        "full_layer_tok_s": round(tok / (t_f * 1e-3), 1),
        "shared_layer_tok_s": round(tok / (t_att * 1e-3), 1),
        "group_FSSS_tok_s": round(tok / ((t_f + 3 * t_att) * 1e-3), 1),
        "group_FFFF_tok_s": round(tok / (4 * t_f * 1e-3), 1),
        "indexer_key_read_GBs": round(key_bytes / (t_idx * 1e-3) / 1e9, 1),
        "gather_GBs": round(gathered / (t_att * 1e-3) / 1e9, 1),
        "gather_frac_hbm": round(gathered / (t_att * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "note": "caches flushed before each timed call; one layer = one call each",
        "serving_paged": {
            "block_size": bs, "pages": "random slots of one pool, shared block table",
            "indexer_topk_ms": round(t_pidx, 4), "sparse_mla_ms": round(t_patt, 4),
            "full_layer_tok_s": round(tok / ((t_pidx + t_patt) * 1e-3), 1),
            "t_identical_to_contiguous": same_t,
        },
    }


COPY_BYTES = 1 << 30   # the calibration copy moves this many bytes each way


def retention_sweep(args, torch, sa, inputs):
    """Layer patterns keeping 1/1, 1/2, 1/4 and 1/8 of the 16 layers Full, at the
    32K-token stack shape: per-layer times of the indexer (Full layers only),
    sparse MLA and the FFN stand-in, the stack time they imply for each pattern,
    and one directly timed F,S,S,S x 4 stack for comparison."""
    wl = inputs.WORKLOADS["stack_32k"]
    dev = torch.device("cuda:0")
    L, n_layers = wl.Lq, wl.layers
    q, k, w = inputs.indexer_inputs(wl, 0, dev)
    qa, kv = inputs.attention_inputs(wl, 0, dev)
    W = inputs.ffn_weight(wl, 0, dev)
    x = inputs.stack_x0(wl, dev)
    t_cache = torch.empty(wl.B, L, wl.topk, dtype=torch.int32, device=dev)
    out = torch.empty(wl.B, L, wl.Hq, wl.Dv, dtype=torch.bfloat16, device=dev)
    scale = 1.0 / math.sqrt(wl.Dqk)
    sa.idx_cache_route("F", 0, q, k, w, t_cache)

    def layer(pattern, i):
        sa.idx_cache_route(pattern, i, q, k, w, t_cache)
        sa.sparse_mla_attn(qa, kv, t_cache, scale, wl.Dv, out=out)
        x1 = x.clone()
        x1[:, :wl.Dv] += out[0].sum(dim=1)
        return x1 + x1 @ W

    def timed(fn, n=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    t_idx = timed(lambda: sa.idx_cache_route("F", 0, q, k, w, t_cache))
    t_att = timed(lambda: sa.sparse_mla_attn(qa, kv, t_cache, scale, wl.Dv, out=out))
    t_ffn = timed(lambda: layer("FS", 1)) - t_att   # head sum, residual and FFN GEMM
    pats = {"1/1": "F" * n_layers, "1/2": "FS" * (n_layers // 2), "1/4": "FSSS" * (n_layers // 4),
            "1/8": "FSSSSSSS" * (n_layers // 8)}
    res = {}
    full = n_layers * (t_idx + t_att + t_ffn)
    for name, pat in pats.items():
        nf = pat.count("F")
        stack = nf * t_idx + n_layers * (t_att + t_ffn)
        res[name] = {"pattern": pat, "full_layers": nf, "indexer_ms": round(nf * t_idx, 3),
                     "indexer_saved_ms": round((n_layers - nf) * t_idx, 3), "stack_ms": round(stack, 3),
                     "speedup_vs_all_full": round(full / stack, 4)}
    measured = timed(lambda: [layer(pats["1/4"], i) for i in range(n_layers)], n=1)
    del q, k, w, qa, kv, out, W, x, t_cache
    return {"workload": "stack_32k", "L": L, "layers": n_layers, "indexer_ms_per_full_layer": round(t_idx, 3),
            "sparse_mla_ms_per_layer": round(t_att, 3), "ffn_and_residual_ms_per_layer": round(t_ffn, 3),
            "patterns": res, "measured_FSSSx4_stack_ms": round(measured, 3),
            "note": "stack_ms = Full layers x indexer + all layers x (sparse MLA + FFN stand-in)"}


def profile_run(args, torch, sa, inputs):
    """Runs one workload a few times with no timing, for rocprofv3."""
    dev = torch.device("cuda:0")
    if args.profile == "prefill":
        headline(args, torch, sa, inputs)
    elif args.profile == "decode":
        wl = inputs.WORKLOADS["decode_200k"]
        q, k, w = inputs.indexer_inputs(wl, 0, dev)
        qa, kv = inputs.attention_inputs(wl, 0, dev)
        t = torch.empty(wl.B, wl.Lq, wl.topk, dtype=torch.int32, device=dev)
        out = torch.empty(wl.B, wl.Lq, wl.Hq, wl.Dv, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(sa.idx_score_topk_workspace(q, k, w, wl.topk), dtype=torch.uint8, device=dev)
        for _ in range(args.warmup + args.steps):
            sa.idx_cache_route("F", 0, q, k, w, t, ws=ws)
            sa.sparse_mla_attn(qa, kv, t, 1.0 / math.sqrt(wl.Dqk), wl.Dv, out=out)
    elif args.profile == "mla_prefill":
        wl = inputs.WORKLOADS["stack_32k"]
        qa, kv = inputs.attention_inputs(wl, 0, dev)
        q, k, w = inputs.indexer_inputs(wl, 0, dev)
        t = sa.idx_score_topk(q, k, w, wl.topk)
        del q, k, w
        out = torch.empty(wl.B, wl.Lq, wl.Hq, wl.Dv, dtype=torch.bfloat16, device=dev)
        for _ in range(args.warmup + args.steps):
            sa.sparse_mla_attn(qa, kv, t, 1.0 / math.sqrt(wl.Dqk), wl.Dv, out=out)
    else:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profiled": args.profile, "runs": args.warmup + args.steps}))


def _counter_kb(run_dir, counter, name_part):
    """Mean per-dispatch value of `counter` over dispatches whose kernel name contains name_part
    (counter values of one dispatch summed over the rows rocprofv3 writes for it)."""
    import csv
    import glob
    per_dispatch = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter and name_part in r.get("Kernel_Name", ""):
                    key = (path, r.get("Dispatch_Id", r.get("Correlation_Id", "")))
                    per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    if not per_dispatch:
        raise SystemExit(f"no {counter} rows for '{name_part}' under {run_dir}")
    return sum(per_dispatch.values()) / len(per_dispatch)


def traffic_from(args):
    """Scales the headline kernel's FETCH_SIZE / WRITE_SIZE by what the same
    counters read for a copy of COPY_BYTES, and records the result."""
    d = args.traffic_from
    kname = "prefill_kernel"
    copy_name = "copyBuffer"   # the device-to-device copy torch issues for dst.copy_(src)
    fetch_kb = _counter_kb(os.path.join(d, "fetch"), "FETCH_SIZE", kname)
    write_kb = _counter_kb(os.path.join(d, "write"), "WRITE_SIZE", kname)
    cf_kb = _counter_kb(os.path.join(d, "copy_fetch"), "FETCH_SIZE", copy_name)
    cw_kb = _counter_kb(os.path.join(d, "copy_write"), "WRITE_SIZE", copy_name)
    f_fetch = cf_kb * 1024.0 / COPY_BYTES
    f_write = cw_kb * 1024.0 / COPY_BYTES
    read_b = fetch_kb * 1024.0 / f_fetch
    write_b = write_kb * 1024.0 / f_write
    rec = {"kernel": kname, "workload": "prefill_64k", "kernel_source_sha": _kernel_sha(),
           "fetch_size_kb": fetch_kb, "write_size_kb": write_kb,
           "copy_bytes_each_way": COPY_BYTES, "copy_fetch_kb": cf_kb, "copy_write_kb": cw_kb,
           "scale_fetch": f_fetch, "scale_write": f_write,
           "read_bytes_per_launch": read_b, "write_bytes_per_launch": write_b,
           "bytes_per_launch": read_b + write_b}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def cpu_baseline(args, inputs, torch):
    """Oracle rows/s on the host, scaled to pairs/s (bounded seeded row sample)."""
    import numpy as np

    import oracle
    wl = inputs.WORKLOADS["prefill_64k"]
    q, k, w = inputs.indexer_inputs(wl, 0, "cuda:0")
    qr = q.cpu().view(torch.uint8).numpy()
    kr = k.cpu().view(torch.uint8).numpy()
    wr = w.cpu().view(torch.int16).numpy()
    del q, k, w
    threads = oracle.default_threads()
    rng = np.random.default_rng(2024)
    order = rng.permutation(wl.Lq)
    done_rows, done_pairs, wall = 0, 0, 0.0
    batch = 2 * threads
    while wall < args.cpu_seconds and done_rows < wl.Lq:
        rows = np.sort(order[done_rows:done_rows + batch]).astype(np.int64)
        t0 = time.perf_counter()
        oracle.indexer_topk(qr, kr, wr, ("fp8", "fp8", "bf16"), wl.topk, rows=rows, nthreads=threads)
        wall += time.perf_counter() - t0
        done_rows += rows.size
        done_pairs += int((rows + 1).sum())
    return {"value": round(done_pairs / wall, 1), "unit": "pairs/s", "cores": threads, "kind": "oracle",
            "sample": f"{done_rows} seeded random query rows of prefill_64k ({done_pairs} causal pairs, "
                      f"fp64 scores + top-k), {wall:.1f} s wall"}


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    import sparse_attention_indexer_lightning_amd as sa
    from sparse_attention_indexer_lightning_amd import inputs

    sa.lib()
    if args.profile:
        profile_run(args, torch, sa, inputs)
        return
    wl, ms, pairs, flops = headline(args, torch, sa, inputs)
    if args.profile_only:
        print(json.dumps({"ms_per_step": ms}))
        return
    achieved = flops / (ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        if rec.get("kernel_source_sha") == _kernel_sha():
            traffic = rec.get("bytes_per_launch")
    line = {
        "metric": "indexer+top-k scored (q,key) pairs/s at L=64K; 200K-ctx sparse decode tok/s",
        "value": round(pairs / (ms * 1e-3), 1),
        "unit": "pairs/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8", "data": "synthetic",
        "config": {"workload": "prefill_64k", "B": wl.B, "L": wl.Lq, "H_I": wl.H, "d_I": wl.D,
                   "topk": wl.topk, "q_k": "fp8_e4m3", "w": "bf16", "pairs_per_step": pairs,
                   "step": "idx_cache_route on a Full layer (fused score + top-k, T written)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                     "kernel": "prefill_kernel<FP8,128,64,u16>",
                     "flops_per_launch": flops},
    }
    if not args.no_decode:
        line["secondary"] = decode(args, torch, sa, inputs)
    if not args.no_sweep:
        line["retention_sweep"] = retention_sweep(args, torch, sa, inputs)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, inputs, torch)
    print(json.dumps(line))


def _kernel_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for n in ("indexer.hip", "device_common.h"):
        with open(os.path.join(ROOT, "sparse_attention_indexer_lightning_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
