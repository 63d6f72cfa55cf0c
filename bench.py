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
``operand_peak`` is the rate of plain dense MFMA chains on this workload's own
operand bytes: the engine clock falls when MFMA operands toggle, so random
operands cap an MFMA-bound kernel below the published ``peak``.  The retention
sweep reports the sparse MLA prefill layer the same way (bf16).

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
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
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
    ap.add_argument("--profile", choices=["prefill", "decode", "mla_prefill", "chunk", "copy"],
                    help="run warmup+steps of one workload (for profiler runs) and exit")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="HBM traffic per launch from rocprofv3 counter runs in DIR (subdirectories fetch/, "
                         "write/, copy_fetch/, copy_write/), scaled by the copy calibration; prints it and, for "
                         "the headline kernel, records it under profiles/; then exits")
    ap.add_argument("--kernels", default="prefill_kernel",
                    help="with --traffic-from: comma-separated kernel-name parts to report")
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
    peak_ops = operand_peak(torch, sa, 0, q, k)
    return wl, ms, pairs, flops, t_cache, peak_ops


def operand_peak(torch, sa, kind, a, b):
    """TFLOP/s of a plain chain of dense MFMAs (idxc_calib_mfma_rate) whose
    operands are bytes of the tensors a and b: on this part the engine clock
    falls when MFMA operands toggle, so random operands cap an MFMA-bound
    kernel below the published peak.  kind 0: fp8 32x32x64, 1: bf16 32x32x16."""
    import ctypes
    L = sa.lib()
    f = L.idxc_calib_mfma_rate
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    blocks = 512                                  # four wavefronts each: two per SIMD
    iters = 6000 if kind == 0 else 12000          # about 6-7 ms per launch
    flop = (2 * 32 * 32 * 64 if kind == 0 else 2 * 32 * 32 * 16) * 16 * iters * blocks * 4
    out = torch.empty(blocks * 256, dtype=torch.float32, device=a.device)
    s = torch.cuda.current_stream()

    def launch():
        rc = f(kind, a.data_ptr(), a.numel() * a.element_size(), b.data_ptr(), b.numel() * b.element_size(), iters,
               blocks, out.data_ptr(), s.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"idxc_calib_mfma_rate failed: {rc}")

    launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(3):
        launch()
    e1.record(s)
    torch.cuda.synchronize()
    return flop * 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12


def decode(args, torch, sa, inputs):
    wl = inputs.WORKLOADS["decode_200k"]
    dev = torch.device("cuda:0")
    q, k, w = inputs.indexer_inputs(wl, 0, dev)
    qa, kv = inputs.attention_inputs(wl, 0, dev)
    t = torch.empty(wl.B, wl.Lq, wl.topk, dtype=torch.int32, device=dev)
    out = torch.empty(wl.B, wl.Lq, wl.Hq, wl.Dv, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(sa.idx_score_topk_workspace(q, k, w, wl.topk), dtype=torch.uint8, device=dev)
    # Cold timing: a read-only pass over 512 MB (twice the 256 MB MALL) before
    # each timed call evicts the caches.  It only reads, so the timed call
    # inherits no dirty lines to write back.
    flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(wl.Dqk)
    sa.idx_cache_route("FSSS", 0, q, k, w, t, ws=ws)
    torch.cuda.synchronize()
    n = max(3, args.steps)

    def timed(fn, cold=True):
        """ms per call.  cold: each call alone after the flush (the flush kernel
        also covers the host's launch latency).  warm: n calls back to back
        between one pair of events."""
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        if not cold:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n
        tot = 0.0
        for _ in range(n):
            torch.sum(flush)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1)
        return tot / n

    f_idx = lambda: sa.idx_cache_route("FSSS", 0, q, k, w, t, ws=ws)   # noqa: E731
    f_att = lambda: sa.sparse_mla_attn(qa, kv, t, scale, wl.Dv, out=out)   # noqa: E731
    t_idx = timed(f_idx)
    t_att = timed(f_att)
    t_idx_warm = timed(f_idx, cold=False)
    t_att_warm = timed(f_att, cold=False)
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
    ceiling = gather_ceiling(torch, sa, kv, t, wl, timed, gathered)
    key_bytes = wl.B * wl.Lk * wl.D
    tok = wl.B * wl.Lq
    layer_bytes = decode_layer_bytes(wl)
    return {
        "workload": "decode_200k", "batch": wl.B, "context": wl.Lk,
        "indexer_topk_ms": round(t_idx, 4), "sparse_mla_ms": round(t_att, 4),
        "indexer_topk_ms_warm": round(t_idx_warm, 4), "sparse_mla_ms_warm": round(t_att_warm, 4),
        "full_layer_roofline": {
            "bound": "hbm", "algorithmic_bytes": layer_bytes, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "achieved": round(layer_bytes / (t_f * 1e-3) / 1e9, 1),
            "frac": round(layer_bytes / (t_f * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "ideal_ms": round(layer_bytes / (PEAK_HBM_GBS * 1e9) * 1e3, 4),
            "bytes": "keys + gathered latent rows + q, w, Q, O and T (score rows in the workspace excluded)"},
        "full_layer_tok_s": round(tok / (t_f * 1e-3), 1),
        "shared_layer_tok_s": round(tok / (t_att * 1e-3), 1),
        "group_FSSS_tok_s": round(tok / ((t_f + 3 * t_att) * 1e-3), 1),
        "group_FFFF_tok_s": round(tok / (4 * t_f * 1e-3), 1),
        "indexer_key_read_GBs": round(key_bytes / (t_idx * 1e-3) / 1e9, 1),
        "gather_GBs": round(gathered / (t_att * 1e-3) / 1e9, 1),
        "gather_frac_hbm": round(gathered / (t_att * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "gather_ceiling": ceiling,
        "gather_frac_of_ceiling": round(gathered / (t_att * 1e-3) / 1e9 / ceiling["cold_GBs"], 4),
        "note": "cold: a read-only pass over 512 MB before each timed call; warm: back to back; one layer = one call each",
        "serving_paged": {
            "block_size": bs, "pages": "random slots of one pool, shared block table",
            "indexer_topk_ms": round(t_pidx, 4), "sparse_mla_ms": round(t_patt, 4),
            "full_layer_tok_s": round(tok / ((t_pidx + t_patt) * 1e-3), 1),
            "t_identical_to_contiguous": same_t,
        },
    }


def gather_ceiling(torch, sa, kv, t, wl, timed, gathered):
    """GB/s of reading exactly the latent rows the decode step's T names
    (idxc_calib_gather_rate: the same rows, 16-byte loads laid out as the
    sparse attention copies them, nothing else to do), cold and warm, best
    over a few grid sizes: what this pattern of random 1152-byte rows allows
    on this part, next to the sparse attention kernel's own gather rate."""
    import ctypes
    assert wl.Lq == 1, "one query per sequence: query b reads rows of sequence b"
    f = sa.lib().idxc_calib_gather_rate
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    shapes = (256, 512, 1024, 2048, 4096)
    out = torch.empty(max(shapes) * 256, dtype=torch.int32, device=kv.device)
    per = {}
    for blocks in shapes:
        def launch(blocks=blocks):
            rc = f(kv.data_ptr(), wl.Dqk * 2, wl.Lk, t.data_ptr(), wl.B * wl.Lq, wl.topk, blocks, out.data_ptr(),
                   torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"idxc_calib_gather_rate failed: {rc}")
        per[blocks] = (gathered / (timed(launch) * 1e-3) / 1e9, gathered / (timed(launch, cold=False) * 1e-3) / 1e9)
    bc = max(per, key=lambda b: per[b][0])
    bw = max(per, key=lambda b: per[b][1])
    return {"kernel": "idxc_calib_gather_rate", "rows": "the decode step's T over its latent cache, 1152-byte rows",
            "cold_GBs": round(per[bc][0], 1), "warm_GBs": round(per[bw][1], 1),
            "blocks_cold": bc, "blocks_warm": bw, "threads_per_block": 256,
            "cold_frac_hbm": round(per[bc][0] / PEAK_HBM_GBS, 4),
            "per_blocks_cold_warm_GBs": {str(b): [round(v[0], 1), round(v[1], 1)] for b, v in per.items()}}


def _prefill_chunk_calls(torch, sa, inputs):
    """Inputs of a serving batch holding one prefill chunk (the last 4096
    positions of a 200,000-token sequence, its indexer keys in 64-row pages at
    random slots of a pool) and two calls on them: idx_score_topk_paged (the
    fused kernel with page lookups) and idx_score_topk over contiguous keys."""
    import dataclasses
    base = inputs.WORKLOADS["decode_200k"]
    C, L = 4096, base.Lk
    wl = dataclasses.replace(base, name="chunk", B=1, Lq=C)
    dev = torch.device("cuda:0")
    q, k, w = inputs.indexer_inputs(wl, 0, dev)
    bs = 64
    npg = (L + bs - 1) // bs
    g = torch.Generator(device="cpu").manual_seed(12)
    perm = torch.randperm(npg, generator=g).to(dev)
    table = perm.view(1, npg).to(torch.int32)
    k_pool = torch.empty(npg, bs, wl.D, dtype=k.dtype, device=dev)
    k_pool[perm.long()] = k.view(npg, bs, wl.D)
    qs = torch.tensor([0, C], dtype=torch.int32, device=dev)
    sl = torch.tensor([L], dtype=torch.int32, device=dev)
    qp, wp = q.view(C, wl.H, wl.D), w.view(C, wl.H)
    ws_bytes = sa.idx_score_topk_paged_workspace(qp, k_pool, wp, table, qs, wl.topk, L)
    wsp = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    tp = torch.empty(C, wl.topk, dtype=torch.int32, device=dev)
    tc = torch.empty(1, C, wl.topk, dtype=torch.int32, device=dev)
    paged = lambda: sa.idx_score_topk_paged(qp, k_pool, table, qs, sl, wp, wl.topk, L, t_out=tp, ws=wsp)
    contig = lambda: sa.idx_score_topk(q, k, w, wl.topk, t_out=tc)
    return paged, contig, tp, tc, (C, L, bs, ws_bytes)


def serving_prefill_chunk(args, torch, sa, inputs):
    """The prefill-chunk serving batch timed through idx_score_topk_paged next
    to idx_score_topk on the same rows over contiguous keys."""
    paged, contig, tp, tc, (C, L, bs, ws_bytes) = _prefill_chunk_calls(torch, sa, inputs)
    ms_paged = time_steps(paged, 5, 1, torch)
    ms_contig = time_steps(contig, 5, 1, torch)
    same = bool(torch.equal(tp, tc[0]))
    pairs = causal_pairs(C, L)
    return {"chunk_queries": C, "context": L, "block_size": bs, "pages": "random slots of one pool",
            "paged_ms": round(ms_paged, 3), "contiguous_ms": round(ms_contig, 3),
            "paged_pairs_per_s": round(pairs / (ms_paged * 1e-3), 1), "t_identical_to_contiguous": same,
            "workspace_bytes": ws_bytes,
            "note": "the fused kernel reads each 64-key block's page from the block table; no score rows stored"}


def decode_layer_bytes(wl) -> int:
    """Algorithmic HBM bytes of one Full decode layer: every key of every
    sequence once, the selected latent rows once, the indexer queries and
    weights, the attention queries and outputs, and T."""
    keys = wl.B * wl.Lk * wl.D                       # fp8
    gathered = wl.B * wl.Lq * wl.topk * wl.Dqk * 2   # bf16 latent rows
    q_i = wl.B * wl.Lq * wl.H * wl.D + wl.B * wl.Lq * wl.H * 2
    q_a = wl.B * wl.Lq * wl.Hq * wl.Dqk * 2
    o = wl.B * wl.Lq * wl.Hq * wl.Dv * 2
    t = wl.B * wl.Lq * wl.topk * 4
    return keys + gathered + q_i + q_a + o + t


COPY_BYTES = 1 << 30   # the calibration copy moves this many bytes each way


def retention_sweep(args, torch, sa, inputs):
    """Layer patterns keeping 1/1, 1/2, 1/4 and 1/8 of the 16 layers Full, at the
    32K-token stack shape, each timed end to end: the stack runs all 16 layers
    with X chained through attention and the FFN stand-in (residual), layer l
    taking input set l mod 4 (four seeded sets of indexer, attention and FFN
    inputs).  Next to each measured time, the model that adds per-layer times
    (Full layers x indexer + all layers x (attention + FFN))."""
    from sparse_attention_indexer_lightning_amd.stack import Stack, compose, layer_inputs
    wl = inputs.WORKLOADS["stack_32k"]
    dev = torch.device("cuda:0")
    n_layers, n_sets = wl.layers, 4
    sets = [layer_inputs(wl, i, dev) for i in range(n_sets)]
    x0 = inputs.stack_x0(wl, dev)
    st = Stack(wl, [sets[l % n_sets] for l in range(n_layers)], x0, residual=True)
    scale = 1.0 / math.sqrt(wl.Dqk)

    def timed(fn, n=2):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    s0 = sets[0]
    t_idx = timed(lambda: sa.idx_cache_route("F", 0, s0["q_i"], s0["k_i"], s0["w"], st.t_cache, ws=st.ws), 3)
    t_att = timed(lambda: sa.sparse_mla_attn(s0["q"], s0["kv"], st.t_cache, scale, wl.Dv, out=st.out), 3)
    t_ffn = timed(lambda: compose(x0, st.out[0], s0["W"], True, False), 3)
    pats = {"1/1": "F" * n_layers, "1/2": "FS" * (n_layers // 2), "1/4": "FSSS" * (n_layers // 4),
            "1/8": "FSSSSSSS" * (n_layers // 8)}
    res = {}
    for name, pat in pats.items():
        nf = pat.count("F")
        res[name] = {"pattern": pat, "full_layers": nf,
                     "stack_ms": round(timed(lambda: st.run(pat)), 3),
                     "modelled_stack_ms": round(nf * t_idx + n_layers * (t_att + t_ffn), 3),
                     "indexer_ms": round(nf * t_idx, 3), "indexer_saved_ms": round((n_layers - nf) * t_idx, 3)}
    mla_flops = wl.B * wl.Lq * wl.Hq * wl.topk * (wl.Dqk + wl.Dv) * 2
    mla_tflops = mla_flops / (t_att * 1e-3) / 1e12
    mla_peak = operand_peak(torch, sa, 1, s0["q"], s0["kv"])
    full = res["1/1"]["stack_ms"]
    for r in res.values():
        r["speedup_vs_all_full"] = round(full / r["stack_ms"], 4)
        r["measured_saving_ms"] = round(full - r["stack_ms"], 3)
    del sets, st
    torch.cuda.empty_cache()
    return {"workload": "stack_32k", "L": wl.Lq, "layers": n_layers, "input_sets": n_sets,
            "indexer_ms_per_full_layer": round(t_idx, 3), "sparse_mla_ms_per_layer": round(t_att, 3),
            "ffn_and_residual_ms_per_layer": round(t_ffn, 3),
            "sparse_mla_roofline": {"bound": "mfma", "achieved": round(mla_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                                    "unit": "TFLOP/s", "frac": round(mla_tflops / PEAK_BF16_TFLOPS, 4),
                                    "operand_peak": round(mla_peak, 1),
                                    "frac_of_operand_peak": round(mla_tflops / mla_peak, 4),
                                    "flops_per_layer": mla_flops},
            "patterns": res,
            "note": "stack_ms: the whole 16-layer stack timed end to end (X chained, layer l on input set l mod 4); "
                    "modelled_stack_ms = Full layers x indexer + all layers x (sparse MLA + FFN stand-in)"}


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
    elif args.profile == "chunk":
        paged, contig = _prefill_chunk_calls(torch, sa, inputs)[:2]
        for _ in range(args.warmup + args.steps):
            paged()
            contig()
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
    """Scales each kernel's FETCH_SIZE / WRITE_SIZE by what the same counters
    read for a device copy of COPY_BYTES each way, and prints the bytes per
    launch; the headline kernel's figure is also recorded in TRAFFIC_FILE."""
    d = args.traffic_from
    copy_name = "copyBuffer"   # the device-to-device copy torch issues for dst.copy_(src)
    cf_kb = _counter_kb(os.path.join(d, "copy_fetch"), "FETCH_SIZE", copy_name)
    cw_kb = _counter_kb(os.path.join(d, "copy_write"), "WRITE_SIZE", copy_name)
    f_fetch = cf_kb * 1024.0 / COPY_BYTES
    f_write = cw_kb * 1024.0 / COPY_BYTES
    out = []
    for kname in [x for x in args.kernels.split(",") if x]:
        fetch_kb = _counter_kb(os.path.join(d, "fetch"), "FETCH_SIZE", kname)
        write_kb = _counter_kb(os.path.join(d, "write"), "WRITE_SIZE", kname)
        read_b = fetch_kb * 1024.0 / f_fetch
        write_b = write_kb * 1024.0 / f_write
        rec = {"kernel": kname, "kernel_source_sha": _kernel_sha(),
               "fetch_size_kb": fetch_kb, "write_size_kb": write_kb,
               "copy_bytes_each_way": COPY_BYTES, "copy_fetch_kb": cf_kb, "copy_write_kb": cw_kb,
               "scale_fetch": f_fetch, "scale_write": f_write,
               "read_bytes_per_launch": read_b, "write_bytes_per_launch": write_b,
               "bytes_per_launch": read_b + write_b}
        if kname == "prefill_kernel":
            rec["workload"] = "prefill_64k"
            with open(TRAFFIC_FILE, "w") as f:
                json.dump(rec, f, indent=1)
        out.append(rec)
    print(json.dumps(out))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def sa_scores_rows(torch, inputs, wl, rows):
    """The fused kernel's fp32 scores of the listed rows of prefill_64k (its
    test-only full score output, written once outside any timed region)."""
    import sparse_attention_indexer_lightning_amd as sa
    q, k, w = inputs.indexer_inputs(wl, 0, "cuda:0")
    scores = torch.empty(wl.B, wl.Lq, wl.Lk, dtype=torch.float32, device="cuda:0")
    sa.idx_score_topk(q, k, w, wl.topk, scores_dbg=scores)
    torch.cuda.synchronize()
    out = scores[0][torch.from_numpy(rows).to(scores.device)].cpu().numpy()
    del scores, q, k, w
    torch.cuda.empty_cache()
    return out


def _score_error(torch, g_rows, sampled):
    """Largest score difference over the sampled rows, as a fraction of
    |oracle| + 0.01 * max|oracle row| (the GPU tests allow 1e-2 for fp8)."""
    import numpy as np
    s_or = np.concatenate([s for _, _, s in sampled])
    worst, worst_abs = 0.0, 0.0
    for g, o in zip(g_rows, s_or):
        fin = np.isfinite(o)
        if not fin.any():
            continue
        scale = np.abs(o[fin]).max()
        err = np.abs(g[fin].astype(np.float64) - o[fin])
        worst = max(worst, float((err / (np.abs(o[fin]) + 0.01 * scale)).max()))
        worst_abs = max(worst_abs, float(err.max()))
    return {"max_err_over_scale": float(f"{worst:.3g}"), "max_abs": float(f"{worst_abs:.3g}"),
            "scale": "|oracle| + 0.01 max|oracle row|; tolerance of the GPU tests 1e-2"}


def cpu_baseline(args, inputs, torch, t_gpu=None):
    """Oracle pairs/s on the host (bounded seeded row sample of prefill_64k):
    once on the CPU share this process is given (OMP_NUM_THREADS, else every
    core), once on one thread.  With ``t_gpu`` (the timed steps' T) the
    sampled rows' oracle T is also compared with it: mean and minimum share
    of the oracle's k indices that the GPU selected, and rows identical."""
    import numpy as np

    import oracle
    wl = inputs.WORKLOADS["prefill_64k"]
    q, k, w = inputs.indexer_inputs(wl, 0, "cuda:0")
    qr = q.cpu().view(torch.uint8).numpy()
    kr = k.cpu().view(torch.uint8).numpy()
    wr = w.cpu().view(torch.int16).numpy()
    del q, k, w
    host_cores = os.cpu_count() or 1
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or host_cores
    threads = max(1, min(host_cores, share))
    rng = np.random.default_rng(2024)
    order = rng.permutation(wl.Lq)

    sampled = []   # (rows, oracle T)

    def run(nthreads, seconds, start):
        done_rows, done_pairs, wall = 0, 0, 0.0
        batch = 2 * nthreads
        while wall < seconds and start + done_rows < wl.Lq:
            rows = np.sort(order[start + done_rows:start + done_rows + batch]).astype(np.int64)
            t0 = time.perf_counter()
            t_or, s_or = oracle.indexer_topk(qr, kr, wr, ("fp8", "fp8", "bf16"), wl.topk, rows=rows,
                                             nthreads=nthreads)
            wall += time.perf_counter() - t0
            sampled.append((rows, t_or, s_or))
            done_rows += rows.size
            done_pairs += int((rows + 1).sum())
        return done_rows, done_pairs, wall

    rows_n, pairs_n, wall_n = run(threads, args.cpu_seconds, 0)
    rows_1, pairs_1, wall_1 = run(1, args.cpu_seconds / 3, rows_n)
    agreement = None
    if t_gpu is not None:
        rows = np.concatenate([r for r, _, _ in sampled])
        t_or = np.concatenate([t for _, t, _ in sampled])
        t_g = t_gpu.reshape(-1, wl.topk)[torch.from_numpy(rows).to(t_gpu.device)].cpu().numpy()
        share = []
        for a, b in zip(t_g, t_or):
            ref = b[b >= 0]
            share.append(np.intersect1d(a[a >= 0], ref).size / max(ref.size, 1))
        share = np.asarray(share)
        agreement = {"rows": int(rows.size), "overlap_mean": round(float(share.mean()), 6),
                     "overlap_min": round(float(share.min()), 6),
                     "rows_identical": int(sum(np.array_equal(a, b) for a, b in zip(t_g, t_or))),
                     "score_error": _score_error(torch, sa_scores_rows(torch, inputs, wl, rows), sampled)}
    return {"value": round(pairs_n / wall_n, 1), "unit": "pairs/s", "cores": threads, "kind": "oracle",
            "t_agreement_with_gpu": agreement,
            "sample": f"{rows_n} seeded random query rows of prefill_64k ({pairs_n} causal pairs, fp64 scores + "
                      f"top-k), {wall_n:.1f} s wall on {threads} threads",
            "host_cpu": _cpu_model(), "host_logical_cores": host_cores,
            "one_thread": {"value": round(pairs_1 / wall_1, 1), "unit": "pairs/s",
                           "sample": f"{rows_1} further rows of the same order ({pairs_1} pairs), {wall_1:.1f} s"}}


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    import sparse_attention_indexer_lightning_amd as sa
    from sparse_attention_indexer_lightning_amd import inputs

    sa.lib()
    if args.profile:
        profile_run(args, torch, sa, inputs)
        return
    wl, ms, pairs, flops, t_head, peak_ops = headline(args, torch, sa, inputs)
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
                     "flops_per_launch": flops,
                     "operand_peak": round(peak_ops, 1), "frac_of_operand_peak": round(achieved / peak_ops, 4),
                     "operand_peak_note": "fp8 32x32x64 MFMA chains on this workload's q and k bytes (engine "
                                          "clock falls with operand toggling); peak stays the published one"},
    }
    if not args.no_decode:
        line["secondary"] = decode(args, torch, sa, inputs)
        line["secondary"]["serving_prefill_chunk"] = serving_prefill_chunk(args, torch, sa, inputs)
    if not args.no_sweep:
        line["retention_sweep"] = retention_sweep(args, torch, sa, inputs)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, inputs, torch, t_head)
    print(json.dumps(line))


def _kernel_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for n in ("indexer.hip", "device_common.h", "select_common.h", "kernels.h"):
        with open(os.path.join(ROOT, "sparse_attention_indexer_lightning_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
