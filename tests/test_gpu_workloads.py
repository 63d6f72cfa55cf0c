"""GPU parity on the five workloads at full size, through the C ABI, in the launch
configuration the benchmark times.  Full comparison where the oracle is fast
(tiny stack); seeded row samples elsewhere, plus the closed-form recency input
at full size (every key enters the streaming selection)."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_lightning_amd as sa
from sparse_attention_indexer_lightning_amd import inputs
from parity_util import (RTOL, check_index_sets, check_scores, check_t_invariants_gpu, indexer_oracle, raw,
                         sample_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _f64(x):
    return oracle.bf16_bits_to_f64(raw(x))


def test_tiny_stack_full():
    """4 layers F,S,S,S: index sets, scores, attention and the final X against the oracle."""
    wl = inputs.WORKLOADS["tiny_stack"]
    L, k = wl.Lq, wl.topk
    scale = 1.0 / math.sqrt(wl.Dqk)
    x = inputs.stack_x0(wl, DEV)
    t_cache = torch.full((1, L, k), -1, dtype=torch.int32, device=DEV)
    layers = []
    for layer, c in enumerate(wl.pattern):
        q, kk, w = inputs.indexer_inputs(wl, layer, DEV)
        qa, kv = inputs.attention_inputs(wl, layer, DEV)
        W = inputs.ffn_weight(wl, layer, DEV)
        layers.append(dict(q_i=raw(q), k_i=raw(kk), w=raw(w), idx_dtypes=("bf16", "bf16", "fp32"),
                           q=raw(qa), kv=raw(kv), W=raw(W)))
        if c == "F":
            scores = torch.empty(1, L, L, dtype=torch.float32, device=DEV)
            sa.idx_score_topk(q, kk, w, k, scores_dbg=scores)
            to, so = indexer_oracle(q, kk, w, k)
            torch.cuda.synchronize()
            check_scores(scores.cpu().numpy()[0], so, RTOL["bf16"], f"layer {layer}")
        assert sa.idx_cache_route(wl.pattern, layer, q, kk, w, t_cache) == (c == "F")
        torch.cuda.synchronize()
        assert np.array_equal(t_cache.cpu().numpy()[0], to), f"layer {layer}: T differs"
        o, _ = sa.sparse_mla_attn(qa, kv, t_cache, scale, wl.Dv)
        x1 = (x.float() + o.float().sum(dim=2)[0]).to(torch.bfloat16)
        x = (x1.float() @ W.float()).to(torch.bfloat16)
    torch.cuda.synchronize()
    xo, ts = oracle.stack(wl.pattern, raw(inputs.stack_x0(wl, DEV)), layers, k, scale, wl.Dv, residual_ffn=False)
    for a, b in zip(ts[1:], ts[:-1]):
        assert np.array_equal(a, b)  # one Full layer: every layer uses its T
    # bf16 rounding of X after every step on both sides: relative Frobenius
    # error within 2e-2 and no element off by more than 5 % of max |X|
    xg, xr = _f64(x), oracle.bf16_bits_to_f64(xo)
    rel = np.linalg.norm(xg - xr) / np.linalg.norm(xr)
    assert rel <= 2e-2, f"final X relative error {rel}"
    assert np.abs(xg - xr).max() <= 0.05 * np.abs(xr).max()


def test_prefill_8k_sampled():
    wl = inputs.WORKLOADS["prefill_8k"]
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    scores = torch.empty(wl.Lq, wl.Lk, dtype=torch.float32, device=DEV)
    t = sa.idx_score_topk(q, k, w, wl.topk, scores_dbg=scores)
    torch.cuda.synchronize()
    check_t_invariants_gpu(t, wl.Lq, wl.Lk, wl.topk)
    rows = sample_rows(wl.Lq, wl.topk, 56, seed=1001)
    to, so = indexer_oracle(q, k, w, wl.topk, rows=rows)
    sg = scores.cpu().numpy()[rows]
    check_scores(sg, so, RTOL["fp8"], "prefill_8k")
    pos = oracle.row_positions(1, wl.Lq, wl.Lk, rows)
    check_index_sets(t.cpu().numpy()[0][rows], to, so, pos, wl.topk, RTOL["fp8"], "prefill_8k")
    # the top-k kernel on the oracle's own score rows is bit-exact
    s_or = torch.from_numpy(so).to(DEV)
    t_or = sa.idx_topk(s_or, wl.topk, row_pos=torch.from_numpy(pos).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(t_or.cpu().numpy(), to)


def test_prefill_64k_sampled():
    wl = inputs.WORKLOADS["prefill_64k"]
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    t = sa.idx_score_topk(q, k, w, wl.topk)
    torch.cuda.synchronize()
    check_t_invariants_gpu(t, wl.Lq, wl.Lk, wl.topk)
    rows = np.array([0, 2047, 2048, 9000, 33333, 51234, 65534, 65535], dtype=np.int64)
    to, so = indexer_oracle(q, k, w, wl.topk, rows=rows)
    pos = oracle.row_positions(1, wl.Lq, wl.Lk, rows)
    check_index_sets(t.cpu().numpy()[0][rows], to, so, pos, wl.topk, RTOL["fp8"], "prefill_64k")


def test_prefill_64k_recency_closed_form():
    """I[t,s] = s at full size: T[t] = {t-k+1..t}; every key enters the selection."""
    wl = inputs.WORKLOADS["prefill_64k"]
    q, k, w = inputs.closed_form_indexer(1, wl.Lq, wl.H, wl.D, "fp8", "recency", device=DEV)
    t = sa.idx_score_topk(q, k, w, wl.topk)
    torch.cuda.synchronize()
    i = torch.arange(wl.Lq, device=DEV)[:, None]
    j = torch.arange(wl.topk, device=DEV)[None, :]
    start = torch.clamp(i - wl.topk + 1, min=0)
    want = torch.where(start + j <= i, start + j, torch.full_like(i + j, -1)).to(torch.int32)
    assert torch.equal(t[0], want)


def test_decode_200k_sampled():
    wl = inputs.WORKLOADS["decode_200k"]
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    t = sa.idx_score_topk(q, k, w, wl.topk)
    torch.cuda.synchronize()
    check_t_invariants_gpu(t, wl.Lq, wl.Lk, wl.topk)
    bs = [0, 13, 31]
    for b in bs:
        to, so = indexer_oracle(q[b:b + 1], k[b:b + 1], w[b:b + 1], wl.topk)
        check_index_sets(t[b].cpu().numpy(), to, so, np.array([wl.Lk - 1]), wl.topk, RTOL["fp8"], f"decode b={b}")
    # sparse MLA over the selected rows, compared on the gathered rows
    qa, kv = inputs.attention_inputs(wl, 0, DEV)
    scale = 1.0 / math.sqrt(wl.Dqk)
    out, _ = sa.sparse_mla_attn(qa, kv, t, scale, wl.Dv)
    torch.cuda.synchronize()
    for b in (0, 7, 31):
        sel = t[b, 0].long()
        kv_sub = kv[b:b + 1, sel]                                  # the 2048 gathered rows
        t_sub = torch.arange(wl.topk, dtype=torch.int32).reshape(1, 1, -1).numpy()
        ro, _ = oracle.sparse_mla_dv(raw(qa[b:b + 1]), raw(kv_sub), t_sub, scale, wl.Dv)
        err = np.abs(_f64(out[b:b + 1]).reshape(ro.shape) - oracle.bf16_bits_to_f64(ro)).max()
        assert err <= 2e-2, f"decode attention b={b}: {err}"


def test_decode_200k_recency_closed_form():
    wl = inputs.WORKLOADS["decode_200k"]
    q, k, w = inputs.closed_form_indexer(4, wl.Lk, wl.H, wl.D, "fp8", "recency", device=DEV)
    q = q[:, -1:].contiguous()
    w = w[:, -1:].contiguous()
    t = sa.idx_score_topk(q, k, w, wl.topk)
    torch.cuda.synchronize()
    want = torch.arange(wl.Lk - wl.topk, wl.Lk, dtype=torch.int32, device=DEV)
    assert all(torch.equal(t[b, 0], want) for b in range(4))


def test_stack_32k_one_group_sampled():
    """One F layer and one S layer of the 16-layer stack at L = 32768: the index
    set on sampled rows, Shared-layer reuse, and attention on sampled queries."""
    wl = inputs.WORKLOADS["stack_32k"]
    L, k = wl.Lq, wl.topk
    q, kk, w = inputs.indexer_inputs(wl, 0, DEV)
    t_cache = torch.full((1, L, k), -1, dtype=torch.int32, device=DEV)
    assert sa.idx_cache_route(wl.pattern, 0, q, kk, w, t_cache)
    torch.cuda.synchronize()
    snap = t_cache.clone()
    assert not sa.idx_cache_route(wl.pattern, 1, None, None, None, t_cache)
    torch.cuda.synchronize()
    assert torch.equal(snap, t_cache)
    check_t_invariants_gpu(t_cache, L, L, k)
    rows = np.array([0, 2047, 2048, 20000, 32767], dtype=np.int64)
    to, so = indexer_oracle(q, kk, w, k, rows=rows)
    pos = oracle.row_positions(1, L, L, rows)
    check_index_sets(t_cache.cpu().numpy()[0][rows], to, so, pos, k, RTOL["fp8"], "stack_32k")
    del q, kk, w
    qa, kv = inputs.attention_inputs(wl, 1, DEV)
    scale = 1.0 / math.sqrt(wl.Dqk)
    out, _ = sa.sparse_mla_attn(qa, kv, t_cache, scale, wl.Dv)
    torch.cuda.synchronize()
    for i in (0, 5000, 32767):
        ro, _ = oracle.sparse_mla_dv(raw(qa[:, i:i + 1]), raw(kv), t_cache[:, i:i + 1].cpu().numpy(), scale, wl.Dv)
        err = np.abs(_f64(out[:, i:i + 1]).reshape(ro.shape) - oracle.bf16_bits_to_f64(ro)).max()
        assert err <= 2e-2, f"stack attention query {i}: {err}"
