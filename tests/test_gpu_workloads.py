"""GPU parity on the five workloads at full size, through the C ABI, in the launch
configuration the benchmark times.  Full comparison where the oracle is fast
(tiny stack); seeded random row samples elsewhere (plus the edge rows), the
closed-form recency input at full size (every key enters the streaming
selection), and bitwise determinism of T at the two headline shapes.

Stack workloads compare the library's outputs (each layer's T and attention
output O) with the oracle, and the harness's X after every layer element by
element within the bound of parity_util.stack_layer_bound: once for one layer
applied to the same input (the GPU's X entering the layer), once along the
whole chain from X0 (oracle.stack)."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_lightning_amd as sa
from sparse_attention_indexer_lightning_amd import inputs
from parity_util import (RTOL, check_index_sets, check_scores, check_t_invariants_gpu, harness_layer,
                         indexer_oracle, raw, sample_rows, score_tol, stack_layer_bound)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ATT_TOL = 2e-2    # attention: max-abs on the bf16 output


def _f64(x):
    return oracle.bf16_bits_to_f64(raw(x) if isinstance(x, torch.Tensor) else x)


def _report(what, **vals):
    print(f"[parity] {what}: " + ", ".join(f"{k}={v:.4g}" if isinstance(v, float) else f"{k}={v}"
                                           for k, v in vals.items()), flush=True)


def _row_maxabs(a, b):
    d = np.abs(_f64(a) - _f64(b))
    return d.reshape(d.shape[0], -1).max(axis=1)


def _check_stack(wl, pattern, rows, x0_rows, layers, t_gpu, xs_g, os_g, scale, residual):
    """Per layer: O against the oracle (given the GPU's T, and along the
    oracle's own chain), X after one layer from the GPU's input, and X along
    the chain, each element-wise.  rows: the query rows compared (their X and
    O are in xs_g / os_g, in this order; None: every row).

    Along the chain the oracle uses its own index sets.  Where a row's T
    differs from the GPU's (allowed at near-ties of the k-th score), its
    attention output legitimately differs by more than the attention
    tolerance, so that tolerance is asserted on the rows whose T agree; the X
    bound uses every row's measured O difference and holds for all rows."""
    L, k = wl.Lq, wl.topk
    rows_a = np.arange(L) if rows is None else np.asarray(rows)
    xo, ts_o, xs_o, os_o = oracle.stack(pattern, x0_rows, layers, k, scale, wl.Dv, residual, rows=rows,
                                        per_layer=True)
    e_chain = np.zeros(x0_rows.shape)
    x_in_g = x0_rows
    worst = dict(step_x=0.0, chain_x=0.0, o_given_t=0.0, o_chain_same_t=0.0, o_chain_other_t=0.0,
                 rows_t_differ=0, x_rel_chain=0.0)
    for l in range(len(pattern)):
        W = _f64(layers[l]["W"])
        # one layer from the GPU's own input X and index set
        x_st, o_st, det = oracle.stack_layer(x_in_g, t_gpu[l], layers[l], scale, wl.Dv, residual, rows=rows,
                                             detail=True)
        d_o = _row_maxabs(os_g[l], o_st)
        assert d_o.max() <= ATT_TOL, f"layer {l}: attention given the GPU's T, max-abs {d_o.max()}"
        e = stack_layer_bound(0.0, det, _f64(o_st), _f64(oracle.f64_to_bf16_bits(det["pre_x1"])), W, d_o,
                              residual)
        err = np.abs(_f64(xs_g[l]) - _f64(x_st))
        assert np.all(err <= e), f"layer {l}: X from the same input off by {err.max()} (bound {e[err > e][:3]})"
        # the same layer along the oracle's chain from X0
        same_t = np.all(ts_o[l][0, rows_a] == t_gpu[l][0, rows_a], axis=1)
        d_oc = _row_maxabs(os_g[l], os_o[l])
        if same_t.any():
            assert d_oc[same_t].max() <= ATT_TOL, f"layer {l}: attention along the chain, max-abs {d_oc.max()}"
        worst["o_chain_same_t"] = max(worst["o_chain_same_t"], float(d_oc[same_t].max(initial=0.0)))
        worst["o_chain_other_t"] = max(worst["o_chain_other_t"], float(d_oc[~same_t].max(initial=0.0)))
        worst["rows_t_differ"] = max(worst["rows_t_differ"], int((~same_t).sum()))
        x_prev_o = x0_rows if l == 0 else xs_o[l - 1]
        _, _, det_c = oracle.stack_layer(x_prev_o, ts_o[l], layers[l], scale, wl.Dv, residual, rows=rows,
                                         detail=True)
        e_chain = stack_layer_bound(e_chain, det_c, _f64(os_o[l]),
                                    _f64(oracle.f64_to_bf16_bits(det_c["pre_x1"])), W, d_oc, residual)
        err_c = np.abs(_f64(xs_g[l]) - _f64(xs_o[l]))
        assert np.all(err_c <= e_chain), f"layer {l}: X along the chain off by {err_c.max()}"
        if float(err.max()) > worst["step_x"]:
            i = np.unravel_index(np.argmax(err), err.shape)
            worst["step_x_at_abs_x"] = float(abs(_f64(x_st)[i]))
            worst["step_x_bound_there"] = float(e[i])
        worst["x_abs_max"] = max(worst.get("x_abs_max", 0.0), float(np.abs(_f64(x_st)).max()))
        worst["step_x"] = max(worst["step_x"], float(err.max()))
        worst["chain_x"] = max(worst["chain_x"], float(err_c.max()))
        worst["o_given_t"] = max(worst["o_given_t"], float(d_o.max()))
        x_in_g = xs_g[l]
    xr = _f64(xo)
    worst["x_rel_chain"] = float(np.linalg.norm(_f64(xs_g[-1]) - xr) / np.linalg.norm(xr))
    return ts_o, worst


def test_tiny_stack_full():
    """4 layers F,S,S,S, every row: scores, index sets (bit-exact), attention and X after every layer."""
    wl = inputs.WORKLOADS["tiny_stack"]
    L, k = wl.Lq, wl.topk
    scale = 1.0 / math.sqrt(wl.Dqk)
    x = inputs.stack_x0(wl, DEV)
    x0 = raw(x)
    t_cache = torch.full((1, L, k), -1, dtype=torch.int32, device=DEV)
    layers, t_gpu, xs_g, os_g = [], [], [], []
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
        t_gpu.append(t_cache.cpu().numpy().copy())
        o, _ = sa.sparse_mla_attn(qa, kv, t_cache, scale, wl.Dv)
        x = harness_layer(x, o[0], W, False, torch)
        torch.cuda.synchronize()
        os_g.append(raw(o[0]))
        xs_g.append(raw(x))
    ts_o, worst = _check_stack(wl, wl.pattern, None, x0, layers, t_gpu, xs_g, os_g, scale, False)
    for l in range(len(wl.pattern)):
        assert np.array_equal(ts_o[l], t_gpu[l]), f"layer {l}: T along the oracle's chain differs"
    _report("tiny_stack", **worst)


def test_prefill_8k_sampled():
    wl = inputs.WORKLOADS["prefill_8k"]
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    scores = torch.empty(wl.B, wl.Lq, wl.Lk, dtype=torch.float32, device=DEV)
    t = sa.idx_score_topk(q, k, w, wl.topk, scores_dbg=scores)
    torch.cuda.synchronize()
    check_t_invariants_gpu(t, wl.Lq, wl.Lk, wl.topk)
    rows = sample_rows(wl.Lq, wl.topk, 128, seed=1001)
    to, so = indexer_oracle(q, k, w, wl.topk, rows=rows)
    sg = scores.cpu().numpy()[0][rows]
    check_scores(sg, so, RTOL["fp8"], "prefill_8k")
    pos = oracle.row_positions(1, wl.Lq, wl.Lk, rows)
    ov = check_index_sets(t.cpu().numpy()[0][rows], to, so, pos, wl.topk, RTOL["fp8"], "prefill_8k")
    # the top-k kernel on the oracle's own score rows is bit-exact
    s_or = torch.from_numpy(so).to(DEV)
    t_or = sa.idx_topk(s_or, wl.topk, row_pos=torch.from_numpy(pos).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(t_or.cpu().numpy(), to)
    # largest score error as a fraction of its tolerance (1.0 = at the tolerance)
    frac = 0.0
    for r in range(so.shape[0]):
        fin = np.isfinite(so[r])
        tol = score_tol(so[r], RTOL["fp8"])[fin]
        frac = max(frac, float((np.abs(sg[r][fin].astype(np.float64) - so[r][fin]) / tol).max()))
    _report("prefill_8k", rows=len(rows), overlap=ov, score_err_over_tol=frac)


def test_prefill_64k_sampled():
    """128 seeded random rows plus the edge rows, in the benchmark's launch."""
    wl = inputs.WORKLOADS["prefill_64k"]
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    t = torch.empty(wl.B, wl.Lq, wl.topk, dtype=torch.int32, device=DEV)
    assert sa.idx_cache_route("F", 0, q, k, w, t)
    torch.cuda.synchronize()
    check_t_invariants_gpu(t, wl.Lq, wl.Lk, wl.topk)
    rows = sample_rows(wl.Lq, wl.topk, 128, seed=1002)
    assert len(rows) >= 128
    to, so = indexer_oracle(q, k, w, wl.topk, rows=rows)
    pos = oracle.row_positions(1, wl.Lq, wl.Lk, rows)
    ov = check_index_sets(t.cpu().numpy()[0][rows], to, so, pos, wl.topk, RTOL["fp8"], "prefill_64k")
    exact = sum(np.array_equal(t.cpu().numpy()[0][r], to[i]) for i, r in enumerate(rows))
    _report("prefill_64k", rows=len(rows), overlap=ov, rows_identical=exact)
    # bitwise determinism at full size (sampled threshold and batched compactions included)
    t2 = torch.empty_like(t)
    sa.idx_cache_route("F", 0, q, k, w, t2)
    torch.cuda.synchronize()
    assert torch.equal(t, t2), "T differs between two identical launches"


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


def test_decode_200k_all_sequences():
    """All 32 sequences: T against the oracle, attention element-wise (given the
    GPU's T, on the gathered rows), and bitwise determinism of T."""
    wl = inputs.WORKLOADS["decode_200k"]
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    ws = torch.empty(sa.idx_score_topk_workspace(q, k, w, wl.topk), dtype=torch.uint8, device=DEV)
    t = torch.empty(wl.B, wl.Lq, wl.topk, dtype=torch.int32, device=DEV)
    assert sa.idx_cache_route("F", 0, q, k, w, t, ws=ws)
    t2 = torch.empty_like(t)
    sa.idx_cache_route("F", 0, q, k, w, t2, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(t, t2), "decode T differs between two identical launches"
    check_t_invariants_gpu(t, wl.Lq, wl.Lk, wl.topk)
    to, so = indexer_oracle(q, k, w, wl.topk)
    pos = np.full(wl.B, wl.Lk - 1)
    ov = check_index_sets(t.cpu().numpy().reshape(wl.B, wl.topk), to, so, pos, wl.topk, RTOL["fp8"], "decode")
    qa, kv = inputs.attention_inputs(wl, 0, DEV)
    scale = 1.0 / math.sqrt(wl.Dqk)
    out, lse = sa.sparse_mla_attn(qa, kv, t, scale, wl.Dv,
                                  lse=torch.empty(wl.B, wl.Lq, wl.Hq, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    worst, worst_lse = 0.0, 0.0
    for b in range(wl.B):
        sel = t[b, 0].long()
        kv_sub = kv[b:b + 1, sel]                                  # the 2048 gathered rows
        t_sub = np.arange(wl.topk, dtype=np.int32).reshape(1, 1, -1)
        ro, rl = oracle.sparse_mla_dv(raw(qa[b:b + 1]), raw(kv_sub), t_sub, scale, wl.Dv)
        err = float(np.abs(_f64(out[b:b + 1]).reshape(ro.shape) - _f64(ro)).max())
        assert err <= ATT_TOL, f"decode attention b={b}: {err}"
        gl = lse[b, 0].cpu().numpy()
        assert np.allclose(gl, rl[0], rtol=1e-4, atol=1e-3), f"decode lse b={b}"
        el = float(np.abs(gl.astype(np.float64) - rl[0]).max())
        worst, worst_lse = max(worst, err), max(worst_lse, el)
    _report("decode_200k", sequences=wl.B, overlap=ov, attention_maxabs=worst, lse_maxabs=worst_lse)


def test_decode_200k_recency_closed_form():
    wl = inputs.WORKLOADS["decode_200k"]
    q, k, w = inputs.closed_form_indexer(4, wl.Lk, wl.H, wl.D, "fp8", "recency", device=DEV)
    q = q[:, -1:].contiguous()
    w = w[:, -1:].contiguous()
    t = sa.idx_score_topk(q, k, w, wl.topk)
    torch.cuda.synchronize()
    want = torch.arange(wl.Lk - wl.topk, wl.Lk, dtype=torch.int32, device=DEV)
    assert all(torch.equal(t[b, 0], want) for b in range(4))


def test_stack_32k_fsss_group_sampled():
    """One F,S,S,S group of the 16-layer stack at L = 32768 with its own seeded
    inputs per layer and X chained through the FFN stand-in (residual): the
    Full layer's T on >= 64 seeded random rows plus the edge rows, Shared
    layers leaving the cache untouched, attention and X of every layer on those
    rows against the oracle (rows are independent, so the oracle computes only
    them)."""
    wl = inputs.WORKLOADS["stack_32k"]
    L, k = wl.Lq, wl.topk
    pattern = wl.pattern[:4]
    scale = 1.0 / math.sqrt(wl.Dqk)
    rows = sample_rows(L, k, 64, seed=1004)
    assert len(rows) >= 64
    x = inputs.stack_x0(wl, DEV)
    x0_rows = raw(x[rows])
    t_cache = torch.full((1, L, k), -1, dtype=torch.int32, device=DEV)
    layers, t_gpu, xs_g, os_g = [], [], [], []
    rows_dev = torch.from_numpy(rows).to(DEV)
    for layer, c in enumerate(pattern):
        lay = {}
        if c == "F":
            q, kk, w = inputs.indexer_inputs(wl, layer, DEV)
            assert sa.idx_cache_route(pattern, layer, q, kk, w, t_cache)
            torch.cuda.synchronize()
            check_t_invariants_gpu(t_cache, L, L, k)
            lay.update(q_i=raw(q), k_i=raw(kk), w=raw(w), idx_dtypes=("fp8", "fp8", "bf16"))
            to, so = indexer_oracle(q, kk, w, k, rows=rows)
            pos = oracle.row_positions(1, L, L, rows)
            ov = check_index_sets(t_cache.cpu().numpy()[0][rows], to, so, pos, k, RTOL["fp8"], "stack_32k F")
            del q, kk, w
        else:
            snap = t_cache.clone()
            assert not sa.idx_cache_route(pattern, layer, None, None, None, t_cache)
            torch.cuda.synchronize()
            assert torch.equal(snap, t_cache), f"Shared layer {layer} changed the cache"
            del snap
        t_gpu.append(t_cache.cpu().numpy())
        qa, kv = inputs.attention_inputs(wl, layer, DEV)
        W = inputs.ffn_weight(wl, layer, DEV)
        o, _ = sa.sparse_mla_attn(qa, kv, t_cache, scale, wl.Dv)
        x = harness_layer(x, o[0], W, True, torch)
        torch.cuda.synchronize()
        lay.update(q=raw(qa[:, rows_dev]), kv=raw(kv), W=raw(W))
        layers.append(lay)
        os_g.append(raw(o[0, rows_dev]))
        xs_g.append(raw(x[rows_dev]))
        del qa, kv, o, W
    torch.cuda.empty_cache()
    ts_o, worst = _check_stack(wl, pattern, rows, x0_rows, layers, t_gpu, xs_g, os_g, scale, True)
    _report("stack_32k FSSS", rows=len(rows), overlap=ov, **worst)
