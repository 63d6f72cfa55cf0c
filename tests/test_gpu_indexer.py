"""GPU parity of the indexer + top-k and the router, through the C ABI, on small
and edge-case shapes the oracle computes in full."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_lightning_amd as sa
from sparse_attention_indexer_lightning_amd import inputs
from parity_util import (RTOL, check_index_sets, check_scores, check_t_invariants_gpu, enc_of,
                         indexer_oracle)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run_full(q, k, w, topk, dbg=True):
    B, Lq = q.shape[:2]
    Lk = k.shape[1]
    scores = torch.empty(B, Lq, Lk, dtype=torch.float32, device=DEV) if dbg else None
    t = sa.idx_score_topk(q, k, w, topk, scores_dbg=scores)
    torch.cuda.synchronize()
    return t, scores


def compare_all_rows(q, k, w, topk, what, exact_sets=False):
    B, Lq = q.shape[:2]
    Lk = k.shape[1]
    t, scores = run_full(q, k, w, topk)
    # the launch without the test-only score row (the production variant of
    # the fused sweep) gives the same T
    t_nodbg, _ = run_full(q, k, w, topk, dbg=False)
    assert torch.equal(t, t_nodbg), what
    to, so = indexer_oracle(q, k, w, topk)
    rt = RTOL[enc_of(q)]
    check_scores(scores.cpu().numpy().reshape(B * Lq, Lk), so, rt, what)
    tg = t.cpu().numpy().reshape(B * Lq, topk)
    pos = oracle.row_positions(B, Lq, Lk)
    if exact_sets:
        assert np.array_equal(tg, to), what
    else:
        check_index_sets(tg, to, so, pos, topk, rt, what)
    check_t_invariants_gpu(t, Lq, Lk, topk)
    return tg, to


def _golden():
    with open(os.path.join(GOLDEN, "hand_example_8tok.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("enc,H,D", [("fp8", 64, 128), ("bf16", 4, 32), ("bf16", 16, 64)])
def test_hand_example_through_router(enc, H, D):
    g = _golden()
    L, k = g["L"], g["topk"]
    qdt = torch.float8_e4m3fn if enc == "fp8" else torch.bfloat16
    wdt = torch.bfloat16 if enc == "fp8" else torch.float32
    keys = torch.zeros(1, L, D)
    keys[0, :, :2] = torch.tensor(g["keys"], dtype=torch.float32)
    q = torch.zeros(1, L, H, D)
    q[0, :, 0, 0] = 1.0
    q[0, :, 1, 1] = 1.0
    t_cache = torch.full((1, L, k), 12345, dtype=torch.int32, device=DEV)
    for layer, c in enumerate(g["pattern"]):
        ww = g["w_even_odd_by_layer"][str(layer)]
        w = torch.zeros(1, L, H)
        for t in range(L):
            w[0, t, :2] = torch.tensor(ww["even"] if t % 2 == 0 else ww["odd"], dtype=torch.float32)
        before = t_cache.clone()
        did = sa.idx_cache_route(g["pattern"], layer, q.to(qdt).to(DEV), keys.to(qdt).to(DEV),
                                 w.to(wdt).to(DEV), t_cache)
        torch.cuda.synchronize()
        assert did == (c == "F")
        if c == "S":
            assert torch.equal(before, t_cache), "a Shared layer modified the cache"
        src = g["expected"]["T_by_layer"][str(layer)]
        assert t_cache[0].cpu().tolist() == g["expected"][src]["T"], (enc, layer)


@pytest.mark.parametrize("enc,H,D", [("bf16", 4, 32), ("bf16", 8, 32), ("bf16", 16, 64), ("bf16", 32, 128),
                                     ("bf16", 64, 32), ("fp8", 16, 128), ("fp8", 32, 128), ("fp8", 64, 128)])
def test_head_counts_and_dims(enc, H, D):
    wl = inputs.Workload("t", 1, 300, 300, H, D, 40, enc, "bf16" if enc == "fp8" else "fp32", 11)
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    compare_all_rows(q, k, w, 40, f"{enc} H={H} D={D}")


@pytest.mark.parametrize("B,Lq,Lk,topk", [
    (1, 50, 50, 64),        # every row shorter than k: pure padding
    (1, 40, 40, 8),         # one partial key block (keys past the end read as zeros)
    (1, 64, 64, 64),        # exactly one key block, k = every key
    (2, 65, 65, 33),        # one block and one key, batch
    (1, 777, 777, 100),     # ragged length, several key blocks
    (3, 130, 130, 17),      # batch
    (1, 300, 1000, 256),    # chunked prefill: queries at the end of a longer context
    (1, 200, 200, 1),       # k = 1
    (2, 3, 5000, 300),      # decode-shaped (split-key path) with B > 1, Lq > 1
    (1, 1, 3000, 2048),     # single decode query
    (2, 300, 6000, 2048),   # sampled starting threshold, batch, queries at the end of the context
    (1, 64, 5000, 512),     # sampled threshold with a smaller k (rank r = 35 of the sample)
    (2, 2, 4097, 512),      # decode-shaped, score rows not a multiple of 4 floats (scores written directly)
])
def test_edge_shapes_fp8(B, Lq, Lk, topk):
    wl = inputs.Workload("e", B, Lq, Lk, 64, 128, topk, "fp8", "bf16", 5)
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    compare_all_rows(q, k, w, topk, f"B={B} Lq={Lq} Lk={Lk} k={topk}")


def test_long_context_32bit_indices():
    """Lk > 65536: the fused kernel keeps 16-bit candidate indices with a
    per-row table of where each 65,536-key segment starts in the buffer."""
    wl = inputs.Workload("l", 1, 40, 70000, 64, 128, 2048, "fp8", "bf16", 6)
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    t, scores = run_full(q, k, w, 2048)
    rows = np.array([0, 17, 39], dtype=np.int64)
    to, so = indexer_oracle(q, k, w, 2048, rows=rows)
    sg = scores.cpu().numpy().reshape(40, -1)[rows]
    check_scores(sg, so, RTOL["fp8"], "Lk=70000")
    pos = oracle.row_positions(1, 40, 70000, rows)
    check_index_sets(t.cpu().numpy().reshape(40, -1)[rows], to, so, pos, 2048, RTOL["fp8"], "Lk=70000")


@pytest.mark.parametrize("enc", ["fp8", "bf16"])
@pytest.mark.parametrize("kind", ["recency", "reverse", "ties", "negzero_ties"])
@pytest.mark.parametrize("Lq,Lk", [(700, 700), (2, 9000)])
def test_closed_forms(enc, kind, Lq, Lk):
    """Scores with a known order: recency (I = s) inserts every key into the
    streaming selection, reverse (I = -s) only the first k; ties must resolve
    to the lowest indices, also when every score is -0."""
    H, D, k = (64, 128, 256) if enc == "fp8" else (4, 32, 64)
    q, kk, w = inputs.closed_form_indexer(1, Lk, H, D, enc, kind, device=DEV)
    q = q[:, Lk - Lq:].contiguous()
    w = w[:, Lk - Lq:].contiguous()
    t, scores = run_full(q, kk, w, k)
    tg = t.cpu().numpy().reshape(Lq, k)
    sg = scores.cpu().numpy().reshape(Lq, Lk)
    for i in range(Lq):
        p = Lk - Lq + i
        n = min(k, p + 1)
        if kind == "recency":
            want = np.arange(p + 1 - n, p + 1)
            assert np.array_equal(sg[i, : p + 1], np.arange(p + 1, dtype=np.float32))
        else:
            want = np.arange(n)
        assert np.array_equal(tg[i, :n], want), (kind, i)
        assert np.all(tg[i, n:] == -1)
        assert np.all(np.isneginf(sg[i, p + 1:]))


def test_determinism():
    wl = inputs.Workload("d", 1, 1500, 1500, 64, 128, 512, "fp8", "bf16", 9)
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    t1, s1 = run_full(q, k, w, 512)
    t2, s2 = run_full(q, k, w, 512)
    t3, _ = run_full(q, k, w, 512, dbg=False)
    assert torch.equal(t1, t2) and torch.equal(t1, t3)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))


def test_fused_and_split_paths_agree():
    """The fused prefill kernel and the split-key path agree: the same queries
    scored by both give scores within the score tolerance of each other and
    index sets that differ only at keys within it of the k-th score.  (The two
    kernels sum in different fp32 orders: the 64-head fused kernel splits the
    ReLU as w*|x|/2 + w*x/2 with the linear half on an MFMA, so their scores are
    not bit-identical.)"""
    wl = inputs.Workload("a", 2, 4, 6000, 64, 128, 700, "fp8", "bf16", 12)
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    t_split, s_split = run_full(q, k, w, 700)           # Lq <= 4: split-key path
    # the same queries as the tail of a longer query block: fused path
    wl2 = inputs.Workload("a", 2, 40, 6000, 64, 128, 700, "fp8", "bf16", 12)
    q2 = torch.zeros(2, 40, 64, 128, dtype=q.dtype, device=DEV)
    w2 = torch.zeros(2, 40, 64, dtype=w.dtype, device=DEV)
    q2[:, 36:] = q
    w2[:, 36:] = w
    t_fused, s_fused = run_full(q2.contiguous(), k, w2.contiguous(), 700)
    sg = s_fused[:, 36:].cpu().numpy().reshape(8, -1)
    so = s_split.cpu().numpy().reshape(8, -1).astype(np.float64)
    check_scores(sg, so, RTOL["fp8"], "fused vs split")
    pos = oracle.row_positions(2, 4, 6000)
    check_index_sets(t_fused[:, 36:].cpu().numpy().reshape(8, -1), t_split.cpu().numpy().reshape(8, -1), so, pos,
                     700, RTOL["fp8"], "fused vs split")
    del wl2


def test_sampled_threshold_fallback():
    """The 64-head fused sweep starts each long row from a threshold taken on
    every 32nd key block.  Here the keys of those blocks get four times the
    norm, so the sample's threshold lies above nearly every other score: the
    rows end with fewer than k candidates and their workgroups sweep again
    without the sample.  T must be the exact top-k of the kernel's own scores
    and agree with the oracle."""
    Lq, Lk, topk = 24, 12000, 2048
    wl = inputs.Workload("s", 1, Lq, Lk, 64, 128, topk, "fp8", "bf16", 21)
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    kf = k.float()
    sampled = (torch.arange(Lk, device=DEV) // 64) % 32 == 0
    kf[:, sampled] = (kf[:, sampled] * 4).clamp(-448, 448)
    k = kf.to(torch.float8_e4m3fn).contiguous()
    t, scores = run_full(q, k, w, topk)
    pos = oracle.row_positions(1, Lq, Lk)
    sg = scores.cpu().numpy().reshape(Lq, Lk)
    tg = t.cpu().numpy().reshape(Lq, topk)
    assert np.array_equal(tg, oracle.topk(sg, pos, topk))
    rows = np.array([0, 11, 23], dtype=np.int64)
    to, so = indexer_oracle(q, k, w, topk, rows=rows)
    check_scores(sg[rows], so, RTOL["fp8"], "sampled fallback")
    check_index_sets(tg[rows], to, so, pos[rows], topk, RTOL["fp8"], "sampled fallback")


@pytest.mark.parametrize("kind", ["ties", "reverse"])
def test_sampled_threshold_closed_forms(kind):
    """Long rows with k = 2048 take the sampled starting threshold.  With every
    score equal the threshold is the tie value itself, no key beats it, and
    the workgroups sweep again without the sample (ties then go to the lowest
    indices); with I = -s the sample's threshold admits exactly the keys
    below the r-th sampled one."""
    Lq, Lk, k = 16, 6000, 2048
    q, kk, w = inputs.closed_form_indexer(1, Lk, 64, 128, "fp8", kind, device=DEV)
    q = q[:, Lk - Lq:].contiguous()
    w = w[:, Lk - Lq:].contiguous()
    t, _ = run_full(q, kk, w, k)
    tg = t.cpu().numpy().reshape(Lq, k)
    assert np.array_equal(tg, np.tile(np.arange(k, dtype=np.int32), (Lq, 1))), kind


def test_long_context_segments_vs_oracle():
    """Four key segments (Lk = 200,000): sampled rows against the oracle."""
    Lq, Lk = 48, 200000
    wl = inputs.Workload("s", 1, Lq, Lk, 64, 128, 2048, "fp8", "bf16", 9)
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    t, scores = run_full(q, k, w, 2048)
    rows = np.array([0, 21, 47], dtype=np.int64)
    to, so = indexer_oracle(q, k, w, 2048, rows=rows)
    sg = scores.cpu().numpy().reshape(Lq, -1)[rows]
    check_scores(sg, so, RTOL["fp8"], "Lk=200000")
    pos = oracle.row_positions(1, Lq, Lk, rows)
    check_index_sets(t.cpu().numpy().reshape(Lq, -1)[rows], to, so, pos, 2048, RTOL["fp8"], "Lk=200000")


@pytest.mark.parametrize("kind", ["recency", "reverse", "ties"])
def test_long_context_segments_closed_forms(kind):
    """Closed forms over three key segments: I = s puts every selected key in
    the last segment (the earlier ones end up empty), I = -s and all-equal
    scores keep every selected key in the first (later segments never
    reached); T is known exactly."""
    Lq, Lk, k = 8, 140000, 2048
    q, kk, w = inputs.closed_form_indexer(1, Lk, 64, 128, "fp8", kind, device=DEV)
    q = q[:, Lk - Lq:].contiguous()
    w = w[:, Lk - Lq:].contiguous()
    t, _ = run_full(q, kk, w, k, dbg=False)
    tg = t.cpu().numpy().reshape(Lq, k)
    for i in range(Lq):
        pos = Lk - Lq + i
        want = np.arange(pos - k + 1, pos + 1, dtype=np.int32) if kind == "recency" else np.arange(k, dtype=np.int32)
        assert np.array_equal(tg[i], want), (kind, i)
