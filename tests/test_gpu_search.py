"""The greedy Full/Shared search (itoverdose.com, "IndexCache: Wie DeepSeek
O(NL²)-Kosten in Sparse Attention um 75% reduziert", section "Training-freie
Optimierung: Greedy-Suche mit minimalem Verlust") driven by a layer stack run
on the GPU through the library, against the same search over the oracle's
stack.

Loss of a pattern: relative deviation of its final X from the all-Full final X.
The GPU and the oracle evaluate it on stacks whose X differ by bf16 rounding
only, so the two loss values of one pattern differ by at most
    tol(p) = (e_p + e_F (1 + loss)) / ||X_oracle(all F)|| (+ slack),
e_p = ||X_gpu(p) - X_oracle(p)|| (triangle inequality on the two quotients).
Both searches must visit the same patterns; where their choices part, the two
chosen candidates must be tied within those tolerances (both are then valid
greedy steps), and the comparison stops there."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_indexer_lightning_amd import inputs
from sparse_attention_indexer_lightning_amd.search import greedy_pattern, stack_deviation_loss
from sparse_attention_indexer_lightning_amd.stack import Stack, layer_inputs
from parity_util import raw

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _oracle_loss(wl, layers_raw, x0_raw, scale):
    memo = {}
    ref = {}

    def run(p):
        if p not in memo:
            xo, _ = oracle.stack(p, x0_raw, layers_raw, wl.topk, scale, wl.Dv, wl.residual_ffn)
            memo[p] = oracle.bf16_bits_to_f64(xo)
        return memo[p]

    def loss(p):
        if "F" not in ref:
            ref["F"] = run("F" * len(layers_raw))
        x = run(p)
        return float(np.linalg.norm(x - ref["F"]) / np.linalg.norm(ref["F"]))

    loss.x = memo
    return loss


def test_greedy_search_on_gpu_stack_matches_oracle_search():
    n = 6
    wl = dataclasses.replace(inputs.WORKLOADS["tiny_stack"], name="tiny_stack_6", layers=n, pattern="F" * n)
    scale = 1.0 / math.sqrt(wl.Dqk)
    layers = [layer_inputs(wl, l, DEV) for l in range(n)]
    x0 = inputs.stack_x0(wl, DEV)
    st = Stack(wl, layers, x0, residual=wl.residual_ffn, fp32_ffn=True)
    loss_g = stack_deviation_loss(st)
    path_g = greedy_pattern(n, loss_g, n_full=1)
    torch.cuda.synchronize()

    layers_raw = [dict(q_i=raw(d["q_i"]), k_i=raw(d["k_i"]), w=raw(d["w"]), idx_dtypes=("bf16", "bf16", "fp32"),
                       q=raw(d["q"]), kv=raw(d["kv"]), W=raw(d["W"])) for d in layers]
    loss_o = _oracle_loss(wl, layers_raw, raw(x0), scale)
    path_o = greedy_pattern(n, loss_o, n_full=1)

    ref_o = loss_o.x["F" * n]
    nref = np.linalg.norm(ref_o)
    xg_ref = oracle.bf16_bits_to_f64(raw(st.run("F" * n)))
    e_f = np.linalg.norm(xg_ref - ref_o)

    def tol(p):
        xg = oracle.bf16_bits_to_f64(raw(st.run(p)))
        e_p = np.linalg.norm(xg - loss_o.x[p])
        return (e_p + e_f * (1 + loss_o(p))) / nref * 1.01 + 1e-12

    # every pattern both searches evaluated: the two losses agree within tol
    common = set(loss_g.memo) & set(loss_o.x)
    assert len(common) >= n
    for p in common:
        assert abs(loss_g.memo[p] - loss_o(p)) <= tol(p), (p, loss_g.memo[p], loss_o(p), tol(p))
    # the paths agree step by step, or part only at a tie
    steps = 0
    for (pg, lg), (po, lo) in zip(path_g, path_o):
        if pg != po:
            assert pg in loss_o.x, "the GPU's choice was not a candidate of the oracle's step"
            assert loss_o(pg) - loss_o(po) <= tol(pg) + tol(po), (pg, po, loss_o(pg), loss_o(po))
            break
        steps += 1
    print(f"[parity] greedy search: {steps} of {len(path_o)} steps identical; GPU path "
          + " -> ".join(f"{p}:{l:.4f}" for p, l in path_g), flush=True)
    assert path_g[-1][0].count("F") == 1 and path_g[0][0] == "F" * n
