"""A layer stack run through the library: the IndexCache inference loop of
itoverdose.com, "IndexCache: Wie DeepSeek O(NL²)-Kosten in Sparse Attention um
75% reduziert", section "Einfache Implementierung, enorme Effizienzgewinne":
per layer, a Full layer runs the indexer and top-k into the one index cache
and a Shared layer reuses it (``idx_cache_route``), sparse MLA attends over the
selected rows (``sparse_mla_attn``), then the FFN step.

No trained model exists here, so the stack follows the synthetic reading used
throughout this repository: every layer's indexer and attention inputs are
seeded tensors independent of X; X1 = bf16(X + pad(sum over heads of O)) and
X = bf16(X1 W) or bf16(X1 + X1 W) with a seeded bf16 W standing in for the FFN.
The indexer, router and attention run in the library's kernels; the head sum
and the FFN stand-in are torch operations (a GEMM on hipBLASLt), which are not
part of the path the library implements.

Used by the retention-ratio sweep of the benchmark (every pattern timed end to
end) and as the loss of the greedy Full/Shared search (``search.py``).
"""
from __future__ import annotations

import math

import torch

from . import idx_cache_route, idx_score_topk_workspace, sparse_mla_attn
from . import inputs as _inputs


def layer_inputs(wl, layer: int, device, need_indexer: bool = True) -> dict:
    """Seeded inputs of one layer of workload ``wl`` (indexer q, k, w only when
    ``need_indexer``; attention q and latent kv; FFN stand-in W)."""
    d = {}
    if need_indexer:
        d["q_i"], d["k_i"], d["w"] = _inputs.indexer_inputs(wl, layer, device)
    d["q"], d["kv"] = _inputs.attention_inputs(wl, layer, device)
    d["W"] = _inputs.ffn_weight(wl, layer, device)
    return d


def compose(x, o, W, residual: bool, fp32_ffn: bool):
    """FFN step of one layer after attention: X1 = bf16(X + pad(sum_h O)), then
    X = bf16(X1 W) or bf16(X1 + X1 W).  x bf16 [L, Dm], o bf16 [L, Hq, Dv],
    W bf16 [Dm, Dm].  The head sum and the X + pad(S) add run in fp32 with one
    rounding to bf16.  fp32_ffn: the product X1 W in fp32 with one rounding
    of the result (as the oracle rounds); otherwise a bf16 GEMM with fp32
    accumulation (hipBLASLt), the residual fused into its epilogue."""
    Dv = o.shape[-1]
    s = torch.zeros(x.shape, dtype=torch.float32, device=x.device)
    s[:, :Dv] = torch.sum(o, dim=1, dtype=torch.float32)
    x1 = (x.float() + s).to(torch.bfloat16)
    del s
    if fp32_ffn:
        x1f = x1.float()
        y = x1f @ W.float()
        return ((x1f + y) if residual else y).to(torch.bfloat16)
    return torch.addmm(x1, x1, W) if residual else x1 @ W


class Stack:
    """A stack of len(pattern) layers over one workload's shapes.

    ``layers[l]`` holds layer l's input tensors (``layer_inputs``); the same
    dict may serve several layers (rotating input sets).  ``run(pattern)``
    runs the stack from ``x0`` and returns the final X; every layer routes
    through the one index cache ``t_cache``.
    """

    def __init__(self, wl, layers, x0, residual: bool, fp32_ffn: bool = False):
        self.wl = wl
        self.layers = layers
        self.x0 = x0
        self.residual = residual
        self.fp32_ffn = fp32_ffn
        dev = x0.device
        self.scale = 1.0 / math.sqrt(wl.Dqk)
        self.t_cache = torch.full((wl.B, wl.Lq, wl.topk), -1, dtype=torch.int32, device=dev)
        self.out = torch.empty(wl.B, wl.Lq, wl.Hq, wl.Dv, dtype=torch.bfloat16, device=dev)
        first = next(l for l in layers if "q_i" in l)
        n = idx_score_topk_workspace(first["q_i"], first["k_i"], first["w"], wl.topk)
        self.ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)

    def run(self, pattern: str, keep_layers: bool = False):
        """Final X (bf16 [L, Dm]) of the stack with the given F/S pattern; with
        ``keep_layers`` also the list of per-layer (T copy, O copy, X)."""
        if len(pattern) != len(self.layers):
            raise ValueError(f"pattern of {len(pattern)} layers for a stack of {len(self.layers)}")
        x = self.x0
        kept = []
        for l, lay in enumerate(self.layers):
            if pattern[l] == "F":
                idx_cache_route(pattern, l, lay["q_i"], lay["k_i"], lay["w"], self.t_cache, ws=self.ws)
            else:
                idx_cache_route(pattern, l, None, None, None, self.t_cache)
            sparse_mla_attn(lay["q"], lay["kv"], self.t_cache, self.scale, self.wl.Dv, out=self.out)
            x = compose(x, self.out[0], lay["W"], self.residual, self.fp32_ffn)
            if keep_layers:
                kept.append((self.t_cache.clone(), self.out[0].clone(), x))
        return (x, kept) if keep_layers else x


def relative_deviation(x, x_ref) -> float:
    """||X - X_ref|| / ||X_ref|| (Frobenius, in float64): how far a pattern's
    final X lies from the all-Full stack's, the loss of the greedy search."""
    a = x.double()
    b = x_ref.double()
    return float(torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b))
