"""Pin of the oracle's layer stack (oracle.stack) against the hand-worked
two-layer example in tests/golden/hand_stack_2layer.json.

The example follows the inference loop of itoverdose.com, "IndexCache: Wie
DeepSeek O(NL²)-Kosten in Sparse Attention um 75% reduziert", section "Einfache
Implementierung, enorme Effizienzgewinne".  With topk = 1 every attention
output is one latent row exactly, and every value is a small integer, so the
final X is known exactly for all four combinations of Full/Shared second layer
and plain/residual FFN.  A Shared layer that recomputed its own index set, an
FFN applied before the attention update, a dropped residual or a head sum
taken over the wrong axis each change some entry.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_stack_2layer.json")


def _g():
    with open(GOLDEN) as f:
        return json.load(f)


def _bf16_bits(a) -> np.ndarray:
    return torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _layers(g):
    L, H, D, Hq, Dqk = g["L"], g["H"], g["D"], g["Hq"], g["Dqk"]
    keys = np.array(g["keys"], np.float32)[None]                     # [1, L, D]
    q_i = np.zeros((1, L, H, D), np.float32)
    for h in range(H):
        q_i[0, :, h, :] = np.array(g["q_per_row"][h], np.float32)
    q_att = np.broadcast_to(np.array(g["attn_q_per_row_head"], np.float32), (1, L, Hq, Dqk)).copy()
    layers = []
    for l in range(2):
        w = np.broadcast_to(np.array(g["w_by_layer"][str(l)], np.float32), (1, L, H)).copy()
        layers.append(dict(q_i=q_i, k_i=keys, w=w, idx_dtypes=("fp32",) * 3,
                           q=_bf16_bits(q_att), kv=_bf16_bits(np.array(g["kv_by_layer"][str(l)])[None]),
                           W=_bf16_bits(g["W_by_layer"][str(l)])))
    return layers


@pytest.mark.parametrize("pattern", ["FS", "FF"])
@pytest.mark.parametrize("residual", [False, True])
def test_two_layer_stack_hand_example(pattern, residual):
    g = _g()
    x0 = _bf16_bits(g["X0"])
    xo, ts = oracle.stack(pattern, x0, _layers(g), g["topk"], 0.5, g["Dv"], residual_ffn=residual)
    key = f"{pattern}_{'residual' if residual else 'plain'}"
    assert oracle.bf16_bits_to_f64(xo).tolist() == g["expected"][key], key
    assert ts[0].reshape(g["L"], 1).tolist() == g["expected"]["T0"]
    want1 = g["expected"]["T0"] if pattern == "FS" else g["expected"]["T1"]
    assert ts[1].reshape(g["L"], 1).tolist() == want1


def test_shared_layer_result_differs_from_recomputing():
    """The example is built so that a Shared layer that ran its own indexer
    would land on the Full-layer answer instead: the two outcomes differ."""
    g = _g()
    for res in ("plain", "residual"):
        assert g["expected"][f"FS_{res}"] != g["expected"][f"FF_{res}"]
    assert g["expected"]["T0"] != g["expected"]["T1"]


def _rand_bits(g, shape, std=1.0):
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("residual", [False, True])
def test_row_subset_equals_full_stack(residual):
    """Per-layer inputs do not depend on X, so each row's path through the
    stack is independent of the others: computing a subset of rows gives
    exactly those rows of the full stack, for every layer's X and T."""
    g = torch.Generator().manual_seed(5)
    L, H, D, k, Hq, Dqk, Dv, Dm = 40, 4, 16, 6, 4, 24, 16, 24
    layers = []
    for _ in range(3):
        layers.append(dict(q_i=_rand_bits(g, (1, L, H, D)), k_i=_rand_bits(g, (1, L, D)),
                           w=torch.rand((1, L, H), generator=g).numpy(), idx_dtypes=("bf16", "bf16", "fp32"),
                           q=_rand_bits(g, (1, L, Hq, Dqk)), kv=_rand_bits(g, (1, L, Dqk)),
                           W=_rand_bits(g, (Dm, Dm), Dm ** -0.5)))
    x0 = _rand_bits(g, (L, Dm))
    xf, tf, xsf, osf = oracle.stack("FSF", x0, layers, k, Dqk ** -0.5, Dv, residual, per_layer=True)
    rows = np.array([31, 0, 7, 39, 12])
    sub = [dict(lay, q=np.ascontiguousarray(lay["q"][:, rows])) for lay in layers]
    xr, tr, xsr, osr = oracle.stack("FSF", np.ascontiguousarray(x0[rows]), sub, k, Dqk ** -0.5, Dv, residual,
                               rows=rows, per_layer=True)
    assert np.array_equal(xr, xf[rows])
    for a, b in zip(xsr, xsf):
        assert np.array_equal(a, b[rows])
    for a, b in zip(tr, tf):
        assert np.array_equal(a[0, rows], b[0, rows])
    for a, b in zip(osr, osf):
        assert np.array_equal(a, b[rows])
