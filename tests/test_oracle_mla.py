"""Pins for the oracle's sparse MLA attention and layer stack.

  * dense equivalence: when the index set holds every causal key, sparse MLA is
    ordinary causal softmax attention, which torch's scaled_dot_product_attention
    computes on the CPU in float64;
  * closed forms: q = 0 gives the mean of the selected value rows; a single
    index returns that row; permuting the index set changes nothing; one
    dominant logit returns (nearly) that row; -1 entries are skipped.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _bf16(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f64(bits: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_f64(bits)


def _bf16_ulp_close(a, b, ulps=1.0):
    """|a-b| within `ulps` bf16 units of the larger magnitude (one rounding each)."""
    scale = np.maximum(np.abs(a), np.abs(b))
    return np.all(np.abs(a - b) <= ulps * scale * 2.0 ** -8 + 1e-30)


@pytest.mark.parametrize("Dqk,Dv,Hq", [(32, 32, 4), (64, 48, 3)])
def test_dense_equivalence_with_sdpa(Dqk, Dv, Hq):
    g = torch.Generator().manual_seed(1)
    B, L = 2, 21
    q = torch.randn(B, L, Hq, Dqk, generator=g)
    kv = torch.randn(B, L, Dqk, generator=g)
    qb, kvb = _bf16(q), _bf16(kv)
    k = 32  # >= every p+1, so the index set is all causal keys, -1 padded
    t = np.full((B, L, k), -1, np.int32)
    for i in range(L):
        t[:, i, : i + 1] = np.arange(i + 1)
    scale = 1.0 / math.sqrt(Dqk)
    out, lse = oracle.sparse_mla_dv(qb, kvb, t, scale, Dv)
    qd = torch.from_numpy(_f64(qb)).permute(0, 2, 1, 3)           # B,H,L,D
    kd = torch.from_numpy(_f64(kvb))[:, None].expand(B, Hq, L, Dqk)
    vd = kd[..., :Dv]
    ref = F.scaled_dot_product_attention(qd, kd, vd, is_causal=True, scale=scale)
    ref = ref.permute(0, 2, 1, 3).reshape(B * L, Hq, Dv).numpy()
    assert _bf16_ulp_close(_f64(out), ref, 1.0)
    logits = torch.einsum("bhld,bhsd->bhls", qd, kd) * scale
    mask = torch.ones(L, L, dtype=torch.bool).tril()
    ref_lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)
    ref_lse = ref_lse.permute(0, 2, 1).reshape(B * L, Hq).numpy()
    assert np.allclose(lse, ref_lse, rtol=1e-6, atol=1e-6)


def test_closed_forms():
    g = torch.Generator().manual_seed(2)
    B, Lq, Lk, Hq, D, k = 1, 3, 50, 2, 32, 8
    kv = _bf16(torch.randn(B, Lk, D, generator=g))
    kvd = _f64(kv)[0]
    t = np.array([[[5, 9, 13, 40, 41, 2, 7, 30],
                   [11, -1, -1, -1, -1, -1, -1, -1],
                   [3, 4, -1, 8, -1, 20, -1, -1]]], np.int32)
    # q = 0: uniform weights -> mean of the selected value rows
    q0 = _bf16(torch.zeros(B, Lq, Hq, D))
    out, lse = oracle.sparse_mla(q0, kv, t, 0.125)
    o = _f64(out)
    for i in range(Lq):
        sel = [j for j in t[0, i] if j >= 0]
        assert _bf16_ulp_close(o[i, 0], kvd[sel].mean(axis=0), 1.0)
        assert np.allclose(lse[i], math.log(len(sel)))
    # single valid index: the output is that row, exactly
    q = _bf16(torch.randn(B, Lq, Hq, D, generator=g))
    out, lse = oracle.sparse_mla(q, kv, t, 0.125)
    assert np.array_equal(_f64(out)[1, 1], kvd[11])
    # permutation of the index set (and moving the -1 holes) changes nothing
    tp = t.copy()
    tp[0, 0] = t[0, 0][::-1]
    tp[0, 2] = np.array([-1, 20, -1, 8, 4, -1, 3, -1])
    out2, lse2 = oracle.sparse_mla(q, kv, tp, 0.125)
    assert np.array_equal(out, out2) or _bf16_ulp_close(_f64(out), _f64(out2), 1.0)
    assert np.allclose(lse, lse2, rtol=1e-6)
    # one dominant logit: the output collapses onto that row (max-subtraction keeps it finite)
    qd = np.zeros((B, Lq, Hq, D))
    qd[0, 0, 0] = kvd[40] * 400.0
    out3, lse3 = oracle.sparse_mla(_bf16(torch.from_numpy(qd)), kv, t, 1.0)
    assert np.all(np.isfinite(lse3))
    assert _bf16_ulp_close(_f64(out3)[0, 0], kvd[40], 1.0)


def test_empty_index_set_yields_zero():
    kv = _bf16(torch.ones(1, 4, 32))
    q = _bf16(torch.ones(1, 1, 2, 32))
    t = np.full((1, 1, 3), -1, np.int32)
    out, lse = oracle.sparse_mla(q, kv, t, 1.0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_stack_shared_layers_reuse_last_full():
    """Invariant of the stack: every Shared layer's T is the last Full layer's T."""
    rng = np.random.default_rng(0)
    L, H, D, k, Dm = 24, 2, 4, 5, 4
    layers = []
    for _ in range(5):
        layers.append(dict(
            q_i=rng.standard_normal((1, L, H, D)).astype(np.float32),
            k_i=rng.standard_normal((1, L, D)).astype(np.float32),
            w=rng.random((1, L, H)).astype(np.float32), idx_dtypes=("fp32",) * 3,
            q=_bf16(torch.from_numpy(rng.standard_normal((1, L, 2, Dm)))),
            kv=_bf16(torch.from_numpy(rng.standard_normal((1, L, Dm)))),
            W=_bf16(torch.from_numpy(rng.standard_normal((Dm, Dm)) / 2))))
    x0 = _bf16(torch.from_numpy(rng.standard_normal((L, Dm))))
    x, ts = oracle.stack("FSSFS", x0, layers, k, 0.5, Dm, residual_ffn=True)
    assert np.array_equal(ts[0], ts[1]) and np.array_equal(ts[1], ts[2])
    assert np.array_equal(ts[3], ts[4]) and not np.array_equal(ts[0], ts[3])
    # a stale T on a Shared layer would change the result
    x2, _ = oracle.stack("FSSSS", x0, layers, k, 0.5, Dm, residual_ffn=True)
    assert not np.array_equal(x, x2)
