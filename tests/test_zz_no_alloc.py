"""The allocation-free entry point idx_score_topk_noalloc against idx_score_topk
(workspace passed in), through the C ABI: T must be identical, on two calls in
a row with the second smaller than the first (the static scratch keeps the
first call's contents), on a prefill-shaped call that needs no scratch, and
the size limit is enforced."""
import pytest
import torch

import sparse_attention_indexer_lightning_amd as sa
from sparse_attention_indexer_lightning_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _decode_inputs(B, Lk, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = (torch.randn(B, 1, 64, 128, generator=g, device=DEV) / 128 ** 0.5).to(torch.float8_e4m3fn)
    k = (torch.randn(B, Lk, 128, generator=g, device=DEV) / 128 ** 0.5).to(torch.float8_e4m3fn)
    w = (torch.randn(B, 1, 64, generator=g, device=DEV) * 0.1).to(torch.bfloat16)
    return q, k, w


def _both(q, k, w, topk):
    t_ref = sa.idx_score_topk(q, k, w, topk)
    t = torch.full_like(t_ref, -7)
    sa.idx_score_topk_noalloc(q, k, w, topk, t)
    torch.cuda.synchronize()
    return t, t_ref


def test_decode_calls_large_then_small():
    wl = inputs.WORKLOADS["decode_200k"]
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)          # 32 x 200,000 keys: ~77 MB of scratch
    t, t_ref = _both(q, k, w, wl.topk)
    assert torch.equal(t, t_ref)
    del q, k, w
    q, k, w = _decode_inputs(4, 30000, seed=5)          # smaller, over the first call's leftovers
    t, t_ref = _both(q, k, w, 2048)
    assert torch.equal(t, t_ref)
    q, k, w = _decode_inputs(3, 1500, seed=6)           # rows shorter than k: all keys, -1 padding
    t, t_ref = _both(q, k, w, 2048)
    assert torch.equal(t, t_ref)


def test_prefill_shaped_call_needs_no_scratch():
    wl = inputs.WORKLOADS["prefill_8k"]
    q, k, w = inputs.indexer_inputs(wl, 0, DEV)
    t, t_ref = _both(q, k, w, wl.topk)
    assert torch.equal(t, t_ref)


def test_request_beyond_the_scratch_is_rejected():
    q, k, w = _decode_inputs(64, 1, seed=7)
    big_k = torch.empty(64, 600000, 128, dtype=torch.float8_e4m3fn, device=DEV)   # 64 x 600,000 fp32 scores > 128 MiB
    t = torch.empty(64, 1, 2048, dtype=torch.int32, device=DEV)
    with pytest.raises(sa.IdxcError) as e:
        sa.idx_score_topk_noalloc(q, big_k, w, 2048, t)
    assert e.value.status == -9
