"""GPU parity of sparse MLA attention against the oracle (max-abs <= 2e-2 on the
bf16 output, log-sum-exp within 1e-3)."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_lightning_amd as sa
from parity_util import raw

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ATOL = 2e-2


def _bf16_np(x: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits_to_f64(raw(x))


def run_and_compare(B, Lq, Lk, Hq, Dqk, Dv, k, t_kind="random", seed=0, rope_growth=0.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn(B, Lq, Hq, Dqk, generator=g, device=DEV).to(torch.bfloat16)
    kv = torch.randn(B, Lk, Dqk, generator=g, device=DEV)
    if rope_growth:
        # the key-only columns of row s scaled by 1 + rope_growth * s / Lk: with
        # T in ascending order the logits keep growing along the index set.  The
        # softmax then rests on a few rows, so the output is about one value row:
        # values are scaled by 1/4 to keep it below about 1.5, where one bf16 ulp
        # (2^-7 at most) stays below the 2e-2 max-abs bound
        kv[:, :, Dv:] *= 1.0 + rope_growth * torch.arange(Lk, device=DEV, dtype=torch.float32)[None, :, None] / Lk
        kv[:, :, :Dv] *= 0.25
    kv = kv.to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    t = np.full((B, Lq, k), -1, np.int32)
    for b in range(B):
        for i in range(Lq):
            if t_kind == "random":
                n = int(rng.integers(0, min(k, Lk) + 1))
                t[b, i, :n] = rng.choice(Lk, size=n, replace=False)
                rng.shuffle(t[b, i])
            elif t_kind == "full":
                n = min(k, Lk)
                t[b, i, :n] = rng.choice(Lk, size=n, replace=False)
            elif t_kind == "sorted":
                n = min(k, Lk)
                t[b, i, :n] = np.sort(rng.choice(Lk, size=n, replace=False))
            elif t_kind == "dup":
                t[b, i] = rng.integers(0, min(Lk, k // 4 + 1), size=k)
            elif t_kind == "beyond":
                # valid rows mixed with indices at or past Lk, which select nothing
                n = min(k, Lk) // 2
                t[b, i, :n] = rng.choice(Lk, size=n, replace=False)
                t[b, i, n:] = rng.choice([Lk, Lk + 1, Lk + 4093, 1 << 30, 2 ** 31 - 1], size=k - n)
                rng.shuffle(t[b, i])
    tt = torch.from_numpy(t).to(DEV)
    t = np.where(t >= Lk, -1, t)    # the oracle's form of the same index set
    scale = 1.0 / math.sqrt(Dqk)
    lse = torch.empty(B, Lq, Hq, dtype=torch.float32, device=DEV)
    out, _ = sa.sparse_mla_attn(q, kv, tt, scale, Dv, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_mla_dv(raw(q), raw(kv), t, scale, Dv)
    go = _bf16_np(out).reshape(ro.shape)
    err = np.abs(go - oracle.bf16_bits_to_f64(ro)).max()
    assert err <= ATOL, f"max-abs error {err}"
    gl = lse.cpu().numpy().reshape(rl.shape)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert np.allclose(gl[fin], rl[fin], rtol=1e-4, atol=1e-3)
    return err


@pytest.mark.parametrize("Hq", [4, 8, 20])
def test_small_latent(Hq):
    run_and_compare(2, 33, 400, Hq, 32, 32, 64)


@pytest.mark.parametrize("Hq,k", [(16, 64), (128, 200), (32, 2048)])
def test_mla_latent(Hq, k):
    run_and_compare(1, 3, 3000, Hq, 576, 512, k, seed=Hq)


def test_mla_full_index_sets():
    run_and_compare(2, 2, 5000, 128, 576, 512, 2048, t_kind="full", seed=3)


def test_empty_index_set():
    run_and_compare(1, 2, 100, 16, 576, 512, 64, t_kind="empty")


# Shapes served by the 64-heads-per-workgroup kernel (Hq a multiple of 64):
# few queries split each index set into chunks merged by a second kernel,
# many queries run one workgroup per (query, 64 heads).
@pytest.mark.parametrize("B,Lq,Hq,k", [
    (1, 3, 64, 2048),     # 16 chunks of 128 rows
    (1, 3, 64, 1000),     # 8 chunks, the last one ragged
    (1, 1, 192, 300),     # three head blocks, ragged tiles
    (2, 1, 128, 37),      # one partial tile
    (2, 128, 64, 96),     # one chunk per query, 256 workgroups
])
def test_mla_wide(B, Lq, Hq, k):
    run_and_compare(B, Lq, 4000, Hq, 576, 512, k, seed=B * 1000 + Lq + Hq + k)


def test_mla_wide_full_index_sets():
    run_and_compare(1, 2, 2100, 64, 576, 512, 2048, t_kind="full", seed=11)


def test_mla_wide_repeated_indices():
    # each occurrence of an index is one more term of the softmax
    run_and_compare(1, 2, 3000, 64, 576, 512, 512, t_kind="dup", seed=12)


@pytest.mark.parametrize("B,Lq,k", [
    (1, 2, 2048),     # decode shape: 16 chunks per (query, 64 heads) and the merge
    (1, 300, 1024),   # one chunk per query, 32 tiles in one workgroup
])
def test_mla_wide_growing_logits(B, Lq, k):
    """Logits that keep growing along the (ascending) index set: the softmax
    reference is raised many times in the middle of a sweep (each raise by more
    than 2^8), so the rescale of the accumulated output and row sums runs
    repeatedly."""
    run_and_compare(B, Lq, 4000, 64, 576, 512, k, t_kind="sorted", seed=21 + Lq, rope_growth=200.0)


def test_mla_wide_empty_index_set():
    run_and_compare(2, 2, 100, 64, 576, 512, 256, t_kind="empty")


@pytest.mark.parametrize("B,Lq,Hq,Dqk,Dv,k", [
    (2, 5, 8, 32, 32, 64),        # small latent kernel
    (1, 3, 16, 576, 512, 200),    # 16-head latent kernel
    (1, 3, 64, 576, 512, 1000),   # 64-head kernel, chunked + merge
    (2, 40, 128, 576, 512, 96),   # 64-head kernel, one chunk per query
])
def test_indices_at_or_beyond_lk_are_skipped(B, Lq, Hq, Dqk, Dv, k):
    run_and_compare(B, Lq, 700, Hq, Dqk, Dv, k, t_kind="beyond", seed=Hq + k)
