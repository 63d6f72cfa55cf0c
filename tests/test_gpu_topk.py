"""GPU parity of the standalone row top-k: bit-exact against the oracle on the
same fp32 score matrix (ties, -0, short rows, long rows)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_lightning_amd as sa

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(scores: np.ndarray, pos, k):
    s = torch.from_numpy(np.ascontiguousarray(scores, dtype=np.float32)).to(DEV)
    p = None if pos is None else torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int32)).to(DEV)
    t = sa.idx_topk(s, k, row_pos=p)
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("R,Lk,k", [(64, 3000, 100), (16, 257, 256), (33, 5000, 2048), (5, 1, 1)])
def test_small_integer_scores_with_ties(R, Lk, k):
    rng = np.random.default_rng(R * 7 + Lk)
    s = rng.integers(-5, 6, (R, Lk)).astype(np.float32)
    s[s == 0] = np.where(rng.random((s == 0).sum()) < 0.5, -0.0, 0.0)
    pos = rng.integers(-1, Lk, R).astype(np.int32)
    pos[0] = Lk - 1
    assert np.array_equal(run(s, pos, k), oracle.topk(s, pos, k))
    assert np.array_equal(run(s, None, k), oracle.topk(s, None, k))


def test_gaussian_rows_long():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((4, 200000)).astype(np.float32)
    s[:, ::1000] = 3.5  # plateau of equal scores near the top
    pos = np.array([199999, 150000, 2047, 100], np.int32)
    assert np.array_equal(run(s, pos, 2048), oracle.topk(s, pos, 2048))


def test_extreme_values():
    s = np.array([[np.inf, -np.inf, 3.4e38, -3.4e38, 1e-45, -1e-45, 0.0, -0.0, 1.0, 2.0] * 30], np.float32)
    for k in (1, 5, 37, 299, 300):
        assert np.array_equal(run(s, None, k), oracle.topk(s, None, k))


def test_all_equal_rows():
    for v in (0.0, -0.0, 1.5, -2.0):
        s = np.full((3, 4097), v, np.float32)
        t = run(s, None, 2048)
        assert np.array_equal(t, np.tile(np.arange(2048, dtype=np.int32), (3, 1)))


@pytest.mark.parametrize("R,Lk", [(1, 65536), (2, 70001)])
def test_all_equal_rows_split_path(R, Lk):
    """All-equal long rows take the split path with every key a candidate (more
    than the LDS capacity: the HBM select runs); ties go to the lower index."""
    for v in (0.0, 1.5):
        s = np.full((R, Lk), v, np.float32)
        if v == 0.0:
            s[:, 1::2] = -0.0                     # -0 and +0 are equal keys
        t = run(s, None, 2048)
        assert np.array_equal(t, np.tile(np.arange(2048, dtype=np.int32), (R, 1)))
        pos = np.full(R, Lk - 3, np.int32)
        assert np.array_equal(run(s, pos, 2048), oracle.topk(s, pos, 2048))


@pytest.mark.parametrize("R,Lk", [(32, 200000), (3, 70001), (100, 16384), (1, 1000000)])
def test_split_rows(R, Lk):
    """Few long rows: the split path (bounds per split, candidate collection, per-row select)."""
    rng = np.random.default_rng(R + Lk)
    s = rng.standard_normal((R, Lk)).astype(np.float32)
    s[:, 5::997] = np.float32(2.75)          # ties near the cut
    s[0, : Lk // 2] = np.float32(-1.0)        # one row whose top-k sits in its second half
    pos = rng.integers(0, Lk, R).astype(np.int32)
    pos[0] = Lk - 1
    pos[-1] = 4096 * 3 + 17                   # ends inside a split
    assert np.array_equal(run(s, pos, 2048), oracle.topk(s, pos, 2048))
    assert np.array_equal(run(s, None, 2048), oracle.topk(s, None, 2048))
    assert np.array_equal(run(s, None, 64), oracle.topk(s, None, 64))


def test_split_rows_increasing():
    """Sorted rows: every split's bound is loose; candidates exceed LDS and the HBM fallback runs."""
    s = np.tile(np.arange(100000, dtype=np.float32), (4, 1))
    s[1] = s[1][::-1]
    assert np.array_equal(run(s, None, 2048), oracle.topk(s, None, 2048))
