"""GPU parity of the cross-layer overlap diagnostic against the oracle (exact counts)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_lightning_amd as sa
from sparse_attention_indexer_lightning_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def sorted_rows(rng, R, k, universe, fill):
    t = np.full((R, k), -1, np.int32)
    for r in range(R):
        n = int(fill[r])
        t[r, :n] = np.sort(rng.choice(universe, n, replace=False))
    return t


@pytest.mark.parametrize("R,k,universe", [(1, 1, 3), (37, 64, 200), (513, 2048, 5000), (9, 2048, 2100)])
def test_random_sets(R, k, universe):
    rng = np.random.default_rng(R * 31 + k)
    fill_a = rng.integers(0, k + 1, R)
    fill_a[0] = k
    a = sorted_rows(rng, R, k, universe, fill_a)
    b = sorted_rows(rng, R, k, universe, rng.integers(0, k + 1, R))
    ga = torch.from_numpy(a).to(DEV)
    gb = torch.from_numpy(b).to(DEV)
    got = sa.idx_overlap(ga, gb).cpu().numpy()
    assert np.array_equal(got, oracle.overlap(a, b))
    assert np.array_equal(sa.idx_overlap(ga, ga).cpu().numpy(), (a >= 0).sum(1))      # identical
    assert np.array_equal(sa.idx_overlap(gb, ga).cpu().numpy(), got)                 # symmetric


def test_index_sets_of_two_layers():
    """T of two Full layers of the small stack workload (seeded q/k/w per layer)."""
    wl = inputs.WORKLOADS["tiny_stack"]
    ts = []
    for layer in range(2):
        q, k, w = inputs.indexer_inputs(wl, layer, DEV)
        ts.append(sa.idx_score_topk(q, k, w, wl.topk))
    torch.cuda.synchronize()
    got = sa.idx_overlap(ts[0], ts[1]).cpu().numpy()
    want = oracle.overlap(ts[0].cpu().numpy(), ts[1].cpu().numpy())
    assert np.array_equal(got, want)
    m = sa.overlap_matrix(ts)
    assert abs(m[0, 0].item() - 1.0) < 1e-12 and abs(m[1, 1].item() - 1.0) < 1e-12
    valid = (ts[0] >= 0).sum(-1).clamp(min=1).double().cpu().numpy()
    assert abs(m[0, 1].item() - float((want / valid).mean())) < 1e-12
