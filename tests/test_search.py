"""Host tests of the greedy Full/Shared search driver."""
import itertools

import pytest

from sparse_attention_indexer_lightning_amd.search import greedy_pattern


def test_additive_loss_matches_brute_force():
    """With a loss that adds a fixed cost per Shared layer, greedy removal is
    optimal: every prefix of the path is the cheapest pattern of its size."""
    cost = [0.0, 5.0, 1.0, 3.0, 0.5, 4.0, 2.0, 6.0]
    n = len(cost)

    def loss(p):
        return sum(c for c, x in zip(cost, p) if x == "S")

    path = greedy_pattern(n, loss, n_full=1)
    assert path[0][0] == "F" * n and path[-1][0] == "F" + "S" * (n - 1)
    for pat, val in path:
        nf = pat.count("F")
        best = min(loss("".join("F" if (i == 0 or i in keep) else "S" for i in range(n)))
                   for keep in itertools.combinations(range(1, n), nf - 1))
        assert val == pytest.approx(best)
    # order of conversion follows the costs
    order = [next(i for i in range(n) if a[i] != b[i]) for (a, _), (b, _) in zip(path, path[1:])]
    assert order == sorted(range(1, n), key=lambda i: cost[i])


def test_evaluation_count_and_layer0_fixed():
    calls = []

    def loss(p):
        calls.append(p)
        assert p[0] == "F"
        return float(len(p) - p.count("F")) ** 1.5 + 0.01 * p.find("S")

    n = 10
    path = greedy_pattern(n, loss, n_full=3)
    assert path[-1][0].count("F") == 3
    # 1 + sum over steps of the remaining candidates
    assert len(calls) == 1 + sum(range(n - 1, 2, -1))
    assert all(b[1] >= a[1] for a, b in zip(path, path[1:]))   # this loss grows with each conversion


def test_argument_checks():
    with pytest.raises(ValueError):
        greedy_pattern(0, lambda p: 0.0)
    with pytest.raises(ValueError):
        greedy_pattern(4, lambda p: 0.0, n_full=0)
    assert greedy_pattern(1, lambda p: 1.0) == [("F", 1.0)]
