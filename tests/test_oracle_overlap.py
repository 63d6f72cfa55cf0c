"""Pins of the oracle's cross-layer overlap (a set intersection written out)."""
import numpy as np

import oracle


def test_hand_worked_rows():
    a = np.array([[0, 3, 5, 9, -1, -1],
                  [1, 2, 3, 4, 5, 6],
                  [-1, -1, -1, -1, -1, -1]], np.int32)
    b = np.array([[3, 4, 5, 8, 9, -1],
                  [7, 8, 9, 10, 11, 12],
                  [0, 1, 2, -1, -1, -1]], np.int32)
    # row 0: {0,3,5,9} & {3,4,5,8,9} = {3,5,9}; row 1: disjoint; row 2: a is empty
    assert oracle.overlap(a, b).tolist() == [3, 0, 0]


def test_identical_nested_and_symmetric():
    rng = np.random.default_rng(0)
    for _ in range(20):
        k = int(rng.integers(1, 64))
        n = int(rng.integers(0, k + 1))
        a = np.full((1, k), -1, np.int32)
        a[0, :n] = np.sort(rng.choice(1000, n, replace=False))
        assert oracle.overlap(a, a)[0] == n                      # identical sets
        m = int(rng.integers(0, n + 1))
        b = np.full((1, k), -1, np.int32)
        b[0, :m] = np.sort(rng.choice(a[0, :n], m, replace=False)) if m else []
        assert oracle.overlap(a, b)[0] == m                      # b nested in a
        c = np.full((1, k), -1, np.int32)
        c[0, :n] = a[0, :n] + 1000                                # shifted: disjoint
        assert oracle.overlap(a, c)[0] == 0
        d = np.full((1, k), -1, np.int32)
        j = int(rng.integers(0, k + 1))
        d[0, :j] = np.sort(rng.choice(1200, j, replace=False))
        assert oracle.overlap(a, d)[0] == oracle.overlap(d, a)[0]  # symmetric
