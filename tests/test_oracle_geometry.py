"""Pins of the geometry guard oracle against the hand-built cases of
tests/golden/tree_geometry.txt (the classes named in lucebox PR #506,
Safety boundary)."""
import os

import numpy as np

from oracle import geometry as og


def load_cases(golden_dir):
    cases = []
    with open(os.path.join(golden_dir, "tree_geometry.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, arr, n, chain_v, tree_v = [c.strip() for c in line.split("|")]
            n = int(n)
            if arr == "NULL":
                parent = None
            elif arr == "-":
                parent = np.zeros(0, dtype=np.int32)
            elif arr.startswith("@chain"):
                parent = np.arange(-1, int(arr[6:]) - 1, dtype=np.int32)
            else:
                parent = np.array([int(x) for x in arr.split()], dtype=np.int32)
            cases.append((name, parent, n, chain_v, tree_v))
    return cases


def test_golden_geometry(golden_dir):
    names = {v: k for k, v in og.NAMES.items()}
    cases = load_cases(golden_dir)
    assert len(cases) >= 15
    for name, parent, n, chain_v, tree_v in cases:
        assert og.check_tree(parent, n, True) == names[chain_v], name
        assert og.check_tree(parent, n, False) == names[tree_v], name


def test_accepted_arrays_are_acyclic_trees():
    rng = np.random.default_rng(0)
    for _ in range(2000):
        T = int(rng.integers(1, 9))
        parent = rng.integers(-2, T + 1, T).astype(np.int32)
        if og.check_tree(parent, T, False) == og.OK:
            for i in range(T):
                seen, n = 0, i
                while n >= 0:
                    n = parent[n]
                    seen += 1
                    assert seen <= T
            assert parent[0] == -1 and np.sum(parent == -1) == 1
