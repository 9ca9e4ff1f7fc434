"""Pins of the acceptance oracle: numpy.argmax, hand-built NaN/inf/-0 rows,
brute-force root-path enumeration and hand-worked golden cases."""
import os

import numpy as np
import pytest

from oracle import accept as oa
from synth import (TINY_CHAIN, QWEN_STACK_TREE, QWEN_STACK_CHAIN, gen_accept, scaled, bf16_bits)


def test_argmax_matches_numpy_without_nan():
    rng = np.random.default_rng(5)
    for _ in range(50):
        row = rng.integers(-4, 5, 300).astype(np.float32)   # many ties
        assert oa.argmax_row(row) == int(np.argmax(row))
        assert oa.argmax_row_fast(row) == int(np.argmax(row))
    rows = bf16_bits(rng.standard_normal((7, 1000)).astype(np.float32))
    f = (rows.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(oa.argmax_rows(rows), np.argmax(f, axis=1))


@pytest.mark.parametrize("row,exp", [
    ([np.nan, 1.0, np.nan], 1),
    ([np.nan, np.nan], 0),
    ([-np.inf, np.nan], 0),
    ([np.nan, -np.inf], 1),
    ([-0.0, 0.0], 0),
    ([0.0, -0.0], 0),
    ([1.0, np.inf, np.inf], 1),
    ([np.nan, -np.inf, -np.inf, np.nan], 1),
    ([-3.0, -2.0, np.nan, -2.0], 1),
])
def test_argmax_special_values(row, exp):
    r32 = np.array(row, dtype=np.float32)
    assert oa.argmax_row(r32) == exp
    assert oa.argmax_row_fast(r32) == exp
    assert oa.argmax_row(bf16_bits(r32) if not np.isnan(r32).any() else r32) == exp


def _parse_ints(s):
    return np.array([int(x) for x in s.split()], dtype=np.int32)


def test_golden_cases(golden_dir):
    n = 0
    with open(os.path.join(golden_dir, "accept_cases.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, par, tok, am, node, ln, path, bonus = [c.strip() for c in line.split("|")]
            parent, tokens, argmax = _parse_ints(par), _parse_ints(tok), _parse_ints(am)
            r = oa.accept(argmax, tokens, parent)
            exp_path = _parse_ints(path)
            assert r.accept_node == int(node), name
            assert r.accept_len == int(ln), name
            assert np.array_equal(r.path[:len(exp_path)], exp_path) and np.all(r.path[len(exp_path):] == -1), name
            assert r.bonus == int(bonus), name
            rb = oa.brute_force_accept(argmax, tokens, parent)
            assert (rb.accept_node, rb.accept_len, rb.bonus) == (r.accept_node, r.accept_len, r.bonus), name
            n += 1
    assert n >= 8


def _random_tree(rng, T):
    parent = np.full(T, -1, dtype=np.int32)
    for i in range(1, T):
        parent[i] = rng.integers(0, i)
    return parent


def test_walk_equals_brute_force_random():
    rng = np.random.default_rng(9)
    for trial in range(400):
        T = int(rng.integers(1, 12))
        parent = _random_tree(rng, T) if trial % 2 else np.arange(-1, T - 1, dtype=np.int32)
        tokens = rng.integers(0, 3, T).astype(np.int32)
        argmax = rng.integers(0, 3, T).astype(np.int32)
        r = oa.accept(argmax, tokens, parent)
        rb = oa.brute_force_accept(argmax, tokens, parent)
        assert r.accept_node == rb.accept_node and r.accept_len == rb.accept_len
        assert np.array_equal(r.path, rb.path) and r.bonus == rb.bonus


def test_chain_accept_counts_leading_matches():
    rng = np.random.default_rng(10)
    for _ in range(200):
        T = int(rng.integers(1, 18))
        tokens = rng.integers(0, 2, T).astype(np.int32)
        argmax = rng.integers(0, 2, T).astype(np.int32)
        j = 0
        while j + 1 < T and tokens[j + 1] == argmax[j]:
            j += 1
        r = oa.accept(argmax, tokens)
        assert r.accept_node == j and r.accept_len == j and r.bonus == argmax[j]
        assert np.array_equal(r.path[:j + 1], np.arange(j + 1))


@pytest.mark.parametrize("wl", [TINY_CHAIN, scaled(QWEN_STACK_TREE, vocab=4096), scaled(QWEN_STACK_CHAIN, vocab=4096)])
def test_generator_plant_is_recovered(wl):
    """The generator plants a unique maximum and a target node; the oracle's
    argmax and acceptance recover exactly what was planted."""
    for req in range(6):
        ai = gen_accept(wl, req)
        am = oa.argmax_rows(ai.logits)
        assert np.array_equal(am, ai.planted_argmax)
        r = oa.accept(am, ai.tokens, ai.parent)
        assert r.accept_node == ai.planted_node
        # the planted maximum is unique in each row
        rows = ai.logits
        f = (rows.astype(np.uint32) << 16).view(np.float32) if rows.dtype == np.uint16 else rows
        for t in range(f.shape[0]):
            assert np.sum(f[t] == f[t].max()) == 1
        if wl.logits_distinct:
            for t in range(f.shape[0]):
                assert np.unique(f[t]).size == f.shape[1]


def test_generator_tree_constraints():
    """Draft trees of the tree workload: root first, parents before children,
    depth at most 8, at most 3 children per node, sibling tokens distinct."""
    from synth import gen_tree_parent
    w = scaled(QWEN_STACK_TREE, vocab=4096)
    for req in range(20):
        par = gen_tree_parent(w, req)
        assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, w.n_pos))
        depth = np.zeros(w.n_pos, dtype=int)
        for i in range(1, w.n_pos):
            depth[i] = depth[par[i]] + 1
        assert depth.max() <= w.tree_max_depth
        kids = np.bincount(par[1:], minlength=w.n_pos)
        assert kids.max() <= w.tree_max_children
        ai = gen_accept(w, req, with_logits=False)
        for p in range(w.n_pos):
            sib = ai.tokens[1:][par[1:] == p]
            assert len(set(sib.tolist())) == len(sib)
