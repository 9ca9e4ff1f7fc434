"""Pins of the GDN oracle against facts that do not come from the oracle itself.

Each test would fail on a plausible slip in oracle/gdn.py: a dropped decay on
the erase term, a sign error, S k versus k^T S (transposed operand), the
wrong key-head grouping, a wrong parent index, or a missing per-position
float32 rounding.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import gdn as og
from synth import F32, BF16, gen_unit, scaled, TINY_CHAIN, QWEN_LAYER_CHAIN, gen_tree_parent

RNG = np.random.default_rng(1234)


def rel_err(g, o):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    return np.max(np.abs(g - o)) / max(np.max(np.abs(o)), 2.0 ** -126)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_inputs(T, Hk, Hv, dk, dv, rng=RNG):
    q = _unit(rng.standard_normal((T, Hk, dk))).astype(np.float32)
    k = _unit(rng.standard_normal((T, Hk, dk))).astype(np.float32)
    v = rng.standard_normal((T, Hv, dv)).astype(np.float32)
    a = rng.uniform(0.05, 0.95, (T, Hv)).astype(np.float32)
    b = rng.uniform(0.05, 0.95, (T, Hv)).astype(np.float32)
    s = (rng.standard_normal((Hv, dv, dk)) * 0.02).astype(np.float32)
    return q, k, v, a, b, s


def test_hand_worked_golden(golden_dir):
    """Values worked by hand in tests/golden/gdn_hand_worked.json match bit-exactly."""
    with open(os.path.join(golden_dir, "gdn_hand_worked.json")) as f:
        data = json.load(f)
    for case in data["cases"]:
        S = np.array(case["S0"], dtype=np.float32)[None]
        for st in case["steps"]:
            q = np.array(st["q"], dtype=np.float32)[None]
            k = np.array(st["k"], dtype=np.float32)[None]
            v = np.array(st["v"], dtype=np.float32)[None]
            a = np.array([st["a"]], dtype=np.float32)
            b = np.array([st["b"]], dtype=np.float32)
            S, o = og.gdn_position(S, q, k, v, a, b)
            assert np.array_equal(S[0], np.array(st["S"], dtype=np.float32)), case["name"]
            assert np.array_equal(o[0], np.array(st["o"], dtype=np.float32)), case["name"]


def test_single_step_dense_closed_form():
    """T=1: S1 = a S0 (I - b k k^T) + b v k^T with dense matrix products."""
    dk = dv = 16
    q, k, v, a, b, s = _rand_inputs(1, 2, 4, dk, dv)
    ckpt, out = og.gdn_span(s, q, k, v, a, b)
    I = np.eye(dk)
    for h in range(4):
        g = h // 2
        kk = k[0, g].astype(np.float64)[:, None]
        S1 = a[0, h] * s[h].astype(np.float64) @ (I - b[0, h] * kk @ kk.T) \
            + b[0, h] * v[0, h].astype(np.float64)[:, None] @ kk.T
        assert rel_err(ckpt[0, h], S1) < 2e-7
        o = S1 @ q[0, g].astype(np.float64)
        assert rel_err(out[0, h], o) < 2e-6


def test_two_step_composition_dense():
    """K=1 (T=2): the two-fold composition of the dense step, rounding the
    state to float32 between the positions (the checkpoint precision)."""
    dk = dv = 8
    q, k, v, a, b, s = _rand_inputs(2, 1, 1, dk, dv)
    ckpt, out = og.gdn_span(s, q, k, v, a, b)
    I = np.eye(dk)
    S = s[0].astype(np.float64)
    for t in range(2):
        kk = k[t, 0].astype(np.float64)[:, None]
        S = a[t, 0] * S @ (I - b[t, 0] * kk @ kk.T) + b[t, 0] * v[t, 0].astype(np.float64)[:, None] @ kk.T
        S = S.astype(np.float32).astype(np.float64)
        assert rel_err(ckpt[t, 0], S) < 2e-7


def test_identity_gate_leaves_state():
    """a=1, b=0: every checkpoint equals the initial state and o_t = S0 q_t."""
    q, k, v, a, b, s = _rand_inputs(5, 2, 4, 8, 8)
    a[:] = 1.0
    b[:] = 0.0
    ckpt, out = og.gdn_span(s, q, k, v, a, b)
    for t in range(5):
        assert np.array_equal(ckpt[t], s)
        for h in range(4):
            np.testing.assert_allclose(out[t, h], s[h].astype(np.float64) @ q[t, h // 2], rtol=1e-6, atol=1e-9)


def test_zero_decay_writes_outer_product():
    q, k, v, a, b, s = _rand_inputs(3, 1, 2, 8, 8)
    a[:] = 0.0
    ckpt, _ = og.gdn_span(s, q, k, v, a, b)
    for t in range(3):
        for h in range(2):
            exp = b[t, h] * np.outer(v[t, h].astype(np.float64), k[t, 0].astype(np.float64))
            assert rel_err(ckpt[t, h], exp) < 2e-7


def test_delta_rule_write_unit_key():
    """Unit k (exactly: 0.6, 0.8), a=b=1: S_t k_t = v_t (the stored value)."""
    dk = dv = 6
    q, k, v, a, b, s = _rand_inputs(2, 1, 1, dk, dv)
    k[:] = 0.0
    k[0, 0, 0], k[0, 0, 1] = 0.6, 0.8
    k[1, 0, 2], k[1, 0, 5] = 0.8, -0.6
    a[:] = 1.0
    b[:] = 1.0
    ckpt, _ = og.gdn_span(s, q, k, v, a, b)
    for t in range(2):
        got = ckpt[t, 0].astype(np.float64) @ k[t, 0].astype(np.float64)
        np.testing.assert_allclose(got, v[t, 0], rtol=0, atol=1e-6)


def test_invariants_along_and_orthogonal_to_key():
    """S_t u = a S_{t-1} u for u orthogonal to k; along k:
    S_t k = a S_{t-1} k (1 - b k.k) + b v (k.k)."""
    dk = dv = 8
    q, k, v, a, b, s = _rand_inputs(1, 1, 1, dk, dv)
    k[:] = 0.0
    k[0, 0, :2] = [0.5, 0.25]            # not unit, exact
    ortho = np.zeros(dk)
    ortho[:2] = [-0.25, 0.5]
    ortho[5] = 1.0
    ckpt, _ = og.gdn_span(s, q, k, v, a, b)
    S0 = s[0].astype(np.float64)
    S1 = ckpt[0, 0].astype(np.float64)
    kk = k[0, 0].astype(np.float64)
    np.testing.assert_allclose(S1 @ ortho, a[0, 0] * (S0 @ ortho), rtol=1e-6, atol=1e-8)
    kk2 = kk @ kk
    np.testing.assert_allclose(S1 @ kk, a[0, 0] * (S0 @ kk) * (1 - b[0, 0] * kk2) + b[0, 0] * v[0, 0] * kk2,
                               rtol=1e-6, atol=1e-7)


def _f32_frac(x):
    return Fraction(float(np.float32(x)))


def _round_f32_exact(x: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32, ties to the even
    significand, deciding between the two neighbours with exact arithmetic
    (no intermediate float64 rounding)."""
    f = np.float32(float(x))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - x)
        key = (d, int(np.asarray(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


@pytest.mark.parametrize("d,T", [(2, 1), (2, 3), (3, 2), (3, 3)])
def test_exact_rational_brute_force(d, T):
    """Exact rationals with the literal product formula S (I - b k k^T) on
    dyadic inputs, rounding to float32 after each position as the checkpoint
    does; the oracle must agree bit-exactly."""
    rng = np.random.default_rng(d * 10 + T)
    dy = lambda *shape: (rng.integers(-8, 9, shape) / 8.0).astype(np.float32)
    q, k, v = dy(T, 1, d), dy(T, 1, d), dy(T, 1, d)
    a = (rng.integers(0, 5, (T, 1)) / 4.0).astype(np.float32)
    b = (rng.integers(0, 5, (T, 1)) / 4.0).astype(np.float32)
    s = dy(1, d, d)
    ckpt, out = og.gdn_span(s, q, k, v, a, b)
    S = [[_f32_frac(s[0, i, j]) for j in range(d)] for i in range(d)]
    for t in range(T):
        kk = [_f32_frac(k[t, 0, j]) for j in range(d)]
        vv = [_f32_frac(v[t, 0, j]) for j in range(d)]
        qq = [_f32_frac(q[t, 0, j]) for j in range(d)]
        at, bt = _f32_frac(a[t, 0]), _f32_frac(b[t, 0])
        M = [[(1 if i == j else 0) - bt * kk[i] * kk[j] for j in range(d)] for i in range(d)]
        SM = [[sum(S[i][m] * M[m][j] for m in range(d)) for j in range(d)] for i in range(d)]
        S = [[at * SM[i][j] + bt * vv[i] * kk[j] for j in range(d)] for i in range(d)]
        S = [[_f32_frac(float(S[i][j])) for j in range(d)] for i in range(d)]
        o = [sum(S[i][j] * qq[j] for j in range(d)) for i in range(d)]
        for i in range(d):
            for j in range(d):
                assert ckpt[t, 0, i, j] == np.float32(float(S[i][j]))
            assert out[t, 0, i] == np.float32(float(o[i]))


def test_key_head_grouping_contiguous():
    """Value head h uses key head h // (Hv/Hk): duplicating each key head over
    its group and running with Hk == Hv gives the same result."""
    q, k, v, a, b, s = _rand_inputs(3, 2, 4, 8, 8)
    ck1, o1 = og.gdn_span(s, q, k, v, a, b)
    q2 = np.repeat(q, 2, axis=1)
    k2 = np.repeat(k, 2, axis=1)
    ck2, o2 = og.gdn_span(s, q2, k2, v, a, b)
    assert np.array_equal(ck1, ck2) and np.array_equal(o1, o2)
    # and it is not the interleaved grouping h % Hk
    k3 = np.tile(k, (1, 2, 1))
    q3 = np.tile(q, (1, 2, 1))
    ck3, _ = og.gdn_span(s, q3, k3, v, a, b)
    assert not np.array_equal(ck1, ck3)


def test_power_of_two_scaling_exact():
    """Scaling state and v by 2 scales every checkpoint and output by 2."""
    q, k, v, a, b, s = _rand_inputs(4, 2, 4, 8, 8)
    ck1, o1 = og.gdn_span(s, q, k, v, a, b)
    ck2, o2 = og.gdn_span(s * 2, q, k, v * 2, a, b)
    assert np.array_equal(ck2, ck1 * 2) and np.array_equal(o2, o1 * 2)


def test_q_scale_power_of_two():
    q, k, v, a, b, s = _rand_inputs(3, 1, 2, 8, 8)
    ck1, o1 = og.gdn_span(s, q, k, v, a, b)
    ck2, o2 = og.gdn_span(s, q, k, v, a, b, q_scale=0.5)
    assert np.array_equal(ck1, ck2) and np.array_equal(o2, o1 * 0.5)


def test_split_span_composition():
    """span(T) equals span(j) followed by span(T-j) from checkpoint j-1
    (verify equals step-by-step decode)."""
    q, k, v, a, b, s = _rand_inputs(7, 2, 4, 8, 8)
    ck, out = og.gdn_span(s, q, k, v, a, b)
    for j in (1, 3, 6):
        ck_b, out_b = og.gdn_span(ck[j - 1], q[j:], k[j:], v[j:], a[j:], b[j:])
        assert np.array_equal(ck_b, ck[j:]) and np.array_equal(out_b, out[j:])
    # and one position at a time
    S = s
    for t in range(7):
        c1, o1 = og.gdn_span(S, q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1])
        assert np.array_equal(c1[0], ck[t]) and np.array_equal(o1[0], out[t])
        S = c1[0]


def test_tree_node_equals_chain_over_root_path():
    w = scaled(TINY_CHAIN, tree=True, n_pos=12, d_k=8, d_v=8, n_kheads=2, n_vheads=4)
    u = gen_unit(w, 0, 0)
    parent = gen_tree_parent(w, 0)
    assert any(parent[t] != t - 1 for t in range(1, 12)), "tree must branch"
    ck, out = og.gdn_span(u.state, u.q, u.k, u.v, u.a, u.b, parent)
    for node in range(12):
        path = []
        n = node
        while n >= 0:
            path.append(n)
            n = parent[n]
        path = path[::-1]
        idx = np.array(path)
        ckc, outc = og.gdn_span(u.state, u.q[idx], u.k[idx], u.v[idx], u.a[idx], u.b[idx])
        assert np.array_equal(ckc[-1], ck[node]) and np.array_equal(outc[-1], out[node])


def test_explicit_chain_parent_equals_default():
    w = scaled(TINY_CHAIN, d_k=8, d_v=8)
    u = gen_unit(w, 0, 0)
    ck1, o1 = og.gdn_span(u.state, u.q, u.k, u.v, u.a, u.b)
    ck2, o2 = og.gdn_span(u.state, u.q, u.k, u.v, u.a, u.b, np.arange(-1, w.n_pos - 1))
    assert np.array_equal(ck1, ck2) and np.array_equal(o1, o2)


def test_bf16_inputs_widen_exactly():
    """bf16 bit patterns are widened exactly: the oracle on bf16 inputs equals
    the oracle on the same values given as float32."""
    w = scaled(QWEN_LAYER_CHAIN, n_kheads=2, n_vheads=4, d_k=16, d_v=16, n_pos=4)
    u = gen_unit(w, 0, 0)
    assert u.q.dtype == np.uint16
    f = lambda x: (x.astype(np.uint32) << 16).view(np.float32)
    ck1, o1 = og.gdn_span(u.state, u.q, u.k, u.v, u.a, u.b)
    ck2, o2 = og.gdn_span(u.state, f(u.q), f(u.k), f(u.v), f(u.a), f(u.b))
    assert np.array_equal(ck1, ck2) and np.array_equal(o1, o2)


def test_nonexpansive_with_unit_keys():
    """With unit-norm k and 0 < a, b < 1 the map S -> a S (I - b k k^T) is a
    contraction, so the difference of two runs from different states shrinks."""
    q, k, v, a, b, s = _rand_inputs(6, 1, 1, 8, 8)
    s2 = s + np.float32(0.01)
    ck1, _ = og.gdn_span(s, q, k, v, a, b)
    ck2, _ = og.gdn_span(s2, q, k, v, a, b)
    prev = np.linalg.norm(s2.astype(np.float64) - s)
    for t in range(6):
        cur = np.linalg.norm(ck2[t].astype(np.float64) - ck1[t])
        assert cur <= prev * (1 + 1e-5)
        prev = cur


@pytest.mark.parametrize("d,T,seed", [(2, 3, 0), (3, 3, 1), (3, 2, 2)])
def test_exact_rational_full_mantissa(d, T, seed):
    """Exact rationals on random float32 inputs with full 24-bit significands,
    so that the new state is almost never a float32 value: the checkpoint must
    be the exact state rounded to float32 (nearest, ties to even), the output
    must be computed from that rounded checkpoint, and the next position must
    start from it. The inputs are checked to be ones where taking the output
    from the unrounded state would change some output bits, so a slip there
    cannot pass."""
    rng = np.random.default_rng(100 + seed)
    f32 = lambda *shape: rng.uniform(-1.0, 1.0, shape).astype(np.float32)
    q, k, v, s = f32(T, 1, d), f32(T, 1, d), f32(T, 1, d), f32(1, d, d)
    a = rng.uniform(0.1, 0.99, (T, 1)).astype(np.float32)
    b = rng.uniform(0.1, 0.99, (T, 1)).astype(np.float32)
    ckpt, out = og.gdn_span(s, q, k, v, a, b)
    S = [[_f32_frac(s[0, i, j]) for j in range(d)] for i in range(d)]
    differs = 0
    for t in range(T):
        kk = [_f32_frac(k[t, 0, j]) for j in range(d)]
        vv = [_f32_frac(v[t, 0, j]) for j in range(d)]
        qq = [_f32_frac(q[t, 0, j]) for j in range(d)]
        at, bt = _f32_frac(a[t, 0]), _f32_frac(b[t, 0])
        M = [[(1 if i == j else 0) - bt * kk[i] * kk[j] for j in range(d)] for i in range(d)]
        exact = [[at * sum(S[i][m] * M[m][j] for m in range(d)) + bt * vv[i] * kk[j] for j in range(d)]
                 for i in range(d)]
        rounded = [[_round_f32_exact(exact[i][j]) for j in range(d)] for i in range(d)]
        S = [[Fraction(float(rounded[i][j])) for j in range(d)] for i in range(d)]
        for i in range(d):
            o_exact = _round_f32_exact(sum(S[i][j] * qq[j] for j in range(d)))
            o_unrounded = _round_f32_exact(sum(exact[i][j] * qq[j] for j in range(d)))
            differs += int(o_exact != o_unrounded)
            assert out[t, 0, i] == o_exact, (t, i)
            for j in range(d):
                assert ckpt[t, 0, i, j] == rounded[i][j], (t, i, j)
    assert differs > 0, "inputs must make the output depend on the checkpoint rounding"
