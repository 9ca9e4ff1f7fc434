"""Pins of the fused-layer oracle: with a conv that only passes the current
input, the layer must equal the GDN oracle run on channel slices that are
passed through SiLU (scipy's logistic) and L2-normalised (numpy's norm)
independently of the oracle's own code — this fixes the q | k | v split order
and where the normalisation sits."""
import numpy as np
from scipy.special import expit

from oracle import fused as ofu, gdn as ogdn
from synth import QWEN_LAYER_CHAIN, gen_tree_parent, gen_unit, scaled, bf16_to_f32


def test_identity_conv_equals_gdn_on_slices():
    Hk, Hv, dk, dv, T = 2, 4, 16, 8, 5
    C = 2 * Hk * dk + Hv * dv
    rng = np.random.default_rng(3)
    x = rng.standard_normal((T, C)).astype(np.float32)
    w = np.zeros((C, 4), dtype=np.float32)
    w[:, 3] = 1.0
    cs = rng.standard_normal((3, C)).astype(np.float32)
    a = rng.uniform(0.1, 0.9, (T, Hv)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (T, Hv)).astype(np.float32)
    state = (rng.standard_normal((Hv, dv, dk)) * 0.1).astype(np.float32)
    ck, out, _ = ofu.layer_span(x, w, cs, a, b, state, Hk, Hv, dk, dv, q_scale=0.25, eps=1e-6)
    y = x.astype(np.float64) * expit(x.astype(np.float64))
    y = y.astype(np.float32).astype(np.float64)
    q = y[:, :Hk * dk].reshape(T, Hk, dk)
    k = y[:, Hk * dk:2 * Hk * dk].reshape(T, Hk, dk)
    v = y[:, 2 * Hk * dk:].reshape(T, Hv, dv)
    qn = q / np.sqrt(np.linalg.norm(q, axis=-1, keepdims=True) ** 2 + 1e-6)
    kn = k / np.sqrt(np.linalg.norm(k, axis=-1, keepdims=True) ** 2 + 1e-6)
    ck2, out2 = ogdn.gdn_span(state, qn, kn, v, a, b, q_scale=0.25)
    np.testing.assert_allclose(ck, ck2, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(out, out2, rtol=1e-6, atol=1e-7)
    # the split order matters: swapping the q and k channel blocks changes the result
    xs = x.copy()
    xs[:, :Hk * dk], xs[:, Hk * dk:2 * Hk * dk] = x[:, Hk * dk:2 * Hk * dk], x[:, :Hk * dk]
    ck3, _, _ = ofu.layer_span(xs, w, cs, a, b, state, Hk, Hv, dk, dv, q_scale=0.25)
    assert not np.allclose(ck3, ck)


def test_normalised_rows_have_unit_norm():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 3, 32)) * 5
    n = np.linalg.norm(ofu.l2norm_rows(x, 0.0), axis=-1)
    np.testing.assert_allclose(n, 1.0, rtol=1e-12)
    assert np.all(np.abs(ofu.l2norm_rows(np.zeros((2, 8)), 1e-6)) == 0)


def test_tree_layer_node_equals_chain_over_root_path():
    w_ = scaled(QWEN_LAYER_CHAIN, n_kheads=2, n_vheads=4, d_k=16, d_v=16, n_pos=10, tree=True,
                conv_channels=2 * 2 * 16 + 4 * 16)
    u = gen_unit(w_, 0, 0)
    rng = np.random.default_rng(5)
    wt = (rng.standard_normal((w_.conv_channels, 4)) * 0.5).astype(np.float32)
    parent = gen_tree_parent(w_, 0)
    f = lambda t: (t.astype(np.uint32) << 16).view(np.float32) if t.dtype == np.uint16 else t
    x, cs, a, b = f(u.x), f(u.conv_state), f(u.a), f(u.b)
    ck, out, _ = ofu.layer_span(x, wt, cs, a, b, u.state, 2, 4, 16, 16, parent=parent)
    for node in (int(np.argmax(parent)), 9):
        path, n = [], node
        while n >= 0:
            path.append(n)
            n = parent[n]
        idx = np.array(path[::-1])
        ckc, outc, _ = ofu.layer_span(x[idx], wt, cs, a[idx], b[idx], u.state, 2, 4, 16, 16)
        assert np.array_equal(ckc[-1], ck[node]) and np.array_equal(outc[-1], out[node])


def test_l2norm_hand_worked_values():
    """Closed forms worked by hand, with eps large enough to matter: eps is
    added to the sum of squares under the square root. Rows:
      [3, 4],  eps 0      -> /5           = [0.6, 0.8]
      [3, 4],  eps 11     -> /sqrt(36)=6  = [0.5, 2/3]
      [1, 0],  eps 3      -> /sqrt(4)=2   = [0.5, 0]
      [2,0,0,0], eps 5    -> /sqrt(9)=3   = [2/3, 0, 0, 0]
      [0, 0],  eps 1      -> [0, 0]
      small norm [3e-4, 4e-4], eps 1e-6: sum of squares 2.5e-7, plus eps
      1.25e-6, root sqrt(5)/2 * 1e-3, so [0.6, 0.8] / sqrt(5).
    Putting eps outside the root (x / (|x| + eps)) gives [3/16, 1/4] for the
    second row and [0.5988..., 0.7984...] for the small-norm row."""
    import math
    cases = [([3.0, 4.0], 0.0, [0.6, 0.8]),
             ([3.0, 4.0], 11.0, [0.5, 2.0 / 3.0]),
             ([1.0, 0.0], 3.0, [0.5, 0.0]),
             ([2.0, 0.0, 0.0, 0.0], 5.0, [2.0 / 3.0, 0.0, 0.0, 0.0]),
             ([0.0, 0.0], 1.0, [0.0, 0.0]),
             ([3e-4, 4e-4], 1e-6, [0.6 / math.sqrt(5.0), 0.8 / math.sqrt(5.0)])]
    for x, eps, exp in cases:
        got = ofu.l2norm_rows(np.array([x]), eps)[0]
        np.testing.assert_allclose(got, exp, rtol=1e-14, atol=0, err_msg=f"{x}, eps {eps}")


def test_layer_normalises_q_and_k_with_eps_under_the_root():
    """Through the whole layer: identity conv without SiLU, eps = 2.4375, and
    q and k rows whose sum of squares is 1.5625, so |x|^2 + eps = 4 and the
    root is 2: q [0.75, 1] -> [0.375, 0.5] and k [1.25, 0] -> [0.625, 0],
    exact dyadics worked by hand. The layer must equal the GDN oracle fed
    those rows, bit for bit. With eps outside the root the rows would be
    divided by 1.25 + 2.4375 instead."""
    Hk, Hv, dk, dv, T = 1, 2, 2, 2, 2
    C = 2 * Hk * dk + Hv * dv
    x = np.zeros((T, C), dtype=np.float32)
    x[:, 0:2] = [0.75, 1.0]                                        # q
    x[:, 2:4] = [1.25, 0.0]                                        # k
    x[:, 4:] = [[1.0, -2.0, 0.5, 3.0], [2.0, 1.0, -1.0, 0.25]]     # v of two heads
    w = np.zeros((C, 4), dtype=np.float32)
    w[:, 3] = 1.0
    cs = np.zeros((3, C), dtype=np.float32)
    a = np.array([[0.5, 0.75], [0.25, 1.0]], dtype=np.float32)
    b = np.array([[0.5, 0.25], [1.0, 0.5]], dtype=np.float32)
    state = np.array([[[1.0, 2.0], [3.0, -1.0]], [[0.5, 0.0], [-2.0, 4.0]]], dtype=np.float32)
    ck, out, _ = ofu.layer_span(x, w, cs, a, b, state, Hk, Hv, dk, dv, eps=2.4375, silu=False)
    qn = np.tile(np.array([0.375, 0.5], dtype=np.float32), (T, Hk, 1))
    kn = np.tile(np.array([0.625, 0.0], dtype=np.float32), (T, Hk, 1))
    v = x[:, 4:].reshape(T, Hv, dv)
    ck2, out2 = ogdn.gdn_span(state, qn, kn, v, a, b)
    assert np.array_equal(ck, ck2) and np.array_equal(out, out2)
