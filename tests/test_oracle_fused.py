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
