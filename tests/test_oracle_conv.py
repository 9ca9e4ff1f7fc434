"""Pins of the conv oracle: numpy.convolve on the concatenated sequence,
state slices, scipy's logistic for silu, and tree windows along root paths."""
import numpy as np
import pytest
from scipy.special import expit

from oracle import conv as oc
from synth import TINY_CHAIN, QWEN_LAYER_CHAIN, gen_unit, gen_conv_weight, gen_tree_parent, scaled, bf16_to_f32


def _f64(x):
    x = np.asarray(x)
    return bf16_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


@pytest.mark.parametrize("wl", [TINY_CHAIN, scaled(QWEN_LAYER_CHAIN, conv_channels=256)])
def test_chain_matches_numpy_convolve(wl):
    u = gen_unit(wl, 0, 0)
    w = gen_conv_weight(wl, 0)
    y, ck = oc.conv_span(u.x, w, u.conv_state)
    seq = np.concatenate([u.conv_state, u.x], axis=0)       # [W-1+T, C]
    seqf, wf = _f64(seq), _f64(w)
    T, C = u.x.shape
    Wd = w.shape[1]
    ref = np.empty((T, C))
    for c in range(C):
        ref[:, c] = np.convolve(seqf[:, c], wf[c][::-1], mode="valid")
    err = np.max(np.abs(y - ref)) / np.max(np.abs(ref))
    assert err < 1e-7
    for t in range(T):
        assert np.array_equal(ck[t], seq[t + 1:t + Wd])


def test_silu_flag_uses_logistic():
    wl = scaled(TINY_CHAIN, conv_channels=64)
    u = gen_unit(wl, 0, 0)
    w = gen_conv_weight(wl, 0)
    y_lin, ck1 = oc.conv_span(u.x, w, u.conv_state)
    y_act, ck2 = oc.conv_span(u.x, w, u.conv_state, silu=True)
    assert np.array_equal(ck1, ck2)
    z = y_lin.astype(np.float64)
    np.testing.assert_allclose(y_act, z * expit(z), rtol=2e-7, atol=1e-30)


def test_tree_windows_follow_root_path():
    wl = scaled(TINY_CHAIN, tree=True, n_pos=14, conv_channels=32)
    u = gen_unit(wl, 0, 0)
    w = gen_conv_weight(wl, 0)
    parent = gen_tree_parent(wl, 0)
    y, ck = oc.conv_span(u.x, w, u.conv_state, parent)
    for node in range(14):
        path, n = [], node
        while n >= 0:
            path.append(n)
            n = parent[n]
        idx = np.array(path[::-1])
        yc, ckc = oc.conv_span(u.x[idx], w, u.conv_state)
        assert np.array_equal(yc[-1], y[node]) and np.array_equal(ckc[-1], ck[node])


def test_weight_tap_orientation():
    """w[c][W-1] multiplies the current input: with a one-hot last tap y = x."""
    wl = scaled(TINY_CHAIN, conv_channels=16)
    u = gen_unit(wl, 0, 0)
    w = np.zeros((16, 4), dtype=np.float32)
    w[:, 3] = 1.0
    y, _ = oc.conv_span(u.x, w, u.conv_state)
    assert np.array_equal(y, u.x)
    w[:, 3] = 0.0
    w[:, 0] = 1.0   # oldest tap: the conv state for the first three positions
    y, _ = oc.conv_span(u.x, w, u.conv_state)
    assert np.array_equal(y[0], u.conv_state[0]) and np.array_equal(y[3], u.x[0])
