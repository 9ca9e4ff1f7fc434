"""Pins of the rollback oracle: replay from the pre-span state equals the
span's own checkpoint of the accepted node (the replay/checkpoint equivalence
that fast rollback relies on), for chains and trees."""
import numpy as np

from oracle import accept as oa, conv as oc, gdn as og, rollback as orb
from synth import TINY_CHAIN, gen_unit, gen_conv_weight, gen_tree_parent, scaled


def test_replay_equals_checkpoint_chain():
    wl = scaled(TINY_CHAIN, d_k=16, d_v=16)
    u = gen_unit(wl, 0, 0)
    ck, _ = og.gdn_span(u.state, u.q, u.k, u.v, u.a, u.b)
    for j in range(wl.n_pos):
        path = np.arange(j + 1)
        assert np.array_equal(orb.replay_state(u.state, u.q, u.k, u.v, u.a, u.b, path), ck[j])


def test_replay_equals_checkpoint_tree():
    wl = scaled(TINY_CHAIN, tree=True, n_pos=13, d_k=8, d_v=8, conv_channels=24)
    u = gen_unit(wl, 0, 0)
    w = gen_conv_weight(wl, 0)
    parent = gen_tree_parent(wl, 0)
    ck, _ = og.gdn_span(u.state, u.q, u.k, u.v, u.a, u.b, parent)
    _, cck = oc.conv_span(u.x, w, u.conv_state, parent)
    for node in range(13):
        am = np.zeros(13, dtype=np.int32)
        path, n = [], node
        while n >= 0:
            path.append(n)
            n = parent[n]
        path = np.array(path[::-1] + [-1] * (13 - len(path)))
        assert np.array_equal(orb.replay_state(u.state, u.q, u.k, u.v, u.a, u.b, path), ck[node])
        assert np.array_equal(orb.replay_conv_state(u.conv_state, u.x, path), cck[node])


def test_conv_replay_pads_from_state():
    wl = scaled(TINY_CHAIN, conv_channels=8)
    u = gen_unit(wl, 0, 0)
    got = orb.replay_conv_state(u.conv_state, u.x, [0])
    assert np.array_equal(got, np.stack([u.conv_state[1], u.conv_state[2], u.x[0]]))
    got = orb.replay_conv_state(u.conv_state, u.x, [0, 1, 2, 3, -1])
    assert np.array_equal(got, u.x[1:4])
