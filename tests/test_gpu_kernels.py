"""GPU parity of every entry point against the CPU oracle, at sizes the oracle
finishes in seconds (several row blocks, chunks and a ragged tail), plus the
GPU's own exactness properties. Calls go through the C ABI (ctypes binding).

Bars: integers, indices, copies and conv states bit-exact; float results
within max relative error 1e-4 per tile (tests/gpu_util.py).
"""
import numpy as np
import pytest

import oracle
from oracle import accept as oacc, conv as oconv, gdn as ogdn, ring as oring, rollback as orb
from synth import (F32, BF16, TINY_CHAIN, QWEN_LAYER_CHAIN, QWEN_STACK_TREE, QWEN_STACK_CHAIN, bf16_bits,
                   gen_accept, gen_conv_weight, gen_tree_parent, gen_unit, scaled)
from tests.gpu_util import assert_tiles, say, to_numpy, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hrs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import hybrid_recurrent_state_amd as m
    return m


def _torch():
    import torch
    return torch


# ---------------------------------------------------------------------------
# GDN


def gpu_gdn(hrs, units, parent=None, capture=True, q_scale=1.0, state=None):
    torch = _torch()
    st = lambda name: to_torch(np.stack([getattr(u, name) for u in units]))
    q, k, v, a, b = st("q"), st("k"), st("v"), st("a"), st("b")
    state_t = st("state") if state is None else to_torch(state)
    R, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    ckpt = torch.full((R, T, Hv, dv, dk), float("nan"), device="cuda") if capture else None
    out = torch.full((R, T, Hv, dv), float("nan"), device="cuda")
    hrs.gdn_verify_span(q, k, v, a, b, state_t, ckpt, out, parent=parent, q_scale=q_scale)
    torch.cuda.synchronize()
    return (to_numpy(ckpt) if capture else None), to_numpy(out), to_numpy(state_t)


def check_gdn_vs_oracle(units, ck, out, parents=None, q_scale=1.0, what=""):
    for r, u in enumerate(units):
        par = None if parents is None else parents[r]
        ock, oout = ogdn.gdn_span(u.state, u.q, u.k, u.v, u.a, u.b, par, q_scale)
        e1 = assert_tiles(ck[r], ock, 2, f"{what} ckpt r={r}")
        e2 = assert_tiles(out[r], oout, 1, f"{what} out r={r}")
        say(f"{what} r={r}: ckpt err {e1:.2e}, out err {e2:.2e}")


def test_gdn_tiny_chain_f32(hrs):
    w = TINY_CHAIN
    units = [gen_unit(w, 0, 0)]
    ck, out, st = gpu_gdn(hrs, units)
    check_gdn_vs_oracle(units, ck, out, what="tiny f32")
    assert np.array_equal(st[0], units[0].state), "state must be read only in capture mode"


def test_gdn_qwen_layer_chain_bf16_r3(hrs):
    w = scaled(QWEN_LAYER_CHAIN, n_req=3)
    units = [gen_unit(w, 0, r) for r in range(3)]
    ck, out, _ = gpu_gdn(hrs, units)
    check_gdn_vs_oracle(units, ck, out, what="qwen layer bf16")


def test_gdn_grouped_heads_dk64_f32(hrs):
    w = scaled(TINY_CHAIN, n_kheads=2, n_vheads=8, d_k=64, d_v=48, n_pos=6)
    units = [gen_unit(w, 0, r) for r in range(2)]
    ck, out, _ = gpu_gdn(hrs, units)
    check_gdn_vs_oracle(units, ck, out, what="grouped dk64")


@pytest.mark.parametrize("T", [33, 64])
def test_gdn_long_span_crosses_lds_windows(hrs, T):
    w = scaled(QWEN_LAYER_CHAIN, n_kheads=2, n_vheads=4, n_pos=T)
    units = [gen_unit(w, 0, 0)]
    ck, out, _ = gpu_gdn(hrs, units)
    check_gdn_vs_oracle(units, ck, out, what=f"T={T}")


def test_gdn_q_scale(hrs):
    w = scaled(QWEN_LAYER_CHAIN, n_kheads=4, n_vheads=8, n_pos=5)
    units = [gen_unit(w, 0, 0)]
    ck, out, _ = gpu_gdn(hrs, units, q_scale=0.0883883)
    check_gdn_vs_oracle(units, ck, out, q_scale=0.0883883, what="q_scale")


def test_gdn_tree_qwen_r2(hrs):
    w = scaled(QWEN_STACK_TREE, n_layers=1, n_req=2)
    units = [gen_unit(w, 0, r) for r in range(2)]
    parents = np.stack([gen_tree_parent(w, r) for r in range(2)])
    assert not np.array_equal(parents[0], parents[1])
    ck, out, _ = gpu_gdn(hrs, units, parent=parents)
    check_gdn_vs_oracle(units, ck, out, parents=parents, what="tree")


TREE_SHAPES = {
    "comb": [-1] + [0] * 11,                                   # one slot reused by 11 children
    "binary": [-1, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5],
    "overflow": [-1] + list(range(10)) + list(range(10)),      # 10 live branch points > 8 stash slots
    "late-siblings": [-1, 0, 1, 2, 3, 4, 5, 6, 2, 8, 4, 0, 11],
}


@pytest.mark.parametrize("shape", sorted(TREE_SHAPES))
@pytest.mark.parametrize("n_req", [1, 3])
def test_gdn_tree_shapes(hrs, shape, n_req):
    """Stash schedule: slot reuse, slot overflow to checkpoint reloads, late
    siblings; R=1 uses 16-row units, R=3 the one-block-per-CU grid."""
    par = np.array(TREE_SHAPES[shape], dtype=np.int32)
    T = len(par)
    w = scaled(QWEN_LAYER_CHAIN, n_req=n_req, n_pos=T)
    units = [gen_unit(w, 0, r) for r in range(n_req)]
    parents = np.tile(par, (n_req, 1))
    ck, out, _ = gpu_gdn(hrs, units, parent=parents)
    check_gdn_vs_oracle(units, ck, out, parents=parents, what=f"tree {shape}")


def test_gdn_random_long_trees(hrs):
    rng = np.random.default_rng(33)
    for T in (40, 64):
        par = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, T)], dtype=np.int32)
        w = scaled(QWEN_LAYER_CHAIN, n_kheads=4, n_vheads=8, n_pos=T)
        units = [gen_unit(w, 0, 0)]
        ck, out, _ = gpu_gdn(hrs, units, parent=par[None])
        check_gdn_vs_oracle(units, ck, out, parents=par[None], what=f"random tree T={T}")


def _mixed_trees(rng, n_req, T):
    """Per request a random tree of T positions: uniform parents (wide, many
    live branch points), a deep chain with side branches, or a pure chain."""
    out = []
    for r in range(n_req):
        kind = r % 3
        if kind == 0:
            par = [-1] + [int(rng.integers(0, i)) for i in range(1, T)]
        elif kind == 1:
            par = [-1] + [i - 1 if rng.random() < 0.7 else int(rng.integers(0, i)) for i in range(1, T)]
        else:
            par = list(range(-1, T - 1))
        out.append(par)
    return np.asarray(out, dtype=np.int32)


def test_gdn_tree_batch_split_over_launches(hrs):
    """20 requests of 64-position trees: the tree geometry of at most 16
    requests fits one launch, so the span runs as a 16-request launch (one
    block per CU) and a 4-request launch (16-row units with staging-only
    waves); wide trees need the checkpoint-reload variant."""
    rng = np.random.default_rng(71)
    R, T = 20, 64
    w = scaled(QWEN_LAYER_CHAIN, n_req=R, n_kheads=2, n_vheads=4, n_pos=T)
    units = [gen_unit(w, 0, r) for r in range(R)]
    parents = _mixed_trees(rng, R, T)
    say(f"tree batch R={R} T={T}")
    ck, out, _ = gpu_gdn(hrs, units, parent=parents)
    check_gdn_vs_oracle(units, ck, out, parents=parents, what="tree batch")


def test_gdn_random_shapes(hrs):
    """Seeded sweep over shapes the library accepts (d_k 64/128, d_v a
    multiple of 16 up to 256, 1-4 value heads per key head, 1-5 requests,
    1-40 positions, chain or random tree, bf16 or f32 inputs), each against
    the oracle: launch shapes and unit counts beyond the model's."""
    rng = np.random.default_rng(2024)
    for i in range(12):
        dk = int(rng.choice([64, 128]))
        dv = int(rng.choice([16, 32, 48, 64, 96, 128, 256]))
        Hk = int(rng.choice([1, 2, 3]))
        Hv = Hk * int(rng.choice([1, 2, 4]))
        R = int(rng.integers(1, 6))
        T = int(rng.integers(1, 41))
        dt = BF16 if rng.random() < 0.6 else F32
        tree = T > 2 and rng.random() < 0.5
        w = scaled(QWEN_LAYER_CHAIN, n_req=R, n_pos=T, n_kheads=Hk, n_vheads=Hv, d_k=dk, d_v=dv, dtype=dt,
                   conv_channels=16, seed=100 + i)
        units = [gen_unit(w, 0, r) for r in range(R)]
        parents = None
        if tree:
            parents = np.array([[-1] + [int(rng.integers(0, t)) for t in range(1, T)] for _ in range(R)],
                               dtype=np.int32)
        what = f"shape {i}: R={R} T={T} Hk={Hk} Hv={Hv} dk={dk} dv={dv} {dt} {'tree' if tree else 'chain'}"
        say(what)
        ck, out, _ = gpu_gdn(hrs, units, parent=parents)
        check_gdn_vs_oracle(units, ck, out, parents=parents, what=what)


def test_gdn_tree_with_chain_parent_equals_chain(hrs):
    w = scaled(QWEN_LAYER_CHAIN, n_req=2)
    units = [gen_unit(w, 0, r) for r in range(2)]
    ck1, o1, _ = gpu_gdn(hrs, units)
    chain = np.tile(np.arange(-1, w.n_pos - 1, dtype=np.int32), (2, 1))
    ck2, o2, _ = gpu_gdn(hrs, units, parent=chain)
    assert np.array_equal(ck1, ck2) and np.array_equal(o1, o2)


def test_gdn_tree_node_equals_chain_over_root_path(hrs):
    w = scaled(QWEN_STACK_TREE, n_layers=1, n_kheads=4, n_vheads=8)
    u = gen_unit(w, 0, 0)
    parent = gen_tree_parent(w, 0)
    ck, out, _ = gpu_gdn(hrs, [u], parent=parent[None])
    depth = np.zeros(w.n_pos, dtype=int)
    for t in range(1, w.n_pos):
        depth[t] = depth[parent[t]] + 1
    for node in [int(np.argmax(depth)), w.n_pos - 1, 1]:
        path, n = [], node
        while n >= 0:
            path.append(n)
            n = parent[n]
        idx = np.array(path[::-1])
        sub = type(u)(q=u.q[idx], k=u.k[idx], v=u.v[idx], a=u.a[idx], b=u.b[idx], state=u.state, x=u.x,
                      conv_state=u.conv_state)
        ckc, outc, _ = gpu_gdn(hrs, [sub])
        assert np.array_equal(ckc[0, -1], ck[0, node]) and np.array_equal(outc[0, -1], out[0, node]), node


@pytest.mark.parametrize("n_kheads,n_vheads", [(4, 8), (16, 32)])
@pytest.mark.parametrize("tree", [False, True])
def test_gdn_degenerate_gates(hrs, n_kheads, n_vheads, tree):
    """Gates and keys at the rule's degenerate values, against the oracle and
    against what the rule then reduces to, exactly: a = b = 0 forgets the
    state (S' = 0), a = 1 with b = 0 keeps it (S' = S of the parent), k = 0
    only decays it (S' = a S of the parent, one rounding), and a = 0 with
    b = 1 writes v k^T alone (a product of two bf16 values: exact in f32).
    Two launch shapes: 16-row units at 8 value heads, 32-row units on one
    block per CU at 2 requests x 32 value heads."""
    T = 12
    w = scaled(QWEN_LAYER_CHAIN, n_req=2, n_kheads=n_kheads, n_vheads=n_vheads, n_pos=T)
    parent = (np.array([-1, 0, 1, 1, 3, 2, 5, 4, 7, 0, 9, 10], dtype=np.int32) if tree
              else np.arange(-1, T - 1, dtype=np.int32))
    forget, keep, no_key, write_only = (9, 5, 8, 11) if tree else (2, 5, 7, 9)
    one, zero = bf16_bits(np.float32(1.0)), np.uint16(0)
    units = []
    for r in range(2):
        u = gen_unit(w, 0, r)
        a, b, k = u.a.copy(), u.b.copy(), u.k.copy()
        a[forget], b[forget] = zero, zero
        a[keep], b[keep] = one, zero
        k[no_key] = zero
        a[write_only], b[write_only] = zero, one
        units.append(type(u)(q=u.q, k=k, v=u.v, a=a, b=b, state=u.state, x=u.x, conv_state=u.conv_state))
    parents = np.tile(parent, (2, 1))
    ck, out, _ = gpu_gdn(hrs, units, parent=parents if tree else None)
    check_gdn_vs_oracle(units, ck, out, parents=parents if tree else None, what="degenerate gates")
    f32 = lambda bits: (bits.astype(np.uint32) << 16).view(np.float32)
    group = n_vheads // n_kheads
    for r, u in enumerate(units):
        assert np.all(ck[r, forget] == 0) and np.all(out[r, forget] == 0), "a = b = 0 must forget the state"
        assert np.array_equal(ck[r, keep], ck[r, parent[keep]]), "a = 1, b = 0 must keep the parent's state"
        a_nk = f32(u.a[no_key])                                     # [Hv]
        assert np.array_equal(ck[r, no_key], a_nk[:, None, None] * ck[r, parent[no_key]]), "k = 0: S' = a S"
        vk = f32(u.v[write_only])[:, :, None] * np.repeat(f32(u.k[write_only]), group, axis=0)[:, None, :]
        assert np.array_equal(ck[r, write_only], vk), "a = 0, b = 1: S' = v k^T"


def test_gdn_decode_steps_equal_span(hrs):
    """span(T) with capture == T single-position calls without capture that
    advance the state in place (verify == decode), bit for bit."""
    w = scaled(QWEN_LAYER_CHAIN, n_req=2, n_pos=6)
    units = [gen_unit(w, 0, r) for r in range(2)]
    ck, out, _ = gpu_gdn(hrs, units)
    state = np.stack([u.state for u in units])
    for t in range(w.n_pos):
        step = [type(u)(q=u.q[t:t + 1], k=u.k[t:t + 1], v=u.v[t:t + 1], a=u.a[t:t + 1], b=u.b[t:t + 1],
                        state=u.state, x=u.x, conv_state=u.conv_state) for u in units]
        _, o1, state = gpu_gdn(hrs, step, capture=False, state=state)
        assert np.array_equal(o1[:, 0], out[:, t]), t
        assert np.array_equal(state, ck[:, t]), t


def test_gdn_power_of_two_scaling_and_determinism(hrs):
    w = scaled(QWEN_LAYER_CHAIN, n_kheads=4, n_vheads=8)
    u = gen_unit(w, 0, 0)
    ck1, o1, _ = gpu_gdn(hrs, [u])
    ck1b, o1b, _ = gpu_gdn(hrs, [u])
    assert np.array_equal(ck1, ck1b) and np.array_equal(o1, o1b), "not deterministic"
    # v x 2 in bf16 is exact (exponent shift)
    v2 = bf16_bits((np.asarray((u.v.astype(np.uint32) << 16).view(np.float32)) * 2).astype(np.float32))
    u2 = type(u)(q=u.q, k=u.k, v=v2, a=u.a, b=u.b, state=u.state * np.float32(2), x=u.x, conv_state=u.conv_state)
    ck2, o2, _ = gpu_gdn(hrs, [u2])
    assert np.array_equal(ck2, ck1 * 2) and np.array_equal(o2, o1 * 2)


def test_gdn_every_checkpoint_written_and_guard_bands(hrs):
    """NaN sentinels: every checkpoint and output element is written, and
    nothing outside the buffers changes."""
    torch = _torch()
    w = scaled(QWEN_LAYER_CHAIN, n_req=2, n_kheads=4, n_vheads=8)
    units = [gen_unit(w, 0, r) for r in range(2)]
    st = lambda name: to_torch(np.stack([getattr(x, name) for x in units]))
    R, T, Hv, dv, dk = 2, w.n_pos, 8, 128, 128
    G = 4096
    flat = torch.full((G + R * T * Hv * dv * dk + G,), float("nan"), device="cuda")
    oflat = torch.full((G + R * T * Hv * dv + G,), float("nan"), device="cuda")
    ckpt = flat[G:G + R * T * Hv * dv * dk].view(R, T, Hv, dv, dk)
    out = oflat[G:G + R * T * Hv * dv].view(R, T, Hv, dv)
    hrs.gdn_verify_span(st("q"), st("k"), st("v"), st("a"), st("b"), st("state"), ckpt, out)
    torch.cuda.synchronize()
    assert not torch.isnan(ckpt).any() and not torch.isnan(out).any()
    assert torch.isnan(flat[:G]).all() and torch.isnan(flat[-G:]).all()
    assert torch.isnan(oflat[:G]).all() and torch.isnan(oflat[-G:]).all()


# ---------------------------------------------------------------------------
# conv


def gpu_conv(hrs, units, wt, parent=None, capture=True, silu=False, conv_state=None):
    torch = _torch()
    x = to_torch(np.stack([u.x for u in units]))
    cs = to_torch(np.stack([u.conv_state for u in units]) if conv_state is None else conv_state)
    R, T, C = x.shape
    wdev = to_torch(wt)
    ck = torch.empty((R, T, 3, C), dtype=x.dtype, device="cuda") if capture else None
    y = torch.full((R, T, C), float("nan"), device="cuda")
    hrs.conv1d_verify_span(x, wdev, cs, ck, y, parent=parent, silu=silu)
    torch.cuda.synchronize()
    return to_numpy(y), (to_numpy(ck) if capture else None), to_numpy(cs)


@pytest.mark.parametrize("wl,silu", [(TINY_CHAIN, False), (TINY_CHAIN, True),
                                     (scaled(QWEN_LAYER_CHAIN, n_req=2, n_pos=6, conv_channels=1024), False),
                                     (scaled(QWEN_LAYER_CHAIN, n_req=1, n_pos=1, conv_channels=1024), True),
                                     (scaled(QWEN_LAYER_CHAIN, n_req=2), False),
                                     (scaled(QWEN_LAYER_CHAIN, n_req=2), True),
                                     (scaled(QWEN_LAYER_CHAIN, conv_channels=776, n_pos=3), False)])
def test_conv_chain_vs_oracle(hrs, wl, silu):
    units = [gen_unit(wl, 0, r) for r in range(wl.n_req)]
    wt = gen_conv_weight(wl, 0)
    y, ck, cs_after = gpu_conv(hrs, units, wt, silu=silu)
    for r, u in enumerate(units):
        oy, ock = oconv.conv_span(u.x, wt, u.conv_state, silu=silu)
        assert_tiles(y[r], oy, 1, f"conv y r={r}")
        assert np.array_equal(ck[r], ock), "conv checkpoints are exact copies"
        assert np.array_equal(cs_after[r], u.conv_state), "conv_state is read only in capture mode"


def test_conv_tree_vs_oracle(hrs):
    w = scaled(QWEN_STACK_TREE, n_layers=1, n_req=2, conv_channels=1024)
    units = [gen_unit(w, 0, r) for r in range(2)]
    wt = gen_conv_weight(w, 0)
    parents = np.stack([gen_tree_parent(w, r) for r in range(2)])
    y, ck, _ = gpu_conv(hrs, units, wt, parent=parents)
    for r, u in enumerate(units):
        oy, ock = oconv.conv_span(u.x, wt, u.conv_state, parents[r])
        assert_tiles(y[r], oy, 1, "conv tree y")
        assert np.array_equal(ck[r], ock)


def test_conv_tree_batch_split_over_launches(hrs):
    """20 requests of 64-position trees: the window-source tables of at most
    16 requests fit one launch."""
    rng = np.random.default_rng(72)
    R, T = 20, 64
    w = scaled(QWEN_LAYER_CHAIN, n_req=R, n_pos=T, conv_channels=1024)
    units = [gen_unit(w, 0, r) for r in range(R)]
    wt = gen_conv_weight(w, 0)
    parents = _mixed_trees(rng, R, T)
    y, ck, _ = gpu_conv(hrs, units, wt, parent=parents, silu=True)
    for r, u in enumerate(units):
        oy, ock = oconv.conv_span(u.x, wt, u.conv_state, parents[r], silu=True)
        assert_tiles(y[r], oy, 1, f"conv tree batch y r={r}")
        assert np.array_equal(ck[r], ock), f"conv tree batch checkpoints r={r}"


def test_conv_random_shapes(hrs):
    """Seeded sweep: channels 8-8200 (partial blocks), 1-64 positions, 1-4
    requests, chain or random tree, SiLU on or off, bf16 or f32; outputs
    within the tolerance and checkpoints bit-exact against the oracle."""
    rng = np.random.default_rng(909)
    for i in range(10):
        C = 8 * int(rng.integers(1, 1026))
        T = int(rng.integers(1, 65))
        R = int(rng.integers(1, 5))
        dt = F32 if rng.random() < 0.3 else BF16
        silu = bool(rng.random() < 0.5)
        tree = T > 2 and rng.random() < 0.5
        w = scaled(QWEN_LAYER_CHAIN, n_req=R, n_pos=T, conv_channels=C, dtype=dt, n_kheads=1, n_vheads=1, d_k=64,
                   d_v=16, seed=700 + i)
        units = [gen_unit(w, 0, r) for r in range(R)]
        wt = gen_conv_weight(w, 0)
        parents = None
        if tree:
            parents = np.array([[-1] + [int(rng.integers(0, t)) for t in range(1, T)] for _ in range(R)],
                               dtype=np.int32)
        say(f"conv shape {i}: R={R} T={T} C={C} {dt} silu={silu} {'tree' if tree else 'chain'}")
        y, ck, _ = gpu_conv(hrs, units, wt, parent=parents, silu=silu)
        for r, u in enumerate(units):
            oy, ock = oconv.conv_span(u.x, wt, u.conv_state, None if parents is None else parents[r], silu=silu)
            assert_tiles(y[r], oy, 1, f"conv shape {i} y r={r}")
            assert np.array_equal(ck[r], ock), f"conv shape {i} checkpoints r={r}"


@pytest.mark.parametrize("T", [1, 2, 5])
def test_conv_in_place_decode(hrs, T):
    w = scaled(QWEN_LAYER_CHAIN, n_req=2, n_pos=T, conv_channels=2048)
    units = [gen_unit(w, 0, r) for r in range(2)]
    wt = gen_conv_weight(w, 0)
    y1, ck, _ = gpu_conv(hrs, units, wt)
    y2, _, cs = gpu_conv(hrs, units, wt, capture=False)
    assert np.array_equal(y1, y2)
    assert np.array_equal(cs, ck[:, T - 1])
    for r, u in enumerate(units):
        assert np.array_equal(cs[r], orb.replay_conv_state(u.conv_state, u.x, np.arange(T)))


# ---------------------------------------------------------------------------
# accept


def gpu_accept(hrs, logits, tokens, parent=None):
    torch = _torch()
    lg = to_torch(logits)
    R, T, V = lg.shape
    tok = to_torch(np.ascontiguousarray(tokens, dtype=np.int32))
    outs = [torch.full(s, -7, dtype=torch.int32, device="cuda") for s in [(R, T), (R,), (R,), (R, T), (R,)]]
    nbytes = hrs.accept_greedy_workspace_bytes(R, T, V, hrs.HRS_BF16 if lg.dtype == torch.bfloat16 else hrs.HRS_F32,
                                               parent)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    hrs.accept_greedy(lg, tok, *outs, ws, parent=parent)
    torch.cuda.synchronize()
    return [to_numpy(o) for o in outs]


def check_accept(got, logits, tokens, parent=None):
    am, node, ln, path, bonus = got
    R = tokens.shape[0]
    oam = oacc.argmax_rows(logits)
    assert np.array_equal(am, oam), "argmax"
    for r in range(R):
        par = None if parent is None else parent[r]
        res = oacc.accept(oam[r], tokens[r], par)
        assert (node[r], ln[r], bonus[r]) == (res.accept_node, res.accept_len, res.bonus), r
        assert np.array_equal(path[r], res.path), r


def test_accept_tiny_distinct_f32(hrs):
    w = TINY_CHAIN
    ai = gen_accept(w, 0)
    got = gpu_accept(hrs, ai.logits[None], ai.tokens[None])
    check_accept(got, ai.logits[None], ai.tokens[None])
    assert got[1][0] == ai.planted_node


def test_accept_full_vocab_chain_bf16_r4(hrs):
    w = scaled(QWEN_STACK_CHAIN, n_req=4)
    acc = [gen_accept(w, r) for r in range(4)]
    lg = np.stack([a.logits for a in acc])
    tok = np.stack([a.tokens for a in acc])
    got = gpu_accept(hrs, lg, tok)
    check_accept(got, lg, tok)
    assert [int(x) for x in got[1]] == [a.planted_node for a in acc]


def test_accept_tree_ragged_vocab(hrs):
    w = scaled(QWEN_STACK_TREE, n_req=3, vocab=20008)
    acc = [gen_accept(w, r) for r in range(3)]
    lg = np.stack([a.logits for a in acc])
    tok = np.stack([a.tokens for a in acc])
    par = np.stack([a.parent for a in acc])
    got = gpu_accept(hrs, lg, tok, parent=par)
    check_accept(got, lg, tok, par)
    assert [int(x) for x in got[1]] == [a.planted_node for a in acc]


def test_accept_random_matches_brute_force(hrs):
    rng = np.random.default_rng(21)
    R, T, V = 8, 12, 64
    par = np.stack([np.concatenate([[-1], [rng.integers(0, i) for i in range(1, T)]]) for _ in range(R)]).astype(np.int32)
    tok = rng.integers(0, 3, (R, T)).astype(np.int32)
    lg = rng.standard_normal((R, T, V)).astype(np.float32)
    lg[:, :, :3] += 3.0 * rng.random((R, T, 3)).astype(np.float32)   # argmax mostly in {0,1,2}
    got = gpu_accept(hrs, lg, tok, parent=par)
    check_accept(got, lg, tok, par)
    oam = oacc.argmax_rows(lg)
    for r in range(R):
        bf = oacc.brute_force_accept(oam[r], tok[r], par[r])
        assert got[1][r] == bf.accept_node


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_accept_special_values(hrs, dtype):
    V = 2 * 16384 + 64   # two whole 16384-logit chunks and a ragged one
    rows = np.full((8, V), -5.0, dtype=np.float32)
    rows[0, 3] = np.nan; rows[0, 10] = 1.0                 # NaN never wins
    rows[1, :] = np.nan                                      # all NaN -> 0
    rows[2, :] = -np.inf; rows[2, 7] = np.nan               # -inf row with a NaN -> first -inf (0)
    rows[3, 20000] = 2.0; rows[3, 100] = 2.0                 # tie across chunks -> lowest
    rows[4, 16383] = 3.0; rows[4, 16384] = 3.0               # tie at a chunk boundary
    rows[5, :] = 0.0; rows[5, :5] = -0.0                    # -0 == +0 -> index 0
    rows[6, V - 1] = np.inf; rows[6, V - 2] = np.inf         # inf ties -> lowest
    rows[7, V - 1] = 7.0                                     # max in the ragged last chunk
    logits = rows if dtype == F32 else bf16_bits(np.nan_to_num(rows, nan=0.0))
    if dtype == BF16:
        logits = logits.copy()
        nanbits = np.uint16(0x7FC0)
        logits[0, 3] = nanbits; logits[1, :] = nanbits; logits[2, 7] = nanbits
    tok = np.zeros((1, 8), dtype=np.int32)
    got = gpu_accept(hrs, logits[None], tok)
    expect = [10, 0, 0, 100, 16383, 0, V - 2, V - 1]
    assert list(got[0][0]) == expect
    assert list(oacc.argmax_rows(logits)) == expect


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_accept_signalling_nan_patterns(hrs, dtype):
    """NaN bit patterns whose quiet bit is clear (a bf16 NaN widens to such a
    float32) never win either, before or after the true maximum, in the same
    or another chunk; a row of them alone gives 0."""
    V = 16384 + 1024
    if dtype == F32:
        pats = np.array([0x7F800001, 0xFF800001, 0x7FBFFFFF, 0x7FC00000], dtype=np.uint32)
        rows = np.full((5, V), -3.0, dtype=np.float32)
        bits = rows.view(np.uint32)
    else:
        pats = np.array([0x7F81, 0xFF81, 0x7FBF, 0xFFFF], dtype=np.uint16)
        rows = bf16_bits(np.full((5, V), -3.0, dtype=np.float32))
        bits = rows
    bits[0, 5] = pats[0]; rows_max = {0: 4000}
    bits[1, 16400] = pats[1]; rows_max[1] = 17
    bits[2, :] = pats[2]                                # every entry NaN -> 0
    bits[3, 0] = pats[0]; bits[3, 1] = pats[2]; rows_max[3] = 16383
    bits[4, ::3] = pats[3]; rows_max[4] = V - 1
    for r, i in rows_max.items():
        if dtype == F32:
            rows[r, i] = 1.5
        else:
            rows[r, i] = bf16_bits(np.float32(1.5))
    tok = np.zeros((1, 5), dtype=np.int32)
    got = gpu_accept(hrs, rows[None], tok)
    expect = [4000, 17, 0, 16383, V - 1]
    assert list(oacc.argmax_rows(rows)) == expect
    assert list(got[0][0]) == expect



@pytest.mark.parametrize("V", [8, 16384, 32768, 16384 + 8])
def test_accept_vocab_at_chunk_boundaries(hrs, V):
    """Vocabularies that end exactly at a pass-1 chunk boundary (one or two
    whole 16384-logit chunks), a single 8-logit slice, and one slice past a
    boundary: every row's argmax equals the oracle's, with the maximum in the
    first slot, the last slot, a tie across the last boundary, and random."""
    rng = np.random.default_rng(V)
    rows = rng.standard_normal((5, V)).astype(np.float32)
    rows[0, 0] = 9.0
    rows[1, V - 1] = 9.0
    rows[2, V - 1] = 9.0; rows[2, max(0, V - 16385)] = 9.0   # tie: the lower index wins
    logits = bf16_bits(rows)
    tok = np.zeros((1, 5), dtype=np.int32)
    say(f"accept vocab {V}")
    got = gpu_accept(hrs, logits[None], tok)
    expect = list(oacc.argmax_rows(logits))
    assert expect[0] == 0 and expect[1] == V - 1 and expect[2] == max(0, V - 16385)
    assert list(got[0][0]) == expect

def test_accept_workspace_reused_across_calls(hrs):
    """Workspace contents are ignored on entry: one buffer serves consecutive
    calls of different sizes, with garbage written into it between them, and
    every result equals the oracle's."""
    torch = _torch()
    big = scaled(QWEN_STACK_CHAIN, n_req=5, vocab=24576)
    small = scaled(QWEN_STACK_TREE, n_req=2, vocab=8200)
    nbytes = max(hrs.accept_greedy_workspace_bytes(5, big.n_pos, big.vocab, hrs.HRS_BF16),
                 hrs.accept_greedy_workspace_bytes(2, small.n_pos, small.vocab, hrs.HRS_BF16))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for w in (big, small, big):
        ws.fill_(0xA5)
        acc = [gen_accept(w, r) for r in range(w.n_req)]
        lg = np.stack([a.logits for a in acc])
        tok = np.stack([a.tokens for a in acc])
        par = np.stack([a.parent for a in acc]) if w.tree else None
        R, T = tok.shape
        outs = [torch.full(sh, -7, dtype=torch.int32, device="cuda") for sh in [(R, T), (R,), (R,), (R, T), (R,)]]
        hrs.accept_greedy(to_torch(lg), to_torch(tok), *outs, ws, parent=par)
        torch.cuda.synchronize()
        check_accept([to_numpy(o) for o in outs], lg, tok, par)
        assert [int(x) for x in to_numpy(outs[1])] == [a.planted_node for a in acc]


def test_accept_tree_batch_over_two_launches(hrs):
    """64-position trees for 50 requests: the parent table of one walk launch
    holds 48 of them, so the walk runs as two launches over the requests'
    keys and outputs."""
    rng = np.random.default_rng(33)
    R, T, V = 50, 64, 1024
    par = np.stack([np.concatenate([[-1], [rng.integers(max(0, i - 3), i) for i in range(1, T)]])
                    for _ in range(R)]).astype(np.int32)
    lg = rng.standard_normal((R, T, V)).astype(np.float32)
    oam = oacc.argmax_rows(lg)
    tok = np.zeros((R, T), dtype=np.int32)
    for r in range(R):
        for t in range(1, T):
            # the draft matches its parent's argmax on most positions
            tok[r, t] = oam[r, par[r, t]] if rng.random() < 0.8 else (oam[r, par[r, t]] + 1) % V
    got = gpu_accept(hrs, lg, tok, parent=par)
    check_accept(got, lg, tok, par)


# ---------------------------------------------------------------------------
# rollback


@pytest.mark.parametrize("Hv,dv,dk,C", [(4, 64, 64, 64),      # state exactly one 64 KiB block
                                          (3, 48, 64, 24),      # 36 KiB state: one partial block
                                          (3, 112, 128, 1000)])  # 2.6 blocks, odd conv width
def test_rollback_copies_checkpoint_and_flags_bad_index(hrs, Hv, dv, dk, C):
    torch = _torch()
    L, R, T = 2, 3, 5
    rng = np.random.default_rng(4)
    ckpt = rng.standard_normal((L, R, T, Hv, dv, dk)).astype(np.float32)
    state0 = rng.standard_normal((L, R, Hv, dv, dk)).astype(np.float32)
    cck = bf16_bits(rng.standard_normal((L, R, T, 3, C)).astype(np.float32))
    cs0 = bf16_bits(rng.standard_normal((L, R, 3, C)).astype(np.float32))
    node = np.array([2, 7, 0], dtype=np.int32)
    d_ck, d_st, d_cck, d_cs = to_torch(ckpt), to_torch(state0), to_torch(cck), to_torch(cs0)
    status = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    hrs.rollback_restore(d_ck, d_st, d_cck, d_cs, to_torch(node), status)
    torch.cuda.synchronize()
    st, cs, stat = to_numpy(d_st), to_numpy(d_cs), to_numpy(status)
    assert stat[0] == 1
    for l in range(L):
        for r in range(R):
            if node[r] < T:
                assert np.array_equal(st[l, r], ckpt[l, r, node[r]])
                assert np.array_equal(cs[l, r], cck[l, r, node[r]])
            else:
                assert np.array_equal(st[l, r], state0[l, r]) and np.array_equal(cs[l, r], cs0[l, r])
    node2 = np.array([4, 1, 3], dtype=np.int32)
    hrs.rollback_restore(d_ck, d_st, None, None, to_torch(node2), status)
    torch.cuda.synchronize()
    assert to_numpy(status)[0] == 0
    assert np.array_equal(to_numpy(d_st)[:, 1], ckpt[:, 1, 1])


def test_rollback_equals_replay_after_span(hrs):
    """GDN + conv span, then rollback to the accepted node: equals the oracle's
    replay of the accepted path from the pre-span state (chain and tree)."""
    torch = _torch()
    for w, tree in ((scaled(QWEN_LAYER_CHAIN, n_req=2), False),
                    (scaled(QWEN_STACK_TREE, n_layers=1, n_req=2), True)):
        units = [gen_unit(w, 0, r) for r in range(2)]
        wt = gen_conv_weight(w, 0)
        parents = np.stack([gen_tree_parent(w, r) for r in range(2)]) if tree else None
        st = lambda name: to_torch(np.stack([getattr(u, name) for u in units]))
        R, T, Hv, dv, dk, C = 2, w.n_pos, w.n_vheads, w.d_v, w.d_k, w.conv_channels
        state, cs = st("state"), st("conv_state")
        ckpt = torch.empty((1, R, T, Hv, dv, dk), device="cuda")
        cck = torch.empty((1, R, T, 3, C), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((R, T, Hv, dv), device="cuda")
        y = torch.empty((R, T, C), device="cuda")
        hrs.conv1d_verify_span(st("x"), to_torch(wt), cs, cck[0], y, parent=parents)
        hrs.gdn_verify_span(st("q"), st("k"), st("v"), st("a"), st("b"), state, ckpt[0], out, parent=parents)
        node = np.array([gen_accept(w, r, with_logits=False).planted_node for r in range(2)], dtype=np.int32)
        status = torch.zeros(4, dtype=torch.int32, device="cuda")
        hrs.rollback_restore(ckpt, state[None], cck, cs[None], to_torch(node), status)
        torch.cuda.synchronize()
        got_s, got_c = to_numpy(state), to_numpy(cs)
        assert to_numpy(status)[0] == 0
        for r, u in enumerate(units):
            path, n = [], int(node[r])
            while n >= 0:
                path.append(n)
                n = (parents[r][n] if tree else n - 1)
            path = path[::-1]
            ref = orb.replay_state(u.state, u.q, u.k, u.v, u.a, u.b, path)
            assert_tiles(got_s[r], ref, 2, f"rollback state r={r} tree={tree}")
            assert np.array_equal(got_c[r], orb.replay_conv_state(u.conv_state, u.x, path))


# ---------------------------------------------------------------------------
# ring


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_ring_set_get_vs_oracle(hrs, dtype):
    rng = np.random.default_rng(8)
    n_rings, S, D = 4, 64, 320
    raw = rng.standard_normal((n_rings, S, D)).astype(np.float32)
    ring0 = bf16_bits(raw) if dtype == BF16 else raw
    pk_raw = rng.standard_normal((40, D)).astype(np.float32)
    packed = bf16_bits(pk_raw) if dtype == BF16 else pk_raw
    runs = [(0, 60, 9, 0), (1, 3, 20, 9), (2, 63, 2, 29), (3, 10, 9, 31)]   # runs 0 and 2 wrap
    ring = to_torch(ring0)
    pk = to_torch(packed)
    _torch().cuda.synchronize()
    hrs.ring_set_2d(ring, pk, runs)
    out = to_torch(np.zeros_like(packed))
    hrs.ring_get_2d(ring, out, runs)
    _torch().cuda.synchronize()
    exp_ring = oring.ring_set(ring0, packed, runs)
    assert np.array_equal(to_numpy(ring), exp_ring)
    assert np.array_equal(to_numpy(out), oring.ring_get(exp_ring, np.zeros_like(packed), runs))


def test_ring_run_longer_than_one_launch_extent(hrs):
    """A run of 68,000 rows (more than the 65,535 rows one grid dimension of a
    launch holds) into a 70,000-slot ring, beside a wrapping run: set and get
    against the oracle."""
    rng = np.random.default_rng(9)
    n_rings, S, D = 2, 70000, 8
    ring0 = bf16_bits(rng.standard_normal((n_rings, S, D)).astype(np.float32))
    packed = bf16_bits(rng.standard_normal((68050, D)).astype(np.float32))
    runs = [(0, 1000, 68000, 0), (1, 69990, 50, 68000)]   # run 1 wraps
    say("ring 2 x 70000 slots, runs of 68000 and 50 rows")
    ring = to_torch(ring0)
    pk = to_torch(packed)
    _torch().cuda.synchronize()
    hrs.ring_set_2d(ring, pk, runs)
    out = to_torch(np.zeros_like(packed))
    hrs.ring_get_2d(ring, out, runs)
    _torch().cuda.synchronize()
    exp_ring = oring.ring_set(ring0, packed, runs)
    assert np.array_equal(to_numpy(ring), exp_ring)
    assert np.array_equal(to_numpy(out), oring.ring_get(exp_ring, np.zeros_like(packed), runs))


def test_gdn_persistent_multi_window_chain(hrs):
    """8 requests of the Qwen shape (one 12-wave block per CU walking 1024
    32-row units) over 40 positions (two LDS windows per unit): the producer
    waves stage window 2 and the next unit while the consumers run; sampled
    requests against the oracle, the rest against the 4-wave launch of the
    same requests one at a time."""
    import torch
    w = scaled(QWEN_LAYER_CHAIN, n_req=8, n_pos=40)
    units = [gen_unit(w, 0, r) for r in range(w.n_req)]
    say("persistent chain R=8 T=40")
    ck, out, _ = gpu_gdn(hrs, units)
    check_gdn_vs_oracle([units[0], units[5]], ck[[0, 5]], out[[0, 5]], what="persistent T=40")
    for r in range(w.n_req):
        ck1, out1, _ = gpu_gdn(hrs, [units[r]])
        assert np.array_equal(ck[r], ck1[0]) and np.array_equal(out[r], out1[0]), r


def test_gdn_persistent_zero_copy_invalid_node(hrs):
    """Zero-copy start on the persistent launch: an out-of-range index writes
    nothing for that request and is counted; the others equal the copied start."""
    import torch
    w = scaled(QWEN_LAYER_CHAIN, n_req=8, n_pos=17)
    units = [gen_unit(w, 0, r) for r in range(w.n_req)]
    st = lambda name: to_torch(np.stack([getattr(u, name) for u in units]))
    R, T, Hv, d = 8, 17, 32, 128
    gen = torch.Generator(device="cuda").manual_seed(11)
    prev = torch.randn((R, 5, Hv, d, d), device="cuda", generator=gen) * 0.02
    node = torch.tensor([4, 0, 2, 9, 1, 3, 4, -1], dtype=torch.int32, device="cuda")   # requests 3 and 7 invalid
    status = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    ckpt = torch.full((R, T, Hv, d, d), float("nan"), device="cuda")
    out = torch.full((R, T, Hv, d), float("nan"), device="cuda")
    hrs.gdn_verify_span_from(prev, node, st("q"), st("k"), st("v"), st("a"), st("b"), ckpt, out, status=status)
    idx = [4, 0, 2, 0, 1, 3, 4, 0]
    state = torch.stack([prev[r, idx[r]] for r in range(R)]).contiguous()
    ck_ref = torch.empty_like(ckpt)
    out_ref = torch.empty_like(out)
    hrs.gdn_verify_span(st("q"), st("k"), st("v"), st("a"), st("b"), state, ck_ref, out_ref)
    torch.cuda.synchronize()
    assert int(to_numpy(status)[0]) == 2
    for r in range(R):
        if r in (3, 7):
            assert torch.isnan(ckpt[r]).all() and torch.isnan(out[r]).all(), r
        else:
            assert torch.equal(ckpt[r], ck_ref[r]) and torch.equal(out[r], out_ref[r]), r


def test_gdn_persistent_dk64_bf16(hrs):
    """d_k = d_v = 64 on the persistent producer/consumer launch (4 requests x
    32 value heads x 2 row blocks = 256 units of 32 rows), bf16."""
    w = scaled(QWEN_LAYER_CHAIN, n_req=4, n_pos=20, d_k=64, d_v=64)
    units = [gen_unit(w, 0, r) for r in range(w.n_req)]
    say("persistent dk64 R=4 T=20")
    ck, out, _ = gpu_gdn(hrs, units, q_scale=0.125)
    check_gdn_vs_oracle(units, ck, out, q_scale=0.125, what="persistent dk64")


def test_gdn_span_prefix_equals_shorter_span(hrs):
    """The first j+1 checkpoints and outputs of a 17-position span equal a
    (j+1)-position span over the same inputs, bit for bit (the arithmetic of a
    position does not depend on the span length or the launch shape)."""
    w = scaled(QWEN_LAYER_CHAIN, n_req=8)
    units = [gen_unit(w, 0, r) for r in range(w.n_req)]
    ck, out, _ = gpu_gdn(hrs, units)
    for j in (0, 4, 15):
        short = [scaled_unit(u, j + 1) for u in units]
        cks, outs, _ = gpu_gdn(hrs, short)
        assert np.array_equal(ck[:, :j + 1], cks) and np.array_equal(out[:, :j + 1], outs), j


def scaled_unit(u, n):
    import dataclasses
    return dataclasses.replace(u, q=u.q[:n], k=u.k[:n], v=u.v[:n], a=u.a[:n], b=u.b[:n], x=u.x[:n])
