"""GPU parity of the fused layer entry point (conv, SiLU, split, q/k L2 norm
and the gated delta rule in one kernel) against the fused-layer oracle,
through the C ABI. Bar: max relative error 1e-4 per tile for checkpoints and
outputs; the zero-copy start must equal the copied start bit for bit."""
import numpy as np
import pytest

from oracle import fused as ofu
from synth import (F32, QWEN_LAYER_CHAIN, QWEN_STACK_TREE, TINY_CHAIN, gen_conv_weight, gen_tree_parent, gen_unit,
                   scaled)
from tests.gpu_util import assert_tiles, say, to_numpy, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hrs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import hybrid_recurrent_state_amd as m
    return m


def layer_workload(w, **kw):
    """The workload with its conv channels set to the layer's q | k | v width."""
    w = scaled(w, **kw)
    return scaled(w, conv_channels=2 * w.n_kheads * w.d_k + w.n_vheads * w.d_v)


def run_layer(hrs, w, parents=None, q_scale=1.0, silu=True, eps=1e-6, layer=0):
    import torch
    units = [gen_unit(w, layer, r) for r in range(w.n_req)]
    st = lambda name: to_torch(np.stack([getattr(u, name) for u in units]))
    x, cs, a, b, state = st("x"), st("conv_state"), st("a"), st("b"), st("state")
    wc = gen_conv_weight(w, layer)
    R, T, Hv, dv, dk = w.n_req, w.n_pos, w.n_vheads, w.d_v, w.d_k
    ckpt = torch.full((R, T, Hv, dv, dk), float("nan"), device="cuda")
    out = torch.full((R, T, Hv, dv), float("nan"), device="cuda")
    par = None if parents is None else np.stack(parents)
    say(f"layer span {w.name}: R={R} T={T} Hk={w.n_kheads} Hv={Hv} dk={dk} dv={dv} tree={parents is not None}")
    hrs.gdn_layer_verify_span(x, to_torch(wc), cs, a, b, ckpt, out, w.n_kheads, dk, state=state, parent=par,
                              q_scale=q_scale, l2_eps=eps, silu=silu)
    torch.cuda.synchronize()
    return units, wc, to_numpy(ckpt), to_numpy(out)


def check_layer(w, units, wc, ck, out, parents=None, q_scale=1.0, silu=True, eps=1e-6, what=""):
    for r, u in enumerate(units):
        par = None if parents is None else parents[r]
        ock, oout, _ = ofu.layer_span(u.x, wc, u.conv_state, u.a, u.b, u.state, w.n_kheads, w.n_vheads, w.d_k,
                                      w.d_v, parent=par, q_scale=q_scale, eps=eps, silu=silu)
        e1 = assert_tiles(ck[r], ock, 2, f"{what} ckpt r={r}")
        e2 = assert_tiles(out[r], oout, 1, f"{what} out r={r}")
        say(f"{what} r={r}: ckpt err {e1:.2e}, out err {e2:.2e}")


@pytest.mark.parametrize("silu", [True, False])
def test_layer_tiny_chain_f32(hrs, silu):
    w = layer_workload(TINY_CHAIN, n_req=2)
    units, wc, ck, out = run_layer(hrs, w, q_scale=0.125, silu=silu)
    check_layer(w, units, wc, ck, out, q_scale=0.125, silu=silu, what="tiny chain")


def test_layer_qwen_chain_bf16(hrs):
    w = layer_workload(QWEN_LAYER_CHAIN, n_req=2)
    assert w.conv_channels == 8192
    units, wc, ck, out = run_layer(hrs, w, q_scale=128 ** -0.5)
    check_layer(w, units, wc, ck, out, q_scale=128 ** -0.5, what="qwen chain")


def test_layer_qwen_tree_bf16(hrs):
    w = layer_workload(QWEN_STACK_TREE, n_req=2, n_layers=1)
    parents = [gen_tree_parent(w, r) for r in range(w.n_req)]
    units, wc, ck, out = run_layer(hrs, w, parents=parents)
    check_layer(w, units, wc, ck, out, parents=parents, what="qwen tree")


@pytest.mark.parametrize("T,tree", [(40, False), (64, True), (33, True)])
def test_layer_long_spans_cross_lds_windows(hrs, T, tree):
    w = layer_workload(TINY_CHAIN, n_req=2, n_pos=T, n_kheads=1, n_vheads=4, d_k=128, d_v=32, tree=tree,
                       tree_max_depth=64)
    parents = [gen_tree_parent(w, r) for r in range(w.n_req)] if tree else None
    units, wc, ck, out = run_layer(hrs, w, parents=parents)
    check_layer(w, units, wc, ck, out, parents=parents, what=f"T={T} tree={tree}")


def test_layer_tree_batch_split_over_launches(hrs):
    # 26 requests of a 23-position tree need two launches of the tree geometry.
    w = layer_workload(QWEN_STACK_TREE, n_req=26, n_layers=1, n_kheads=1, n_vheads=2, d_k=64, d_v=16, dtype=F32)
    parents = [gen_tree_parent(w, r) for r in range(w.n_req)]
    units, wc, ck, out = run_layer(hrs, w, parents=parents, q_scale=0.5)
    check_layer(w, units, wc, ck, out, parents=parents, q_scale=0.5, what="26-request tree")


def test_layer_grouped_heads_dk64(hrs):
    w = layer_workload(TINY_CHAIN, n_req=3, n_kheads=2, n_vheads=8, d_k=64, d_v=48)
    units, wc, ck, out = run_layer(hrs, w, eps=1e-3)
    check_layer(w, units, wc, ck, out, eps=1e-3, what="grouped dk64")


def test_layer_from_checkpoint_equals_from_state(hrs):
    import torch
    w = layer_workload(QWEN_LAYER_CHAIN, n_req=3, n_pos=9, n_kheads=4, n_vheads=8)
    units = [gen_unit(w, 0, r) for r in range(w.n_req)]
    st = lambda name: to_torch(np.stack([getattr(u, name) for u in units]))
    x, cs, a, b = st("x"), st("conv_state"), st("a"), st("b")
    wc = to_torch(gen_conv_weight(w, 0))
    R, T, Hv, d = w.n_req, w.n_pos, w.n_vheads, w.d_k
    gen = torch.Generator(device="cuda").manual_seed(5)
    prev = torch.randn((R, 6, Hv, d, d), device="cuda", generator=gen) * 0.02
    node = torch.tensor([5, 0, 7], dtype=torch.int32, device="cuda")    # request 2 out of range
    status = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    ck = torch.full((R, T, Hv, d, d), float("nan"), device="cuda")
    out = torch.full((R, T, Hv, d), float("nan"), device="cuda")
    hrs.gdn_layer_verify_span(x, wc, cs, a, b, ck, out, w.n_kheads, d, src_ckpt=prev, src_node=node,
                              status=status)
    state = torch.stack([prev[0, 5], prev[1, 0], prev[2, 0]]).contiguous()
    ck_ref = torch.empty_like(ck)
    out_ref = torch.empty_like(out)
    hrs.gdn_layer_verify_span(x, wc, cs, a, b, ck_ref, out_ref, w.n_kheads, d, state=state)
    torch.cuda.synchronize()
    assert int(to_numpy(status)[0]) == 1
    assert torch.equal(ck[:2], ck_ref[:2]) and torch.equal(out[:2], out_ref[:2])
    assert torch.isnan(ck[2]).all() and torch.isnan(out[2]).all()


@pytest.mark.parametrize("tree", [False, True])
def test_fused_step_equals_layer_calls(hrs, tree):
    """Three fused zero-copy steps: every layer's span equals a direct
    gdn_layer_verify_span call from the materialised state and the conv state
    as rebuilt, bit for bit; the first step also matches the oracle."""
    import torch
    from hybrid_recurrent_state_amd.step import FusedVerifyStep, StepBuffers
    from synth.device import fill_step, step_shape
    base = QWEN_STACK_TREE if tree else scaled(QWEN_LAYER_CHAIN, vocab=4096)
    w = layer_workload(base, n_layers=2, n_req=2, n_kheads=4, n_vheads=8, vocab=4096)
    bufs = StepBuffers(step_shape(w))
    loaded = fill_step(bufs, w)
    step = FusedVerifyStep(bufs, parent=loaded.parent, runs=loaded.runs, q_scale=0.25)
    L, R = w.n_layers, w.n_req
    par = None if loaded.parent is None else np.asarray(loaded.parent)
    for i in range(3):
        state0 = bufs.state.clone() if i == 0 else None
        if i > 0:
            step.materialize()
            state0 = bufs.state.clone()
        cs0 = bufs.conv_state.clone()
        acc, bonus = step.run()
        say(f"fused step {i}: accepted {list(map(int, acc))}")
        ck = step.current_ckpt()
        for l in range(L):
            ck_ref = torch.empty_like(ck[l])
            out_ref = torch.empty_like(bufs.out[l])
            hrs.gdn_layer_verify_span(bufs.x[l], bufs.w[l], cs0[l], bufs.a[l], bufs.b[l], ck_ref, out_ref,
                                      w.n_kheads, w.d_k, state=state0[l].contiguous(), parent=par, q_scale=0.25)
            torch.cuda.synchronize()
            assert torch.equal(ck[l], ck_ref), (i, l)
            assert torch.equal(bufs.out[l], out_ref), (i, l)
            if i == 0:
                xs, ws, css, a_, b_, st_ = (to_numpy(t) for t in (bufs.x[l], bufs.w[l], cs0[l], bufs.a[l],
                                                                  bufs.b[l], state0[l]))
                for r in range(R):
                    pr = None if par is None else par[r]
                    ock, oout, _ = ofu.layer_span(xs[r], ws, css[r], a_[r], b_[r], st_[r], w.n_kheads, w.n_vheads,
                                                  w.d_k, w.d_v, parent=pr, q_scale=0.25)
                    assert_tiles(to_numpy(ck[l, r]), ock, 2, f"step ckpt l={l} r={r}")
                    assert_tiles(to_numpy(bufs.out[l, r]), oout, 1, f"step out l={l} r={r}")


def test_layer_persistent_multi_window(hrs):
    """8 requests (persistent producer/consumer launch) over 40 positions:
    two windows per unit, fused staging by the producer waves; two requests
    against the oracle, every request against its own single-request launch."""
    import torch
    w = layer_workload(QWEN_LAYER_CHAIN, n_req=8, n_pos=40)
    units, wc, ck, out = run_layer(hrs, w, q_scale=0.3)
    check_layer(w, [units[1], units[6]], wc, ck[[1, 6]], out[[1, 6]], q_scale=0.3, what="fused persistent T=40")
    for r in range(w.n_req):
        u = units[r]
        x, cs, a, b, state = (to_torch(t[None]) for t in (u.x, u.conv_state, u.a, u.b, u.state))
        ck1 = torch.empty((1, w.n_pos, w.n_vheads, w.d_v, w.d_k), device="cuda")
        out1 = torch.empty((1, w.n_pos, w.n_vheads, w.d_v), device="cuda")
        hrs.gdn_layer_verify_span(x, to_torch(wc), cs, a, b, ck1, out1, w.n_kheads, w.d_k, state=state, q_scale=0.3)
        torch.cuda.synchronize()
        assert np.array_equal(ck[r], to_numpy(ck1)[0]) and np.array_equal(out[r], to_numpy(out1)[0]), r


def test_layer_persistent_dk64(hrs):
    """Fused layer with d_k = d_v = 64 (q/k rows are 4-lane DPP groups) on the
    persistent launch: 4 requests x 32 value heads x 2 row blocks."""
    w = layer_workload(QWEN_LAYER_CHAIN, n_req=4, n_pos=20, d_k=64, d_v=64)
    units, wc, ck, out = run_layer(hrs, w, q_scale=0.125)
    check_layer(w, units, wc, ck, out, q_scale=0.125, what="fused persistent dk64")


def test_layer_random_shapes(hrs):
    """Seeded sweep over layer shapes (d_k 64/128, d_v 16-128, 1-4 value
    heads per key head, 1-4 requests, 1-40 positions, chain or random tree,
    bf16 or f32, SiLU on or off), each against the fused-layer oracle."""
    rng = np.random.default_rng(4048)
    for i in range(8):
        dk = int(rng.choice([64, 128]))
        dv = int(rng.choice([16, 32, 48, 64, 128]))
        Hk = int(rng.choice([1, 2]))
        Hv = Hk * int(rng.choice([1, 2, 4]))
        R = int(rng.integers(1, 5))
        T = int(rng.integers(1, 41))
        dt = TINY_CHAIN.dtype if rng.random() < 0.4 else QWEN_LAYER_CHAIN.dtype
        tree = T > 2 and rng.random() < 0.5
        silu = bool(rng.random() < 0.7)
        q_scale = float(2.0 ** -int(rng.integers(0, 4)))
        w = layer_workload(TINY_CHAIN, n_req=R, n_pos=T, n_kheads=Hk, n_vheads=Hv, d_k=dk, d_v=dv, dtype=dt,
                           seed=300 + i)
        parents = None
        if tree:
            parents = [np.array([-1] + [int(rng.integers(0, t)) for t in range(1, T)], dtype=np.int32)
                       for _ in range(R)]
        what = f"layer shape {i}: R={R} T={T} Hk={Hk} Hv={Hv} dk={dk} dv={dv} {dt} silu={silu}"
        units, wc, ck, out = run_layer(hrs, w, parents=parents, q_scale=q_scale, silu=silu)
        check_layer(w, units, wc, ck, out, parents=parents, q_scale=q_scale, silu=silu, what=what)
