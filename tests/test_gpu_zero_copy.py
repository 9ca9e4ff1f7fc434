"""Zero-copy rollback and compact conv state: over several consecutive verify
steps, the zero-copy step (spans start from the previous span's checkpoint at
the accepted position; conv state rebuilt from the accepted path) must produce
bit for bit what the checkpoint-copy step produces, and the materialised state
must equal the copied one. Sampled (layer, request) units of every step are
also checked against the oracle, whose state between steps is the replay of
the accepted path from the previous step's state (openinfer PR #626, What
Changed: conservative commit; lucebox PR #506, Summary: restore without
replay). Graph replays of the zero-copy and fused steps are checked the same
way. Invalid indices leave outputs untouched and are counted in the status
word."""
import numpy as np
import pytest

from oracle import rollback as orb
from synth import QWEN_STACK_CHAIN, QWEN_STACK_TREE, QWEN_LAYER_CHAIN, bf16_bits, gen_unit, scaled
from tests.gpu_util import say, to_numpy, to_torch
from tests.step_oracle import TrackedUnit, unit_slices

pytestmark = pytest.mark.gpu


def make(w, zero_copy, fused=False):
    from hybrid_recurrent_state_amd.step import FusedVerifyStep, StepBuffers, VerifyStep, ZeroCopyVerifyStep
    from synth.device import fill_step, step_shape
    bufs = StepBuffers(step_shape(w))
    loaded = fill_step(bufs, w)
    cls = FusedVerifyStep if fused else (ZeroCopyVerifyStep if zero_copy else VerifyStep)
    return bufs, cls(bufs, parent=loaded.parent, runs=loaded.runs), loaded


ZC_WORKLOADS = [
    (scaled(QWEN_STACK_CHAIN, n_layers=3, n_req=3, vocab=4096, ring_slots=64, ring_width=256), [(0, 1), (2, 2)]),
    (scaled(QWEN_STACK_TREE, n_layers=2, n_req=2, vocab=4096), [(1, 1)]),
]


@pytest.mark.parametrize("w,samples", ZC_WORKLOADS)
def test_zero_copy_steps_equal_copy_steps(w, samples):
    import torch
    std_bufs, std, _ = make(w, False)
    zc_bufs, zc, loaded = make(w, True)
    units = [TrackedUnit(w, loaded, l, r) for (l, r) in samples]
    for i in range(3):
        acc_s, bon_s = std.run()
        acc_z, bon_z = zc.run()
        assert np.array_equal(acc_s, acc_z) and np.array_equal(bon_s, bon_z), i
        for name in ("argmax", "accept_node", "path", "y", "out", "conv_state"):
            assert np.array_equal(to_numpy(getattr(std_bufs, name)), to_numpy(getattr(zc_bufs, name))), (i, name)
        assert np.array_equal(to_numpy(std_bufs.ckpt), to_numpy(zc.current_ckpt())), (i, "ckpt")
        if w.ring_slots:
            assert np.array_equal(to_numpy(std_bufs.packed_out), to_numpy(zc_bufs.packed_out)), i
        for tu in units:
            assert int(acc_z[tu.r]) == tu.acc.accept_len
            tu.check(i, *unit_slices(zc_bufs, zc.current_ckpt(), tu.l, tu.r), what="zero-copy")
        say(f"step {i}: accepted {list(map(int, acc_z))}")
    zc.materialize()
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy(std_bufs.state), to_numpy(zc_bufs.state))
    assert to_numpy(zc_bufs.status)[0] == 0
    for tu in units:
        tu.check_state(to_numpy(zc_bufs.state[tu.l, tu.r]), what="zero-copy")


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("w,samples", ZC_WORKLOADS)
def test_zero_copy_graph_replays(w, samples, fused):
    """Two captured graphs (one per checkpoint-buffer parity) replayed
    alternately, with unrelated eager work and host syncs between replays:
    every replay equals the eagerly launched step bit for bit, and sampled
    units equal the oracle."""
    import torch
    if fused:
        w = scaled(w, conv_channels=2 * w.n_kheads * w.d_k + w.n_vheads * w.d_v)
    e_bufs, eager, _ = make(w, True, fused)
    g_bufs, graphed, loaded = make(w, True, fused)
    graphed.capture_graph()
    units = [TrackedUnit(w, loaded, l, r, fused=fused) for (l, r) in samples]
    scratch = torch.randn(1 << 20, device="cuda")
    for i in range(4):
        acc_e, bon_e = eager.run()
        acc_g, bon_g = graphed.replay()      # step 0 eagerly (from state), then graph parities 0, 1, 0
        assert np.array_equal(acc_e, acc_g) and np.array_equal(bon_e, bon_g), i
        names = ("argmax", "accept_node", "path", "out", "conv_state") + (() if fused else ("y",))
        for name in names:
            assert np.array_equal(to_numpy(getattr(e_bufs, name)), to_numpy(getattr(g_bufs, name))), (i, name)
        assert np.array_equal(to_numpy(eager.current_ckpt()), to_numpy(graphed.current_ckpt())), (i, "ckpt")
        for tu in units:
            tu.check(i, *unit_slices(g_bufs, graphed.current_ckpt(), tu.l, tu.r, with_y=not fused),
                     what=("fused" if fused else "zero-copy") + " graph")
        scratch.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        say(f"replay {i}: accepted {list(map(int, acc_g))}")


def test_span_from_invalid_node_writes_nothing():
    import torch
    import hybrid_recurrent_state_amd as hrs
    w = scaled(QWEN_LAYER_CHAIN, n_req=2, n_kheads=4, n_vheads=8, n_pos=5)
    units = [gen_unit(w, 0, r) for r in range(2)]
    st = lambda name: to_torch(np.stack([getattr(u, name) for u in units]))
    R, T, Hv, d = 2, 5, 8, 128
    prev = torch.randn(R, 7, Hv, d, d, device="cuda")
    node = torch.tensor([3, 9], dtype=torch.int32, device="cuda")      # request 1 out of range
    ckpt = torch.full((R, T, Hv, d, d), float("nan"), device="cuda")
    out = torch.full((R, T, Hv, d), float("nan"), device="cuda")
    status = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    hrs.gdn_verify_span_from(prev, node, st("q"), st("k"), st("v"), st("a"), st("b"), ckpt, out, status=status)
    # reference: the plain span from the copied state of request 0
    state = prev[:, 3].contiguous()
    ck_ref = torch.empty_like(ckpt)
    out_ref = torch.empty_like(out)
    hrs.gdn_verify_span(st("q"), st("k"), st("v"), st("a"), st("b"), state, ck_ref, out_ref)
    torch.cuda.synchronize()
    assert to_numpy(status)[0] == 1
    assert torch.equal(ckpt[0], ck_ref[0]) and torch.equal(out[0], out_ref[0])
    assert torch.isnan(ckpt[1]).all() and torch.isnan(out[1]).all()


def test_conv_state_advance_vs_replay():
    import torch
    import hybrid_recurrent_state_amd as hrs
    rng = np.random.default_rng(12)
    L, R, T, C = 2, 5, 6, 1032
    x = bf16_bits(rng.standard_normal((L, R, T, C)).astype(np.float32))
    cs = bf16_bits(rng.standard_normal((L, R, 3, C)).astype(np.float32))
    parent = np.array([-1, 0, 1, 0, 3, 4], dtype=np.int32)
    nodes = [0, 1, 2, 5, 4]                       # path lengths 1, 2, 3, 4, 3 (tree paths)
    paths = np.full((R, T), -1, dtype=np.int32)
    lens = np.zeros(R, dtype=np.int32)
    for r, u in enumerate(nodes):
        p, n = [], u
        while n >= 0:
            p.append(n)
            n = parent[n]
        p = p[::-1]
        paths[r, :len(p)] = p
        lens[r] = len(p) - 1
    lens_bad = lens.copy()
    lens_bad[4] = T                                 # out of range: request 4 untouched
    x_d, cs_d = to_torch(x), to_torch(cs)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    hrs.conv_state_advance(x_d, cs_d, to_torch(paths), to_torch(lens_bad), status=status)
    torch.cuda.synchronize()
    got = to_numpy(cs_d)
    assert to_numpy(status)[0] == 1
    for l in range(L):
        for r in range(R):
            if r == 4:
                assert np.array_equal(got[l, r], cs[l, r])
            else:
                exp = orb.replay_conv_state(cs[l, r], x[l, r], paths[r])
                assert np.array_equal(got[l, r], exp), (l, r)
