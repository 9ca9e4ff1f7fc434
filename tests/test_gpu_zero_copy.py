"""Zero-copy rollback and compact conv state: over several consecutive verify
steps, the zero-copy step (spans start from the previous span's checkpoint at
the accepted position; conv state rebuilt from the accepted path) must produce
bit for bit what the checkpoint-copy step produces, and the materialised state
must equal the copied one. Invalid indices leave outputs untouched and are
counted in the status word."""
import numpy as np
import pytest

from oracle import rollback as orb
from synth import QWEN_STACK_CHAIN, QWEN_STACK_TREE, QWEN_LAYER_CHAIN, bf16_bits, gen_unit, scaled
from tests.gpu_util import say, to_numpy, to_torch

pytestmark = pytest.mark.gpu


def make(w, zero_copy):
    from hybrid_recurrent_state_amd.step import StepBuffers, VerifyStep, ZeroCopyVerifyStep
    from synth.device import fill_step, step_shape
    bufs = StepBuffers(step_shape(w))
    loaded = fill_step(bufs, w)
    cls = ZeroCopyVerifyStep if zero_copy else VerifyStep
    return bufs, cls(bufs, parent=loaded.parent, runs=loaded.runs)


@pytest.mark.parametrize("w", [
    scaled(QWEN_STACK_CHAIN, n_layers=3, n_req=3, vocab=4096, ring_slots=64, ring_width=256),
    scaled(QWEN_STACK_TREE, n_layers=2, n_req=2, vocab=4096),
])
def test_zero_copy_steps_equal_copy_steps(w):
    import torch
    std_bufs, std = make(w, False)
    zc_bufs, zc = make(w, True)
    for i in range(3):
        acc_s, bon_s = std.run()
        acc_z, bon_z = zc.run()
        assert np.array_equal(acc_s, acc_z) and np.array_equal(bon_s, bon_z), i
        for name in ("argmax", "accept_node", "path", "y", "out", "conv_state"):
            assert np.array_equal(to_numpy(getattr(std_bufs, name)), to_numpy(getattr(zc_bufs, name))), (i, name)
        assert np.array_equal(to_numpy(std_bufs.ckpt), to_numpy(zc.current_ckpt())), (i, "ckpt")
        if w.ring_slots:
            assert np.array_equal(to_numpy(std_bufs.packed_out), to_numpy(zc_bufs.packed_out)), i
        say(f"step {i}: accepted {list(map(int, acc_z))}")
    zc.materialize()
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy(std_bufs.state), to_numpy(zc_bufs.state))
    assert to_numpy(zc_bufs.status)[0] == 0


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
