"""Full-size parity: each named workload at its real size, run through the
same VerifyStep launch sequence that bench.py times (one step: 48 x (conv,
GDN), acceptance, rollback, ring), then checked against the oracle.

The oracle cannot redo a whole 16 x 48-layer step in seconds, so:
  * acceptance (argmax of every row, accepted node, length, path, bonus) is
    checked for every request, bit-exact;
  * checkpoints, outputs, conv outputs and conv checkpoints are checked on
    sampled (layer, request) units, all positions and heads of each;
  * the rolled-back state of the sampled units is checked against the
    oracle's replay of the accepted path, and bit-exactly against the step's
    own checkpoint of the accepted node;
  * the feature ring is checked completely (every slot).
"""
import numpy as np
import pytest

from oracle import accept as oacc, conv as oconv, gdn as ogdn, ring as oring, rollback as orb
from synth import WORKLOADS, WORKLOAD_ORDER, gen_conv_weight, gen_unit
from tests.gpu_util import assert_tiles, say, to_numpy

pytestmark = pytest.mark.gpu

SAMPLES = {
    0: [(0, 0)],
    1: [(0, 0)],
    2: [(0, 0), (23, 0), (47, 0)],
    3: [(0, 0), (47, 15), (23, 7), (11, 4)],
    4: [(0, 0), (29, 0), (47, 0)],
}


def run_workload(idx):
    import torch
    import hybrid_recurrent_state_amd  # noqa: F401
    from hybrid_recurrent_state_amd.step import StepBuffers, VerifyStep
    from synth.device import fill_step, step_shape
    w = WORKLOADS[WORKLOAD_ORDER[idx]]
    say(f"workload {w.name}: allocating and filling")
    bufs = StepBuffers(step_shape(w))
    loaded = fill_step(bufs, w, keep_ring=bool(w.ring_slots))
    step = VerifyStep(bufs, parent=loaded.parent, runs=loaded.runs)
    say("one step")
    acc_len, bonus = step.run()
    torch.cuda.synchronize()
    return w, bufs, loaded, acc_len, bonus


@pytest.mark.parametrize("idx", [0, 1, 2, 4, 3])
def test_full_size_step(idx):
    w, bufs, loaded, acc_len, bonus = run_workload(idx)
    R, T = w.n_req, w.n_pos
    parents = loaded.parent
    # -- acceptance, every request -------------------------------------------
    node = to_numpy(bufs.accept_node)
    if w.vocab:
        am = to_numpy(bufs.argmax)
        path = to_numpy(bufs.path)
        for r in range(R):
            ai = loaded.accept[r]
            oam = oacc.argmax_rows(ai.logits)
            assert np.array_equal(am[r], oam), f"argmax r={r}"
            res = oacc.accept(oam, ai.tokens, None if parents is None else parents[r])
            assert node[r] == res.accept_node and acc_len[r] == res.accept_len and bonus[r] == res.bonus, r
            assert np.array_equal(path[r], res.path), r
            assert res.accept_node == ai.planted_node
        say(f"accept ok: accepted lengths {list(map(int, acc_len))}")
    else:
        assert [int(x) for x in node] == [a.planted_node for a in loaded.accept]
    assert to_numpy(bufs.status)[0] == 0
    # -- sampled units ----------------------------------------------------------
    for (l, r) in SAMPLES[idx]:
        u = gen_unit(w, l, r)
        par = None if parents is None else parents[r]
        ck = to_numpy(bufs.ckpt[l, r])
        out = to_numpy(bufs.out[l, r])
        ock, oout = ogdn.gdn_span(u.state, u.q, u.k, u.v, u.a, u.b, par)
        e1 = assert_tiles(ck, ock, 2, f"ckpt l={l} r={r}")
        e2 = assert_tiles(out, oout, 1, f"out l={l} r={r}")
        wt = gen_conv_weight(w, l)
        oy, occ = oconv.conv_span(u.x, wt, u.conv_state, par)
        e3 = assert_tiles(to_numpy(bufs.y[l, r]), oy, 1, f"conv y l={l} r={r}")
        assert np.array_equal(to_numpy(bufs.conv_ckpt[l, r]), occ), f"conv ckpt l={l} r={r}"
        # rollback: restored state == own checkpoint (bit-exact) == oracle replay
        u_node = int(node[r])
        st = to_numpy(bufs.state[l, r])
        assert np.array_equal(st, ck[u_node])
        rpath, n = [], u_node
        while n >= 0:
            rpath.append(n)
            n = (par[n] if par is not None else n - 1)
        ref = orb.replay_state(u.state, u.q, u.k, u.v, u.a, u.b, rpath[::-1])
        e4 = assert_tiles(st, ref, 2, f"rollback l={l} r={r}")
        assert np.array_equal(to_numpy(bufs.conv_state[l, r]),
                              orb.replay_conv_state(u.conv_state, u.x, rpath[::-1]))
        say(f"unit l={l} r={r}: ckpt {e1:.1e} out {e2:.1e} conv {e3:.1e} rollback {e4:.1e}")
    # -- ring ---------------------------------------------------------------------
    if w.ring_slots:
        ring = to_numpy(bufs.ring)
        exp = oring.ring_set(loaded.ring0, loaded.packed, loaded.runs)
        assert np.array_equal(ring, exp), "ring contents"
        got = to_numpy(bufs.packed_out)
        assert np.array_equal(got, oring.ring_get(exp, np.zeros_like(loaded.packed), loaded.runs))
        say("ring ok")


@pytest.mark.parametrize("fused", [False, True])
def test_full_size_zero_copy_and_fused_steps(fused):
    """The NEXT-row steps bench.py times, at the 16-request x 48-layer size:
    the zero-copy step (spans start in place from the previous step's accepted
    checkpoint, conv state rebuilt from the accepted path) and the same step
    with every layer fused into one kernel. Two consecutive steps (the first
    from the initial state, the second zero-copy); every request's acceptance
    and sampled (layer, request) units of both steps against the oracle, the
    second from the oracle's replay of the first step's accepted path."""
    import torch
    from hybrid_recurrent_state_amd.step import FusedVerifyStep, StepBuffers, ZeroCopyVerifyStep
    from synth.device import fill_step, step_shape
    from tests.step_oracle import TrackedUnit, unit_slices
    torch.cuda.empty_cache()
    w = WORKLOADS[WORKLOAD_ORDER[3]]
    assert w.conv_channels == 2 * w.n_kheads * w.d_k + w.n_vheads * w.d_v
    say(f"workload {w.name} ({'fused' if fused else 'zero-copy'} step): allocating and filling")
    bufs = StepBuffers(step_shape(w))
    loaded = fill_step(bufs, w)
    cls = FusedVerifyStep if fused else ZeroCopyVerifyStep
    step = cls(bufs, parent=loaded.parent, runs=loaded.runs)
    units = [TrackedUnit(w, loaded, l, r, fused=fused) for (l, r) in [(0, 3), (47, 12), (30, 8)]]
    for i in range(2):
        say(f"step {i}")
        acc_len, bonus = step.run()
        torch.cuda.synchronize()
        for r in range(w.n_req):
            res = oacc.accept(oacc.argmax_rows(loaded.accept[r].logits), loaded.accept[r].tokens)
            assert acc_len[r] == res.accept_len and bonus[r] == res.bonus, (i, r)
        for tu in units:
            tu.check(i, *unit_slices(bufs, step.current_ckpt(), tu.l, tu.r, with_y=not fused),
                     what="full-size " + ("fused" if fused else "zero-copy"))
    del step, bufs
    torch.cuda.empty_cache()
