"""Graph launch of the verify step: replaying the captured HIP graph must give
exactly the results of launching the same step eagerly, on every replay, with
unrelated eager GPU work and host synchronisations between the replays, and
sampled (layer, request) units of every replay must equal the oracle (each
replay starts from the state the previous replay's rollback restored, which
the oracle defines as the replay of the accepted path)."""
import numpy as np
import pytest

from synth import QWEN_STACK_CHAIN, QWEN_STACK_TREE, scaled
from tests.gpu_util import say, to_numpy
from tests.step_oracle import TrackedUnit, unit_slices

pytestmark = pytest.mark.gpu

FIELDS = ["ckpt", "out", "y", "conv_ckpt", "state", "conv_state", "argmax", "accept_node", "accept_len",
          "path", "bonus", "ring", "packed_out"]


def make(w):
    from hybrid_recurrent_state_amd.step import StepBuffers, VerifyStep
    from synth.device import fill_step, step_shape
    bufs = StepBuffers(step_shape(w))
    loaded = fill_step(bufs, w)
    return bufs, VerifyStep(bufs, parent=loaded.parent, runs=loaded.runs), loaded


@pytest.mark.parametrize("w,samples", [
    (scaled(QWEN_STACK_CHAIN, n_layers=3, n_req=2, vocab=4096, ring_slots=64, ring_width=256), [(2, 1)]),
    (scaled(QWEN_STACK_TREE, n_layers=2, n_req=2, vocab=4096), [(0, 1)]),
])
def test_graph_replay_equals_eager(w, samples):
    import torch
    eager_bufs, eager, _ = make(w)
    graph_bufs, graphed, loaded = make(w)
    graphed.capture_graph()
    units = [TrackedUnit(w, loaded, l, r) for (l, r) in samples]
    scratch = torch.randn(1 << 20, device="cuda")
    for i in range(3):
        acc_e, bonus_e = eager.run()
        acc_g, bonus_g = graphed.replay()
        assert np.array_equal(acc_e, acc_g) and np.array_equal(bonus_e, bonus_g), i
        for name in FIELDS:
            a, b = getattr(eager_bufs, name), getattr(graph_bufs, name)
            if a is None:
                continue
            assert np.array_equal(to_numpy(a), to_numpy(b)), (i, name)
        for tu in units:
            tu.check(i, *unit_slices(graph_bufs, graph_bufs.ckpt, tu.l, tu.r), what="graph")
            # the copy rollback restored the accepted checkpoint into the state
            tu.check_state(to_numpy(graph_bufs.state[tu.l, tu.r]), what="graph")
        scratch.mul_(1.0001).add_(0.5)     # unrelated eager work between replays
        torch.cuda.synchronize()
        say(f"replay {i}: accepted {list(map(int, acc_g))}")
