"""Graph launch of the verify step: replaying the captured HIP graph must give
exactly the results of launching the same step eagerly, on every replay, with
unrelated eager GPU work and host synchronisations between the replays."""
import numpy as np
import pytest

from synth import QWEN_STACK_CHAIN, QWEN_STACK_TREE, scaled
from tests.gpu_util import say, to_numpy

pytestmark = pytest.mark.gpu

FIELDS = ["ckpt", "out", "y", "conv_ckpt", "state", "conv_state", "argmax", "accept_node", "accept_len",
          "path", "bonus", "ring", "packed_out"]


def make(w):
    from hybrid_recurrent_state_amd.step import StepBuffers, VerifyStep
    from synth.device import fill_step, step_shape
    bufs = StepBuffers(step_shape(w))
    loaded = fill_step(bufs, w)
    return bufs, VerifyStep(bufs, parent=loaded.parent, runs=loaded.runs)


@pytest.mark.parametrize("w", [
    scaled(QWEN_STACK_CHAIN, n_layers=3, n_req=2, vocab=4096, ring_slots=64, ring_width=256),
    scaled(QWEN_STACK_TREE, n_layers=2, n_req=2, vocab=4096),
])
def test_graph_replay_equals_eager(w):
    import torch
    eager_bufs, eager = make(w)
    graph_bufs, graphed = make(w)
    graphed.capture_graph()
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
        scratch.mul_(1.0001).add_(0.5)     # unrelated eager work between replays
        torch.cuda.synchronize()
        say(f"replay {i}: accepted {list(map(int, acc_g))}")
