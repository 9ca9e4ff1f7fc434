"""accept_greedy_noalloc (the acceptance entry point that allocates nothing)
against accept_greedy with a caller workspace, through the C ABI: the same
inputs give bit-identical outputs on two calls in a row, the second one
smaller than the first, and a size beyond the library's fixed array is
rejected before anything is launched."""
import ctypes

import numpy as np
import pytest

from synth import QWEN_STACK_CHAIN, QWEN_STACK_TREE, gen_accept, scaled
from tests.gpu_util import say, to_numpy, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hrs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import hybrid_recurrent_state_amd as m
    return m


def _outputs(R, T, fill):
    import torch
    return [torch.full(s, fill, dtype=torch.int32, device="cuda") for s in [(R, T), (R,), (R,), (R, T), (R,)]]


def run_both(hrs, w):
    import torch
    acc = [gen_accept(w, r) for r in range(w.n_req)]
    lg = to_torch(np.stack([a.logits for a in acc]))
    tok = to_torch(np.stack([a.tokens for a in acc]))
    par = np.stack([a.parent for a in acc]) if w.tree else None
    R, T, V = lg.shape
    say(f"accept_greedy_noalloc vs accept_greedy: {w.name} R={R} T={T} V={V} tree={w.tree}")
    ref = _outputs(R, T, -7)
    nbytes = hrs.accept_greedy_workspace_bytes(R, T, V, hrs.HRS_BF16, par)
    assert 0 < nbytes <= hrs.ACCEPT_NOALLOC_MAX_BYTES
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    hrs.accept_greedy(lg, tok, *ref, ws, parent=par)
    got = _outputs(R, T, -9)
    d, _keep = hrs.accept_desc(R, T, V, hrs.HRS_BF16, par)
    st = hrs.lib.accept_greedy_noalloc(ctypes.byref(d), lg.data_ptr(), tok.data_ptr(), *[o.data_ptr() for o in got],
                                       torch.cuda.current_stream().cuda_stream)
    assert st == hrs.HRS_OK, hrs.strerror(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("argmax", "accept_node", "accept_len", "path", "bonus"), ref, got):
        assert np.array_equal(to_numpy(a), to_numpy(b)), name
    assert [int(x) for x in to_numpy(got[1])] == [a.planted_node for a in acc]


def test_noalloc_equals_workspace_call_twice_second_smaller(hrs):
    run_both(hrs, scaled(QWEN_STACK_CHAIN, n_req=16))    # 16 x 17 rows of 151,936 bf16 logits
    run_both(hrs, scaled(QWEN_STACK_TREE, n_req=1))      # then one 23-node tree: smaller


def test_noalloc_rejects_sizes_beyond_the_array(hrs):
    import torch
    R, T, V = 256, 64, 151936        # 16,384 rows x 10 chunks x 8 B = 1.25 MiB of keys
    d, _keep = hrs.accept_desc(R, T, V, hrs.HRS_BF16)
    assert hrs.lib.accept_greedy_workspace_bytes(ctypes.byref(d)) > hrs.ACCEPT_NOALLOC_MAX_BYTES
    small = torch.zeros(64, dtype=torch.int32, device="cuda")   # never read: rejected before any launch
    p = small.data_ptr()
    st = hrs.lib.accept_greedy_noalloc(ctypes.byref(d), p, p, p, p, p, p, p, torch.cuda.current_stream().cuda_stream)
    assert st == hrs.HRS_EINVAL
