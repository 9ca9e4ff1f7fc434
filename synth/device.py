"""Copy seeded synthetic workloads into device buffers (tests and bench).

Pure data movement: numpy arrays from ``synth`` are uploaded into the
``StepBuffers`` tensors of the GPU library. bf16 data travels as its 16-bit
patterns, so both sides see identical bits.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

from . import Workload, gen_accept, gen_conv_weight, gen_ring, gen_unit, BF16


def to_torch(arr: np.ndarray, device="cuda"):
    import torch
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(arr).to(device)


def to_numpy(t) -> np.ndarray:
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def step_shape(w: Workload):
    from hybrid_recurrent_state_amd.step import StepShape
    return StepShape(n_layers=w.n_layers, n_req=w.n_req, n_pos=w.n_pos, n_kheads=w.n_kheads,
                     n_vheads=w.n_vheads, d_k=w.d_k, d_v=w.d_v, bf16=(w.dtype == BF16),
                     conv_channels=w.conv_channels, conv_width=w.conv_width, vocab=w.vocab,
                     ring_slots=w.ring_slots, ring_width=w.ring_width)


@dataclasses.dataclass
class Loaded:
    parent: Optional[np.ndarray]     # [R, T] for trees, else None
    accept: List                     # AcceptInputs per request
    runs: List[tuple]
    ring0: Optional[np.ndarray]      # initial ring contents (host copy) if kept
    packed: Optional[np.ndarray]


def fill_step(bufs, w: Workload, keep_ring: bool = False, log=None) -> Loaded:
    """Fill every buffer of ``bufs`` with the workload's seeded inputs."""
    import torch
    L, R = w.n_layers, w.n_req
    for l in range(L):
        units = [gen_unit(w, l, r) for r in range(R)]
        for name in ("q", "k", "v", "a", "b", "state", "x", "conv_state"):
            stacked = np.stack([getattr(u, name) for u in units])
            getattr(bufs, name)[l].copy_(to_torch(stacked, "cpu"))
        bufs.w[l].copy_(to_torch(gen_conv_weight(w, l), "cpu"))
        if log and (l % 8 == 7 or l == L - 1):
            log(f"inputs: layer {l + 1}/{L} uploaded")
    acc = [gen_accept(w, r, with_logits=w.vocab > 0) for r in range(R)]
    bufs.tokens.copy_(torch.from_numpy(np.stack([a.tokens for a in acc])))
    if w.vocab:
        bufs.logits.copy_(to_torch(np.stack([a.logits for a in acc]), "cpu"))
    else:
        bufs.accept_node.copy_(torch.from_numpy(np.array([a.planted_node for a in acc], dtype=np.int32)))
    parent = np.stack([a.parent for a in acc]) if w.tree else None
    runs, ring0, packed = [], None, None
    if w.ring_slots:
        ri = gen_ring(w, with_ring=True)
        runs = ri.runs
        bufs.ring.copy_(to_torch(ri.ring, "cpu"))
        bufs.packed_in.copy_(to_torch(ri.packed, "cpu"))
        bufs.packed_out.zero_()
        packed = ri.packed
        ring0 = ri.ring if keep_ring else None
    torch.cuda.synchronize()
    return Loaded(parent=parent, accept=acc, runs=runs, ring0=ring0, packed=packed)
