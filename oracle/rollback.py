"""Rollback to the accepted node: the oracle (test infrastructure only).

The conservative commit restores the canonical pre-span state and replays the
accepted target span through normal decode (openinfer PR #626, What Changed).
Fast rollback instead keeps an F32 SSM checkpoint of every verified position
and restores the accepted one without replay (lucebox PR #506, Summary;
lucebox PR #533, Sustained performance: replay=0.000s), together with the
conv state (lucebox PR #533, Changes).

The oracle computes the replay definition, never the checkpoint index: the
rolled-back recurrent state is the pre-span state advanced, one position at a
time, along the root path of the accepted node; the rolled-back conv state is
the last W-1 inputs along that path, padded from the pre-span conv state.
The GPU restore (a copy of checkpoint[accepted]) must reproduce it.

Pins (tests/test_oracle_rollback.py): replay equals the span's own
checkpoint at the accepted node for chains and trees, accepted length 0
returns the state after the root alone, and the conv state equals a slice of
the concatenated input sequence. Parity pinned.
"""
from __future__ import annotations

import numpy as np

from .gdn import gdn_position


def replay_state(state, q, k, v, a, b, path, q_scale: float = 1.0) -> np.ndarray:
    """Advance ``state`` through the positions listed in ``path`` (root first).

    ``path`` entries < 0 are ignored (unused tail). Returns float32.
    """
    S = np.array(state, dtype=np.float32, copy=True)
    for t in path:
        t = int(t)
        if t < 0:
            break
        S, _ = gdn_position(S, q[t], k[t], v[t], a[t], b[t], q_scale)
    return S


def replay_conv_state(conv_state, x, path) -> np.ndarray:
    """Last W-1 inputs along ``path`` with the pre-span conv state in front."""
    rows = [conv_state[i] for i in range(conv_state.shape[0])]
    for t in path:
        t = int(t)
        if t < 0:
            break
        rows.append(x[t])
    keep = rows[len(rows) - conv_state.shape[0]:]
    return np.stack(keep, axis=0).astype(conv_state.dtype)
