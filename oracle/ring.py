"""Feature ring set/get: the oracle (test infrastructure only).

The draft conditions on target hidden features kept in a per-request ring of
slots. Synchronising the ring is batched as one get_2d and one set_2d per
non-wrapping run instead of two host/device transfers and a stream sync per
token (lucebox PR #533, Changes). A run of n rows starting at slot p occupies
slots (p + i) mod S, i = 0..n-1; a run that wraps is two non-wrapping runs.

Definition: set writes ring[r][(p + i) mod S] = packed[row + i]; every other
slot keeps its value. get returns packed[row + i] = ring[r][(p + i) mod S].

Pins (tests/test_oracle_ring.py): per-row Python loop versus slice
assignment over the split runs; untouched slots unchanged; set then get is
the identity on the written rows. Parity pinned.
"""
from __future__ import annotations

import numpy as np


def ring_set(ring: np.ndarray, packed: np.ndarray, runs) -> np.ndarray:
    """Return a copy of ``ring`` [R, S, D] with ``runs`` written from ``packed``."""
    out = np.array(ring, copy=True)
    S = out.shape[1]
    for ring_id, start, n_rows, row in runs:
        for i in range(n_rows):
            out[ring_id, (start + i) % S] = packed[row + i]
    return out


def ring_get(ring: np.ndarray, packed: np.ndarray, runs) -> np.ndarray:
    """Return a copy of ``packed`` [N, D] with ``runs`` read from ``ring``."""
    out = np.array(packed, copy=True)
    S = ring.shape[1]
    for ring_id, start, n_rows, row in runs:
        for i in range(n_rows):
            out[row + i] = ring[ring_id, (start + i) % S]
    return out


def split_runs(runs, n_slots: int):
    """Each run as at most two non-wrapping (ring_id, start, n_rows, row) runs."""
    out = []
    for ring_id, start, n_rows, row in runs:
        first = min(n_rows, n_slots - start)
        out.append((ring_id, start, first, row))
        if n_rows > first:
            out.append((ring_id, 0, n_rows - first, row + first))
    return out
