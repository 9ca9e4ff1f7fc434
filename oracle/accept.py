"""Greedy acceptance over a chain or a draft tree: the oracle (test infrastructure only).

Greedy verification keeps the draft tokens that the target itself would have
produced: a draft token is accepted when it equals the target's argmax at its
parent position, and acceptance stops at the first mismatch
(openinfer PR #626, Summary: a single active greedy request whose output
matches plain greedy decoding). With a DDTree (lucebox PR #533, Sustained
performance: DDTree budget 16) the accepted result is the deepest node whose
whole root path matches. The target's argmax at the accepted node is the
bonus token that the next step starts from.

Readings:
  * node 0 is the committed root token and is always matched; the accepted
    length is the depth of the accepted node (number of accepted drafts);
  * argmax ties go to the lowest index; NaN never wins (it orders below
    -inf); a row that is all NaN yields index 0; -0 equals +0;
  * among equally deep matched nodes the lowest index wins;
  * the path is root -> accepted node; unused entries are -1.

Pins (tests/test_oracle_accept.py): numpy.argmax on rows without NaN;
hand-built NaN/inf/-0 rows; exhaustive root-path enumeration
(``brute_force_accept``) on random and hand-built trees; hand-worked cases in
tests/golden/accept_cases.txt. Parity pinned.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from .common import widen


def argmax_row(row) -> int:
    """Index of the largest value; lowest index on ties; NaN never wins."""
    vals = widen(row)
    best = -1
    best_val = 0.0
    for i in np.flatnonzero(~np.isnan(vals)):
        val = vals[i]
        if best < 0 or val > best_val:
            best, best_val = int(i), val
    return 0 if best < 0 else best


def argmax_row_fast(row) -> int:
    """Same definition as ``argmax_row`` with vectorised numpy steps."""
    vals = widen(row)
    ok = ~np.isnan(vals)
    if not ok.any():
        return 0
    m = np.max(vals[ok])
    return int(np.flatnonzero(ok & (vals == m))[0])


def argmax_rows(logits) -> np.ndarray:
    """Row argmax of a [..., V] array -> int32 [...]."""
    arr = np.asarray(logits)
    flat = arr.reshape(-1, arr.shape[-1])
    out = np.array([argmax_row_fast(r) for r in flat], dtype=np.int32)
    return out.reshape(arr.shape[:-1])


@dataclasses.dataclass
class AcceptResult:
    accept_node: int
    accept_len: int
    path: np.ndarray    # [T] int32: root..accepted node, then -1
    bonus: int


def _root_path(parent, u: int) -> List[int]:
    path = []
    while u >= 0:
        path.append(u)
        u = int(parent[u])
    return path[::-1]


def accept(argmax: np.ndarray, tokens: np.ndarray,
           parent: Optional[np.ndarray] = None) -> AcceptResult:
    """Deepest matched node (then lowest index) for one request."""
    T = len(tokens)
    if parent is None:
        parent = np.arange(-1, T - 1)
    matched = [False] * T
    depth = [0] * T
    matched[0] = True
    for t in range(1, T):
        p = int(parent[t])
        depth[t] = depth[p] + 1
        matched[t] = matched[p] and int(tokens[t]) == int(argmax[p])
    best = 0
    for t in range(T):
        if matched[t] and depth[t] > depth[best]:
            best = t
    path = np.full(T, -1, dtype=np.int32)
    rp = _root_path(parent, best)
    path[:len(rp)] = rp
    return AcceptResult(accept_node=best, accept_len=depth[best], path=path,
                        bonus=int(argmax[best]))


def brute_force_accept(argmax: np.ndarray, tokens: np.ndarray,
                       parent: np.ndarray) -> AcceptResult:
    """Enumerate every node's root path; keep the longest path whose every
    edge (p -> c) has tokens[c] == argmax[p]; ties to the lowest end node."""
    T = len(tokens)
    best, best_len = 0, 0
    for u in range(T):
        rp = _root_path(parent, u)
        if all(int(tokens[c]) == int(argmax[p]) for p, c in zip(rp[:-1], rp[1:])):
            if len(rp) - 1 > best_len:
                best, best_len = u, len(rp) - 1
    path = np.full(T, -1, dtype=np.int32)
    rp = _root_path(parent, best)
    path[:len(rp)] = rp
    return AcceptResult(accept_node=best, accept_len=best_len, path=path,
                        bonus=int(argmax[best]))
