"""Gated DeltaNet verify span: the oracle (test infrastructure only).

Recurrence: the gated delta rule (Yang, Kautz, Hatamizadeh, "Gated Delta
Networks: Improving Mamba2 with Delta Rule", ICLR 2025). For each value head,
with state S (d_v rows by d_k columns), key k_t, value v_t, query q_t, decay
a_t and write strength b_t:

    S_t = a_t * S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,    o_t = S_t q_t.

Expanding the product, with u = S_{t-1} k_t:

    S_t = a_t S_{t-1} + b_t (v_t - a_t u) k_t^T.

The span is the committed root token plus the K drafts (T = K + 1
positions), verified through the recurrent layers of the target
(lucebox PR #533, Sustained performance: verify phase). The state after every
position is kept as a float32 checkpoint so a later rollback can restore the
accepted one without replay (lucebox PR #506, Summary; Memory trade-off). In a
draft tree (lucebox PR #533, Changes and Verification: DDTree), node t starts
from its parent's checkpoint, the root from the pre-span state.

Readings where the pages say nothing (each listed in the design notes):
  * S has d_v rows and d_k columns (forced by v k^T and S q).
  * a_t and b_t are scalars per (position, value head).
  * value head h uses key head h // (Hv / Hk) (contiguous groups).
  * q is multiplied by q_scale (default 1) after widening; no
    normalisation happens here (the inputs are made unit-norm upstream).
  * the state is rounded to float32 once per position: that rounded value is
    the checkpoint, the output is computed from it, and the next position
    starts from it.

Pins (tests/test_oracle_gdn.py): dense closed form of one step with matrix
products; two-fold composition; a=1,b=0 leaves the state unchanged; a=0
writes b v k^T; unit k with a=b=1 stores v at k; the invariants along k and
orthogonal to k; exact rational brute force on tiny shapes; chain-as-tree
equality; split-span composition. Parity pinned.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .common import to_f32, widen


def gdn_position(P: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                 a: np.ndarray, b: np.ndarray, q_scale: float = 1.0
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """One position for all value heads.

    P: [Hv, d_v, d_k] float32 state the position starts from.
    q, k: [Hk, d_k]; v: [Hv, d_v]; a, b: [Hv] (float32 or bf16 bits).
    Returns (S_t as float32 [Hv, d_v, d_k], o_t as float32 [Hv, d_v]).
    """
    Hv = P.shape[0]
    Hk = k.shape[0]
    group = Hv // Hk
    qf, kf, vf, af, bf = widen(q), widen(k), widen(v), widen(a), widen(b)
    S_out = np.empty(P.shape, dtype=np.float32)
    o_out = np.empty(P.shape[:2], dtype=np.float32)
    for h in range(Hv):
        g = h // group
        s = P[h].astype(np.float64)
        kk = kf[g]
        qq = qf[g] * float(q_scale)
        u = s @ kk
        s_new = af[h] * s + bf[h] * np.outer(vf[h] - af[h] * u, kk)
        S_out[h] = to_f32(s_new)
        o_out[h] = to_f32(S_out[h].astype(np.float64) @ qq)
    return S_out, o_out


def gdn_span(state: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
             a: np.ndarray, b: np.ndarray, parent: Optional[np.ndarray] = None,
             q_scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """The verify span of one (layer, request).

    state: [Hv, d_v, d_k] float32 pre-span state.
    q, k: [T, Hk, d_k]; v: [T, Hv, d_v]; a, b: [T, Hv].
    parent: [T] int, parent[0] = -1 and parent[t] < t; None means a chain
    (parent[t] = t - 1).
    Returns ckpt [T, Hv, d_v, d_k] float32 and out [T, Hv, d_v] float32.
    """
    T = q.shape[0]
    if parent is None:
        parent = np.arange(-1, T - 1)
    ckpt = np.empty((T,) + state.shape, dtype=np.float32)
    out = np.empty((T,) + state.shape[:2], dtype=np.float32)
    for t in range(T):
        p = int(parent[t])
        P = state if p < 0 else ckpt[p]
        ckpt[t], out[t] = gdn_position(P, q[t], k[t], v[t], a[t], b[t], q_scale)
    return ckpt, out
