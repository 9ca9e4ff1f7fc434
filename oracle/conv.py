"""Causal depthwise conv1d over the verify span: the oracle (test infrastructure only).

The Qwen3.5/3.6 hybrid layers keep, beside the recurrent state, a short conv
state: the last W-1 inputs of a causal depthwise convolution
(openinfer PR #626, What Changed: "full-attention KV, recurrent state, conv
state"; lucebox PR #533, Changes: split SSM and convolution state restored on
device). Verifying a draft block must capture that conv state at every
position, like the SSM checkpoints (lucebox PR #506, Summary), so rollback
can restore it.

Definition for one (layer, request), channel c, width W:
    window_t = [cs_p[0], ..., cs_p[W-2], x_t]   (oldest first)
    y_t[c]   = sum_m w[c][m] * window_t[m][c]     (float64, then float32)
    cs_t     = window_t[1:]                        (the new conv state)
where cs_p is the conv state after the parent position p (the pre-span conv
state for the root). Optionally y is passed through silu(z) = z / (1 + e^-z)
before rounding.

Readings: w[c][W-1] multiplies the current input (left-padded causal
convolution); there is no bias; silu is an opt-in flag; the conv state has
the input's dtype, so every captured state is an exact copy of inputs.

Pins (tests/test_oracle_conv.py): numpy.convolve on the concatenated chain
sequence; the captured states are slices of that sequence; tree node windows
equal the chain over the node's root path. Parity pinned.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .common import to_f32, widen


def conv_span(x: np.ndarray, w: np.ndarray, conv_state: np.ndarray,
              parent: Optional[np.ndarray] = None, silu: bool = False
              ) -> Tuple[np.ndarray, np.ndarray]:
    """x: [T, C]; w: [C, W]; conv_state: [W-1, C] (same dtype as x).

    Returns y [T, C] float32 and conv_ckpt [T, W-1, C] in x's dtype (exact
    copies of inputs).
    """
    T, C = x.shape
    W = w.shape[1]
    if parent is None:
        parent = np.arange(-1, T - 1)
    wf = widen(w)
    ckpt = np.empty((T, W - 1, C), dtype=x.dtype)
    y = np.empty((T, C), dtype=np.float32)
    for t in range(T):
        p = int(parent[t])
        prev = conv_state if p < 0 else ckpt[p]
        window = np.concatenate([prev, x[t:t + 1]], axis=0)   # [W, C], raw dtype
        wv = widen(window)
        acc = np.zeros(C, dtype=np.float64)
        for m in range(W):
            acc += wf[:, m] * wv[m]
        if silu:
            acc = acc / (1.0 + np.exp(-acc))
        y[t] = to_f32(acc)
        ckpt[t] = window[1:]
    return y, ckpt
