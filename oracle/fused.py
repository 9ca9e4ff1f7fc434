"""One Gated DeltaNet layer's verify span in the layer's own order: the oracle
(test infrastructure only).

In the Qwen3.5/3.6 hybrid layers the recurrent block's projected q, k and v
channels pass together through the causal depthwise conv with SiLU, are split
back into q, k and v heads, q and k are scaled to unit L2 norm per head, and
the gated delta rule runs on the result (the conv state and the recurrent state
are the hybrid state of openinfer PR #626, "feat(qwen35): add opt-in DFlash
speculative decoding", What Changed; the conv width 4 and the verify span as in
the rest of this oracle).

Definition (composition of the pinned pieces, nothing fused):
    y              = conv_span(x, w, conv_state, parent, silu)   (float32 [T, C])
    q, k, v        = y[:, :Hk*dk], y[:, Hk*dk:2*Hk*dk], y[:, 2*Hk*dk:] as heads
    q_hat, k_hat   = q / sqrt(|q|^2 + eps), k / sqrt(|k|^2 + eps)   (float64, per head)
    ckpt, out      = gdn_span(state, q_hat, k_hat, v, a, b, parent, q_scale)
Channel order [q heads | k heads | v heads], head-major inside each group.

Readings: the conv output stays float32 (no rounding to bf16 between the conv
and the recurrence); eps is added to the sum of squares (default 1e-6); q_scale
multiplies the normalised q.

Pins (tests/test_oracle_fused.py): with a conv that passes the current input
only, the layer equals the GDN oracle on silu / L2-normalised channel slices
computed independently (scipy's logistic, numpy's norm), which fixes the split
order and the place of the normalisation; normalised rows have unit norm.
Parity pinned.
"""
from __future__ import annotations

import numpy as np

from .conv import conv_span
from .gdn import gdn_span


def l2norm_rows(x: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def layer_span(x, w, conv_state, a, b, state, n_kheads: int, n_vheads: int, d_k: int, d_v: int,
               parent=None, q_scale: float = 1.0, eps: float = 1e-6, silu: bool = True):
    """x [T, C] (C = 2*Hk*dk + Hv*dv), w [C, W], conv_state [W-1, C], a, b [T, Hv],
    state [Hv, dv, dk] float32. Returns (ckpt [T,Hv,dv,dk] f32, out [T,Hv,dv] f32,
    conv_ckpt [T, W-1, C])."""
    T = x.shape[0]
    y, conv_ckpt = conv_span(x, w, conv_state, parent, silu=silu)
    yf = y.astype(np.float64)
    nq = n_kheads * d_k
    q = yf[:, :nq].reshape(T, n_kheads, d_k)
    k = yf[:, nq:2 * nq].reshape(T, n_kheads, d_k)
    v = yf[:, 2 * nq:2 * nq + n_vheads * d_v].reshape(T, n_vheads, d_v)
    ckpt, out = gdn_span(state, l2norm_rows(q, eps), l2norm_rows(k, eps), v, a, b, parent, q_scale)
    return ckpt, out, conv_ckpt
