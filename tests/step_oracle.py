"""Oracle side of multi-step GPU tests (a helper module, not collected).

Tracks sampled (layer, request) units of a workload through consecutive
verify steps with the oracle's plain definitions: each step's span runs from
the state the previous step's rollback defines, and that rollback is the
replay of the accepted root path (the conservative commit of openinfer PR
#626, What Changed, which the checkpoint restore of lucebox PR #506, Summary,
must reproduce without replay). Inputs, logits and drafts are the same in
every step, as the GPU step buffers are not refilled between steps.
"""
from __future__ import annotations

import numpy as np

from oracle import accept as oacc, conv as oconv, fused as ofu, gdn as ogdn, rollback as orb
from synth import gen_conv_weight, gen_unit
from tests.gpu_util import assert_tiles, say, to_numpy


class TrackedUnit:
    """One (layer, request) unit followed through consecutive steps.

    fused: the unit's layer is the fused one (conv with SiLU, q/k/v split,
    q/k L2 norm, gated delta rule); else the conv span (no SiLU) and the GDN
    span run on their separate inputs."""

    def __init__(self, w, loaded, layer: int, req: int, fused: bool = False, silu: bool = True,
                 eps: float = 1e-6):
        self.w, self.l, self.r, self.fused, self.silu, self.eps = w, layer, req, fused, silu, eps
        self.u = gen_unit(w, layer, req)
        self.wt = gen_conv_weight(w, layer)
        self.parent = None if loaded.parent is None else loaded.parent[req]
        ai = loaded.accept[req]
        am = oacc.argmax_rows(ai.logits) if w.vocab else ai.planted_argmax
        self.acc = oacc.accept(am, ai.tokens, self.parent)
        self.path = [int(t) for t in self.acc.path if t >= 0]
        self.state = self.u.state
        self.conv_state = self.u.conv_state

    def expected(self):
        """Oracle outputs of the next step from the tracked state:
        (ckpt [T,Hv,dv,dk], out [T,Hv,dv], y [T,C] or None)."""
        u, w = self.u, self.w
        if self.fused:
            ck, out, _ = ofu.layer_span(u.x, self.wt, self.conv_state, u.a, u.b, self.state, w.n_kheads,
                                        w.n_vheads, w.d_k, w.d_v, parent=self.parent, eps=self.eps, silu=self.silu)
            return ck, out, None
        ck, out = ogdn.gdn_span(self.state, u.q, u.k, u.v, u.a, u.b, self.parent)
        y, _ = oconv.conv_span(u.x, self.wt, self.conv_state, self.parent)
        return ck, out, y

    def advance(self):
        """Roll the tracked states forward to the accepted node by replay."""
        u, w = self.u, self.w
        idx = np.array(self.path)
        if self.fused:
            ck, _, _ = ofu.layer_span(u.x[idx], self.wt, self.conv_state, u.a[idx], u.b[idx], self.state,
                                      w.n_kheads, w.n_vheads, w.d_k, w.d_v, eps=self.eps, silu=self.silu)
            new_state = ck[-1]
        else:
            new_state = orb.replay_state(self.state, u.q, u.k, u.v, u.a, u.b, self.path)
        self.conv_state = orb.replay_conv_state(self.conv_state, u.x, self.path)
        self.state = new_state

    def check(self, step: int, ckpt, out, y=None, conv_state=None, what: str = ""):
        """Compare the GPU's step outputs of this unit with the oracle's, then
        advance. ckpt/out/y: the unit's slices as numpy arrays; conv_state:
        the GPU conv state after the step's rollback (bit-exact)."""
        ock, oout, oy = self.expected()
        tag = f"{what} step {step} l={self.l} r={self.r}"
        e1 = assert_tiles(ckpt, ock, 2, f"{tag} ckpt")
        e2 = assert_tiles(out, oout, 1, f"{tag} out")
        msg = f"{tag}: ckpt {e1:.1e} out {e2:.1e}"
        if y is not None and oy is not None:
            msg += f" y {assert_tiles(y, oy, 1, f'{tag} y'):.1e}"
        self.advance()
        if conv_state is not None:
            assert np.array_equal(conv_state, self.conv_state), f"{tag} conv state"
        say(msg)

    def check_state(self, state, what: str = ""):
        """The GPU's materialised (rolled-back) recurrent state of this unit
        against the oracle's replay."""
        e = assert_tiles(state, self.state, 2, f"{what} state l={self.l} r={self.r}")
        say(f"{what} materialised state l={self.l} r={self.r}: {e:.1e}")


def unit_slices(bufs, ckpt_buf, l: int, r: int, with_y: bool = True):
    """numpy copies of one unit's step outputs from the step buffers."""
    ck = to_numpy(ckpt_buf[l, r])
    out = to_numpy(bufs.out[l, r])
    y = to_numpy(bufs.y[l, r]) if with_y else None
    cs = to_numpy(bufs.conv_state[l, r])
    return ck, out, y, cs
