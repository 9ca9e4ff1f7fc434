"""One verify step over a stack of GDN layers, on one stream, one host sync.

Order of the step (all on the caller's stream):
  for each layer: conv1d_verify_span, then gdn_verify_span (checkpoints on)
  accept_greedy over the target logits
  rollback_restore of every layer to the accepted position (index stays on
  the device)
  ring_set_2d, ring_get_2d of the step's hidden-feature rows
then one device-to-host copy of the accepted lengths and bonus tokens,
which is the step's only synchronisation (lucebox PR #533, "feat: DFlash
support for tensor-parallel Qwen3.6 targets", Changes: restore SSM and conv
state on device and synchronize once after rollback).

Buffers are allocated once by ``StepBuffers`` (device memory through torch)
and every descriptor and pointer of the step is computed once by
``VerifyStep``, so launching a step is a fixed sequence of C calls.

Variants: ``ZeroCopyVerifyStep`` starts
each span from the previous span's accepted checkpoint in place (no rollback
copy, conv state rebuilt from the accepted path) and ``FusedVerifyStep`` adds
one fused kernel per layer (conv, SiLU, q/k/v split, q/k L2 norm and the
gated delta rule) to it.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import List, Optional, Sequence

import numpy as np

from . import (AcceptDesc, ConvAdvanceDesc, ConvDesc, GdnDesc, GdnLayerDesc, HRS_BF16, HRS_CHAIN, HRS_F32, HRS_TREE,
               HrsError, RingDesc, RingRun, RollbackDesc, SpanSource, accept_greedy_workspace_bytes, lib)


@dataclasses.dataclass(frozen=True)
class StepShape:
    n_layers: int
    n_req: int
    n_pos: int
    n_kheads: int
    n_vheads: int
    d_k: int
    d_v: int
    bf16: bool                 # q/k/v/a/b and conv dtype (state is always f32)
    conv_channels: int
    conv_width: int = 4
    vocab: int = 0             # 0: no logits; accept_node is provided directly
    ring_slots: int = 0        # 0: no feature ring
    ring_width: int = 0

    @property
    def gdn_bytes_per_layer(self) -> int:
        """Algorithmic HBM bytes of one gdn_verify_span call with capture:
        read q, k, v, a, b and the state once; write every checkpoint and
        every output once."""
        R, T, Hk, Hv, dk, dv = self.n_req, self.n_pos, self.n_kheads, self.n_vheads, self.d_k, self.d_v
        e = 2 if self.bf16 else 4
        reads = R * T * (2 * Hk * dk + Hv * dv + 2 * Hv) * e + R * Hv * dv * dk * 4
        writes = R * T * Hv * dv * dk * 4 + R * T * Hv * dv * 4
        return reads + writes

    @property
    def layer_bytes_per_layer(self) -> int:
        """Algorithmic HBM bytes of one fused gdn_layer_verify_span call: read
        x, the conv weights, the conv state, a, b and the initial state once;
        write every checkpoint and every output once (q, k, v and the conv
        output never reach memory)."""
        R, T, Hv, dk, dv, C, W = (self.n_req, self.n_pos, self.n_vheads, self.d_k, self.d_v, self.conv_channels,
                                  self.conv_width)
        e = 2 if self.bf16 else 4
        reads = (R * T * C + C * W + R * (W - 1) * C + 2 * R * T * Hv) * e + R * Hv * dv * dk * 4
        writes = R * T * Hv * dv * dk * 4 + R * T * Hv * dv * 4
        return reads + writes

    @property
    def conv_bytes_per_layer(self) -> int:
        R, T, C, W = self.n_req, self.n_pos, self.conv_channels, self.conv_width
        e = 2 if self.bf16 else 4
        return R * T * C * e + C * W * e + R * (W - 1) * C * e + R * T * (W - 1) * C * e + R * T * C * 4

    @property
    def accept_bytes(self) -> int:
        e = 2 if self.bf16 else 4
        return self.n_req * self.n_pos * self.vocab * e

    @property
    def rollback_bytes(self) -> int:
        """Read + write of one checkpoint per (layer, request), state and conv."""
        e = 2 if self.bf16 else 4
        per = self.n_vheads * self.d_v * self.d_k * 4 + (self.conv_width - 1) * self.conv_channels * e
        return 2 * self.n_layers * self.n_req * per

    @property
    def ring_bytes(self) -> int:
        """set + get: each moves n_req * n_pos rows in and out."""
        return 2 * 2 * self.n_req * self.n_pos * self.ring_width * 2


class StepBuffers:
    """Device buffers of one step, laid out [L, ...] per layer (torch owned)."""

    def __init__(self, shape: StepShape, device="cuda"):
        import torch
        s = shape
        dt = torch.bfloat16 if s.bf16 else torch.float32
        L, R, T, Hk, Hv, dk, dv, C, W = (s.n_layers, s.n_req, s.n_pos, s.n_kheads, s.n_vheads, s.d_k, s.d_v,
                                         s.conv_channels, s.conv_width)
        e = lambda *shp, dtype=dt: torch.empty(shp, dtype=dtype, device=device)
        self.shape = s
        self.q = e(L, R, T, Hk, dk)
        self.k = e(L, R, T, Hk, dk)
        self.v = e(L, R, T, Hv, dv)
        self.a = e(L, R, T, Hv)
        self.b = e(L, R, T, Hv)
        self.state = e(L, R, Hv, dv, dk, dtype=torch.float32)
        self.ckpt = e(L, R, T, Hv, dv, dk, dtype=torch.float32)
        self.out = e(L, R, T, Hv, dv, dtype=torch.float32)
        self.x = e(L, R, T, C)
        self.w = e(L, C, W)
        self.conv_state = e(L, R, W - 1, C)
        self.conv_ckpt = e(L, R, T, W - 1, C)
        self.y = e(L, R, T, C, dtype=torch.float32)
        self.tokens = e(R, T, dtype=torch.int32)
        self.argmax = e(R, T, dtype=torch.int32)
        self.accept_node = torch.zeros(R, dtype=torch.int32, device=device)
        self.accept_len = e(R, dtype=torch.int32)
        self.path = e(R, T, dtype=torch.int32)
        self.bonus = e(R, dtype=torch.int32)
        self.status = torch.zeros(4, dtype=torch.int32, device=device)
        self.logits = e(R, T, s.vocab) if s.vocab else None
        self.workspace = None
        if s.vocab:
            nbytes = accept_greedy_workspace_bytes(R, T, s.vocab, HRS_BF16 if s.bf16 else HRS_F32)
            self.workspace = torch.empty(max(16, nbytes), dtype=torch.uint8, device=device)
        self.ring = e(R, s.ring_slots, s.ring_width, dtype=torch.bfloat16) if s.ring_slots else None
        self.packed_in = e(R * T, s.ring_width, dtype=torch.bfloat16) if s.ring_slots else None
        self.packed_out = e(R * T, s.ring_width, dtype=torch.bfloat16) if s.ring_slots else None
        # Host mirror of the step's only device-to-host transfer.
        self.host_result = torch.empty(2 * R, dtype=torch.int32, pin_memory=True)
        self.dev_result = torch.empty(2 * R, dtype=torch.int32, device=device)


def _check(st: int, name: str) -> None:
    if st != 0:
        raise HrsError(st, name)


class VerifyStep:
    """Precomputed launch sequence of one verify step.

    parent: None (chain) or host ints [R, T] (draft trees, one per request).
    runs: ring runs (ring_id, start_pos, n_rows, packed_row) for set and get.
    """

    def __init__(self, bufs: StepBuffers, parent=None, runs: Optional[Sequence[tuple]] = None,
                 silu: bool = False, q_scale: float = 1.0):
        s = bufs.shape
        self.bufs = bufs
        L, R, T = s.n_layers, s.n_req, s.n_pos
        self.topo = HRS_TREE if parent is not None else HRS_CHAIN
        dt = HRS_BF16 if s.bf16 else HRS_F32
        if parent is not None:
            self._parent = np.ascontiguousarray(np.broadcast_to(np.asarray(parent, dtype=np.int32), (R, T)))
            par_p = self._parent.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        else:
            self._parent, par_p = None, None
        self.gdn_desc = GdnDesc(R, T, s.n_kheads, s.n_vheads, s.d_k, s.d_v, dt, q_scale, self.topo, par_p)
        self.conv_desc = ConvDesc(R, T, s.conv_channels, s.conv_width, dt, int(silu), self.topo, par_p)
        self.accept_desc = AcceptDesc(R, T, s.vocab, dt, self.topo, par_p) if s.vocab else None
        self.rb_desc = RollbackDesc(L, R, T, s.n_vheads, s.d_k, s.d_v, s.conv_channels, s.conv_width, dt)
        self.runs = list(runs or [])
        if s.ring_slots and self.runs:
            self._runs_arr = (RingRun * len(self.runs))(*[RingRun(*map(int, r)) for r in self.runs])
            self.ring_desc = RingDesc(R, s.ring_slots, s.ring_width, HRS_BF16, R * T, len(self.runs),
                                      self._runs_arr)
        else:
            self.ring_desc = None

        b = bufs
        ptr = lambda t, l: t[l].data_ptr()
        self.layer_args: List[tuple] = []
        for l in range(L):
            self.layer_args.append((
                (ptr(b.x, l), ptr(b.w, l), ptr(b.conv_state, l), ptr(b.conv_ckpt, l), ptr(b.y, l)),
                (ptr(b.q, l), ptr(b.k, l), ptr(b.v, l), ptr(b.a, l), ptr(b.b, l), ptr(b.state, l),
                 ptr(b.ckpt, l), ptr(b.out, l)),
            ))
        if s.vocab:
            self.accept_args = (b.logits.data_ptr(), b.tokens.data_ptr(), b.argmax.data_ptr(),
                                b.accept_node.data_ptr(), b.accept_len.data_ptr(), b.path.data_ptr(),
                                b.bonus.data_ptr(), b.workspace.data_ptr(),
                                b.workspace.numel())
        self.rb_args = (b.ckpt.data_ptr(), b.state.data_ptr(), b.conv_ckpt.data_ptr(), b.conv_state.data_ptr(),
                        b.accept_node.data_ptr(), b.status.data_ptr())
        self.gdn_p = ctypes.byref(self.gdn_desc)
        self.conv_p = ctypes.byref(self.conv_desc)
        self.rb_p = ctypes.byref(self.rb_desc)

    # -- pieces -------------------------------------------------------------
    def launch_layer(self, l: int, stream: int, events=None) -> None:
        """conv then GDN of layer l. events: optional (start, stop) raw
        hipEvent_t handles recorded by the GDN dispatch itself."""
        conv_a, gdn_a = self.layer_args[l]
        _check(lib.conv1d_verify_span(self.conv_p, *conv_a, stream), "conv1d_verify_span")
        if events is None:
            _check(lib.gdn_verify_span(self.gdn_p, *gdn_a, stream), "gdn_verify_span")
        else:
            _check(lib.gdn_verify_span_timed(self.gdn_p, *gdn_a, stream, events[0], events[1]), "gdn_verify_span")

    def launch_conv(self, l: int, stream: int) -> None:
        """The conv span of layer l alone."""
        _check(lib.conv1d_verify_span(self.conv_p, *self.layer_args[l][0], stream), "conv1d_verify_span")

    def launch_gdn(self, l: int, stream: int, events=None) -> None:
        """The GDN span of layer l alone (its inputs as the step leaves them).
        events: optional (start, stop) raw hipEvent_t handles recorded by the
        dispatch itself."""
        if events is None:
            _check(lib.gdn_verify_span(self.gdn_p, *self.layer_args[l][1], stream), "gdn_verify_span")
        else:
            _check(lib.gdn_verify_span_timed(self.gdn_p, *self.layer_args[l][1], stream, events[0], events[1]),
                   "gdn_verify_span")

    def launch_accept(self, stream: int) -> None:
        if self.accept_desc is not None:
            _check(lib.accept_greedy(ctypes.byref(self.accept_desc), *self.accept_args, stream), "accept_greedy")

    def launch_rollback(self, stream: int) -> None:
        _check(lib.rollback_restore(self.rb_p, *self.rb_args, stream), "rollback_restore")

    def launch_ring(self, stream: int) -> None:
        if self.ring_desc is None:
            return
        b = self.bufs
        _check(lib.ring_set_2d(ctypes.byref(self.ring_desc), b.ring.data_ptr(), b.packed_in.data_ptr(), stream),
               "ring_set_2d")
        _check(lib.ring_get_2d(ctypes.byref(self.ring_desc), b.ring.data_ptr(), b.packed_out.data_ptr(), stream),
               "ring_get_2d")

    # -- whole step -----------------------------------------------------------
    def launch(self, stream=None, gdn_events=None) -> None:
        """Issue the whole step on ``stream`` (torch stream or raw handle); no sync.

        gdn_events: optional list of (start, stop) raw hipEvent_t handles per
        layer (see ``event_handle``), recorded by each GDN dispatch.
        """
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        h = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        for l in range(self.bufs.shape.n_layers):
            self.launch_layer(l, h, None if gdn_events is None else gdn_events[l])
        self.launch_accept(h)
        self.launch_rollback(h)
        self.launch_ring(h)

    def _gather(self) -> None:
        """Device-side gather of accepted lengths and bonus tokens into one buffer."""
        b = self.bufs
        R = self.bufs.shape.n_req
        b.dev_result[:R].copy_(b.accept_len)
        b.dev_result[R:].copy_(b.bonus)

    def _host(self):
        b = self.bufs
        R = self.bufs.shape.n_req
        b.host_result.copy_(b.dev_result)   # blocking copy into pinned memory
        return b.host_result[:R].numpy().copy(), b.host_result[R:].numpy().copy()

    def finish(self):
        """The step's single host sync: accepted lengths and bonus tokens."""
        self._gather()
        return self._host()

    def run(self, stream=None):
        self.launch(stream)
        return self.finish()

    # -- graph launch ---------------------------------------------------------
    def capture_graph(self) -> None:
        """Record the whole step (every kernel and the device-side gather of
        the results) into one HIP graph. Buffers, descriptors and pointers
        are fixed, so replaying the graph is exactly one step. The graph holds
        kernel launches and device copies only (no memset nodes)."""
        import torch
        self.graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(self.graph, stream=side):
            self.launch(side)
            self._gather()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()

    def replay(self):
        """One step by graph replay, then the step's single host sync."""
        self.graph.replay()
        return self._host()


class ZeroCopyVerifyStep(VerifyStep):
    """Verify step with zero-copy rollback (gdn_verify_span_from) and compact
    conv state (conv1d_verify_span_nocapture + conv_state_advance).

    Two checkpoint buffers alternate between steps: step i writes buffer i % 2
    and its spans start from buffer (i - 1) % 2 at the accepted position that
    step i - 1's acceptance left in ``accept_node`` (the first step starts from
    ``state``). Nothing is copied to roll back; the conv state is rebuilt from
    the x rows along the accepted path. ``materialize()`` writes the canonical
    recurrent state into ``state`` (rollback_restore) when a caller needs it.
    Needs logits (acceptance produces the path the conv state follows).
    """

    def __init__(self, bufs: StepBuffers, parent=None, runs: Optional[Sequence[tuple]] = None,
                 silu: bool = False, q_scale: float = 1.0):
        import torch
        super().__init__(bufs, parent, runs, silu, q_scale)
        s = bufs.shape
        if not s.vocab:
            raise ValueError("zero-copy rollback needs logits: the conv state follows the accepted path")
        L, R, T = s.n_layers, s.n_req, s.n_pos
        if getattr(bufs, "ckpt2", None) is None:
            bufs.ckpt2 = torch.empty_like(bufs.ckpt)
        self.ckpts = (bufs.ckpt, bufs.ckpt2)
        b = bufs
        dt = HRS_BF16 if s.bf16 else HRS_F32
        self.adv_desc = ConvAdvanceDesc(L, R, T, s.conv_channels, s.conv_width, dt)
        self.adv_p = ctypes.byref(self.adv_desc)
        self.adv_args = (b.x.data_ptr(), b.conv_state.data_ptr(), b.path.data_ptr(), b.accept_len.data_ptr(), None)
        ptr = lambda t, l: t[l].data_ptr()
        self.conv_args = [(ptr(b.x, l), ptr(b.w, l), ptr(b.conv_state, l), ptr(b.y, l)) for l in range(L)]
        # [c][l]: inputs and outputs of layer l when writing checkpoint buffer c.
        self.srcs = [[SpanSource(ptr(self.ckpts[1 - c], l), b.accept_node.data_ptr(), T) for l in range(L)]
                     for c in range(2)]
        self.gdn_io = [[(ptr(b.q, l), ptr(b.k, l), ptr(b.v, l), ptr(b.a, l), ptr(b.b, l), ptr(self.ckpts[c], l),
                         ptr(b.out, l)) for l in range(L)] for c in range(2)]
        self.first = True
        self.cur = 0

    def launch_layer(self, l: int, stream: int, events=None) -> None:
        _check(lib.conv1d_verify_span_nocapture(self.conv_p, *self.conv_args[l], stream),
               "conv1d_verify_span_nocapture")
        q, k, v, a, bb, ck, out = self.gdn_io[self.cur][l]
        if self.first:
            _check(lib.gdn_verify_span(self.gdn_p, q, k, v, a, bb, self.layer_args[l][1][5], ck, out, stream),
                   "gdn_verify_span")
        else:
            _check(lib.gdn_verify_span_from(self.gdn_p, ctypes.byref(self.srcs[self.cur][l]), q, k, v, a, bb, ck,
                                            out, None, stream), "gdn_verify_span_from")

    def launch_rollback(self, stream: int) -> None:
        # The rollback of the recurrent state is the next step's source index;
        # only the conv state is rebuilt.
        _check(lib.conv_state_advance(self.adv_p, *self.adv_args, stream), "conv_state_advance")

    def launch(self, stream=None, gdn_events=None) -> None:
        super().launch(stream, gdn_events=None)
        self.first = False
        self.cur ^= 1

    def current_ckpt(self):
        """Checkpoint buffer written by the last launched step."""
        return self.ckpts[self.cur ^ 1]

    def materialize(self, stream=None) -> None:
        """state <- checkpoint of the accepted position of the last step (all layers)."""
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        h = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        s = self.bufs.shape
        d = RollbackDesc(s.n_layers, s.n_req, s.n_pos, s.n_vheads, s.d_k, s.d_v, 0, 0, HRS_F32)
        b = self.bufs
        _check(lib.rollback_restore(ctypes.byref(d), self.current_ckpt().data_ptr(), b.state.data_ptr(), None, None,
                                    b.accept_node.data_ptr(), b.status.data_ptr(), h), "rollback_restore")

    def capture_graph(self) -> None:
        """Record two HIP graphs, one per checkpoint-buffer parity: graph c
        writes buffer c and starts every span from buffer 1 - c at the
        accepted position the previous step left in ``accept_node``. Replays
        alternate between them, as eager steps alternate buffers. The first
        step of a speculation starts from ``state`` and is launched eagerly
        (``replay`` does that by itself when no step has run yet)."""
        import torch
        first, cur = self.first, self.cur
        self.graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        try:
            self.first = False
            for c in (0, 1):
                self.cur = c
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    VerifyStep.launch(self, side)
                    self._gather()
                self.graphs.append(g)
        finally:
            self.first, self.cur = first, cur
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()

    def replay(self):
        """One step by replaying the graph of the current buffer parity (the
        first step of a speculation eagerly), then the step's single host
        sync."""
        if self.first:
            return self.run()
        self.graphs[self.cur].replay()
        self.cur ^= 1
        return self._host()


class FusedVerifyStep(ZeroCopyVerifyStep):
    """Zero-copy verify step whose layers run in their own order in one kernel
    each (gdn_layer_verify_span: conv, SiLU, split, q/k L2 norm and the gated
    delta rule). q, k and v are computed on the chip from x, so the q, k, v
    and y buffers are not used. Rollback as in ZeroCopyVerifyStep: the next
    spans start from the accepted checkpoint, the conv state is rebuilt from
    the accepted path (conv_state_advance).
    """

    def __init__(self, bufs: StepBuffers, parent=None, runs: Optional[Sequence[tuple]] = None,
                 silu: bool = True, q_scale: float = 1.0, l2_eps: float = 1e-6):
        super().__init__(bufs, parent, runs, silu, q_scale)
        s = bufs.shape
        if s.conv_channels != 2 * s.n_kheads * s.d_k + s.n_vheads * s.d_v:
            raise ValueError("the fused layer needs conv channels = 2*Hk*d_k + Hv*d_v (q | k | v)")
        self.layer_desc = GdnLayerDesc(self.gdn_desc, s.conv_width, int(silu), float(l2_eps))
        self.layer_p = ctypes.byref(self.layer_desc)
        b = bufs
        L = s.n_layers
        ptr = lambda t, l: t[l].data_ptr()
        self.fused_in = [(ptr(b.x, l), ptr(b.w, l), ptr(b.conv_state, l), ptr(b.a, l), ptr(b.b, l))
                         for l in range(L)]
        self.fused_out = [[(ptr(self.ckpts[c], l), ptr(b.out, l)) for l in range(L)] for c in range(2)]

    def launch_layer(self, l: int, stream: int, events=None) -> None:
        ck, out = self.fused_out[self.cur][l]
        if self.first:
            state, src = self.layer_args[l][1][5], None
        else:
            state, src = None, ctypes.byref(self.srcs[self.cur][l])
        _check(lib.gdn_layer_verify_span(self.layer_p, *self.fused_in[l], state, src, ck, out, None, stream),
               "gdn_layer_verify_span")
