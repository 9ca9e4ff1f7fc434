"""Python binding of libhrs: verify-span checkpoints, greedy acceptance and
on-device rollback for Gated DeltaNet layers on MI355X (gfx950).

Argument marshalling only. Every function here takes torch tensors that
live on the GPU, checks that they are contiguous and of the expected dtype,
and passes raw pointers, sizes and the current HIP stream to the C ABI in
include/hrs.h; all computation happens in the HIP kernels of libhrs.so. A
negative status from the library raises ``HrsError``.

The library must be built first (``python hybrid_recurrent_state_amd/csrc/build.py``
or ``__graft_entry__.build()``); importing this package without it raises
ImportError, so nothing silently falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhrs.so")

HRS_OK, HRS_EINVAL, HRS_EGEOMETRY, HRS_EALIGN, HRS_EDEVICE, HRS_EUNSUPPORTED = 0, -1, -2, -3, -4, -5
HRS_F32, HRS_BF16 = 0, 1
HRS_CHAIN, HRS_TREE = 0, 1
HRS_MAX_POS = 64
GEOMETRY_CLASSES = {0: "OK", 1: "NULL", 2: "TRUNCATED", 3: "ROOT", 4: "RANGE", 5: "FORWARD", 6: "NOT_CHAIN"}


class HrsError(RuntimeError):
    def __init__(self, status: int, func: str):
        self.status = status
        detail = ""
        if status == HRS_EDEVICE:
            detail = f"; HIP error {lib.hrs_last_hip_error()}: {lib.hrs_last_hip_error_string().decode()}"
        super().__init__(f"{func}: {strerror(status)} (status {status}){detail}")


# --- C structs (mirror include/hrs.h) -------------------------------------
_i32 = ctypes.c_int32
_p = ctypes.c_void_p


class GdnDesc(ctypes.Structure):
    _fields_ = [("n_req", _i32), ("n_pos", _i32), ("n_kheads", _i32), ("n_vheads", _i32),
                ("d_k", _i32), ("d_v", _i32), ("in_dtype", _i32), ("q_scale", ctypes.c_float),
                ("topo", _i32), ("parent", ctypes.POINTER(_i32))]


class ChunkedDesc(ctypes.Structure):
    _fields_ = [("gdn", GdnDesc), ("log_gates", _i32), ("out_dtype", _i32)]


class GdnLayerDesc(ctypes.Structure):
    _fields_ = [("gdn", GdnDesc), ("conv_width", _i32), ("silu", _i32), ("l2_eps", ctypes.c_float)]


class ConvDesc(ctypes.Structure):
    _fields_ = [("n_req", _i32), ("n_pos", _i32), ("channels", _i32), ("width", _i32),
                ("dtype", _i32), ("silu", _i32), ("topo", _i32), ("parent", ctypes.POINTER(_i32))]


class AcceptDesc(ctypes.Structure):
    _fields_ = [("n_req", _i32), ("n_pos", _i32), ("vocab", _i32), ("logit_dtype", _i32),
                ("topo", _i32), ("parent", ctypes.POINTER(_i32))]


class SpanSource(ctypes.Structure):
    _fields_ = [("ckpt", _p), ("node", _p), ("n_pos", _i32)]


class ConvAdvanceDesc(ctypes.Structure):
    _fields_ = [("n_layers", _i32), ("n_req", _i32), ("n_pos", _i32), ("channels", _i32), ("width", _i32),
                ("dtype", _i32)]


class RollbackDesc(ctypes.Structure):
    _fields_ = [("n_layers", _i32), ("n_req", _i32), ("n_pos", _i32), ("n_vheads", _i32),
                ("d_k", _i32), ("d_v", _i32), ("conv_channels", _i32), ("conv_width", _i32),
                ("conv_dtype", _i32)]


class RingRun(ctypes.Structure):
    _fields_ = [("ring_id", _i32), ("start_pos", _i32), ("n_rows", _i32), ("packed_row", _i32)]


class RingDesc(ctypes.Structure):
    _fields_ = [("n_rings", _i32), ("n_slots", _i32), ("width", _i32), ("dtype", _i32),
                ("n_packed_rows", _i32), ("n_runs", _i32), ("runs", ctypes.POINTER(RingRun))]


# Exported symbols and their signatures (every function of include/hrs.h).
_SIGNATURES = {
    "hrs_validate_tree": (_i32, [ctypes.POINTER(_i32), _i32, _i32, ctypes.POINTER(_i32)]),
    "gdn_verify_span": (_i32, [ctypes.POINTER(GdnDesc), _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "gdn_verify_span_timed": (_i32, [ctypes.POINTER(GdnDesc), _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "gdn_verify_span_from": (_i32, [ctypes.POINTER(GdnDesc), ctypes.POINTER(SpanSource), _p, _p, _p, _p, _p, _p,
                                    _p, _p, _p]),
    "gdn_span_chunked_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(ChunkedDesc)]),
    "gdn_span_chunked": (_i32, [ctypes.POINTER(ChunkedDesc), _p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t,
                                _p]),
    "gdn_layer_verify_span": (_i32, [ctypes.POINTER(GdnLayerDesc), _p, _p, _p, _p, _p, _p,
                                     ctypes.POINTER(SpanSource), _p, _p, _p, _p]),
    "conv1d_verify_span_nocapture": (_i32, [ctypes.POINTER(ConvDesc), _p, _p, _p, _p, _p]),
    "conv_state_advance": (_i32, [ctypes.POINTER(ConvAdvanceDesc), _p, _p, _p, _p, _p, _p]),
    "conv1d_verify_span": (_i32, [ctypes.POINTER(ConvDesc), _p, _p, _p, _p, _p, _p]),
    "accept_greedy_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(AcceptDesc)]),
    "accept_greedy": (_i32, [ctypes.POINTER(AcceptDesc), _p, _p, _p, _p, _p, _p, _p, _p,
                             ctypes.c_size_t, _p]),
    "accept_greedy_noalloc": (_i32, [ctypes.POINTER(AcceptDesc), _p, _p, _p, _p, _p, _p, _p, _p]),
    "rollback_restore": (_i32, [ctypes.POINTER(RollbackDesc), _p, _p, _p, _p, _p, _p, _p]),
    "ring_set_2d": (_i32, [ctypes.POINTER(RingDesc), _p, _p, _p]),
    "ring_get_2d": (_i32, [ctypes.POINTER(RingDesc), _p, _p, _p]),
    "hrs_strerror": (ctypes.c_char_p, [_i32]),
    "hrs_abi_version": (_i32, []),
    "hrs_last_hip_error": (_i32, []),
    "hrs_last_hip_error_string": (ctypes.c_char_p, []),
}
EXPORTED = tuple(_SIGNATURES)


def _hip_runtimes_mapped():
    """Distinct HIP runtime files mapped into this process."""
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    found.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return found


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python hybrid_recurrent_state_amd/csrc/build.py`")
    # torch owns device memory and streams. Its HIP runtime must be the one
    # this library binds to: load torch first, so that the library's
    # libamdhip64.so.7 dependency resolves (by soname) to the runtime that is
    # already in the process instead of a second copy from /opt/rocm.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are loaded ({sorted(runtimes)}); libhrs must share torch's")
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def strerror(status: int) -> str:
    return lib.hrs_strerror(int(status)).decode()


def abi_version() -> int:
    return int(lib.hrs_abi_version())


def _check(status: int, func: str) -> None:
    if status != HRS_OK:
        raise HrsError(status, func)


# --- marshalling helpers --------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return HRS_F32
    if t.dtype == torch.bfloat16:
        return HRS_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


class _Checks:
    """Rejects, before anything is launched, a tensor that the kernels would
    read or write out of bounds or as the wrong type. Calls check each
    tensor's shape (the library takes every size from the leading tensor),
    dtype and layout; on_gpu() then checks that all of them are on the GPU."""

    def __init__(self):
        self.seen = []

    def __call__(self, name: str, t, shape=None, dtypes=None, optional: bool = False) -> None:
        if t is None:
            if optional:
                return
            raise ValueError(f"{name} is required")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
        if dtypes is not None and t.dtype not in dtypes:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        self.seen.append((name, t))

    def status(self, status, optional: bool = True) -> None:
        self("status", status, None, _i32t(), optional)
        if status is not None and status.numel() < 1:
            raise ValueError("status needs at least one int32")

    def on_gpu(self) -> None:
        for name, t in self.seen:
            if not t.is_cuda:
                raise ValueError(f"{name} must be a GPU tensor")


def _in_dtypes(name: str, t):
    """The input dtype of a call (f32 or bf16), checked on its leading tensor."""
    torch = _torch()
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"{name}: dtype {t.dtype}, expected torch.float32 or torch.bfloat16")
    return (t.dtype,)


def _f32():
    return (_torch().float32,)


def _i32t():
    return (_torch().int32,)


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _parent_array(parent, n_req: int, n_pos: int):
    """Host int32 [n_req * n_pos] array (a single [n_pos] row is repeated).

    The library reads exactly n_req * n_pos entries, so any other size is
    rejected here instead of being over-read or silently truncated."""
    if parent is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(parent, dtype=np.int32)).reshape(-1)
    if arr.size == n_pos and n_req > 1:
        arr = np.ascontiguousarray(np.tile(arr, n_req))
    if arr.size != n_req * n_pos:
        raise ValueError(f"parent: {arr.size} entries, expected {n_pos} (one row for every request) "
                         f"or {n_req * n_pos} ({n_req} requests x {n_pos} positions)")
    return arr, arr.ctypes.data_as(ctypes.POINTER(_i32))


# --- entry points (same names as the C ABI) -------------------------------

def validate_tree(parent, n_pos: Optional[int] = None, require_chain: bool = False):
    """Run the host geometry guard. Returns (status, class name)."""
    cls = _i32(-1)
    if parent is None:
        st = lib.hrs_validate_tree(None, int(n_pos or 0), int(require_chain), ctypes.byref(cls))
    else:
        arr = np.ascontiguousarray(np.asarray(parent, dtype=np.int32)).reshape(-1)
        n = arr.size if n_pos is None else int(n_pos)
        st = lib.hrs_validate_tree(arr.ctypes.data_as(ctypes.POINTER(_i32)), n, int(require_chain),
                                   ctypes.byref(cls))
    return int(st), GEOMETRY_CLASSES.get(cls.value, "?")


hrs_validate_tree = validate_tree


def event_handle(ev) -> int:
    """Raw hipEvent_t of a torch.cuda.Event (created by recording it once)."""
    if not ev.cuda_event:
        ev.record()
    return ev.cuda_event


def gdn_verify_span(q, k, v, a, b, state, ckpt, out, parent=None, q_scale: float = 1.0, stream=None,
                    events=None):
    """q, k [R,T,Hk,dk]; v [R,T,Hv,dv]; a, b [R,T,Hv] (f32 or bf16);
    state [R,Hv,dv,dk] f32; ckpt [R,T,Hv,dv,dk] f32 or None; out [R,T,Hv,dv] f32.
    parent: None (chain) or host ints [R,T] / [T] (tree).
    events: optional (start, stop) torch.cuda.Event pair recorded by the
    kernel dispatch itself (gdn_verify_span_timed)."""
    R, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dt = _in_dtypes("q", q)
    chk = _Checks()
    chk("q", q, None, dt)
    chk("k", k, (R, T, Hk, dk), dt)
    chk("v", v, (R, T, Hv, dv), dt)
    chk("a", a, (R, T, Hv), dt)
    chk("b", b, (R, T, Hv), dt)
    chk("state", state, (R, Hv, dv, dk), _f32())
    chk("ckpt", ckpt, (R, T, Hv, dv, dk), _f32(), optional=True)
    chk("out", out, (R, T, Hv, dv), _f32())
    par, par_p = _parent_array(parent, R, T)
    chk.on_gpu()
    d = GdnDesc(R, T, Hk, Hv, dk, dv, _dtype_code(q), float(q_scale),
                HRS_TREE if parent is not None else HRS_CHAIN, par_p)
    args = (ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(state), _ptr(ckpt), _ptr(out),
            _stream(stream))
    if events is None:
        st = lib.gdn_verify_span(*args)
    else:
        st = lib.gdn_verify_span_timed(*args, event_handle(events[0]), event_handle(events[1]))
    _check(st, "gdn_verify_span")


def gdn_verify_span_from(src_ckpt, src_node, q, k, v, a, b, ckpt, out, parent=None, status=None,
                         q_scale: float = 1.0, stream=None):
    """Zero-copy rollback: like gdn_verify_span, but request r starts from
    src_ckpt[r][src_node[r]] (src_ckpt [R,Tp,Hv,dv,dk] f32, src_node [R] int32,
    both on the device) instead of a state buffer."""
    R, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dt = _in_dtypes("q", q)
    chk = _Checks()
    chk("q", q, None, dt)
    chk("k", k, (R, T, Hk, dk), dt)
    chk("v", v, (R, T, Hv, dv), dt)
    chk("a", a, (R, T, Hv), dt)
    chk("b", b, (R, T, Hv), dt)
    chk("src_ckpt", src_ckpt, None, _f32())
    chk("src_ckpt", src_ckpt, (R, src_ckpt.shape[1], Hv, dv, dk), _f32())
    chk("src_node", src_node, (R,), _i32t())
    chk("ckpt", ckpt, (R, T, Hv, dv, dk), _f32())
    chk("out", out, (R, T, Hv, dv), _f32())
    chk.status(status)
    par, par_p = _parent_array(parent, R, T)
    chk.on_gpu()
    d = GdnDesc(R, T, Hk, Hv, dk, dv, _dtype_code(q), float(q_scale),
                HRS_TREE if parent is not None else HRS_CHAIN, par_p)
    src = SpanSource(_ptr(src_ckpt), _ptr(src_node), src_ckpt.shape[1])
    st = lib.gdn_verify_span_from(ctypes.byref(d), ctypes.byref(src), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                  _ptr(ckpt), _ptr(out), _ptr(status), _stream(stream))
    _check(st, "gdn_verify_span_from")


def gdn_span_chunked_workspace_bytes(n_req: int, n_pos: int, n_kheads: int, n_vheads: int, d: int = 128) -> int:
    """Device workspace bytes gdn_span_chunked needs for these sizes."""
    g = GdnDesc(n_req, n_pos, n_kheads, n_vheads, d, d, HRS_BF16, 1.0, HRS_CHAIN, None)
    return int(lib.gdn_span_chunked_workspace_bytes(ctypes.byref(ChunkedDesc(g, 0, HRS_F32))))


def gdn_span_chunked(q, k, v, a, b, state, ckpt, out, workspace, q_scale: float = 1.0, log_gates: bool = False,
                     stream=None):
    """Chunked (64-position) gated delta rule over a long chain span: same
    arguments as gdn_verify_span without a parent; ckpt None updates state
    in place. log_gates: `a` holds log decays. out may be f32 or bf16.
    workspace: device tensor of at least gdn_span_chunked_workspace_bytes."""
    R, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    torch = _torch()
    dt = _in_dtypes("q", q)
    chk = _Checks()
    chk("q", q, None, dt)
    chk("k", k, (R, T, Hk, dk), dt)
    chk("v", v, (R, T, Hv, dv), dt)
    chk("a", a, (R, T, Hv), dt)
    chk("b", b, (R, T, Hv), dt)
    chk("state", state, (R, Hv, dv, dk), _f32())
    chk("ckpt", ckpt, (R, T, Hv, dv, dk), _f32(), optional=True)
    chk("out", out, (R, T, Hv, dv), (torch.float32, torch.bfloat16))
    chk("workspace", workspace)
    chk.on_gpu()
    g = GdnDesc(R, T, Hk, Hv, dk, dv, _dtype_code(q), float(q_scale), HRS_CHAIN, None)
    d = ChunkedDesc(g, int(bool(log_gates)), _dtype_code(out))
    nbytes = workspace.numel() * workspace.element_size()
    st = lib.gdn_span_chunked(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(state), _ptr(ckpt),
                              _ptr(out), _ptr(workspace), nbytes, _stream(stream))
    _check(st, "gdn_span_chunked")


def gdn_layer_verify_span(x, conv_w, conv_state, a, b, ckpt, out, n_kheads: int, d_k: int, state=None,
                          src_ckpt=None, src_node=None, parent=None, status=None, q_scale: float = 1.0,
                          l2_eps: float = 1e-6, silu: bool = True, stream=None):
    """One GDN layer in its own order (conv, SiLU, split, q/k L2 norm, gated
    delta rule) in one kernel. x [R,T,C] with C = 2*Hk*dk + Hv*dv, channels
    [q | k | v]; conv_w [C,4]; conv_state [R,3,C] (read only); a, b [R,T,Hv];
    ckpt [R,T,Hv,dv,dk] f32; out [R,T,Hv,dv] f32. The initial state is either
    state [R,Hv,dv,dk] f32 or src_ckpt[r][src_node[r]] (zero-copy)."""
    R, T, C = x.shape
    Hv = a.shape[2]
    dv = (C - 2 * n_kheads * d_k) // Hv
    if Hv < 1 or C != 2 * n_kheads * d_k + Hv * dv:
        raise ValueError(f"x: {C} channels do not split into q, k ({n_kheads} x {d_k} each) and {Hv} v heads")
    dt = _in_dtypes("x", x)
    chk = _Checks()
    chk("x", x, None, dt)
    chk("conv_w", conv_w, (C, conv_w.shape[1] if conv_w is not None and conv_w.dim() == 2 else 4), dt)
    chk("conv_state", conv_state, (R, conv_w.shape[1] - 1, C), dt)
    chk("a", a, (R, T, Hv), dt)
    chk("b", b, (R, T, Hv), dt)
    chk("ckpt", ckpt, (R, T, Hv, dv, d_k), _f32())
    chk("out", out, (R, T, Hv, dv), _f32())
    chk("state", state, (R, Hv, dv, d_k), _f32(), optional=True)
    if src_ckpt is not None:
        chk("src_ckpt", src_ckpt, None, _f32())
        chk("src_ckpt", src_ckpt, (R, src_ckpt.shape[1], Hv, dv, d_k), _f32())
        chk("src_node", src_node, (R,), _i32t())
    chk.status(status)
    par, par_p = _parent_array(parent, R, T)
    chk.on_gpu()
    g = GdnDesc(R, T, n_kheads, Hv, d_k, dv, _dtype_code(x), float(q_scale),
                HRS_TREE if parent is not None else HRS_CHAIN, par_p)
    d = GdnLayerDesc(g, conv_w.shape[1], int(bool(silu)), float(l2_eps))
    src = None
    if src_ckpt is not None:
        src = ctypes.byref(SpanSource(_ptr(src_ckpt), _ptr(src_node), src_ckpt.shape[1]))
    st = lib.gdn_layer_verify_span(ctypes.byref(d), _ptr(x), _ptr(conv_w), _ptr(conv_state), _ptr(a), _ptr(b),
                                   _ptr(state), src, _ptr(ckpt), _ptr(out), _ptr(status), _stream(stream))
    _check(st, "gdn_layer_verify_span")


def conv1d_verify_span_nocapture(x, w, conv_state, y, parent=None, silu: bool = False, stream=None):
    """conv output y only; conv_state [R,W-1,C] is read only."""
    R, T, C = x.shape
    dt = _in_dtypes("x", x)
    chk = _Checks()
    chk("x", x, None, dt)
    chk("w", w, None, dt)
    W = w.shape[1] if w.dim() == 2 else 0
    chk("w", w, (C, W), dt)
    chk("conv_state", conv_state, (R, W - 1, C), dt)
    chk("y", y, (R, T, C), _f32())
    par, par_p = _parent_array(parent, R, T)
    chk.on_gpu()
    d = ConvDesc(R, T, C, W, _dtype_code(x), int(bool(silu)), HRS_TREE if parent is not None else HRS_CHAIN, par_p)
    st = lib.conv1d_verify_span_nocapture(ctypes.byref(d), _ptr(x), _ptr(w), _ptr(conv_state), _ptr(y),
                                          _stream(stream))
    _check(st, "conv1d_verify_span_nocapture")


def conv_state_advance(x, conv_state, path, accept_len, status=None, stream=None):
    """x [L,R,T,C]; conv_state [L,R,W-1,C]; path [R,T], accept_len [R] int32 (device)."""
    L, R, T, C = x.shape
    dt = _in_dtypes("x", x)
    chk = _Checks()
    chk("x", x, None, dt)
    chk("conv_state", conv_state, None, dt)
    chk("conv_state", conv_state, (L, R, conv_state.shape[2], C), dt)
    chk("path", path, (R, T), _i32t())
    chk("accept_len", accept_len, (R,), _i32t())
    chk.status(status)
    chk.on_gpu()
    d = ConvAdvanceDesc(L, R, T, C, conv_state.shape[2] + 1, _dtype_code(x))
    st = lib.conv_state_advance(ctypes.byref(d), _ptr(x), _ptr(conv_state), _ptr(path), _ptr(accept_len),
                                _ptr(status), _stream(stream))
    _check(st, "conv_state_advance")


def conv1d_verify_span(x, w, conv_state, conv_ckpt, y, parent=None, silu: bool = False, stream=None):
    """x [R,T,C]; w [C,W]; conv_state [R,W-1,C]; conv_ckpt [R,T,W-1,C] or None
    (same dtype as x); y [R,T,C] f32. parent: None (chain) or host [R,T]/[T]."""
    R, T, C = x.shape
    dt = _in_dtypes("x", x)
    chk = _Checks()
    chk("x", x, None, dt)
    chk("w", w, None, dt)
    W = w.shape[1] if w.dim() == 2 else 0
    chk("w", w, (C, W), dt)
    chk("conv_state", conv_state, (R, W - 1, C), dt)
    chk("conv_ckpt", conv_ckpt, (R, T, W - 1, C), dt, optional=True)
    chk("y", y, (R, T, C), _f32())
    par, par_p = _parent_array(parent, R, T)
    chk.on_gpu()
    d = ConvDesc(R, T, C, W, _dtype_code(x), int(bool(silu)),
                 HRS_TREE if parent is not None else HRS_CHAIN, par_p)
    st = lib.conv1d_verify_span(ctypes.byref(d), _ptr(x), _ptr(w), _ptr(conv_state), _ptr(conv_ckpt),
                                _ptr(y), _stream(stream))
    _check(st, "conv1d_verify_span")


def accept_desc(n_req: int, n_pos: int, vocab: int, logit_dtype: int, parent=None):
    par, par_p = _parent_array(parent, n_req, n_pos)
    d = AcceptDesc(n_req, n_pos, vocab, logit_dtype, HRS_TREE if parent is not None else HRS_CHAIN, par_p)
    return d, par


def accept_greedy_workspace_bytes(n_req: int, n_pos: int, vocab: int, logit_dtype: int = HRS_BF16,
                                  parent=None) -> int:
    d, _keep = accept_desc(n_req, n_pos, vocab, logit_dtype, parent)
    return int(lib.accept_greedy_workspace_bytes(ctypes.byref(d)))


def accept_greedy(logits, tokens, argmax, accept_node, accept_len, path, bonus, workspace,
                  parent=None, stream=None):
    """logits [R,T,V]; tokens [R,T] int32; outputs int32 device tensors
    argmax [R,T], accept_node [R], accept_len [R], path [R,T], bonus [R];
    workspace: device tensor of at least accept_greedy_workspace_bytes."""
    R, T, V = logits.shape
    chk = _Checks()
    chk("logits", logits, None, _in_dtypes("logits", logits))
    for name, t, shape in (("tokens", tokens, (R, T)), ("argmax", argmax, (R, T)), ("accept_node", accept_node, (R,)),
                           ("accept_len", accept_len, (R,)), ("path", path, (R, T)), ("bonus", bonus, (R,))):
        chk(name, t, shape, _i32t())
    chk("workspace", workspace)
    d, _keep = accept_desc(R, T, V, _dtype_code(logits), parent)
    chk.on_gpu()
    nbytes = workspace.numel() * workspace.element_size()
    st = lib.accept_greedy(ctypes.byref(d), _ptr(logits), _ptr(tokens), _ptr(argmax), _ptr(accept_node),
                           _ptr(accept_len), _ptr(path), _ptr(bonus), _ptr(workspace), nbytes,
                           _stream(stream))
    _check(st, "accept_greedy")


ACCEPT_NOALLOC_MAX_BYTES = 1 << 20


def accept_greedy_noalloc(logits, tokens, argmax, accept_node, accept_len, path, bonus, parent=None, stream=None):
    """accept_greedy without a workspace: the library keeps the keys in a
    fixed device array of ACCEPT_NOALLOC_MAX_BYTES per GPU (no allocation in
    the call). Overlapping calls on one GPU share that array and race."""
    R, T, V = logits.shape
    chk = _Checks()
    chk("logits", logits, None, _in_dtypes("logits", logits))
    for name, t, shape in (("tokens", tokens, (R, T)), ("argmax", argmax, (R, T)), ("accept_node", accept_node, (R,)),
                           ("accept_len", accept_len, (R,)), ("path", path, (R, T)), ("bonus", bonus, (R,))):
        chk(name, t, shape, _i32t())
    d, _keep = accept_desc(R, T, V, _dtype_code(logits), parent)
    chk.on_gpu()
    st = lib.accept_greedy_noalloc(ctypes.byref(d), _ptr(logits), _ptr(tokens), _ptr(argmax), _ptr(accept_node),
                                   _ptr(accept_len), _ptr(path), _ptr(bonus), _stream(stream))
    _check(st, "accept_greedy_noalloc")


def rollback_restore(ckpt, state, conv_ckpt, conv_state, accept_node, status, stream=None):
    """ckpt [L,R,T,Hv,dv,dk] f32 -> state [L,R,Hv,dv,dk]; conv_ckpt
    [L,R,T,W-1,C] -> conv_state [L,R,W-1,C] (both None to skip);
    accept_node [R] int32 device; status [>=1] int32 device."""
    L, R, T, Hv, dv, dk = ckpt.shape
    chk = _Checks()
    chk("ckpt", ckpt, None, _f32())
    chk("state", state, (L, R, Hv, dv, dk), _f32())
    chk("accept_node", accept_node, (R,), _i32t())
    chk.status(status, optional=False)
    if (conv_ckpt is None) != (conv_state is None):
        raise ValueError("conv_ckpt and conv_state go together")
    if conv_ckpt is not None:
        cdt_t = _in_dtypes("conv_ckpt", conv_ckpt)
        chk("conv_ckpt", conv_ckpt, None, cdt_t)
        if conv_ckpt.dim() != 5 or tuple(conv_ckpt.shape[:3]) != (L, R, T):
            raise ValueError(f"conv_ckpt: shape {tuple(conv_ckpt.shape)}, expected ({L}, {R}, {T}, W-1, C)")
        C, W1 = conv_ckpt.shape[4], conv_ckpt.shape[3]
        chk("conv_state", conv_state, (L, R, W1, C), cdt_t)
        cdt = _dtype_code(conv_ckpt)
    else:
        C, W1, cdt = 0, 0, HRS_F32
    chk.on_gpu()
    d = RollbackDesc(L, R, T, Hv, dk, dv, C, W1 + 1 if conv_ckpt is not None else 0, cdt)
    st = lib.rollback_restore(ctypes.byref(d), _ptr(ckpt), _ptr(state), _ptr(conv_ckpt), _ptr(conv_state),
                              _ptr(accept_node), _ptr(status), _stream(stream))
    _check(st, "rollback_restore")


def _ring_desc(ring, packed, runs: Sequence[tuple]):
    n_rings, S, D = ring.shape
    dt = _in_dtypes("ring", ring)
    chk = _Checks()
    chk("ring", ring, None, dt)
    chk("packed", packed, None, dt)
    if packed.dim() != 2 or packed.shape[1] != D:
        raise ValueError(f"packed: shape {tuple(packed.shape)}, expected (rows, {D})")
    chk.on_gpu()
    n_packed_rows = packed.shape[0]
    arr = (RingRun * max(1, len(runs)))(*[RingRun(*map(int, r)) for r in runs])
    d = RingDesc(n_rings, S, D, _dtype_code(ring), n_packed_rows, len(runs), arr)
    return d, arr


def ring_set_2d(ring, packed, runs, stream=None):
    """ring [n_rings,S,D]; packed [N,D]; runs: (ring_id, start_pos, n_rows, packed_row)."""
    d, _keep = _ring_desc(ring, packed, runs)
    _check(lib.ring_set_2d(ctypes.byref(d), _ptr(ring), _ptr(packed), _stream(stream)), "ring_set_2d")


def ring_get_2d(ring, packed, runs, stream=None):
    d, _keep = _ring_desc(ring, packed, runs)
    _check(lib.ring_get_2d(ctypes.byref(d), _ptr(ring), _ptr(packed), _stream(stream)), "ring_get_2d")
