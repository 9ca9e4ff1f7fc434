"""The C-ABI boundary on the host: the library loads, exports every function
include/hrs.h declares, and rejects malformed calls before any launch.

No compute runs here. Device pointers are fake aligned addresses that the
host code never dereferences; a call that got past its checks would try to
launch and return HRS_EDEVICE (no GPU is visible), so seeing the specific
rejection code proves the check ran first, and a well-formed call must end
in HRS_EDEVICE: a launch can never count as a pass.

The module runs only where no GPU is visible. On a machine with a GPU those
well-formed calls would launch kernels on the fake addresses, so the whole
module is skipped there (the GPU tests cover the same entry points with real
buffers).
"""
import ctypes
import os
import re

import numpy as np
import pytest

from tests.conftest import ROOT


def _gpu_visible() -> bool:
    """True when a GPU could be reached. Checks the kernel driver's device
    node first and then torch's device count, neither of which initialises
    the HIP runtime."""
    if os.path.exists("/dev/kfd"):
        return True
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # noqa: BLE001 - no torch: no device through it either
        return False


if _gpu_visible():
    pytest.skip("host-only boundary checks: a GPU is visible, and a call that passes its checks "
                "would launch on fake device addresses", allow_module_level=True)


def _ensure_built():
    lib = os.path.join(ROOT, "hybrid_recurrent_state_amd", "libhrs.so")
    if not os.path.exists(lib):
        import __graft_entry__
        __graft_entry__.build()


_ensure_built()
import hybrid_recurrent_state_amd as hrs  # noqa: E402
from oracle import geometry as ogeo  # noqa: E402
from tests.test_oracle_geometry import load_cases  # noqa: E402

FAKE = 0x7F0000000000      # 16-byte aligned, never dereferenced on the host
MIS = FAKE + 4             # misaligned
P = ctypes.c_void_p


def header_functions():
    with open(os.path.join(ROOT, "include", "hrs.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return")))


def test_every_declared_function_is_exported():
    names = header_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(hrs.lib, n), n
    assert sorted(hrs.EXPORTED) == names
    assert len(hrs._hip_runtimes_mapped()) <= 1, "one HIP runtime per process"


def test_abi_version_and_strerror():
    assert hrs.abi_version() == 1
    for st in (0, -1, -2, -3, -4, -5):
        assert hrs.strerror(st) and hrs.strerror(st) != "unknown status"
    assert hrs.strerror(-99) == "unknown status"


def test_guard_matches_golden_and_oracle(golden_dir):
    codes = {v: k for k, v in ogeo.NAMES.items()}
    for name, parent, n, chain_v, tree_v in load_cases(golden_dir):
        for req_chain, exp in ((True, chain_v), (False, tree_v)):
            st, cls = hrs.validate_tree(parent, n, req_chain)
            assert cls == exp, (name, req_chain, cls)
            assert st == (0 if exp == "OK" else hrs.HRS_EGEOMETRY)
            assert codes[cls] == ogeo.check_tree(parent, n, req_chain)


def test_guard_random_arrays_agree_with_oracle():
    rng = np.random.default_rng(11)
    for _ in range(3000):
        T = int(rng.integers(0, 10))
        parent = rng.integers(-3, T + 2, T).astype(np.int32)
        if rng.random() < 0.5 and T > 0:
            parent = np.arange(-1, T - 1, dtype=np.int32)
            i = int(rng.integers(0, T))
            parent[i] = int(rng.integers(-2, T + 1))
        for req_chain in (True, False):
            st, cls = hrs.validate_tree(parent, T, req_chain)
            assert cls == ogeo.NAMES[ogeo.check_tree(parent, T, req_chain)]


# ---------------------------------------------------------------------------
# Fail-closed entry points


def gdn_call(**kw):
    d = dict(n_req=1, n_pos=4, n_kheads=2, n_vheads=4, d_k=128, d_v=128, in_dtype=hrs.HRS_BF16,
             q_scale=1.0, topo=hrs.HRS_CHAIN, parent=None)
    ptrs = dict(q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, state=FAKE, ckpt=FAKE, out=FAKE)
    for key in list(kw):
        if key in ptrs:
            ptrs[key] = kw.pop(key)
    d.update(kw)
    par = d.pop("parent")
    keep = None
    if par is not None:
        keep = np.ascontiguousarray(np.asarray(par, dtype=np.int32))
        par = keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    desc = hrs.GdnDesc(d["n_req"], d["n_pos"], d["n_kheads"], d["n_vheads"], d["d_k"], d["d_v"],
                       d["in_dtype"], d["q_scale"], d["topo"], par)
    return hrs.lib.gdn_verify_span(ctypes.byref(desc), ptrs["q"], ptrs["k"], ptrs["v"], ptrs["a"], ptrs["b"],
                                   ptrs["state"], ptrs["ckpt"], ptrs["out"], None)


def test_gdn_rejections():
    E = hrs
    assert hrs.lib.gdn_verify_span(None, *([FAKE] * 8), None) == E.HRS_EINVAL
    assert gdn_call(n_req=0) == E.HRS_EINVAL
    assert gdn_call(n_vheads=3) == E.HRS_EINVAL            # Hv % Hk
    assert gdn_call(in_dtype=7) == E.HRS_EINVAL
    assert gdn_call(topo=5) == E.HRS_EINVAL
    assert gdn_call(q=None) == E.HRS_EINVAL
    assert gdn_call(out=None) == E.HRS_EINVAL
    assert gdn_call(n_pos=0) == E.HRS_EGEOMETRY            # truncated
    assert gdn_call(n_pos=65) == E.HRS_EGEOMETRY
    assert gdn_call(topo=E.HRS_TREE, parent=None) == E.HRS_EGEOMETRY   # null geometry
    assert gdn_call(topo=E.HRS_TREE, parent=[-1, 0, 0, 1], ckpt=None) == E.HRS_EINVAL  # tree needs capture
    assert gdn_call(topo=E.HRS_TREE, parent=[-1, 0, 3, 1]) == E.HRS_EGEOMETRY  # forward
    assert gdn_call(topo=E.HRS_TREE, parent=[0, 0, 1, 1]) == E.HRS_EGEOMETRY   # root
    # second request of a batch malformed
    assert gdn_call(n_req=2, topo=E.HRS_TREE, parent=[-1, 0, 0, 1, -1, 0, -1, 2]) == E.HRS_EGEOMETRY
    assert gdn_call(v=MIS) == E.HRS_EALIGN
    assert gdn_call(ckpt=MIS) == E.HRS_EALIGN
    assert gdn_call(d_k=96) == E.HRS_EUNSUPPORTED
    assert gdn_call(d_v=24) == E.HRS_EUNSUPPORTED
    # a well-formed call gets past every check; with no GPU visible the launch fails
    assert gdn_call() == E.HRS_EDEVICE


def conv_call(**kw):
    d = dict(n_req=1, n_pos=4, channels=64, width=4, dtype=hrs.HRS_BF16, silu=0, topo=hrs.HRS_CHAIN, parent=None)
    ptrs = dict(x=FAKE, w=FAKE, cs=FAKE, ck=FAKE, y=FAKE)
    for key in list(kw):
        if key in ptrs:
            ptrs[key] = kw.pop(key)
    d.update(kw)
    par = d.pop("parent")
    keep = None
    if par is not None:
        keep = np.ascontiguousarray(np.asarray(par, dtype=np.int32))
        par = keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    desc = hrs.ConvDesc(d["n_req"], d["n_pos"], d["channels"], d["width"], d["dtype"], d["silu"], d["topo"], par)
    return hrs.lib.conv1d_verify_span(ctypes.byref(desc), ptrs["x"], ptrs["w"], ptrs["cs"], ptrs["ck"],
                                      ptrs["y"], None)


def test_conv_rejections():
    E = hrs
    assert conv_call(channels=12) == E.HRS_EINVAL
    assert conv_call(width=1) == E.HRS_EINVAL
    assert conv_call(x=None) == E.HRS_EINVAL
    assert conv_call(topo=E.HRS_TREE, parent=[-1, 0, 0, 1], ck=None) == E.HRS_EINVAL
    assert conv_call(topo=E.HRS_TREE, parent=[-1, 0, 4, 1]) == E.HRS_EGEOMETRY
    assert conv_call(n_pos=70) == E.HRS_EGEOMETRY
    assert conv_call(y=MIS) == E.HRS_EALIGN
    assert conv_call(width=3) == E.HRS_EUNSUPPORTED
    assert conv_call() == E.HRS_EDEVICE


def accept_call(ws_bytes=None, **kw):
    d = dict(n_req=2, n_pos=5, vocab=1024, logit_dtype=hrs.HRS_BF16, topo=hrs.HRS_CHAIN, parent=None)
    ptrs = dict(logits=FAKE, tokens=FAKE, argmax=FAKE, node=FAKE, ln=FAKE, path=FAKE, bonus=FAKE, ws=FAKE)
    for key in list(kw):
        if key in ptrs:
            ptrs[key] = kw.pop(key)
    d.update(kw)
    par = d.pop("parent")
    keep = None
    if par is not None:
        keep = np.ascontiguousarray(np.asarray(par, dtype=np.int32))
        par = keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    desc = hrs.AcceptDesc(d["n_req"], d["n_pos"], d["vocab"], d["logit_dtype"], d["topo"], par)
    need = hrs.lib.accept_greedy_workspace_bytes(ctypes.byref(desc))
    ws = need if ws_bytes is None else ws_bytes
    return hrs.lib.accept_greedy(ctypes.byref(desc), ptrs["logits"], ptrs["tokens"], ptrs["argmax"], ptrs["node"],
                                 ptrs["ln"], ptrs["path"], ptrs["bonus"], ptrs["ws"], ws, None), need


def test_accept_rejections_and_workspace_size():
    E = hrs
    st, need = accept_call()
    assert need == 2 * 5 * 1 * 8          # one 16384-entry chunk per row, 8-byte keys
    assert st == E.HRS_EDEVICE
    assert accept_call(vocab=151936)[1] == 2 * 5 * 10 * 8
    assert accept_call(vocab=1001)[0] == E.HRS_EINVAL
    assert accept_call(ws_bytes=need - 1)[0] == E.HRS_EINVAL
    assert accept_call(tokens=None)[0] == E.HRS_EINVAL
    assert accept_call(n_pos=0)[0] == E.HRS_EGEOMETRY
    assert accept_call(topo=E.HRS_TREE, parent=[-1, 0, 0, 1, 1, -1, 0, 1, 1, 5])[0] == E.HRS_EGEOMETRY
    assert accept_call(topo=E.HRS_TREE, parent=[-1, 0, 0, 1, 1, -1, 0, 1, 1, 2])[0] == E.HRS_EDEVICE
    assert accept_call(path=MIS)[0] == E.HRS_EALIGN
    assert accept_call(vocab=0)[1] == 0
    # pass-1 blocks (rows x 16384-logit chunks) are bounded by 2^24: the
    # largest vocabulary (2^31 - 8, 2^17 chunks) fits 128 rows, not 192
    vmax = (1 << 31) - 8
    d64 = hrs.AcceptDesc(2, 64, vmax, E.HRS_BF16, E.HRS_CHAIN, None)
    assert hrs.lib.accept_greedy_workspace_bytes(ctypes.byref(d64)) == 128 * (1 << 17) * 8
    assert accept_call(n_req=3, n_pos=64, vocab=vmax) == (E.HRS_EINVAL, 0)


def test_accept_noalloc_rejections():
    """The entry point without a workspace: the same checks as accept_greedy,
    and a size beyond its fixed device array rejected with HRS_EINVAL."""
    E = hrs

    def call(n_req=2, n_pos=5, vocab=1024, logits=FAKE, path=FAKE, parent=None):
        keep = None
        par = None
        if parent is not None:
            keep = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
            par = keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        topo = hrs.HRS_TREE if parent is not None else hrs.HRS_CHAIN
        d = hrs.AcceptDesc(n_req, n_pos, vocab, hrs.HRS_BF16, topo, par)
        return hrs.lib.accept_greedy_noalloc(ctypes.byref(d), logits, FAKE, FAKE, FAKE, FAKE, path, FAKE, None)
    assert hrs.lib.accept_greedy_noalloc(None, *([FAKE] * 7), None) == E.HRS_EINVAL
    assert call(vocab=1001) == E.HRS_EINVAL
    assert call(logits=None) == E.HRS_EINVAL
    assert call(path=MIS) == E.HRS_EALIGN
    assert call(n_pos=0) == E.HRS_EGEOMETRY
    assert call(parent=[-1, 0, 0, 1, 7, -1, 0, 1, 1, 2]) == E.HRS_EGEOMETRY
    # 256 x 64 rows x 10 chunks x 8 B of keys exceed the 1 MiB array; 128 x 64 rows fit
    assert call(n_req=256, n_pos=64, vocab=151936) == E.HRS_EINVAL
    assert hrs.ACCEPT_NOALLOC_MAX_BYTES == 1 << 20
    # a well-formed call gets past every check; with no GPU visible the launch fails
    assert call(n_req=128, n_pos=64, vocab=151936) == E.HRS_EDEVICE
    assert call() == E.HRS_EDEVICE


def rollback_call(**kw):
    d = dict(n_layers=2, n_req=3, n_pos=5, n_vheads=4, d_k=64, d_v=64, conv_channels=64, conv_width=4,
             conv_dtype=hrs.HRS_BF16)
    ptrs = dict(ckpt=FAKE, state=FAKE, cck=FAKE, cs=FAKE, node=FAKE, status=FAKE)
    for key in list(kw):
        if key in ptrs:
            ptrs[key] = kw.pop(key)
    d.update(kw)
    desc = hrs.RollbackDesc(*[d[k] for k in ("n_layers", "n_req", "n_pos", "n_vheads", "d_k", "d_v",
                                              "conv_channels", "conv_width", "conv_dtype")])
    return hrs.lib.rollback_restore(ctypes.byref(desc), ptrs["ckpt"], ptrs["state"], ptrs["cck"], ptrs["cs"],
                                    ptrs["node"], ptrs["status"], None)


def test_rollback_rejections():
    E = hrs
    assert rollback_call(n_layers=0) == E.HRS_EINVAL
    assert rollback_call(n_pos=65) == E.HRS_EINVAL
    assert rollback_call(status=None) == E.HRS_EINVAL
    assert rollback_call(cs=None) == E.HRS_EINVAL          # conv buffers come in pairs
    assert rollback_call(state=MIS) == E.HRS_EALIGN
    assert rollback_call(conv_channels=3, conv_dtype=hrs.HRS_BF16) == E.HRS_EINVAL  # 3 rows x 3 x 2 B not 16-B
    # one (layer, request) state of 2 GiB or more: 64 heads x 4096 x 2048 x 4 B = 2 GiB
    assert rollback_call(n_vheads=64, d_v=4096, d_k=2048) == E.HRS_EINVAL
    assert rollback_call(conv_channels=(1 << 28), conv_dtype=hrs.HRS_F32) == E.HRS_EINVAL   # 3 x 2^28 x 4 B
    assert rollback_call() == E.HRS_EDEVICE
    assert rollback_call(cck=None, cs=None, conv_channels=0) == E.HRS_EDEVICE


def ring_call(setter=True, runs=((0, 14, 5, 0),), n_rings=2, n_slots=16, width=64, dtype=None, n_packed=8,
              ring=FAKE, packed=FAKE):
    arr = (hrs.RingRun * max(1, len(runs)))(*[hrs.RingRun(*r) for r in runs])
    desc = hrs.RingDesc(n_rings, n_slots, width, hrs.HRS_BF16 if dtype is None else dtype, n_packed, len(runs), arr)
    fn = hrs.lib.ring_set_2d if setter else hrs.lib.ring_get_2d
    return fn(ctypes.byref(desc), ring, packed, None)


def test_ring_rejections():
    E = hrs
    for setter in (True, False):
        assert ring_call(setter) == E.HRS_EDEVICE
        assert ring_call(setter, runs=((2, 0, 1, 0),)) == E.HRS_EINVAL      # ring id
        assert ring_call(setter, runs=((0, 16, 1, 0),)) == E.HRS_EINVAL     # start
        assert ring_call(setter, runs=((0, 0, 17, 0),)) == E.HRS_EINVAL     # longer than the ring
        assert ring_call(setter, runs=((0, 0, 5, 4),)) == E.HRS_EINVAL      # past the packed rows
        assert ring_call(setter, width=3) == E.HRS_EINVAL                   # row not 16-byte multiple
        assert ring_call(setter, ring=MIS) == E.HRS_EALIGN
        assert ring_call(setter, runs=()) == E.HRS_OK                       # nothing to copy
        # a run longer than one grid dimension (split on the host before the launch)
        assert ring_call(setter, runs=((0, 5, 70000, 0),), n_slots=80000, n_packed=70000) == E.HRS_EDEVICE
    # set: two runs writing the same slots (wrap overlap) are rejected
    assert ring_call(True, runs=((0, 14, 3, 0), (0, 0, 2, 3))) == E.HRS_EINVAL
    assert ring_call(True, runs=((0, 14, 3, 0), (1, 0, 2, 3))) == E.HRS_EDEVICE
    # get: two runs writing the same packed rows are rejected, same slots are fine
    assert ring_call(False, runs=((0, 14, 3, 0), (1, 0, 2, 2))) == E.HRS_EINVAL
    assert ring_call(False, runs=((0, 14, 3, 0), (0, 14, 3, 3))) == E.HRS_EDEVICE


def test_zero_copy_entry_rejections():
    E = hrs
    desc = hrs.GdnDesc(2, 4, 2, 4, 128, 128, hrs.HRS_BF16, 1.0, hrs.HRS_CHAIN, None)
    ck_bytes = 2 * 4 * 4 * 128 * 128 * 4

    def call(src_ckpt=FAKE + (1 << 32), node=FAKE, n_pos=4, ckpt=FAKE, status=None, src=True):
        s = hrs.SpanSource(src_ckpt, node, n_pos)
        return hrs.lib.gdn_verify_span_from(ctypes.byref(desc), ctypes.byref(s) if src else None, FAKE, FAKE, FAKE,
                                            FAKE, FAKE, ckpt, FAKE, status, None)
    assert call(src=False) == E.HRS_EINVAL
    assert call(src_ckpt=None) == E.HRS_EINVAL
    assert call(node=None) == E.HRS_EINVAL
    assert call(ckpt=None) == E.HRS_EINVAL                  # capture required
    assert call(n_pos=0) == E.HRS_EINVAL
    assert call(n_pos=65) == E.HRS_EINVAL
    assert call(src_ckpt=FAKE + ck_bytes // 2) == E.HRS_EINVAL   # new checkpoints overlap the source
    assert call(src_ckpt=FAKE + ck_bytes) == E.HRS_EDEVICE   # adjacent, no overlap
    assert call(node=MIS) == E.HRS_EALIGN
    assert call(status=MIS) == E.HRS_EALIGN
    assert call() == E.HRS_EDEVICE


def test_conv_nocapture_and_advance_rejections():
    E = hrs
    d = hrs.ConvDesc(1, 4, 64, 4, hrs.HRS_BF16, 0, hrs.HRS_TREE, None)
    assert hrs.lib.conv1d_verify_span_nocapture(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None) == E.HRS_EGEOMETRY
    par = np.array([-1, 0, 0, 1], dtype=np.int32)
    d = hrs.ConvDesc(1, 4, 64, 4, hrs.HRS_BF16, 0, hrs.HRS_TREE, par.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    assert hrs.lib.conv1d_verify_span_nocapture(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None) == E.HRS_EDEVICE
    assert hrs.lib.conv1d_verify_span_nocapture(ctypes.byref(d), FAKE, FAKE, None, FAKE, None) == E.HRS_EINVAL

    def adv(L=2, R=3, T=5, C=64, W=4, dt=hrs.HRS_BF16, x=FAKE, cs=FAKE, path=FAKE, ln=FAKE, st=None):
        a = hrs.ConvAdvanceDesc(L, R, T, C, W, dt)
        return hrs.lib.conv_state_advance(ctypes.byref(a), x, cs, path, ln, st, None)
    assert adv(L=0) == E.HRS_EINVAL
    assert adv(T=65) == E.HRS_EINVAL
    assert adv(C=12) == E.HRS_EINVAL
    assert adv(path=None) == E.HRS_EINVAL
    assert adv(cs=MIS) == E.HRS_EALIGN
    assert adv(W=3) == E.HRS_EUNSUPPORTED
    assert adv() == E.HRS_EDEVICE


def test_layer_entry_rejections():
    E = hrs

    def call(width=4, silu=1, eps=1e-6, x=FAKE, w=FAKE, cs=FAKE, a=FAKE, state=FAKE, src=None, ckpt=FAKE,
             d_k=128, n_vheads=4, topo=hrs.HRS_CHAIN, parent=None, desc=True):
        keep = None
        par = None
        if parent is not None:
            keep = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
            par = keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        g = hrs.GdnDesc(2, 4, 2, n_vheads, d_k, 128, hrs.HRS_BF16, 1.0, topo, par)
        d = hrs.GdnLayerDesc(g, width, silu, eps)
        return hrs.lib.gdn_layer_verify_span(ctypes.byref(d) if desc else None, x, w, cs, a, FAKE, state,
                                             ctypes.byref(src) if src is not None else None, ckpt, FAKE, None,
                                             None)
    assert call(desc=False) == E.HRS_EINVAL
    assert call(width=3) == E.HRS_EUNSUPPORTED
    assert call(state=None) == E.HRS_EINVAL                 # no initial state
    both = hrs.SpanSource(FAKE + (1 << 32), FAKE, 4)
    assert call(src=both) == E.HRS_EINVAL                    # two initial states
    assert call(state=None, src=both) == E.HRS_EDEVICE
    assert call(ckpt=None) == E.HRS_EINVAL                   # capture required
    assert call(x=None) == E.HRS_EINVAL
    assert call(w=None) == E.HRS_EINVAL
    assert call(cs=None) == E.HRS_EINVAL
    assert call(eps=-1.0) == E.HRS_EINVAL
    assert call(eps=float("nan")) == E.HRS_EINVAL
    assert call(n_vheads=3) == E.HRS_EINVAL
    assert call(x=MIS) == E.HRS_EALIGN
    assert call(cs=MIS) == E.HRS_EALIGN
    assert call(a=MIS) == E.HRS_EALIGN
    assert call(d_k=96) == E.HRS_EUNSUPPORTED
    assert call(topo=hrs.HRS_TREE, parent=[-1, 0, 0, 5, -1, 0, 1, 1]) == E.HRS_EGEOMETRY
    assert call(topo=hrs.HRS_TREE, parent=[-1, 0, 0, 1, -1, 0, 1, 1]) == E.HRS_EDEVICE
    assert call() == E.HRS_EDEVICE


def test_chunked_entry_rejections():
    E = hrs

    def call(n_req=1, n_pos=200, Hk=2, Hv=4, dk=128, dv=128, dt=hrs.HRS_BF16, topo=hrs.HRS_CHAIN, q=FAKE, state=FAKE,
             ckpt=None, out=FAKE, desc=True, out_dt=hrs.HRS_F32, log_gates=0, ws=FAKE, ws_bytes=None):
        g = hrs.GdnDesc(n_req, n_pos, Hk, Hv, dk, dv, dt, 1.0, topo, None)
        d = hrs.ChunkedDesc(g, log_gates, out_dt)
        if ws_bytes is None:
            ws_bytes = hrs.lib.gdn_span_chunked_workspace_bytes(ctypes.byref(d))
        return hrs.lib.gdn_span_chunked(ctypes.byref(d) if desc else None, q, FAKE, FAKE, FAKE, FAKE, state, ckpt,
                                        out, ws, ws_bytes, None)
    assert call(desc=False) == E.HRS_EINVAL
    assert call(n_req=0) == E.HRS_EINVAL
    assert call(Hv=3) == E.HRS_EINVAL
    assert call(dt=9) == E.HRS_EINVAL
    assert call(out_dt=5) == E.HRS_EINVAL
    assert call(n_pos=0) == E.HRS_EINVAL
    assert call(n_pos=(1 << 20) + 1) == E.HRS_EINVAL
    assert call(q=None) == E.HRS_EINVAL
    assert call(state=None) == E.HRS_EINVAL
    assert call(out=None) == E.HRS_EINVAL
    assert call(topo=hrs.HRS_TREE) == E.HRS_EUNSUPPORTED
    assert call(topo=7) == E.HRS_EINVAL
    assert call(q=MIS) == E.HRS_EALIGN
    assert call(ckpt=MIS) == E.HRS_EALIGN
    assert call(out=MIS) == E.HRS_EALIGN
    assert call(dk=64, dv=64) == E.HRS_EUNSUPPORTED
    assert call(ws=None) == E.HRS_EINVAL
    assert call(ws_bytes=0) == E.HRS_EINVAL
    assert call(ws_bytes=1 * 4 * 4 * 20992 - 1) == E.HRS_EINVAL
    assert call(ws=MIS) == E.HRS_EALIGN
    assert call(ws_bytes=1 * 4 * 4 * 20992) == E.HRS_EDEVICE
    assert call(n_pos=(1 << 20)) == E.HRS_EDEVICE
    assert call(ckpt=FAKE, out_dt=hrs.HRS_BF16, log_gates=1) == E.HRS_EDEVICE
    assert call() == E.HRS_EDEVICE


def test_binding_rejects_mismatched_tensors_before_launch():
    """The binding checks every tensor against the sizes the library takes from
    the leading one (and dtype, layout and device) before anything launches,
    so a wrong tensor raises instead of being read or written out of bounds."""
    import torch
    R, T, Hk, Hv, d = 2, 3, 1, 2, 64
    f, h = torch.float32, torch.bfloat16
    def span(**over):
        t = dict(q=torch.zeros(R, T, Hk, d, dtype=h), k=torch.zeros(R, T, Hk, d, dtype=h),
                 v=torch.zeros(R, T, Hv, d, dtype=h), a=torch.zeros(R, T, Hv, dtype=h), b=torch.zeros(R, T, Hv, dtype=h),
                 state=torch.zeros(R, Hv, d, d, dtype=f), ckpt=torch.zeros(R, T, Hv, d, d, dtype=f),
                 out=torch.zeros(R, T, Hv, d, dtype=f))
        t.update(over)
        hrs.gdn_verify_span(t["q"], t["k"], t["v"], t["a"], t["b"], t["state"], t["ckpt"], t["out"])
    with pytest.raises(ValueError, match="v: shape"):
        span(v=torch.zeros(R, T + 1, Hv, d, dtype=h))
    with pytest.raises(ValueError, match="out: shape"):
        span(out=torch.zeros(R, T, Hv, d - 1, dtype=f))
    with pytest.raises(TypeError, match="a: dtype"):
        span(a=torch.zeros(R, T, Hv, dtype=f))
    with pytest.raises(TypeError, match="state: dtype"):
        span(state=torch.zeros(R, Hv, d, d, dtype=h))
    with pytest.raises(ValueError, match="contiguous"):
        span(b=torch.zeros(R, Hv, T, dtype=h).transpose(1, 2))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        span()                                   # right shapes, host memory
    with pytest.raises(ValueError, match="state is required"):
        span(state=None)
    x = torch.zeros(R, T, 64, dtype=h)
    with pytest.raises(ValueError, match="conv_state: shape"):
        hrs.conv1d_verify_span(x, torch.zeros(64, 4, dtype=h), torch.zeros(R, 4, 64, dtype=h), None,
                               torch.zeros(R, T, 64, dtype=f))
    with pytest.raises(ValueError, match="tokens: shape"):
        hrs.accept_greedy(torch.zeros(R, T, 64, dtype=h), torch.zeros(R, T + 1, dtype=torch.int32),
                          *[torch.zeros(R, T, dtype=torch.int32)] + [torch.zeros(R, dtype=torch.int32)] * 2 +
                          [torch.zeros(R, T, dtype=torch.int32), torch.zeros(R, dtype=torch.int32),
                           torch.zeros(64, dtype=torch.int64)])
    with pytest.raises(ValueError, match="go together"):
        hrs.rollback_restore(torch.zeros(1, R, T, Hv, d, d), torch.zeros(1, R, Hv, d, d), None,
                             torch.zeros(1, R, 3, 64, dtype=h), torch.zeros(R, dtype=torch.int32),
                             torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="packed: shape"):
        hrs.ring_set_2d(torch.zeros(2, 8, 16, dtype=h), torch.zeros(3, 8, dtype=h), [(0, 0, 3, 0)])


def test_binding_rejects_parent_arrays_of_the_wrong_size():
    """The library reads n_req * n_pos parent entries: the binding accepts one
    row per request or one row repeated for all, and rejects every other size
    (a short list would be over-read on the host, a long one truncated)."""
    import torch
    R, T, Hk, Hv, d = 2, 4, 1, 2, 64
    f, h = torch.float32, torch.bfloat16
    z = lambda *s, dt=h: torch.zeros(*s, dtype=dt)
    span_in = (z(R, T, Hk, d), z(R, T, Hk, d), z(R, T, Hv, d), z(R, T, Hv), z(R, T, Hv), z(R, Hv, d, d, dt=f),
               z(R, T, Hv, d, d, dt=f), z(R, T, Hv, d, dt=f))
    good_row = [-1, 0, 0, 1]
    for bad in (good_row[:3], good_row + [2], good_row * R + [0], (good_row * R)[:-1]):
        with pytest.raises(ValueError, match="parent: "):
            hrs.gdn_verify_span(*span_in, parent=bad)
        with pytest.raises(ValueError, match="parent: "):
            hrs.accept_greedy_workspace_bytes(R, T, 1024, parent=bad)
        with pytest.raises(ValueError, match="parent: "):
            hrs.conv1d_verify_span(z(R, T, 64), z(64, 4), z(R, 3, 64), None, z(R, T, 64, dt=f), parent=bad)
    # the right sizes get past the parent check (and stop at the host tensors)
    for ok in (good_row, good_row * R, np.array([good_row] * R)):
        with pytest.raises(ValueError, match="must be a GPU tensor"):
            hrs.gdn_verify_span(*span_in, parent=ok)
        assert hrs.accept_greedy_workspace_bytes(R, T, 1024, parent=ok) == R * T * 8
