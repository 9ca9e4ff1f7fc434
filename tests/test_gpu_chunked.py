"""GPU parity of the chunked long-span entry point (gdn_span_chunked) against
the GDN oracle (the plain recurrence), through the C ABI: final states,
outputs and, with capture, every checkpoint within max relative error 1e-4
per tile; spans that end inside a chunk, exactly on a chunk boundary and
within the first chunk; spans over more than one 32-chunk segment (the
workspace reused); bf16 (matrix-core k k^T) and f32 inputs; zero decays;
agreement with gdn_verify_span on short spans; workspace contents ignored."""
import numpy as np
import pytest

from oracle import gdn as ogdn
from synth import BF16, F32, QWEN_LAYER_CHAIN, bf16_bits, gen_unit, scaled
from tests.gpu_util import assert_tiles, say, to_numpy, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hrs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import hybrid_recurrent_state_amd as m
    return m


def workspace(hrs, q, v, fill=None):
    """A workspace of exactly the size the library asks for, filled with a
    byte pattern (the kernels must not depend on its contents)."""
    import torch
    R, T, Hk = q.shape[:3]
    n = hrs.gdn_span_chunked_workspace_bytes(R, T, Hk, v.shape[2])
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5 if fill is None else fill)
    return ws


def run(hrs, units, capture, q_scale=1.0):
    import torch
    st = lambda name: to_torch(np.stack([getattr(u, name) for u in units]))
    q, k, v, a, b, state = st("q"), st("k"), st("v"), st("a"), st("b"), st("state")
    R, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    ckpt = torch.full((R, T, Hv, dv, dk), float("nan"), device="cuda") if capture else None
    out = torch.full((R, T, Hv, dv), float("nan"), device="cuda")
    hrs.gdn_span_chunked(q, k, v, a, b, state, ckpt, out, workspace(hrs, q, v), q_scale=q_scale)
    torch.cuda.synchronize()
    return (to_numpy(ckpt) if capture else None), to_numpy(out), to_numpy(state)


def check(units, ck, out, state, capture, q_scale=1.0, what=""):
    for r, u in enumerate(units):
        ock, oout = ogdn.gdn_span(u.state, u.q, u.k, u.v, u.a, u.b, None, q_scale)
        e2 = assert_tiles(out[r], oout, 1, f"{what} out r={r}")
        if capture:
            e1 = assert_tiles(ck[r], ock, 2, f"{what} ckpt r={r}")
            assert np.array_equal(state[r], u.state), "state must be read only with capture"
        else:
            e1 = assert_tiles(state[r], ock[-1], 2, f"{what} final state r={r}")
        say(f"{what} r={r}: state err {e1:.2e}, out err {e2:.2e}")


@pytest.mark.parametrize("T,capture", [(150, False), (150, True), (64, False), (1, True), (65, True)])
def test_chunked_qwen_bf16(hrs, T, capture):
    w = scaled(QWEN_LAYER_CHAIN, n_req=2, n_pos=T, n_kheads=4, n_vheads=8)
    units = [gen_unit(w, 0, r) for r in range(w.n_req)]
    say(f"chunked bf16 R=2 T={T} capture={capture}")
    ck, out, state = run(hrs, units, capture, q_scale=0.5)
    check(units, ck, out, state, capture, q_scale=0.5, what=f"bf16 T={T}")


def test_chunked_f32_grouped(hrs):
    w = scaled(QWEN_LAYER_CHAIN, n_req=1, n_pos=130, n_kheads=2, n_vheads=8, dtype=F32)
    units = [gen_unit(w, 0, 0)]
    ck, out, state = run(hrs, units, True)
    check(units, ck, out, state, True, what="f32 grouped")


def test_chunked_long_span(hrs):
    w = scaled(QWEN_LAYER_CHAIN, n_req=1, n_pos=1000, n_kheads=1, n_vheads=2)
    units = [gen_unit(w, 0, 0)]
    ck, out, state = run(hrs, units, False)
    check(units, ck, out, state, False, what="T=1000")


@pytest.mark.parametrize("T,capture,Hv,dt", [(2048, False, 8, BF16), (2100, False, 2, BF16), (2113, True, 1, BF16),
                                             (2070, False, 2, F32)])
def test_chunked_spans_over_several_segments(hrs, T, capture, Hv, dt):
    """More than 32 chunks: the pre-pass records of the second segment
    overwrite the first's in the workspace, and the second segment starts
    from the state the first left (in place, or the checkpoint before it);
    bf16 inputs (bf16 products against the split state) and f32 inputs."""
    w = scaled(QWEN_LAYER_CHAIN, n_req=2 if capture else 1, n_pos=T, n_kheads=1, n_vheads=Hv, dtype=dt)
    units = [gen_unit(w, 0, r) for r in range(w.n_req)]
    say(f"chunked segments T={T} capture={capture}")
    ck, out, state = run(hrs, units, capture)
    check(units, ck, out, state, capture, what=f"T={T}")


def test_chunked_zero_and_unit_decays(hrs):
    w = scaled(QWEN_LAYER_CHAIN, n_req=1, n_pos=100, n_kheads=2, n_vheads=4)
    u = gen_unit(w, 0, 0)
    a = u.a.copy()
    a[[3, 40, 64, 65, 99], :] = bf16_bits(np.zeros((5, 4), np.float32))        # decay to zero
    a[[10, 11, 12], :] = bf16_bits(np.ones((3, 4), np.float32))                # no decay
    u.a = a
    ck, out, state = run(hrs, [u], True)
    assert np.isfinite(ck).all() and np.isfinite(out).all()
    check([u], ck, out, state, True, what="zero decays")


def test_chunked_matches_recurrent_kernel_on_short_spans(hrs):
    import torch
    w = scaled(QWEN_LAYER_CHAIN, n_req=3, n_pos=17)
    units = [gen_unit(w, 0, r) for r in range(3)]
    st = lambda name: to_torch(np.stack([getattr(u, name) for u in units]))
    q, k, v, a, b, state = st("q"), st("k"), st("v"), st("a"), st("b"), st("state")
    R, T, Hv, d = 3, 17, 32, 128
    ck1 = torch.empty((R, T, Hv, d, d), device="cuda"); out1 = torch.empty((R, T, Hv, d), device="cuda")
    ck2 = torch.empty_like(ck1); out2 = torch.empty_like(out1)
    ws = workspace(hrs, q, v)
    hrs.gdn_span_chunked(q, k, v, a, b, state, ck1, out1, ws)
    hrs.gdn_verify_span(q, k, v, a, b, state, ck2, out2)
    torch.cuda.synchronize()
    c1, c2, o1, o2 = to_numpy(ck1), to_numpy(ck2), to_numpy(out1), to_numpy(out2)
    for r in range(R):
        assert_tiles(c1[r], c2[r], 2, f"chunked vs recurrent ckpt r={r}")
        assert_tiles(o1[r], o2[r], 1, f"chunked vs recurrent out r={r}")
    # the in-place form (chunk-end state in matrix form) ends where the
    # capture form's last checkpoint is, to f32 rounding; one chunk, so the
    # outputs are the same computation
    st2 = state.clone()
    out3 = torch.empty_like(out1)
    ws.fill_(0x5A)
    hrs.gdn_span_chunked(q, k, v, a, b, st2, None, out3, ws)
    torch.cuda.synchronize()
    s2, last = to_numpy(st2), to_numpy(ck1[:, -1])
    for r in range(R):
        assert_tiles(s2[r], last[r], 2, f"in-place vs captured final state r={r}")
    assert torch.equal(out3, out1)


def test_chunked_log_gates(hrs):
    """Log-space gates: `a` holds g = log a (bf16); the oracle runs the
    recurrence on a = exp(g) computed in float64 from the same bf16 values."""
    import torch
    from synth import bf16_to_f32
    w = scaled(QWEN_LAYER_CHAIN, n_req=2, n_pos=90, n_kheads=4, n_vheads=8)
    units = [gen_unit(w, 0, r) for r in range(w.n_req)]
    for u in units:
        g = np.log(bf16_to_f32(u.a).astype(np.float64))
        u.a = bf16_bits(g.astype(np.float32))          # the kernel's input: bf16 log decays
    st = lambda name: to_torch(np.stack([getattr(u, name) for u in units]))
    q, k, v, g, b, state = st("q"), st("k"), st("v"), st("a"), st("b"), st("state")
    R, T, Hv, d = 2, 90, 8, 128
    ckpt = torch.full((R, T, Hv, d, d), float("nan"), device="cuda")
    out = torch.full((R, T, Hv, d), float("nan"), device="cuda")
    hrs.gdn_span_chunked(q, k, v, g, b, state, ckpt, out, workspace(hrs, q, v), log_gates=True)
    torch.cuda.synchronize()
    ck, o = to_numpy(ckpt), to_numpy(out)
    for r, u in enumerate(units):
        a64 = np.exp(bf16_to_f32(u.a).astype(np.float64))
        ock, oout = ogdn.gdn_span(u.state, u.q, u.k, u.v, a64, u.b, None, 1.0)
        e1 = assert_tiles(ck[r], ock, 2, f"log gates ckpt r={r}")
        e2 = assert_tiles(o[r], oout, 1, f"log gates out r={r}")
        say(f"log gates r={r}: ckpt err {e1:.2e}, out err {e2:.2e}")


def test_chunked_log_gates_over_two_segments_with_capture(hrs):
    """Log-space gates with every state captured over 2,100 positions (two
    segments): the second segment starts from the checkpoint before it."""
    import torch
    from synth import bf16_to_f32
    w = scaled(QWEN_LAYER_CHAIN, n_req=1, n_pos=2100, n_kheads=1, n_vheads=1)
    u = gen_unit(w, 0, 0)
    g = np.log(bf16_to_f32(u.a).astype(np.float64))
    u.a = bf16_bits(g.astype(np.float32))
    st = lambda name: to_torch(np.stack([getattr(u, name)]))
    q, k, v, gl, b, state = st("q"), st("k"), st("v"), st("a"), st("b"), st("state")
    ckpt = torch.full((1, 2100, 1, 128, 128), float("nan"), device="cuda")
    out = torch.full((1, 2100, 1, 128), float("nan"), device="cuda")
    hrs.gdn_span_chunked(q, k, v, gl, b, state, ckpt, out, workspace(hrs, q, v), log_gates=True)
    torch.cuda.synchronize()
    a64 = np.exp(bf16_to_f32(u.a).astype(np.float64))
    ock, oout = ogdn.gdn_span(u.state, u.q, u.k, u.v, a64, u.b, None, 1.0)
    e1 = assert_tiles(to_numpy(ckpt)[0], ock, 2, "log gates, two segments, ckpt")
    e2 = assert_tiles(to_numpy(out)[0], oout, 1, "log gates, two segments, out")
    say(f"log gates two segments: ckpt err {e1:.2e}, out err {e2:.2e}")


def test_chunked_bf16_outputs(hrs):
    """bf16 outputs are the f32 outputs of the same computation rounded to the
    nearest bf16 (ties to even), bit for bit; against the oracle, within one
    bf16 rounding (2^-8 of the tile maximum)."""
    import torch
    w = scaled(QWEN_LAYER_CHAIN, n_req=2, n_pos=100, n_kheads=4, n_vheads=8)
    units = [gen_unit(w, 0, r) for r in range(w.n_req)]
    st = lambda name: to_torch(np.stack([getattr(u, name) for u in units]))
    q, k, v, a, b = st("q"), st("k"), st("v"), st("a"), st("b")
    R, T, Hv, d = 2, 100, 8, 128
    out32 = torch.empty((R, T, Hv, d), device="cuda")
    out16 = torch.empty((R, T, Hv, d), device="cuda", dtype=torch.bfloat16)
    s1, s2 = st("state"), st("state")
    hrs.gdn_span_chunked(q, k, v, a, b, s1, None, out32, workspace(hrs, q, v), q_scale=0.5)
    hrs.gdn_span_chunked(q, k, v, a, b, s2, None, out16, workspace(hrs, q, v, fill=0xFF), q_scale=0.5)
    torch.cuda.synchronize()
    o32 = to_numpy(out32)
    o16 = to_numpy(out16)
    o16 = o16 if o16.dtype == np.uint16 else bf16_bits(o16)
    assert np.array_equal(o16, bf16_bits(o32))
    assert torch.equal(s1, s2)
    from synth import bf16_to_f32
    for r, u in enumerate(units):
        _, oout = ogdn.gdn_span(u.state, u.q, u.k, u.v, u.a, u.b, None, 0.5)
        assert_tiles(bf16_to_f32(o16[r]), oout, 1, f"bf16 out r={r}", tol=2.0 ** -8)


def test_chunked_random_shapes(hrs):
    """Seeded sweep: 1-4 requests, 1-300 positions (several chunks, ragged
    last chunk), 1-4 value heads per key head, capture on or off, bf16 or f32
    inputs, power-of-two q scales; each against the GDN oracle."""
    rng = np.random.default_rng(777)
    for i in range(8):
        Hk = int(rng.choice([1, 2]))
        Hv = Hk * int(rng.choice([1, 2, 4]))
        R = int(rng.integers(1, 5))
        T = int(rng.integers(1, 301))
        dt = F32 if rng.random() < 0.3 else BF16
        capture = bool(rng.random() < 0.5)
        q_scale = float(2.0 ** -int(rng.integers(0, 4)))
        w = scaled(QWEN_LAYER_CHAIN, n_req=R, n_pos=T, n_kheads=Hk, n_vheads=Hv, dtype=dt, conv_channels=16,
                   seed=500 + i)
        units = [gen_unit(w, 0, r) for r in range(R)]
        what = f"chunked shape {i}: R={R} T={T} Hk={Hk} Hv={Hv} {dt} capture={capture}"
        say(what)
        ck, out, state = run(hrs, units, capture, q_scale=q_scale)
        check(units, ck, out, state, capture, q_scale=q_scale, what=what)
