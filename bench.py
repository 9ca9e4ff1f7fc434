#!/usr/bin/env python3
"""Benchmark of the GDN verify step on one MI355X.

A step is one pass of the whole hot path over one batch: for each of the 48
layers a conv1d span and a GDN verify span with checkpoints, then greedy
acceptance, rollback of every layer to the accepted checkpoint, the
feature-ring set/get, and the step's single host sync (accepted lengths and
bonus tokens back to the host). Inputs are seeded synthetic data already
resident in HBM when the timed region starts.

Prints ONE JSON line on stdout. Progress goes to stderr.

  python bench.py [--steps K] [--warmup W] [--workload NAME|INDEX] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = 3   # 16 requests x 48 layers, chain K=16, with the feature ring


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=str(DEFAULT_WORKLOAD))
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true", help="skip the measured NEXT-row variants")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other configured workloads (measured after the headline)")
    ap.add_argument("--workload-cpu-seconds", type=float, default=4.0,
                    help="budget of the oracle CPU baseline of each other workload")
    ap.add_argument("--graph", action="store_true",
                    help="launch each step as one captured HIP graph (the same kernels)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before warmup, run a plain device copy of this many MiB three times "
                         "(reference kernel for scaling the FETCH_SIZE/WRITE_SIZE counters)")
    return ap.parse_args()


KERNEL_SOURCES = ["hybrid_recurrent_state_amd/csrc/gdn.hip", "hybrid_recurrent_state_amd/csrc/device.h",
                  "hybrid_recurrent_state_amd/csrc/internal.h"]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str = "gdn_verify_span"):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter passes (profiles/hbm_traffic.json), or None when none were taken
    there or the kernel sources have changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    for rec in data.get("records", []):
        if (rec.get("workload") == workload and rec.get("entry_point") == kernel
                and rec.get("kernel_source_sha256") == kernel_source_hash()):
            return rec.get("traffic_bytes_per_launch")
    return None


def _oracle_units(w, units, seconds: float):
    """Run whole (layer, request) units of the oracle until `seconds` of work
    are spent; returns (units done, verify tokens, seconds of work)."""
    from threadpoolctl import threadpool_limits
    from oracle import accept as oacc, conv as oconv, gdn as ogdn, rollback as orb
    from synth import gen_accept, gen_conv_weight, gen_unit
    done = 0
    t_work = 0.0
    with threadpool_limits(limits=1):
        for (l, r) in units:
            u = gen_unit(w, l, r)
            wt = gen_conv_weight(w, l)
            ai = gen_accept(w, r, with_logits=w.vocab > 0)
            t0 = time.perf_counter()
            par = ai.parent if w.tree else None
            oconv.conv_span(u.x, wt, u.conv_state, par)
            ogdn.gdn_span(u.state, u.q, u.k, u.v, u.a, u.b, par)
            if w.vocab and l == 0:
                am = oacc.argmax_rows(ai.logits)
                res = oacc.accept(am, ai.tokens, par)
            else:
                res = oacc.accept(ai.planted_argmax, ai.tokens, par)
            orb.replay_state(u.state, u.q, u.k, u.v, u.a, u.b, res.path)
            orb.replay_conv_state(u.conv_state, u.x, res.path)
            t_work += time.perf_counter() - t0
            done += 1
            if t_work >= seconds:
                break
    return done, done * w.n_pos, t_work


def _pool_worker(args):
    name, units, seconds = args
    sys.path.insert(0, ROOT)
    from synth import WORKLOADS
    return _oracle_units(WORKLOADS[name], units, seconds)


def cpu_baseline(w, seconds: float):
    """The oracle, as it stands, on a bounded sample of the same workload:
    whole (layer, request) units (conv span, GDN span, acceptance of the
    request, replay rollback along the accepted path). First single-threaded;
    then a pool of worker processes over disjoint units, one per available
    core (at most 16), each for about seconds / workers."""
    units = [(l, r) for r in range(w.n_req) for l in range(w.n_layers)]
    done, tokens, t_work = _oracle_units(w, units, seconds)
    avail = len(os.sched_getaffinity(0))
    out = {"value": tokens / t_work, "unit": "verify tokens/s per layer", "cores": 1, "kind": "oracle",
           "available_cores": avail, "os_cpu_count": os.cpu_count(),
           "sample": f"{done} (layer, request) units of {w.name}: conv span, GDN span, acceptance "
                     f"(argmax once per request), replay rollback; {t_work:.1f} s of CPU work, 1 thread"}
    try:
        import multiprocessing as mp
        n = max(1, min(16, avail, len(units)))
        per = max(1.0, seconds / n)
        chunks = [(w.name, units[i::n], per) for i in range(n)]
        with mp.get_context("spawn").Pool(n) as pool:
            res = pool.map(_pool_worker, chunks)
        rate = sum(tok / t for (_, tok, t) in res if t > 0)
        out["pool"] = {"value": rate, "cores": n, "available_cores": avail,
                       "sample": f"{sum(d for d, _, _ in res)} units over {n} worker processes "
                                 f"({avail} cores available to this process, at most 16 workers), "
                                 f"~{per:.1f} s of work each; rate = sum of per-worker rates"}
    except Exception as e:  # noqa: BLE001 - the pooled figure is optional context
        out["pool"] = {"error": str(e)}
    return out


def chunked_prefill_row(reps: int = 10, T: int = 1024, R: int = 1):
    """f4: one long chain span without capture (prefill length T) on the Qwen
    GDN layer shape, by gdn_span_chunked (a pre-pass over all chunks, then
    the sequential pass; 64-position chunks, matrix cores) and by the recurrent kernel (gdn_verify_span
    without capture, T / 64 launches of 64 positions carrying the state in
    place). Inputs: seeded bf16 q, k (unit norm), v, gates as in synth."""
    import torch
    import hybrid_recurrent_state_amd as hrs
    Hk, Hv, d = 16, 32, 128
    g = torch.Generator(device="cuda").manual_seed(7)
    rn = lambda *shape: torch.randn(*shape, device="cuda", generator=g)
    q = torch.nn.functional.normalize(rn(R, T, Hk, d), dim=-1).to(torch.bfloat16)
    k = torch.nn.functional.normalize(rn(R, T, Hk, d), dim=-1).to(torch.bfloat16)
    v = rn(R, T, Hv, d).to(torch.bfloat16)
    a = torch.sigmoid(-rn(R, T, Hv)).to(torch.bfloat16)
    b = torch.sigmoid(rn(R, T, Hv)).to(torch.bfloat16)
    state0 = rn(R, Hv, d, d) * 0.02
    out = torch.empty(R, T, Hv, d, device="cuda")
    st = state0.clone()
    ws = torch.empty(hrs.gdn_span_chunked_workspace_bytes(R, T, Hk, Hv), dtype=torch.uint8, device="cuda")

    def chunked():
        hrs.gdn_span_chunked(q, k, v, a, b, st, None, out, ws)

    def recurrent():
        for t0 in range(0, T, 64):
            sl = slice(t0, min(T, t0 + 64))
            hrs.gdn_verify_span(q[:, sl], k[:, sl], v[:, sl], a[:, sl], b[:, sl], st, None, out[:, sl])

    if R != 1:
        raise ValueError("the recurrent baseline slices positions of one request")
    res = {}
    # Also one 64-position chunk at 16 requests (both forms a single launch):
    # there the recurrent kernel has parallelism enough and the chunked form
    # pays for its extra matrix work.
    R16, T16 = 16, 64
    q16 = torch.nn.functional.normalize(rn(R16, T16, Hk, d), dim=-1).to(torch.bfloat16)
    k16 = torch.nn.functional.normalize(rn(R16, T16, Hk, d), dim=-1).to(torch.bfloat16)
    v16 = rn(R16, T16, Hv, d).to(torch.bfloat16)
    a16 = torch.sigmoid(-rn(R16, T16, Hv)).to(torch.bfloat16)
    b16 = torch.sigmoid(rn(R16, T16, Hv)).to(torch.bfloat16)
    st16 = rn(R16, Hv, d, d) * 0.02
    out16 = torch.empty(R16, T16, Hv, d, device="cuda")
    ws16 = torch.empty(hrs.gdn_span_chunked_workspace_bytes(R16, T16, Hk, Hv), dtype=torch.uint8, device="cuda")
    for name, fn in (("chunked_r16", lambda: hrs.gdn_span_chunked(q16, k16, v16, a16, b16, st16, None, out16, ws16)),
                     ("recurrent_r16", lambda: hrs.gdn_verify_span(q16, k16, v16, a16, b16, st16, None, out16))):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / reps
    del q16, k16, v16, a16, b16, st16, out16, ws16
    for name, fn in (("chunked", chunked), ("recurrent", recurrent)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / reps
    # both forms from the same state agree (sanity, f32 rounding)
    st.copy_(state0); chunked(); s1 = st.clone(); o1 = out.clone()
    st.copy_(state0); recurrent(); s2 = st.clone()
    rel = float((s1 - s2).abs().max() / s2.abs().max())
    return {"n_req": R, "n_pos": T, "chunked_ms": res["chunked"], "recurrent_ms": res["recurrent"],
            "speedup": res["recurrent"] / res["chunked"], "state_rel_diff": rel,
            "tokens_per_s_per_layer": R * T / (res["chunked"] / 1e3),
            "one_chunk_16_requests": {"n_req": R16, "n_pos": T16, "chunked_ms": res["chunked_r16"],
                                      "recurrent_ms": res["recurrent_r16"],
                                      "speedup": res["recurrent_r16"] / res["chunked_r16"]}}


def row_rates(step, shape, h, L: int, reps: int = 15):
    """Achieved HBM rate of the step's other rows, each timed alone after the
    timed regions: the L conv spans back to back (per layer), acceptance,
    rollback of every layer, ring set + get. Event pairs around each piece,
    median of `reps`; bytes are the algorithmic bytes of the piece."""
    import torch

    def timed(fn, per: int) -> float:
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / per)
        return float(np.median(out)) / 1e3

    def entry(sec: float, nbytes: int, unit: str) -> dict:
        gbs = nbytes / sec / 1e9
        return {"unit_of_work": unit, "us": sec * 1e6, "bytes": nbytes, "achieved_gbs": gbs,
                "frac": gbs / HBM_PEAK_GBS}

    rows = {"conv1d_verify_span": entry(timed(lambda: [step.launch_conv(l, h) for l in range(L)], L),
                                        shape.conv_bytes_per_layer, "one layer (launches back to back)")}
    if shape.vocab:
        rows["accept_greedy"] = entry(timed(lambda: step.launch_accept(h), 1), shape.accept_bytes, "one call")
    rows["rollback_restore"] = entry(timed(lambda: step.launch_rollback(h), 1), shape.rollback_bytes,
                                     "one call (every layer)")
    if shape.ring_slots:
        rows["ring_set_2d+ring_get_2d"] = entry(timed(lambda: step.launch_ring(h), 1), shape.ring_bytes,
                                                "one set and one get")
    return rows


def store_stream_gbs(mib: int = 2048, reps: int = 10) -> float:
    """Reference ceiling: a plain device store stream (torch's fill of one
    buffer), timed with events over `reps` fills."""
    import torch
    buf = torch.empty(mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    buf.fill_(1.0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        buf.fill_(float(i))
    e1.record()
    torch.cuda.synchronize()
    gbs = reps * buf.numel() * 4 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return gbs


def time_steps(step, stream, K: int, warmup: int, graph: bool = False) -> float:
    """ms per step of K consecutive steps (launch + the single host sync),
    after `warmup` untimed ones; graph=True replays captured graphs (the
    step's capture_graph is called first)."""
    import torch
    if graph:
        step.capture_graph()
    for _ in range(warmup):
        step.replay() if graph else step.run(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        if graph:
            step.replay()
        else:
            step.launch(stream)
            step.finish()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / K



def gdn_launch_stats(step, stream, L: int, K: int) -> dict:
    """Timed region 2 and the untimed splits of one workload's step.

    * K more steps in which every gdn_verify_span dispatch records a
      start/stop event pair itself (gdn_verify_span_timed): the events bracket
      exactly the kernel, but they open short gaps between kernels, so this
      region is not used for the step time. Average and median per launch.
    * Phase split: one step with events between its phases.
    * Per stack: the step's L GDN spans back to back with no other kernel
      between them (launch gaps included), event-timed, median of 3.
    * In the step: the L (conv, GDN) layer pairs back to back minus the L
      conv spans back to back, per layer (event-timed stacks, median of 3):
      the GDN span's share of the step's layer time. (Events recorded by a
      dispatch that follows a different kernel open before that kernel has
      finished, so the per-launch events above overstate a span that
      follows a conv; these differences of stacks do not.)"""
    import torch
    import hybrid_recurrent_state_amd as hrs
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
          for _ in range(K)]
    ev_h = [[(hrs.event_handle(s), hrs.event_handle(e)) for (s, e) in row] for row in ev]
    torch.cuda.synchronize()
    log(f"timing {K} steps with per-launch GDN events")
    t2 = time.perf_counter()
    for i in range(K):
        step.launch(stream, gdn_events=ev_h[i])
        step.finish()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    gdn_ms = np.array([[s.elapsed_time(e) for (s, e) in row] for row in ev])

    ph = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    h = stream.cuda_stream
    ph[0].record()
    for l in range(L):
        step.launch_layer(l, h)
    ph[1].record()
    step.launch_accept(h)
    ph[2].record()
    step.launch_rollback(h)
    ph[3].record()
    step.launch_ring(h)
    ph[4].record()
    torch.cuda.synchronize()
    phases = {"conv+gdn": ph[0].elapsed_time(ph[1]), "accept": ph[1].elapsed_time(ph[2]),
              "rollback": ph[2].elapsed_time(ph[3]), "ring": ph[3].elapsed_time(ph[4])}

    def stack_of(launch) -> float:
        out = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for l in range(L):
                launch(l)
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / L)
        return float(np.median(out))

    stack = [stack_of(lambda l: step.launch_gdn(l, h))]
    layer_stack = stack_of(lambda l: step.launch_layer(l, h))
    conv_stack = stack_of(lambda l: step.launch_conv(l, h))
    # The same span-only stacks with every dispatch timing itself: the
    # kernel's duration when the previous kernel is the same one.
    so = []
    reps = max(1, min(K, 10))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
    evh = [(hrs.event_handle(a), hrs.event_handle(b)) for (a, b) in evs]
    torch.cuda.synchronize()
    for _ in range(reps):
        for l in range(L):
            step.launch_gdn(l, h, evh[l])
        torch.cuda.synchronize()
        so += [evs[l][0].elapsed_time(evs[l][1]) for l in range(L)]
    so = np.array(so)
    return {"avg_s": float(gdn_ms.mean()) / 1e3, "median_s": float(np.median(gdn_ms)) / 1e3,
            "min_s": float(gdn_ms.min()) / 1e3, "stack_s": float(np.median(stack)) / 1e3, "phases": phases,
            "span_only_avg_s": float(so.mean()) / 1e3, "span_only_median_s": float(np.median(so)) / 1e3,
            "layer_stack_s": layer_stack / 1e3, "conv_stack_s": conv_stack / 1e3,
            "in_step_span_s": (layer_stack - conv_stack) / 1e3, "t_events": (t2, t3)}


def measure_workload(name: str, steps: int, warmup: int, cpu_seconds: float) -> dict:
    """One configured workload beside the headline: its own buffers, W warmup
    steps, K timed steps (event-free), then gdn_launch_stats, then the oracle
    on a bounded sample of the same workload (unless cpu_seconds is 0).
    Frees its buffers before returning."""
    import torch
    from synth import WORKLOADS
    from synth.device import fill_step, step_shape
    from hybrid_recurrent_state_amd.step import StepBuffers, VerifyStep
    w = WORKLOADS[name]
    shape = step_shape(w)
    log(f"workload {name}: R={w.n_req} L={w.n_layers} T={w.n_pos}")
    bufs = StepBuffers(shape)
    loaded = fill_step(bufs, w)
    step = VerifyStep(bufs, parent=loaded.parent, runs=loaded.runs)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step.run(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step.launch(stream)
        step.finish()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    L, R, T = w.n_layers, w.n_req, w.n_pos
    gs = gdn_launch_stats(step, stream, L, steps)
    nbytes = shape.gdn_bytes_per_layer
    rec = {"workload": name, "n_req": R, "n_layers": L, "n_pos": T, "topology": "tree" if w.tree else "chain",
           "ms_per_step": ms, "value": R * T * L / (ms / 1e3), "unit": "verify tokens/s per layer",
           "gdn_tokens_per_s_per_layer": R * T / gs["avg_s"],
           "gdn_bytes_per_launch": nbytes, "avg_launch_us": gs["avg_s"] * 1e6,
           "median_launch_us": gs["median_s"] * 1e6, "min_launch_us": gs["min_s"] * 1e6,
           "frac": nbytes / gs["avg_s"] / 1e9 / HBM_PEAK_GBS,
           "stack_us_per_layer": gs["stack_s"] * 1e6, "stack_frac": nbytes / gs["stack_s"] / 1e9 / HBM_PEAK_GBS,
           "span_only_launch_avg_us": gs["span_only_avg_s"] * 1e6,
           "span_only_launch_median_us": gs["span_only_median_s"] * 1e6,
           "span_only_frac": nbytes / gs["span_only_avg_s"] / 1e9 / HBM_PEAK_GBS,
           "in_step_span_us": gs["in_step_span_s"] * 1e6,
           "in_step_span_frac": nbytes / gs["in_step_span_s"] / 1e9 / HBM_PEAK_GBS,
           "layer_stack_us": gs["layer_stack_s"] * 1e6, "conv_stack_us": gs["conv_stack_s"] * 1e6,
           "traffic": measured_traffic(name), "phases_ms": gs["phases"]}
    # The NEXT-row steps on the same buffers: f3 (the step as one graph), f2
    # (zero-copy rollback), f1 (fused layers) and their graph replays.
    nxt = {"f3_hip_graph_step_ms": time_steps(step, stream, steps, warmup, graph=True)}
    if w.vocab:
        from hybrid_recurrent_state_amd.step import FusedVerifyStep, ZeroCopyVerifyStep
        variants = [("f2_zero_copy_step_ms", ZeroCopyVerifyStep)]
        if shape.conv_channels == 2 * w.n_kheads * w.d_k + w.n_vheads * w.d_v:
            variants.append(("f1_fused_layer_step_ms", FusedVerifyStep))
        for key, cls in variants:
            v = cls(bufs, parent=loaded.parent, runs=loaded.runs)
            nxt[key] = time_steps(v, stream, steps, warmup)
            del v
            v = cls(bufs, parent=loaded.parent, runs=loaded.runs)
            v.run(stream)
            nxt[key.replace("_step_ms", "_graph_step_ms")] = time_steps(v, stream, steps, warmup, graph=True)
            del v
        bufs.ckpt2 = None
    rec["next_rows"] = nxt
    log(f"  next rows {nxt}")
    log(f"  step {ms:.3f} ms, gdn launch avg {rec['avg_launch_us']:.2f} us (frac {rec['frac']:.3f}), "
        f"stack {rec['stack_us_per_layer']:.2f} us (frac {rec['stack_frac']:.3f}), span-only launches avg "
        f"{rec['span_only_launch_avg_us']:.2f} us (frac {rec['span_only_frac']:.3f}), in the step "
        f"{rec['in_step_span_us']:.2f} us (frac {rec['in_step_span_frac']:.3f})")
    del step, bufs
    torch.cuda.empty_cache()
    if cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(w, cpu_seconds)
    return rec



def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this path has no multi-GPU mode "
              "(requests, layers and heads shard with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch
    from synth import WORKLOADS, WORKLOAD_ORDER
    from synth.device import fill_step, step_shape
    import hybrid_recurrent_state_amd as hrs
    from hybrid_recurrent_state_amd.step import StepBuffers, VerifyStep

    name = WORKLOAD_ORDER[int(args.workload)] if args.workload.isdigit() else args.workload
    w = WORKLOADS[name]
    shape = step_shape(w)
    log(f"workload {name}: R={w.n_req} L={w.n_layers} T={w.n_pos} Hk={w.n_kheads} Hv={w.n_vheads} "
        f"d={w.d_k} C={w.conv_channels} V={w.vocab} ring={w.ring_slots}x{w.ring_width}")
    torch.cuda.set_device(0)
    bufs = StepBuffers(shape)
    loaded = fill_step(bufs, w, log=log)
    step = VerifyStep(bufs, parent=loaded.parent, runs=loaded.runs)
    stream = torch.cuda.current_stream()

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calibrate_copy_mib} MiB read + {args.calibrate_copy_mib} MiB written, x3")
        del src, dst

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step.run(stream)
    torch.cuda.synchronize()

    L, K = w.n_layers, args.steps
    # Timed region 1 (throughput): K whole steps, nothing inserted between kernels.
    if args.graph:
        step.capture_graph()
        for _ in range(args.warmup):
            step.replay()
    log(f"timing {K} steps" + (" (graph replay)" if args.graph else ""))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        if args.graph:
            step.replay()
        else:
            step.launch(stream)
            step.finish()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    # Timed region 2 (roofline of the dominant kernel), phase split and
    # per-stack timing: see gdn_launch_stats.
    gs = gdn_launch_stats(step, stream, L, K)
    gdn_avg_s, gdn_med_s, stack_s, phases = gs["avg_s"], gs["median_s"], gs["stack_s"], gs["phases"]
    t2, t3 = gs["t_events"]
    h = stream.cuda_stream

    rows = row_rates(step, shape, h, L)

    R, T = w.n_req, w.n_pos
    value = R * T * L / (ms_per_step / 1e3)
    gdn_bytes = shape.gdn_bytes_per_layer
    achieved = gdn_bytes / gdn_avg_s / 1e9
    traffic = measured_traffic(name)
    store_gbs = store_stream_gbs()
    log(f"store-stream reference {store_gbs:.0f} GB/s")
    log(f"step {ms_per_step:.3f} ms (with GDN events {(t3 - t2) * 1e3 / K:.3f} ms); gdn launch avg "
        f"{gdn_avg_s * 1e6:.1f} us = {achieved:.0f} GB/s; in the step (layer stack - conv stack) "
        f"{gs['in_step_span_s'] * 1e6:.1f} us; traffic {traffic}; phases {phases}")

    next_rows = None
    if not args.no_next:
        next_rows = {}
        # f3: the same step captured once and launched as one HIP graph.
        if not args.graph:
            ms_g = time_steps(step, stream, K, args.warmup, graph=True)
            next_rows["f3_hip_graph_step"] = {"ms_per_step": ms_g, "value": R * T * L / (ms_g / 1e3),
                                              "vs_stream_launch": ms_per_step / ms_g}
            log(f"f3 graph step {ms_g:.3f} ms")
        # f2: zero-copy rollback + compact conv state (same kernels for the spans,
        # nothing copied to roll back; a second checkpoint buffer alternates).
        if w.vocab:
            from hybrid_recurrent_state_amd.step import FusedVerifyStep, ZeroCopyVerifyStep
            zc = ZeroCopyVerifyStep(bufs, parent=loaded.parent, runs=loaded.runs)
            ms_z = time_steps(zc, stream, K, args.warmup)
            next_rows["f2_zero_copy_rollback_step"] = {"ms_per_step": ms_z, "value": R * T * L / (ms_z / 1e3),
                                                       "vs_copy_rollback": ms_per_step / ms_z}
            log(f"f2 zero-copy step {ms_z:.3f} ms")
            del zc
            # f3 on the zero-copy step: two graphs, one per checkpoint-buffer parity.
            zc = ZeroCopyVerifyStep(bufs, parent=loaded.parent, runs=loaded.runs)
            zc.run(stream)
            ms_zg = time_steps(zc, stream, K, args.warmup, graph=True)
            next_rows["f3_hip_graph_zero_copy_step"] = {"ms_per_step": ms_zg, "value": R * T * L / (ms_zg / 1e3),
                                                        "vs_stream_launch": ms_z / ms_zg}
            log(f"f3 graph zero-copy step {ms_zg:.3f} ms")
            del zc
            # f1: the same zero-copy step with every layer fused into one
            # kernel (conv, SiLU, split, q/k L2 norm, gated delta rule).
            if shape.conv_channels == 2 * w.n_kheads * w.d_k + w.n_vheads * w.d_v:
                fs = FusedVerifyStep(bufs, parent=loaded.parent, runs=loaded.runs)
                ms_f = time_steps(fs, stream, K, args.warmup)
                next_rows["f1_fused_layer_step"] = {
                    "ms_per_step": ms_f, "value": R * T * L / (ms_f / 1e3), "vs_zero_copy_step": ms_z / ms_f,
                    "layer_bytes_per_launch": shape.layer_bytes_per_layer,
                    "traffic": measured_traffic(name, "gdn_layer_verify_span")}
                log(f"f1 fused-layer step {ms_f:.3f} ms")
                del fs
                fs = FusedVerifyStep(bufs, parent=loaded.parent, runs=loaded.runs)
                fs.run(stream)
                ms_fg = time_steps(fs, stream, K, args.warmup, graph=True)
                next_rows["f3_hip_graph_fused_step"] = {"ms_per_step": ms_fg, "value": R * T * L / (ms_fg / 1e3),
                                                        "vs_stream_launch": ms_f / ms_fg}
                log(f"f3 graph fused step {ms_fg:.3f} ms")
                del fs
            bufs.ckpt2 = None
            torch.cuda.empty_cache()

    if next_rows is not None:
        # f4: chunked span for long (prefill-length) spans without capture.
        try:
            next_rows["f4_chunked_prefill_span"] = chunked_prefill_row()
            log(f"f4 chunked prefill {next_rows['f4_chunked_prefill_span']}")
        except Exception as e:  # noqa: BLE001 - report, do not lose the main line
            next_rows["f4_chunked_prefill_span"] = {"error": str(e)}
        torch.cuda.empty_cache()

    headline = {"workload": name, "n_req": R, "n_layers": L, "n_pos": T, "topology": "tree" if w.tree else "chain",
                "ms_per_step": ms_per_step, "value": value, "unit": "verify tokens/s per layer",
                "gdn_tokens_per_s_per_layer": R * T / gdn_avg_s, "gdn_bytes_per_launch": gdn_bytes,
                "avg_launch_us": gdn_avg_s * 1e6, "median_launch_us": gdn_med_s * 1e6,
                "min_launch_us": gs["min_s"] * 1e6, "frac": achieved / HBM_PEAK_GBS,
                "stack_us_per_layer": stack_s * 1e6, "stack_frac": gdn_bytes / stack_s / 1e9 / HBM_PEAK_GBS,
                "span_only_launch_avg_us": gs["span_only_avg_s"] * 1e6,
                "span_only_launch_median_us": gs["span_only_median_s"] * 1e6,
                "span_only_frac": gdn_bytes / gs["span_only_avg_s"] / 1e9 / HBM_PEAK_GBS,
                "in_step_span_us": gs["in_step_span_s"] * 1e6,
                "in_step_span_frac": gdn_bytes / gs["in_step_span_s"] / 1e9 / HBM_PEAK_GBS,
                "layer_stack_us": gs["layer_stack_s"] * 1e6, "conv_stack_us": gs["conv_stack_s"] * 1e6,
                "traffic": traffic, "phases_ms": phases}
    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(w, args.cpu_seconds)
        headline["cpu_baseline"] = cpu

    # Every other configured workload, each in its own buffers after the
    # headline's are freed (the oracle on a shorter sample of each).
    workloads = {f"configs{WORKLOAD_ORDER.index(name)}": headline}
    if not args.no_workloads:
        del step, bufs
        torch.cuda.empty_cache()
        for idx, other in enumerate(WORKLOAD_ORDER):
            if other == name:
                continue
            try:
                workloads[f"configs{idx}"] = measure_workload(
                    other, K, args.warmup, 0.0 if args.no_cpu_baseline else args.workload_cpu_seconds)
            except Exception as e:  # noqa: BLE001 - report, do not lose the main line
                workloads[f"configs{idx}"] = {"workload": other, "error": str(e)}
        workloads = dict(sorted(workloads.items()))

    line = {
        "metric": "GDN verify tokens/s per layer + achieved HBM GB/s (fraction of peak), K=16",
        "value": value,
        "unit": "verify tokens/s per layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; Qwen3.6-27B-shaped GDN layers, no weights)",
        "config": {"workload": name, "launch": "hip graph" if args.graph else "stream", "n_req": R, "n_layers": L, "n_pos": T, "draft_tokens": T - 1,
                   "topology": "tree" if w.tree else "chain", "n_kheads": w.n_kheads, "n_vheads": w.n_vheads,
                   "d_k": w.d_k, "d_v": w.d_v, "inputs": w.dtype, "state": "f32",
                   "conv_channels": w.conv_channels, "conv_width": w.conv_width, "vocab": w.vocab,
                   "ring": [w.n_req, w.ring_slots, w.ring_width] if w.ring_slots else None},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "gdn_verify_span", "bytes_per_launch": gdn_bytes,
                     "avg_launch_us": gdn_avg_s * 1e6, "median_launch_us": gdn_med_s * 1e6,
                     "store_stream_gbs": store_gbs, "frac_of_store_stream": achieved / store_gbs,
                     "stack_us_per_layer": stack_s * 1e6,
                     "stack_frac": gdn_bytes / stack_s / 1e9 / HBM_PEAK_GBS,
                     "span_only_launch_avg_us": gs["span_only_avg_s"] * 1e6,
                     "span_only_frac": gdn_bytes / gs["span_only_avg_s"] / 1e9 / HBM_PEAK_GBS,
                     "in_step_span_us": gs["in_step_span_s"] * 1e6,
                     "in_step_span_frac": gdn_bytes / gs["in_step_span_s"] / 1e9 / HBM_PEAK_GBS},
        "gdn_tokens_per_s_per_layer": R * T / gdn_avg_s,
        "draft_tokens_per_s_per_layer": R * (T - 1) * L / (ms_per_step / 1e3),
        "phases_ms": phases,
        "rows": rows,
        "next_rows": next_rows,
        "workloads": workloads,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
