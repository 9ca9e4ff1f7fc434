"""Helpers of the GPU parity tests (not collected as tests)."""
import sys

import numpy as np

from synth.device import to_numpy, to_torch  # noqa: F401

TOL = 1e-4   # max relative error per tile for float results


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def tile_rel_err(g, o, tile_ndim: int) -> float:
    """max over tiles of max|g - o| / max(max|o|, 2^-126); a tile is the last
    ``tile_ndim`` axes (state: one head's d_v x d_k matrix at one position;
    out: one head's d_v vector; conv y: one position's channels)."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    axes = tuple(range(g.ndim - tile_ndim, g.ndim))
    num = np.max(np.abs(g - o), axis=axes)
    den = np.maximum(np.max(np.abs(o), axis=axes), 2.0 ** -126)
    if np.any(np.isnan(g)):
        return float("inf")
    return float(np.max(num / den))


def elementwise_diag(g, o, tile_ndim: int) -> dict:
    """Element-wise relative errors, reported beside the per-tile metric as
    diagnostics (they do not decide pass or fail: near-zero elements make
    element-wise ratios meaningless). ``max_rel_sig``: the largest
    |g - o| / |o| over elements whose |o| is at least 1/64 of their tile's
    largest magnitude; ``frac_over_tol``: the share of all nonzero-reference
    elements whose own ratio exceeds TOL; ``max_ulp32``: the largest distance
    in float32 units in the last place between g and o rounded to float32."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    axes = tuple(range(g.ndim - tile_ndim, g.ndim))
    tile_max = np.max(np.abs(o), axis=axes, keepdims=True)
    diff = np.abs(g - o)
    nz = np.abs(o) > 0
    rel = np.where(nz, diff / np.where(nz, np.abs(o), 1.0), 0.0)
    sig = np.abs(o) >= tile_max / 64
    g32 = g.astype(np.float32).view(np.int32).astype(np.int64)
    o32 = o.astype(np.float32).view(np.int32).astype(np.int64)
    # map sign-magnitude float bits onto a monotone integer line
    g32 = np.where(g32 < 0, -(g32 & 0x7FFFFFFF), g32)
    o32 = np.where(o32 < 0, -(o32 & 0x7FFFFFFF), o32)
    return {"max_rel_sig": float(np.max(rel[sig])) if np.any(sig) else 0.0,
            "frac_over_tol": float(np.mean(rel[nz] > TOL)) if np.any(nz) else 0.0,
            "max_ulp32": int(np.max(np.abs(g32 - o32))) if g32.size else 0}


def assert_tiles(g, o, tile_ndim: int, what: str, tol: float = TOL) -> float:
    err = tile_rel_err(g, o, tile_ndim)
    d = elementwise_diag(g, o, tile_ndim)
    say(f"  {what}: tile {err:.2e} | element-wise: max rel (|o| >= tile max / 64) {d['max_rel_sig']:.2e}, "
        f"share over {TOL:.0e} {d['frac_over_tol']:.2e}, max {d['max_ulp32']} f32 ulp")
    assert err <= tol, f"{what}: max tile relative error {err:.3e} > {tol:.0e}"
    return err
