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


def assert_tiles(g, o, tile_ndim: int, what: str, tol: float = TOL) -> float:
    err = tile_rel_err(g, o, tile_ndim)
    assert err <= tol, f"{what}: max tile relative error {err:.3e} > {tol:.0e}"
    return err
