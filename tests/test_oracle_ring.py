"""Pins of the ring oracle: slice assignment over split non-wrapping runs,
untouched slots, and set/get round trip."""
import numpy as np

from oracle import ring as orr


def test_set_get_against_slices():
    rng = np.random.default_rng(3)
    R, S, D = 3, 16, 5
    ring = rng.integers(0, 1000, (R, S, D)).astype(np.uint16)
    packed = rng.integers(0, 1000, (20, D)).astype(np.uint16)
    runs = [(0, 14, 5, 0), (1, 0, 6, 5), (2, 9, 7, 11), (0, 3, 2, 18)]
    out = orr.ring_set(ring, packed, runs)
    ref = ring.copy()
    touched = np.zeros((R, S), dtype=bool)
    for rid, st, n, row in orr.split_runs(runs, S):
        assert st + n <= S
        ref[rid, st:st + n] = packed[row:row + n]
        touched[rid, st:st + n] = True
    assert np.array_equal(out, ref)
    assert np.array_equal(out[~touched], ring[~touched])
    got = orr.ring_get(out, np.zeros_like(packed), runs)
    for rid, st, n, row in runs:
        assert np.array_equal(got[row:row + n], packed[row:row + n])


def test_split_runs_wrap():
    assert orr.split_runs([(0, 14, 5, 0)], 16) == [(0, 14, 2, 0), (0, 0, 3, 2)]
    assert orr.split_runs([(1, 0, 16, 4)], 16) == [(1, 0, 16, 4)]
