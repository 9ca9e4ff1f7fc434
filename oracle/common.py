"""Input widening for the oracle (test infrastructure only).

bf16 inputs arrive as their 16-bit patterns (``np.uint16``); a bf16 value is
the float32 whose upper 16 bits are that pattern and whose lower 16 bits are
zero, so widening is exact. float32 inputs widen to float64 exactly.
"""
import numpy as np


def widen(x) -> np.ndarray:
    """Exact float64 value of a float32 array or of bf16 bit patterns."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype == np.float32 or x.dtype == np.float64:
        return x.astype(np.float64)
    raise TypeError(f"unsupported input dtype {x.dtype}")


def to_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 to float32, nearest-even (IEEE default)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)
