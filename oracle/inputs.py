"""Exact upcast of stored inputs to fp64 (oracle side).

Stored tensors are either float32 arrays or uint16 arrays holding bfloat16 bit
patterns (the top half of a binary32).  Both widen to fp64 without rounding.
"""
import numpy as np


def as_f64(x):
    """fp64 copy of a float array or of uint16 bf16 bit patterns."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)
