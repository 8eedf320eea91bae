"""bfloat16 storage conversion (a storage format, not layer arithmetic).

bf16 keeps the top 16 bits of an IEEE-754 binary32 value.  Conversion from
fp32 rounds to nearest, ties to even; NaN stays NaN (quiet bit forced).
"""
import numpy as np


def f32_to_bf16_bits(x):
    """Round fp32 values to bf16 (RNE) and return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                      # wraps only for NaN patterns, which are replaced below
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
