"""Decoding of stored element bits to float64 (oracle; test infrastructure only).

The cache stores either IEEE binary32 (fp32) or bfloat16 (the upper 16
bits of a binary32). Decoding is exact: a bf16 pattern ``u`` is the
binary32 pattern ``u << 16``, and every binary32 value is exactly a
float64. The oracle computes on these exact stored values.

Convention for arrays handed to the oracle:
* ``numpy.uint16``  -> bf16 bit patterns
* ``numpy.float32`` -> fp32 values (or ``numpy.uint32`` fp32 bit patterns)
* ``numpy.float64`` -> already widened
"""

import numpy as np


def bf16_bits_to_f64(bits):
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_bits_to_f64(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def widen(x):
    """Stored array (uint16 bf16 bits / float32 / uint32 fp32 bits / float64) -> float64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    if x.dtype == np.uint32:
        return f32_bits_to_f64(x)
    if x.dtype == np.float32:
        return x.astype(np.float64)
    if x.dtype == np.float64:
        return x
    raise TypeError(f"unsupported stored dtype {x.dtype}")
