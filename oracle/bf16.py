"""Exact bfloat16 -> fp64 decoding for the oracle (test infrastructure only).

A bfloat16 value is the upper 16 bits of an IEEE-754 binary32.  Shifting the
16-bit pattern into the high half of a 32-bit word gives that binary32 exactly,
and binary32 -> binary64 is exact, so the oracle sees the very values the GPU
reads.  No rounding happens here.
"""

import numpy as np


def to_f64(x):
    """Return ``x`` as an fp64 ndarray.

    ``x`` may be a float array of any width (converted exactly) or a uint16 /
    int16 array holding bfloat16 bit patterns.
    """
    a = np.asarray(x)
    if a.dtype in (np.uint16, np.int16):
        u32 = a.view(np.uint16).astype(np.uint32) << np.uint32(16)
        return u32.view(np.float32).astype(np.float64)
    return a.astype(np.float64)
