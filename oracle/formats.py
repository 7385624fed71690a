"""Storage-format decoding for the oracle (exact widening to float64).

TEST INFRASTRUCTURE: see the package docstring.

The oracle receives host arrays carrying the exact bits of the device
tensors.  float32 and float16 arrive as numpy float32/float16.  bfloat16
has no numpy dtype, so it arrives as uint16 and is widened here by
placing its 16 bits in the top half of a float32, which is exact: a
bfloat16 is by definition the upper 16 bits of an IEEE binary32.  E4M3
codes (fp8 KV pools) arrive as uint8 and are decoded by oracle.fp8.

Parity: pinned (tests check decoded values of hand-written bit patterns
for +-0, 1, -2, the smallest subnormal, inf and NaN, and that every
float16/float32 widening equals numpy's own exact cast).
"""

import numpy as np

DTYPES = ("f32", "f16", "bf16", "e4m3")

_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "e4m3": np.uint8}


def storage_dtype(dtype):
    """numpy dtype that carries the bits of one element of `dtype`."""
    return _STORAGE[dtype]


def bits_view(arr):
    """Unsigned-integer view of an array's bits (for bit-exact comparison)."""
    a = np.ascontiguousarray(arr)
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])


def to_f64(arr, dtype):
    """Widen storage-format values to float64 exactly."""
    a = np.asarray(arr)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must arrive as uint16 bit patterns")
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f16":
        if a.dtype != np.float16:
            raise TypeError("f16 data must arrive as numpy float16")
        return a.astype(np.float64)
    if dtype == "f32":
        if a.dtype != np.float32:
            raise TypeError("f32 data must arrive as numpy float32")
        return a.astype(np.float64)
    if dtype == "e4m3":
        if a.dtype != np.uint8:
            raise TypeError("e4m3 data must arrive as uint8 codes")
        from .fp8 import e4m3_decode
        return e4m3_decode(a)
    raise ValueError(f"unknown dtype {dtype!r}")
