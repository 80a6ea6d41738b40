"""Exact decoding of the storage dtypes into float64.

TEST INFRASTRUCTURE (see the package header).

bfloat16 is the upper half of an IEEE binary32, so its bits shifted left by
16 are a binary32 with the same value; float16 and float32 widen exactly to
float64.  Pinned by tests/test_oracle_dtypes.py with bit patterns of known
value.
"""

from __future__ import annotations

import numpy as np

STORAGE = ("f32", "f16", "bf16")  # "f64" is accepted too, for hand-made test data


def decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values of a storage array.

    ``raw`` is float32 for "f32", float16 for "f16" and uint16 (the bit
    pattern) for "bf16".
    """
    if dtype == "f64":
        return np.asarray(raw, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(raw, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")
