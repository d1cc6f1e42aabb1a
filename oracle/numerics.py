"""Exact upcasts of stored tensors to float64 (oracle side)."""

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.

    A bf16 value is the upper half of an IEEE binary32, so shifting the 16
    bits into the top of a 32-bit word gives that binary32 exactly.  Widening
    to binary64 is then exact too.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor (bf16 bits or float32) -> float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)
