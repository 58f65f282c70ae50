"""bf16 decoding for the oracle (test infrastructure only).

A bf16 number is the upper 16 bits of an IEEE-754 binary32; widening it is
exact, so the oracle computes on the very values the device receives.
"""
import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
