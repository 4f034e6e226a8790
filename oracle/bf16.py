"""bf16 bit patterns -> exact float64 values (oracle side).

A bf16 value is the top 16 bits of an IEEE float32, so widening is exact:
place the 16 bits above 16 zero bits, read as float32, widen to float64.
"""
import numpy as np


def bf16_to_float64(bits: np.ndarray) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
