"""bfloat16 helpers for the oracle (test infrastructure only).

bf16 is the upper half of an IEEE fp32 word. Widening is exact (append 16 zero bits).
Narrowing rounds to nearest, ties to even, which is how PyTorch and the decode path
store activations and KV entries at bf16 (the W8A16 workload keeps activations in bf16).
"""
import numpy as np


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> uint16 bf16 patterns, round to nearest even; NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, ((u >> np.uint64(16)).astype(np.uint16) | np.uint16(0x40)), r)
    return r.reshape(x.shape)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 and return them as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))
