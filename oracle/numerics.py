"""bf16 storage conversions for the oracle (test infrastructure only).

bf16 is the top half of an IEEE binary32. Widening is exact (append 16 zero
bits); narrowing rounds to nearest, ties to even, on the dropped 16 bits.
"""
import numpy as np


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 storage -> fp32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> uint16 bf16 storage, round to nearest even. NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(
            np.uint16)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> fp32 holding the nearest bf16 value."""
    return bf16_to_f32(f32_to_bf16(x))
