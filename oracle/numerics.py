"""Exact conversions between stored element formats and fp64 (oracle; test
infrastructure only).

bf16 is the top 16 bits of an IEEE binary32; widening is exact.  The values
the oracle attends over are always the exact stored bits widened, never the
fp32 draws they were rounded from.
"""
import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64, exactly (NaN stays NaN)."""
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, rounding the binary32 value to nearest-even.
    Used only to state which bf16 value a rounded output should take."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    r = ((b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)
    r[nan] = np.uint16(0x7FC0)
    return r


def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Raw stored values (float32 array for "f32", uint16 bits for "bf16")
    widened to float64."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(raw)
    raise ValueError(f"unknown dtype {dtype!r}")
