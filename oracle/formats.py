"""Number formats for the oracle -- test infrastructure only.

bf16 is the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits,
7 stored significand bits. Decoding is exact; encoding rounds to nearest with
ties to even, computed from the float64 value directly (no float32 step, so no
double rounding).
"""
import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns as float64."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns (padding of some inputs) decode to NaN
        return u32.view(np.float32).astype(np.float64)


def to_f64(x, dtype: str) -> np.ndarray:
    """Decode an input buffer: "bf16" (uint16 bits), "f32" or "f64"."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype in ("f32", "f64"):
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even); return bit patterns.

    For |x| in [2**e, 2**(e+1)) the bf16 spacing is 2**(e-7); below the
    smallest normal (2**-126) the spacing is 2**-133. The value is scaled to
    units of that spacing (exact), rounded half-to-even, and scaled back.
    Finite inputs only.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("finite values only")
    _, e2 = np.frexp(x)  # x = m * 2**e2, 0.5 <= |m| < 1, so |x| in [2**(e2-1), 2**e2)
    e = np.maximum(e2.astype(np.int64) - 1, -126)
    spacing_exp = e - 7
    r = np.rint(np.ldexp(x, -spacing_exp))  # numpy rint rounds half to even
    y = np.ldexp(r, spacing_exp)
    if np.any(np.abs(y) >= 2.0 ** 128):
        raise OverflowError("value rounds beyond the bf16 range")
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
