"""bf16 <-> float conversions for the oracle (test infrastructure only).

bf16 is the top half of an IEEE binary32: 1 sign bit, 8 exponent bits, 7
stored fraction bits (8 significant bits).  Widening is exact.  Narrowing
rounds to the nearest representable value, ties to even, straight from the
float64 value (no intermediate float32 step).

Pinned by tests/test_oracle_pins.py: every one of the 65,536 bit patterns
round-trips; values half-way between neighbours round to the even one;
torch's own float32 -> bfloat16 conversion agrees on random float32 inputs.
"""
import numpy as np


def to_f64(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def from_f64(x) -> np.ndarray:
    """float64 -> uint16 bf16 bit patterns, round to nearest, ties to even.

    Finite values are scaled so that one unit of the last place of their bf16
    binade is 1, rounded with numpy's rint (half to even), and scaled back.
    Binade: 2^(e-1) <= |x| < 2^e with frexp's e; bf16 keeps 8 significant
    bits, so the quantum is 2^(e-8), but never below the subnormal quantum
    2^-133.  Results beyond the largest finite bf16 become infinities, and NaN
    stays NaN (quiet).
    """
    x0 = np.asarray(x, dtype=np.float64)
    x = np.atleast_1d(x0)
    out = np.empty(x.shape, dtype=np.float64)
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)
    q_exp = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(xf, -q_exp)), q_exp)
    out[fin] = r
    out[~fin] = x[~fin]
    # largest finite bf16 is (2 - 2^-7) * 2^127; rounding past it gives inf
    big = np.abs(out) > (2.0 - 2.0 ** -7) * 2.0 ** 127
    out[big & fin] = np.copysign(np.inf, out[big & fin])
    f32 = out.astype(np.float32)
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    bits[nan] = 0x7FC0
    return bits.reshape(x0.shape)


def round_f64(x) -> np.ndarray:
    """float64 -> nearest bf16 value, returned as float64."""
    return to_f64(from_f64(x))
