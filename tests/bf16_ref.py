"""Independent bf16 rounding formulation used to pin the oracle's converters (tests only).

Round to nearest, ties to even, written as the definition: bracket |x| between the largest
bf16 value not above it (lo) and the next bf16 value (hi = lo + spacing), measure both
distances exactly in fp64, take the nearer one, and on a tie take the candidate whose last kept
mantissa bit is 0. bf16 has 8 significant bits; in the binade [2^(e-1), 2^e) the spacing is
2^(e-8), and below the smallest normal 2^-126 it stays 2^-133. A chosen value of 2^128 or
more is an overflow and becomes Inf.

This shares nothing with the oracle's bit-pattern trick (fp32 path) or its nearbyint scaling
(fp64 path).
"""
import numpy as np


def bf16_rne_reference_f64(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp64 values x (NaN inputs map to 0x7FC0 / 0xFFC0)."""
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    out = np.zeros(x.size, dtype=np.uint16)
    sign = np.signbit(x)
    ax = np.abs(x)
    nan = np.isnan(x)
    inf = np.isinf(x)
    zero = ax == 0.0
    fin = ~(nan | inf | zero)

    a = ax[fin]
    _, e = np.frexp(a)                        # a in [2^(e-1), 2^e)
    q = np.maximum(e - 8, -133)               # spacing exponent
    units = np.floor(np.ldexp(a, -q))         # lo = units * 2^q  (exact)
    lo = np.ldexp(units, q)
    hi = np.ldexp(units + 1.0, q)
    d_lo = a - lo                             # exact: both within one binade of a
    d_hi = hi - a
    lo_even = np.mod(units, 2.0) == 0.0
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)
    chosen = np.where(take_hi, hi, lo)
    with np.errstate(over="ignore"):
        f32 = chosen.astype(np.float32)       # exact (<= 8 significant bits) unless >= 2^128
    f32 = np.where(chosen >= 2.0 ** 128, np.float32(np.inf), f32).astype(np.float32)
    out[fin] = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[inf] = 0x7F80
    out[zero] = 0
    out[nan] = 0x7FC0
    out |= np.where(sign, np.uint16(0x8000), np.uint16(0)).astype(np.uint16)
    return out


def bf16_rne_reference_f32_bits(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint32).reshape(-1)
    with np.errstate(invalid="ignore"):
        x = bits.view(np.float32).astype(np.float64)
    return bf16_rne_reference_f64(x)


def is_bf16_nan(h: np.ndarray) -> np.ndarray:
    h = np.asarray(h, dtype=np.uint16)
    return ((h & 0x7F80) == 0x7F80) & ((h & 0x007F) != 0)
