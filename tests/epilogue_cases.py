"""GEMM operands whose fp32 sums are chosen fp32 bit patterns, exactly, in any summation order:
the inputs of the epilogue rounding sweep (tests only)."""
import numpy as np


def exact_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bits of values that bf16 holds exactly (asserted: the fp32 low half is zero)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert not np.any(b & 0xFFFF)
    return (b >> 16).astype(np.uint16)


def epilogue_case(sign: np.ndarray, f: np.ndarray, ts):
    """A GEMM whose fp32 sums are exactly the fp32 patterns (sign, 127 + t, f) for every row
    (sign, f) and column t, and the bf16 bits they must round to.

    Row r of A is (h, m, l, 0, ...) with h = +-(1 + (f >> 16) / 2^7), m = +-((f >> 8) & 255) / 2^15,
    l = +-(f & 255) / 2^23: three bf16 values with disjoint significant bits whose sum is
    +-(1 + f / 2^23). Column t of B is 2^t in rows 0..2. Every product and partial sum is then
    exact in fp32 for t >= -103 (the smallest part stays a normal number), so C's fp32 value is the
    pattern itself whatever the summation order, and only the epilogue's rounding is tested."""
    sgn = np.where(sign, -1.0, 1.0)
    f = f.astype(np.int64)
    parts = [sgn * (1.0 + (f >> 16) / 128.0), sgn * ((f >> 8) & 255) / 2.0 ** 15,
             sgn * (f & 255) / 2.0 ** 23]
    M, K, N = f.size, 8, len(ts)
    A = np.zeros((M, K), dtype=np.uint16)
    for k, part in enumerate(parts):
        A[:, k] = exact_bf16_bits(part)
    B = np.zeros((K, N), dtype=np.uint16)
    B[:3, :] = exact_bf16_bits(np.array([2.0 ** t for t in ts]))[None, :]
    pattern = ((sign.astype(np.uint32) << 31)[:, None]
               | (np.array([127 + t for t in ts], dtype=np.uint32) << 23)[None, :]
               | f.astype(np.uint32)[:, None])
    return A, B, pattern
