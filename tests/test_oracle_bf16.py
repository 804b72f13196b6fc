"""Pins for the oracle's bf16 converters against an independent formulation and the format's
definition (IEEE 754 binary32 with the low 16 bits dropped: 1 sign, 8 exponent, 7 mantissa)."""
import os

import numpy as np
import pytest

from bf16_ref import bf16_rne_reference_f32_bits, bf16_rne_reference_f64, is_bf16_nan

# Hand-derived cases (bits of an fp32 -> expected bf16), from the format definition:
HAND_CASES = [
    (0x3F800000, 0x3F80),  # 1.0 exact
    (0x3F808000, 0x3F80),  # 1 + 2^-8: halfway between 0x3F80 and 0x3F81 -> even 0x3F80
    (0x3F818000, 0x3F82),  # halfway between 0x3F81 (odd) and 0x3F82 -> 0x3F82
    (0x3F808001, 0x3F81),  # just above halfway -> up
    (0x3F807FFF, 0x3F80),  # just below halfway -> down
    (0xBF808001, 0xBF81),  # sign is independent of rounding magnitude
    (0x7F7F7FFF, 0x7F7F),  # largest finite bf16 stays
    (0x7F7F8000, 0x7F80),  # halfway above largest finite, odd mantissa -> rounds to Inf
    (0x7F7FFFFF, 0x7F80),  # fp32 max -> Inf
    (0x00000001, 0x0000),  # smallest fp32 subnormal -> +0
    (0x00008000, 0x0000),  # halfway between 0 and smallest bf16 subnormal -> even (0)
    (0x00018000, 0x0002),  # halfway between 0x0001 (odd) and 0x0002 -> 0x0002
    (0x00008001, 0x0001),  # above halfway -> smallest bf16 subnormal
    (0x007FFFFF, 0x0080),  # largest fp32 subnormal rounds up to smallest normal
    (0x80000000, 0x8000),  # -0
    (0x7F800000, 0x7F80),  # +Inf
    (0xFF800000, 0xFF80),  # -Inf
]


def test_hand_cases_f32(orc):
    bits = np.array([c[0] for c in HAND_CASES], dtype=np.uint32)
    want = np.array([c[1] for c in HAND_CASES], dtype=np.uint16)
    got = orc.bf16_from_f32_bits(bits)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(bf16_rne_reference_f32_bits(bits), want)


def test_nan_stays_nan(orc):
    bits = np.array([0x7FC00000, 0x7F800001, 0xFF800001, 0x7FFFFFFF, 0x7F80FFFF], dtype=np.uint32)
    got = orc.bf16_from_f32_bits(bits)
    assert is_bf16_nan(got).all()
    assert ((got >> 15) == (bits >> 31)).all()
    got64 = orc.bf16_from_f64(np.array([np.nan, -np.nan]))
    assert is_bf16_nan(got64).all()


def _structured_patterns():
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    rng = np.random.Generator(np.random.PCG64(0xB16))
    lows = np.concatenate([
        np.array([0x0000, 0x0001, 0x3FFF, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xFFFE, 0xFFFF],
                 dtype=np.uint32),
        rng.integers(0, 1 << 16, size=22, dtype=np.uint32),
    ])
    return (hi[:, None] | lows[None, :]).reshape(-1)


def _compare_f32(orc, bits):
    got = orc.bf16_from_f32_bits(bits)
    want = bf16_rne_reference_f32_bits(bits)
    nan_in = np.isnan(bits.view(np.float32))
    assert is_bf16_nan(got[nan_in]).all()
    ok = got[~nan_in] == want[~nan_in]
    if not ok.all():
        i = np.flatnonzero(~ok)[0]
        b = bits[~nan_in][i]
        raise AssertionError(f"fp32 bits {b:#010x}: oracle {got[~nan_in][i]:#06x} "
                             f"reference {want[~nan_in][i]:#06x}")


def test_structured_sweep_f32(orc):
    """Every sign/exponent/mantissa-top combination with low halves around every rounding edge."""
    _compare_f32(orc, _structured_patterns())


def test_random_patterns_f32(orc):
    rng = np.random.Generator(np.random.PCG64(0xC3B16))
    _compare_f32(orc, rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32))


@pytest.mark.skipif(os.environ.get("C3_EXHAUSTIVE") != "1",
                    reason="full 2^32 sweep takes minutes; set C3_EXHAUSTIVE=1")
def test_exhaustive_f32(orc):
    step = 1 << 24
    for start in range(0, 1 << 32, step):
        _compare_f32(orc, np.arange(start, start + step, dtype=np.uint64).astype(np.uint32))


def test_f64_agrees_on_fp32_values(orc):
    """On values exactly representable in fp32 both oracle paths must agree."""
    bits = _structured_patterns()
    bits = bits[~np.isnan(bits.view(np.float32))]
    x = bits.view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(orc.bf16_from_f64(x), orc.bf16_from_f32_bits(bits))


def test_f64_single_rounding(orc):
    """Values just off a bf16 halfway point that fp32 would first round ONTO the halfway point:
    a double rounding (fp64 -> fp32 -> bf16) gets these wrong, a single rounding does not."""
    one_tie = 1.0 + 2.0 ** -8                    # halfway between bf16 1.0 and 1.0078125
    cases = np.array([
        one_tie + 2.0 ** -30,                    # above halfway -> 0x3F81
        one_tie - 2.0 ** -30,                    # below halfway -> 0x3F80
        -(one_tie + 2.0 ** -30),                 # -> 0xBF81
        (1.0 + 3 * 2.0 ** -8) - 2.0 ** -31,      # below the 0x3F81/0x3F82 halfway -> 0x3F81
    ])
    want = np.array([0x3F81, 0x3F80, 0xBF81, 0x3F81], dtype=np.uint16)
    np.testing.assert_array_equal(orc.bf16_from_f64(cases), want)
    np.testing.assert_array_equal(bf16_rne_reference_f64(cases), want)


def test_f64_random(orc):
    rng = np.random.Generator(np.random.PCG64(0x64B16))
    x = np.concatenate([
        rng.standard_normal(1 << 20) * 10.0 ** rng.integers(-40, 39, size=1 << 20),
        rng.standard_normal(1 << 16) * 2.0 ** -130,      # bf16 subnormal range
        rng.standard_normal(1 << 12) * 3.0e38,           # around overflow
    ])
    np.testing.assert_array_equal(orc.bf16_from_f64(x), bf16_rne_reference_f64(x))


def test_decode_exact(orc):
    h = np.arange(1 << 16, dtype=np.uint16)
    f = orc.bf16_to_f32(h)
    finite = np.isfinite(f)
    # decoding then re-rounding is the identity on every non-NaN pattern
    np.testing.assert_array_equal(orc.bf16_from_f32(f[finite]), h[finite])
