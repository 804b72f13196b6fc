"""Pins of the oracle's all-reduce local share (reduce-scatter sum + all-gather of the reduced
chunks) against what mathematics fixes: exact integer sums, exhaustive two-rank sums against
exact sums rounded by the independent bf16 formulation, hand-worked cases that separate rank
order, single rounding and the sign of zero, and the fp32 recursive-summation error bound."""
import math

import numpy as np
import pytest

import oracle
from bf16_ref import bf16_rne_reference_f64
from concurrent_gemm_dma_amd import workloads as wl


def decode(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def encode_exact(x):
    """bf16 bits of values known to be exactly representable (checked)."""
    f = np.asarray(x, np.float32)
    bits = f.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not exactly representable in bf16"
    return (bits >> np.uint32(16)).astype(np.uint16)


def test_single_rank_is_identity(orc):
    x = wl.gen_bf16((4097,), ("normal", 0.0, 1.0), 11)
    assert np.array_equal(oracle.reduce_sum_bf16([x]), x)


@pytest.mark.parametrize("world", [2, 3, 8])
def test_integer_sums_are_exact(orc, world):
    rng = np.random.default_rng(100 + world)
    ints = rng.integers(-16, 17, size=(world, 5000))
    contribs = [encode_exact(ints[r].astype(np.float32)) for r in range(world)]
    want = encode_exact(ints.sum(axis=0).astype(np.float32))  # |sum| <= 128: exact in bf16
    got = oracle.reduce_sum_bf16(contribs)
    # +0 and -0 are both the integer 0; the sum of integers never produces -0 here unless every
    # term is -0, which integer encoding does not produce
    assert np.array_equal(got, want)


def _bf16_grid(exp_lo, exp_hi):
    """Every bf16 pattern (both signs) whose biased exponent lies in [exp_lo, exp_hi]."""
    pats = []
    for e in range(exp_lo, exp_hi + 1):
        for m in range(128):
            pats.append((e << 7) | m)
    pats = np.array(pats, np.uint16)
    return np.concatenate([pats, pats | np.uint16(0x8000)])


def test_two_ranks_exhaustive_against_exact_sums(orc):
    # biased exponents 124..131: any two such values differ by at most 7 in exponent, so their
    # sum needs at most 8 + 7 + 1 significant bits and is exact in fp32 and fp64; the result is
    # then the exact sum rounded once to bf16
    vals = _bf16_grid(124, 131)
    a = np.repeat(vals, vals.size)
    b = np.tile(vals, vals.size)
    exact = decode(a).astype(np.float64) + decode(b).astype(np.float64)
    want = bf16_rne_reference_f64(exact)
    got = oracle.reduce_sum_bf16([a, b])
    assert np.array_equal(got, want)


def test_two_ranks_tiny_values_and_zeros(orc):
    # zero, subnormals and the smallest normals, both signs: sums exact in fp32
    vals = np.concatenate([_bf16_grid(0, 2), np.array([0x0000, 0x8000], np.uint16)])
    a = np.repeat(vals, vals.size)
    b = np.tile(vals, vals.size)
    exact = decode(a).astype(np.float64) + decode(b).astype(np.float64)
    assert np.array_equal(oracle.reduce_sum_bf16([a, b]), bf16_rne_reference_f64(exact))


# Hand-worked cases (values as bf16 bit patterns):
#   1.0 = 0x3F80, 2^24 = 0x4B80, -2^24 = 0xCB80, 2^-8 = 0x3B80, 1 + 2^-7 = 0x3F81,
#   largest finite bf16 = 0x7F7F (about 3.39e38), +Inf = 0x7F80.
HAND = [
    # rank order in fp32: 1 + 2^24 is a tie between 2^24 and 2^24 + 2 and goes to the even 2^24;
    # adding -2^24 then gives 0 (a reversed order, or an fp64 accumulator, would give 1.0)
    ("rank_order", [[0x3F80], [0x4B80], [0xCB80]], 0x0000),
    # one rounding at the end: 1 + 2^-8 + 2^-8 = 1 + 2^-7 exactly in fp32 (rounding to bf16 after
    # each addition would lose both halves: 1 + 2^-8 is a tie that goes to 1.0)
    ("single_rounding", [[0x3F80], [0x3B80], [0x3B80]], 0x3F81),
    # the sum starts from rank 0's value, so a sum of negative zeros stays -0
    ("negative_zero", [[0x8000], [0x8000], [0x8000], [0x8000]], 0x8000),
    # x + (-x) is +0 under round-to-nearest
    ("cancel_to_plus_zero", [[0x3F80], [0xBF80]], 0x0000),
    # two largest finite values overflow fp32 to +Inf
    ("overflow", [[0x7F7F], [0x7F7F]], 0x7F80),
]


@pytest.mark.parametrize("name,contribs,want", HAND, ids=[h[0] for h in HAND])
def test_hand_worked_cases(orc, name, contribs, want):
    got = oracle.reduce_sum_bf16([np.array(c, np.uint16) for c in contribs])
    assert int(got[0]) == want, f"{name}: got {int(got[0]):#06x}, want {want:#06x}"


def test_error_bound_random(orc):
    world, n = 8, 20000
    contribs = [wl.gen_bf16((n,), ("normal", 0.0, 1.0), 300 + r) for r in range(world)]
    got = decode(oracle.reduce_sum_bf16(contribs)).astype(np.float64)
    xs = np.stack([decode(c).astype(np.float64) for c in contribs])
    exact = np.array([math.fsum(xs[:, e]) for e in range(n)])
    absum = np.abs(xs).sum(axis=0)
    u = 2.0 ** -24
    gamma = (world - 1) * u / (1 - (world - 1) * u)
    acc_err = gamma * absum                        # fp32 recursive summation
    round_err = 2.0 ** -8 * (np.abs(exact) + acc_err) + 2.0 ** -134  # half an ulp of bf16
    assert np.all(np.abs(got - exact) <= acc_err + round_err)
    # and the rounding is to nearest: most results are within a quarter of the bound
    assert np.mean(np.abs(got - exact) <= 0.5 * (acc_err + round_err)) > 0.5


@pytest.mark.parametrize("world,rank", [(1, 0), (4, 0), (4, 2), (8, 7)])
def test_allreduce_local_placement(orc, world, rank):
    n = 37
    contribs = [wl.gen_bf16((n,), ("normal", 0.0, 1.0), 400 + r) for r in range(world)]
    peers = [None if i == rank else wl.gen_bf16((n,), ("normal", 0.0, 1.0), 500 + i)
             for i in range(world)]
    reduced, dst = oracle.allreduce_local(contribs, peers, rank)
    assert np.array_equal(reduced, oracle.reduce_sum_bf16(contribs))
    assert dst.size == world * n
    for i in range(world):
        for e in range(n):
            src = reduced[e] if i == rank else peers[i][e]
            assert dst[i * n + e] == src, (i, e)


def test_allreduce_local_rejects_bad_arguments(orc):
    x = np.zeros(4, np.uint16)
    with pytest.raises(ValueError):
        oracle.allreduce_local([x, x], [None], 0)
    with pytest.raises(ValueError):
        oracle.allreduce_local([x, x], [None, x], 2)
    with pytest.raises(ValueError):
        oracle.reduce_sum_bf16([x, np.zeros(5, np.uint16)])
