"""Pins for the oracle GEMM (C = A.B, bf16 in, bf16 out) against things other than itself:
a numpy step-by-step fp32 accumulation, fp64 brute force with the recursive-summation error
bound, exact integer arithmetic, and identity / zero invariants."""
import numpy as np
import pytest

from bf16_ref import bf16_rne_reference_f32_bits, bf16_rne_reference_f64
from concurrent_gemm_dma_amd import workloads as wl

U = 2.0 ** -24  # unit roundoff of fp32


def _rand_bf16(shape, seed, scale=1.0):
    return wl.gen_bf16(shape, ("normal", 0.0, scale), seed)


def _decode(h):
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _numpy_sequential_fp32(A, B):
    """acc <- fl32(acc + a_k * b_k) for k = 0..K-1, elementwise in numpy float32."""
    a = _decode(A)
    b = _decode(B)
    acc = np.zeros((A.shape[0], B.shape[1]), dtype=np.float32)
    for k in range(A.shape[1]):
        prod = (a[:, k:k + 1] * b[k:k + 1, :]).astype(np.float32)  # exact: 8x8-bit mantissas
        acc = (acc + prod).astype(np.float32)
    return acc


SHAPES = [(1, 1, 1), (1, 3, 2), (2, 1, 5), (3, 5, 7), (7, 3, 16), (16, 17, 33), (17, 16, 64),
          (33, 7, 5), (5, 64, 17), (64, 33, 3), (2, 2, 1), (1, 17, 64)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_f32acc_matches_numpy_sequential(orc, M, N, K):
    A = _rand_bf16((M, K), 100 + M * 7 + K)
    B = _rand_bf16((K, N), 200 + N * 11 + K, 0.5)
    C, acc = orc.gemm_f32acc(A, B, want_acc=True)
    ref_acc = _numpy_sequential_fp32(A, B)
    np.testing.assert_array_equal(acc.view(np.uint32), ref_acc.view(np.uint32))
    np.testing.assert_array_equal(C, bf16_rne_reference_f64(ref_acc.astype(np.float64))
                                  .reshape(M, N))


@pytest.mark.parametrize("M,N,K", SHAPES + [(9, 13, 1000)])
def test_f32acc_within_summation_bound(orc, M, N, K):
    """|fl32 sum - exact| <= gamma_K * sum_k |a_k b_k|, gamma_K = K u / (1 - K u)."""
    A = _rand_bf16((M, K), 300 + M + N)
    B = _rand_bf16((K, N), 400 + K)
    _, acc = orc.gemm_f32acc(A, B, want_acc=True)
    a = _decode(A).astype(np.float64)
    b = _decode(B).astype(np.float64)
    exact = a @ b
    absum = np.abs(a) @ np.abs(b)
    gamma = K * U / (1 - K * U)
    assert np.all(np.abs(acc.astype(np.float64) - exact) <= gamma * absum + 1e-300)


@pytest.mark.parametrize("M,N,K", [(5, 7, 3), (16, 17, 33), (3, 64, 200)])
def test_f64acc_brute_force(orc, M, N, K):
    A = _rand_bf16((M, K), 500 + K)
    B = _rand_bf16((K, N), 600 + N)
    C64, s = orc.gemm_f64acc(A, B, want_sum=True)
    exact = _decode(A).astype(np.float64) @ _decode(B).astype(np.float64)
    np.testing.assert_allclose(s, exact, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(C64, bf16_rne_reference_f64(s).reshape(M, N))


def test_transposed_operand_is_caught(orc):
    """A non-square, non-symmetric case where A.B and A.B^T-style index mistakes differ."""
    A = _rand_bf16((6, 6), 700)
    B = _rand_bf16((6, 6), 701)
    C = orc.gemm_f64acc(A, B)
    a, b = _decode(A).astype(np.float64), _decode(B).astype(np.float64)
    assert not np.array_equal(C, bf16_rne_reference_f64(a @ b.T).reshape(6, 6))
    assert not np.array_equal(C, bf16_rne_reference_f64(b @ a).reshape(6, 6))
    np.testing.assert_array_equal(C, bf16_rne_reference_f64(a @ b).reshape(6, 6))


def _identity_bf16(n):
    return np.where(np.eye(n, dtype=bool), np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)


@pytest.mark.parametrize("M,K", [(3, 5), (17, 64), (40, 33)])
def test_identity(orc, M, K):
    A = _rand_bf16((M, K), 800 + M)
    np.testing.assert_array_equal(orc.gemm_f32acc(A, _identity_bf16(K)), A)
    np.testing.assert_array_equal(orc.gemm_f64acc(A, _identity_bf16(K)), A)
    B = _rand_bf16((M, K), 900 + K)
    np.testing.assert_array_equal(orc.gemm_f32acc(_identity_bf16(M), B), B)


def test_zero(orc):
    A = np.zeros((9, 20), dtype=np.uint16)
    B = _rand_bf16((20, 11), 1000)
    C = orc.gemm_f32acc(A, B)
    assert np.all(_decode(C) == 0.0)
    C = orc.gemm_f64acc(A, B)
    assert np.all(_decode(C) == 0.0)


@pytest.mark.parametrize("M,N,K", [(8, 9, 300), (31, 17, 4096)])
def test_integer_exact(orc, M, N, K):
    """Entries in {-2..2}: every partial sum is an integer of magnitude <= 4K < 2^24, so fp32
    accumulation is exact in any order, and the bf16 result is the unique rounding of the exact
    integer (computed here with int64 matmul and rounded with torch's own bf16 cast)."""
    import torch

    A = wl.gen_small_int_bf16((M, K), 1100 + K)
    B = wl.gen_small_int_bf16((K, N), 1200 + K)
    ai = _decode(A).astype(np.int64)
    bi = _decode(B).astype(np.int64)
    exact = ai @ bi
    want = torch.from_numpy(exact.astype(np.float64)).to(torch.bfloat16).view(torch.int16)
    want = want.numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.gemm_f32acc(A, B), want)
    np.testing.assert_array_equal(orc.gemm_f64acc(A, B), want)


def test_row_ranges_and_elements_agree(orc):
    A = _rand_bf16((23, 40), 1300)
    B = _rand_bf16((40, 19), 1301)
    full32 = orc.gemm_f32acc(A, B)
    full64 = orc.gemm_f64acc(A, B)
    np.testing.assert_array_equal(orc.gemm_f32acc(A, B, rows=(5, 17)), full32[5:17])
    rows, cols = wl.sample_indices(23, 19, 50, seed=7, full_rows=(3,), full_cols=(18,))
    c32, c64, s64 = orc.gemm_elems(A, B, rows, cols)
    np.testing.assert_array_equal(c32, full32[rows, cols])
    np.testing.assert_array_equal(c64, full64[rows, cols])
    with pytest.raises(IndexError):
        orc.gemm_elems(A, B, [23], [0])


def test_fp32_and_fp64_references_close(orc):
    """The two accumulation orders differ by at most one bf16 rounding step on these inputs."""
    A = _rand_bf16((32, 512), 1400)
    B = _rand_bf16((512, 48), 1401, 0.02)
    rep = orc.gemm_compare(orc.gemm_f64acc(A, B), orc.gemm_f32acc(A, B), 1e-2)
    assert rep["n_violations"] == 0 and rep["frob_rel"] < 1e-3


def test_epilogue_sweep_construction_is_exact(orc):
    """The epilogue sweep's operands: the exact (fp64) sum of every row and column equals the
    intended fp32 pattern, so the oracle's fp32-accumulate GEMM must round it exactly as the
    independent nearest-even formulation rounds the pattern."""
    from epilogue_cases import epilogue_case

    rng = np.random.Generator(np.random.PCG64(0xE9))
    idx = rng.integers(0, 1 << 24, size=2000).astype(np.uint32)
    sign, f = (idx >> 23).astype(bool), idx & 0x7FFFFF
    ts = list(range(-103, 128)) + [0]
    A, B, pattern = epilogue_case(sign, f, ts)
    exact = orc.bf16_to_f32(A).astype(np.float64) @ orc.bf16_to_f32(B).astype(np.float64)
    np.testing.assert_array_equal(exact, pattern.view(np.float32).astype(np.float64))
    want = bf16_rne_reference_f32_bits(pattern.reshape(-1)).reshape(pattern.shape)
    np.testing.assert_array_equal(orc.gemm_f32acc(A, B), want)
    assert np.any((want & 0x7FFF) == 0x7F80)        # the top exponent's round-ups overflow
