"""c3_gemm_noalloc (the GEMM entry point that allocates nothing, for callers that cannot
allocate) against c3_gemm, through the C ABI.

Both entry points take the same plan and kernels; the only difference is where a K split keeps
its fp32 partials (a fixed device array instead of a per-stream workspace), so C must be
bit-identical to c3_gemm's and within the GEMM tolerance of the oracle
(|d| <= 1e-2 max(1,|ref|) elementwise, relative Frobenius <= 1e-3, against both the fp64- and
the fp32-accumulate definitions). Each case makes two calls in a row on the shared array, the
second on a smaller shape, so partials a first call leaves behind must not leak into the second.
"""
import numpy as np
import pytest

import oracle
from concurrent_gemm_dma_amd import workloads as wl
from gpu_util import bf16_from_dev, empty_bf16, to_dev

pytestmark = pytest.mark.gpu


def sync():
    import torch

    torch.cuda.synchronize()


def operands(M, N, K, seed):
    A = wl.gen_bf16((M, K), ("normal", 0.0, 1.0), seed)
    B = wl.gen_bf16((K, N), ("normal", 0.0, 0.02), seed + 1)
    return A, B


def both(c3, A, B, stream=None):
    """C from c3_gemm_noalloc, then C from c3_gemm, on the same device operands."""
    M, K = A.shape
    N = B.shape[1]
    dA, dB = to_dev(A), to_dev(B)
    dC1, dC2 = empty_bf16((M, N), -1), empty_bf16((M, N), -2)
    sync()
    c3.c3_gemm_noalloc(dA, dB, dC1, M, N, K, stream)
    sync()
    got = bf16_from_dev(dC1)
    c3.c3_gemm(dA, dB, dC2, M, N, K, stream)
    sync()
    return got, bf16_from_dev(dC2)


def check_vs_oracle(A, B, got, full=True):
    if full:
        refs = (oracle.gemm_f64acc(A, B), oracle.gemm_f32acc(A, B))
        vals = got
    else:
        rows, cols = wl.sample_indices(A.shape[0], B.shape[1], 2048, seed=11,
                                       full_rows=(A.shape[0] - 1,), full_cols=(B.shape[1] - 1,))
        c32, c64, _ = oracle.gemm_elems(A, B, rows, cols)
        refs, vals = (c64, c32), got[rows, cols]
    for ref in refs:
        rep = oracle.gemm_compare(ref, vals)
        assert oracle.gemm_within_tolerance(rep), rep


# (first call, second smaller call): K split by the skinny kernel (M <= 64) and by the 256x256
# tile kernel with fewer tiles than CUs, ragged M and N
PAIRS = [
    ((16, 28672, 8192), (16, 1024, 2048)),   # 4 splits (7 MiB of partials), then 8 (0.5 MiB)
    ((32, 4096, 4096), (17, 520, 328)),      # 16 splits (8 MiB), then a ragged skinny shape
    ((384, 520, 4096), (200, 264, 2048)),    # tile kernel, 16 splits (12 MiB), then 16 (3 MiB)
    ((200, 264, 16384), (96, 136, 4096)),    # tile kernel, 57 splits (11 MiB), then 32 (1.6 MiB)
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_two_calls_match_c3_gemm(c3gpu, first, second):
    for i, (M, N, K) in enumerate((first, second)):
        print(f"c3_gemm_noalloc call {i + 1}: {M}x{N}x{K}", flush=True)
        A, B = operands(M, N, K, 9100 + 17 * i + M)
        got, want = both(c3gpu, A, B)
        np.testing.assert_array_equal(got, want, err_msg=f"call {i + 1} {M}x{N}x{K}")
        check_vs_oracle(A, B, got, full=M * N * K <= (1 << 27))


def test_noalloc_unsplit_shape_and_own_stream(c3gpu):
    """A shape with as many tiles as CUs uses no scratch; a library stream works too."""
    import torch

    s = c3gpu.c3_stream_create()
    try:
        for M, N, K in ((4096, 4096, 256), (512, 512, 512)):
            A, B = operands(M, N, K, 9300 + M)
            got, want = both(c3gpu, A, B, s)
            np.testing.assert_array_equal(got, want)
            check_vs_oracle(A, B, got, full=M * N * K <= (1 << 27))
    finally:
        torch.cuda.synchronize()
        c3gpu.c3_stream_destroy(s)


def test_noalloc_refuses_partials_above_the_scratch(c3gpu):
    """64x28672x8192 splits K 4 ways: 28 MiB of partials, above the 16 MiB array. Refused
    before any launch (C untouched); c3_gemm still runs it."""
    M, N, K = 64, 28672, 8192
    A, B = operands(M, N, K, 9400)
    dA, dB = to_dev(A), to_dev(B)
    dC = empty_bf16((M, N), -3)
    sync()
    with pytest.raises(c3gpu.C3Error) as e:
        c3gpu.c3_gemm_noalloc(dA, dB, dC, M, N, K)
    assert e.value.status == c3gpu.C3_E_INVALID
    assert "scratch" in str(e.value)
    sync()
    assert (bf16_from_dev(dC) == np.uint16(0xFFFD)).all()
    c3gpu.c3_gemm(dA, dB, dC, M, N, K)
    sync()
    check_vs_oracle(A, B, bf16_from_dev(dC), full=False)


def test_noalloc_allocates_no_device_memory(c3gpu):
    """Free device memory is the same before and after a split-K c3_gemm_noalloc call (after a
    warm-up call on the same stream), while c3_gemm's first split-K call on that stream
    allocates its workspace there."""
    import torch

    M, N, K = 384, 520, 4096                 # 16 splits: 12.2 MiB of partials
    A, B = operands(M, N, K, 9500)
    dA, dB = to_dev(A), to_dev(B)
    dC = empty_bf16((M, N))
    s = c3gpu.c3_stream_create()
    try:
        c3gpu.c3_gemm_noalloc(dA, dB, dC, M, N, K, s)   # warm-up: kernels loaded, queue in use
        sync()
        free0 = torch.cuda.mem_get_info()[0]
        c3gpu.c3_gemm_noalloc(dA, dB, dC, M, N, K, s)
        sync()
        free1 = torch.cuda.mem_get_info()[0]
        assert free1 == free0, (free0, free1)
        got = bf16_from_dev(dC)
        c3gpu.c3_gemm(dA, dB, dC, M, N, K, s)          # first split-K c3_gemm on s: allocates
        sync()
        free2 = torch.cuda.mem_get_info()[0]
        assert free0 - free2 >= 16 * M * N * 4, (free0, free2)
        np.testing.assert_array_equal(got, bf16_from_dev(dC))
    finally:
        sync()
        c3gpu.c3_stream_destroy(s)
