"""GPU parity of c3_gemm (bf16 MFMA kernels) against the CPU oracle, through the C ABI.

Bar: elementwise |got - ref| <= 1e-2 * max(1, |ref|) and relative Frobenius error <= 1e-3 against
both the fp64-accumulate definition and the fp32-accumulate triple loop; bit-exact where every
partial sum is an exact integer (entries in {-2..2}); bit-exact identity; exact zero;
deterministic (same bits on every run and under any CU mask)."""
import numpy as np
import pytest

import oracle
from concurrent_gemm_dma_amd import workloads as wl
from epilogue_cases import epilogue_case
from gpu_util import bf16_from_dev, empty_bf16, to_dev

pytestmark = pytest.mark.gpu

# (M, N, K): several 256x256 tiles with ragged tails (with fewer tiles than CUs, K is split too),
# skinny shapes (M <= 64) with ragged N and K, and single-element edges.
SHAPES = [
    (1, 8, 8), (3, 24, 40), (16, 264, 136), (17, 520, 328), (33, 1000, 64), (64, 256, 512),
    (64, 8, 2048), (65, 256, 64), (300, 264, 72), (256, 256, 64), (512, 512, 512),
    (600, 520, 328), (1024, 776, 1040), (257, 257 + 7, 8),
]


def run_gemm(c3, A, B, stream=None):
    M, K = A.shape
    N = B.shape[1]
    dA, dB = to_dev(A), to_dev(B)
    dC = empty_bf16((M, N))
    c3.c3_gemm(dA, dB, dC, M, N, K, stream)
    import torch

    torch.cuda.synchronize()
    return bf16_from_dev(dC)


def check_tol(ref, got):
    rep = oracle.gemm_compare(ref, got)
    assert oracle.gemm_within_tolerance(rep), rep
    return rep


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_random_normal(c3gpu, M, N, K):
    A = wl.gen_bf16((M, K), ("normal", 0.0, 1.0), 7000 + M)
    B = wl.gen_bf16((K, N), ("normal", 0.0, 0.02), 7100 + N + K)
    got = run_gemm(c3gpu, A, B)
    rep = check_tol(oracle.gemm_f64acc(A, B), got)
    check_tol(oracle.gemm_f32acc(A, B), got)
    # bf16 against bf16: only sums that straddle a rounding boundary may differ, far under 1%
    assert rep["n_diff"] <= max(2, rep["n"] // 100), rep


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (17, 520, 328), (600, 520, 328)])
def test_gemm_uniform(c3gpu, M, N, K):
    A = wl.gen_bf16((M, K), ("uniform", -1.0, 1.0), 7200 + M)
    B = wl.gen_bf16((K, N), ("uniform", -1.0, 1.0), 7300 + N)
    check_tol(oracle.gemm_f64acc(A, B), run_gemm(c3gpu, A, B))


@pytest.mark.parametrize("M,N,K", [(16, 520, 4096), (300, 264, 2048), (600, 520, 328), (64, 1024, 8192)])
def test_gemm_integer_exact(c3gpu, M, N, K):
    A = wl.gen_small_int_bf16((M, K), 7400 + K)
    B = wl.gen_small_int_bf16((K, N), 7500 + N)
    got = run_gemm(c3gpu, A, B)
    np.testing.assert_array_equal(got, oracle.gemm_f32acc(A, B))


@pytest.mark.parametrize("M,K", [(300, 264), (40, 520)])
def test_gemm_identity(c3gpu, M, K):
    A = wl.gen_bf16((M, K), ("normal", 0.0, 1.0), 7600 + M)
    eye = np.where(np.eye(K, dtype=bool), np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)
    np.testing.assert_array_equal(run_gemm(c3gpu, A, eye), A)
    B = wl.gen_bf16((M, K), ("normal", 0.0, 1.0), 7700 + K)
    eyeM = np.where(np.eye(M, dtype=bool), np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)
    if M % 8 == 0:
        np.testing.assert_array_equal(run_gemm(c3gpu, eyeM, B), B)


def test_gemm_zero(c3gpu):
    A = np.zeros((300, 136), dtype=np.uint16)
    B = wl.gen_bf16((136, 264), ("normal", 0.0, 1.0), 7800)
    got = run_gemm(c3gpu, A, B)
    assert np.all(oracle.bf16_to_f32(got) == 0.0)


@pytest.mark.parametrize("rows,ts", [
    # every sign and mantissa at the lowest covered, the unit and the highest exponent (where
    # the largest mantissas round up to infinity)
    ("all", (-103, -1, 0, 1, 64, 126, 127, 100)),
    # a mantissa sample (every rounding case: round bits 0x0000-0xFFFF below 7 kept bits) at every
    # covered exponent
    ("sample", tuple(range(-103, 128)) + (0,)),
    # the skinny kernel's epilogue (M <= 64)
    ("skinny", tuple(range(-103, 128)) + (0,)),
])
def test_gemm_epilogue_rounding_sweep(c3gpu, rows, ts):
    """The epilogue's fp32 -> bf16 conversion over every fp32 pattern with exponent field
    24..254 (all 2^24 sign x mantissa patterns at eight exponents, a 2^16 sample at all 231),
    bit-exact against the oracle's nearest-even converter. Exponents below 24, subnormals and
    non-finite sums are outside what exact bf16 products can build here."""
    if rows == "all":
        idx = np.arange(1 << 24, dtype=np.uint32)
        sign, f = (idx >> 23).astype(bool), idx & 0x7FFFFF
    elif rows == "sample":
        # every value of the 16 bits rounding drops, with kept bits and sign varied
        low = np.arange(1 << 16, dtype=np.uint32)
        kept = (low * 2654435761 >> 9) & 0x7F
        f = (kept << 16) | low
        sign = (low & 1).astype(bool)
    else:
        low = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000] * 8, np.uint32)
        kept = np.repeat(np.array([0, 1, 0x7E, 0x7F, 2, 3, 0x40, 0x41], np.uint32), 8)
        f = (kept << 16) | low
        sign = (np.arange(64) % 3 == 0)
    block = 1 << 21                                   # the largest M one call takes
    for r0 in range(0, f.size, block):
        A, B, pattern = epilogue_case(sign[r0:r0 + block], f[r0:r0 + block], list(ts))
        print(f"epilogue sweep {rows}: rows {r0}.. M={A.shape[0]} N={B.shape[1]} K=8", flush=True)
        got = run_gemm(c3gpu, A, B).reshape(-1)
        want = oracle.bf16_from_f32_bits(pattern.reshape(-1))
        pattern = pattern.reshape(-1)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (f"{bad.size} mismatches, first at pattern {int(pattern[bad[0]]):#010x}: "
                               f"got {int(got[bad[0]]):#06x}, want {int(want[bad[0]]):#06x}")


def test_gemm_deterministic_and_mask_invariant(c3gpu):
    import torch

    M, N, K = 1024, 776, 1040
    A = wl.gen_bf16((M, K), ("normal", 0.0, 1.0), 7900)
    B = wl.gen_bf16((K, N), ("normal", 0.0, 0.02), 7901)
    first = run_gemm(c3gpu, A, B)
    np.testing.assert_array_equal(first, run_gemm(c3gpu, A, B))
    for keep in (28, 24, 1):
        mask = c3gpu.c3_cu_mask_balanced(keep)
        s = c3gpu.c3_stream_create(mask)
        try:
            np.testing.assert_array_equal(first, run_gemm(c3gpu, A, B, stream=s))
        finally:
            torch.cuda.synchronize()
            c3gpu.c3_stream_destroy(s)
    # the 128x128 tile kernel (the model's choice for this shape) and the skinny path too
    A3 = wl.gen_bf16((1000, 1000), ("normal", 0.0, 1.0), 7904)
    B3 = wl.gen_bf16((1000, 2000), ("normal", 0.0, 0.02), 7905)
    first3 = run_gemm(c3gpu, A3, B3)
    mask = c3gpu.c3_cu_mask_balanced(24)
    s = c3gpu.c3_stream_create(mask)
    try:
        np.testing.assert_array_equal(first3, run_gemm(c3gpu, A3, B3, stream=s))
    finally:
        torch.cuda.synchronize()
        c3gpu.c3_stream_destroy(s)
    A2 = wl.gen_bf16((16, 8192), ("normal", 0.0, 1.0), 7902)
    B2 = wl.gen_bf16((8192, 1032), ("normal", 0.0, 0.02), 7903)
    np.testing.assert_array_equal(run_gemm(c3gpu, A2, B2), run_gemm(c3gpu, A2, B2))


@pytest.mark.parametrize("M,N,K", [(256, 1024, 4096), (300, 520, 1040), (512, 768, 4096),
                                   (200, 264, 1000)])
def test_gemm_split_k(c3gpu, M, N, K, monkeypatch):
    """Fewer 256x256 tiles than CUs: K is split over workgroups (fp32 partials summed in split
    order). Split and unsplit (C3_GEMM_SPLITS=1) results both meet the bar against the oracle,
    and the split result is the same on every run."""
    print(f"split-K GEMM {M}x{N}x{K}", flush=True)
    A = wl.gen_bf16((M, K), ("normal", 0.0, 1.0), 7950 + M)
    B = wl.gen_bf16((K, N), ("normal", 0.0, 0.02), 7951 + N)
    ref = oracle.gemm_f64acc(A, B)
    split = run_gemm(c3gpu, A, B)
    check_tol(ref, split)
    np.testing.assert_array_equal(split, run_gemm(c3gpu, A, B))
    monkeypatch.setenv("C3_GEMM_SPLITS", "1")
    check_tol(ref, run_gemm(c3gpu, A, B))
    # integer-exact operands: every partial sum is exact, so the split sum is too
    monkeypatch.delenv("C3_GEMM_SPLITS")
    Ai = wl.gen_small_int_bf16((M, K), 7960 + K)
    Bi = wl.gen_small_int_bf16((K, N), 7961 + N)
    np.testing.assert_array_equal(run_gemm(c3gpu, Ai, Bi), oracle.gemm_f32acc(Ai, Bi))


@pytest.mark.parametrize("M,N,K,splits", [
    (520, 264, 4136, 1),    # two full tile rows + a partial one; K tail of 8 after 129 full steps
    (520, 264, 4136, 2),    # splits of 2080 and 2056 k: unrolled main loop, then general steps
    (256, 520, 8200, 3),    # one tile row, ragged N, splits of 2752 / 2752 / 2696 k
    (768, 256, 1216, 1),    # exactly 38 steps: two unrolled groups of twelve, 14 general
])
def test_gemm_unrolled_loop_edges(c3gpu, M, N, K, splits, monkeypatch):
    """The tile kernel's unrolled main loop (full tiles, twelve K steps at a time while every load
    stays inside K) next to the general step (partial tiles, the last steps, ragged K), with and
    without K split: bit-exact on integer-valued operands, within the bar on normal ones."""
    print(f"unrolled-loop GEMM {M}x{N}x{K} splits={splits}", flush=True)
    monkeypatch.setenv("C3_GEMM_TILE", "256")
    monkeypatch.setenv("C3_GEMM_SPLITS", str(splits))
    Ai = wl.gen_small_int_bf16((M, K), 8010 + K)
    Bi = wl.gen_small_int_bf16((K, N), 8011 + N)
    np.testing.assert_array_equal(run_gemm(c3gpu, Ai, Bi), oracle.gemm_f32acc(Ai, Bi))
    A = wl.gen_bf16((M, K), ("normal", 0.0, 1.0), 8020 + M)
    B = wl.gen_bf16((K, N), ("normal", 0.0, 0.02), 8021 + N)
    check_tol(oracle.gemm_f64acc(A, B), run_gemm(c3gpu, A, B))


@pytest.mark.parametrize("K", [32 * s for s in range(4, 30)] + [32 * s + 8 for s in (17, 18, 23, 29)]
                         + [32 * s + 24 for s in (18, 25)])
def test_gemm_fast_steps_past_the_last_group(c3gpu, K, monkeypatch):
    """Past the last whole group of twelve unrolled K steps the fast steps go on while every load
    a step issues lies inside K, then the general step takes over: every remainder after one
    group (6..17 steps), K with no whole group at all, odd and even step counts (the last A slab
    half or wholly used) and ragged K (a partial last step). Rows past M go through the fast
    steps too. Bit-exact on integer-valued operands."""
    M, N = 264, 256
    print(f"fast-tail GEMM {M}x{N}x{K}", flush=True)
    monkeypatch.setenv("C3_GEMM_TILE", "256")
    monkeypatch.setenv("C3_GEMM_SPLITS", "1")
    Ai = wl.gen_small_int_bf16((M, K), 8200 + K)
    Bi = wl.gen_small_int_bf16((K, N), 8201 + K)
    np.testing.assert_array_equal(run_gemm(c3gpu, Ai, Bi), oracle.gemm_f32acc(Ai, Bi))


@pytest.mark.parametrize("M,N,K,tile,splits", [
    (300, 520, 1000, "256", "1"),   # 256 tile: partial tile rows and columns, K tail of 8
    (520, 264, 4136, "256", "2"),   # 256 tile, K split: each split's own tail
    (300, 520, 1000, "128", "0"),   # 128 tile
    (40, 520, 1000, "0", "0"),      # skinny
])
def test_gemm_reads_and_writes_only_its_operands(c3gpu, M, N, K, tile, splits, monkeypatch):
    """Every operand is followed in memory by NaN (A, B) or a sentinel (C), with room for any
    over-read or over-write a missing mask could make (a tile of rows past M, a K step past K):
    C must still equal the exact result, which any NaN read into a sum would break, and the
    sentinel after C must be untouched."""
    import torch

    print(f"operand-bounds GEMM {M}x{N}x{K} tile={tile} splits={splits}", flush=True)
    monkeypatch.setenv("C3_GEMM_TILE", tile)
    monkeypatch.setenv("C3_GEMM_SPLITS", splits)
    A = wl.gen_small_int_bf16((M, K), 8100 + K)
    B = wl.gen_small_int_bf16((K, N), 8101 + N)
    nan = np.uint16(0x7FC0)
    dA = to_dev(np.concatenate([A.reshape(-1), np.full(256 * K + 64, nan, np.uint16)]))
    dB = to_dev(np.concatenate([B.reshape(-1), np.full(32 * N + 64, nan, np.uint16)]))
    dC = empty_bf16((M * N + 256 * N,), fill=0x1234)
    c3gpu.c3_gemm(dA, dB, dC, M, N, K, None)
    torch.cuda.synchronize()
    out = bf16_from_dev(dC)
    np.testing.assert_array_equal(out[:M * N].reshape(M, N), oracle.gemm_f32acc(A, B))
    assert np.all(out[M * N:] == 0x1234)


@pytest.mark.parametrize("M,N,K", [(128, 128, 32), (300, 264, 72), (1000, 2000, 1000),
                                   (65, 520, 328), (1024, 776, 1040), (129, 8, 8)])
def test_gemm_tile128(c3gpu, M, N, K, monkeypatch):
    """The 128x128 tile kernel (chosen by the cost model for mid-size shapes; forced here with
    C3_GEMM_TILE=128): oracle tolerance on normal operands, bit-exact on integer-valued ones,
    same bits on every run."""
    print(f"tile-128 GEMM {M}x{N}x{K}", flush=True)
    monkeypatch.setenv("C3_GEMM_TILE", "128")
    A = wl.gen_bf16((M, K), ("normal", 0.0, 1.0), 7970 + M)
    B = wl.gen_bf16((K, N), ("normal", 0.0, 0.02), 7971 + N)
    got = run_gemm(c3gpu, A, B)
    check_tol(oracle.gemm_f64acc(A, B), got)
    np.testing.assert_array_equal(got, run_gemm(c3gpu, A, B))
    Ai = wl.gen_small_int_bf16((M, K), 7980 + K)
    Bi = wl.gen_small_int_bf16((K, N), 7981 + N)
    np.testing.assert_array_equal(run_gemm(c3gpu, Ai, Bi), oracle.gemm_f32acc(Ai, Bi))


def test_gemm_argument_errors(c3gpu):
    import torch

    dA = torch.zeros((64, 64), dtype=torch.int16, device="cuda:0")
    dB = torch.zeros((64, 64), dtype=torch.int16, device="cuda:0")
    dC = torch.zeros((64, 64), dtype=torch.int16, device="cuda:0")
    call = c3gpu.call
    ptr = lambda t: t.data_ptr()
    assert call("c3_gemm", ptr(dA), ptr(dB), ptr(dC), 64, 64, 60, None) == c3gpu.C3_E_INVALID  # K%8
    assert call("c3_gemm", ptr(dA), ptr(dB), ptr(dC), 64, 60, 64, None) == c3gpu.C3_E_INVALID  # N%8
    assert call("c3_gemm", ptr(dA) + 2, ptr(dB), ptr(dC), 64, 64, 64, None) == c3gpu.C3_E_INVALID
    assert call("c3_gemm", None, ptr(dB), ptr(dC), 64, 64, 64, None) == c3gpu.C3_E_INVALID
    assert call("c3_gemm", ptr(dA), ptr(dB), ptr(dC), 0, 64, 64, None) == c3gpu.C3_E_INVALID
    assert call("c3_gemm", ptr(dA), ptr(dB), ptr(dA), 64, 64, 64, None) == c3gpu.C3_E_OVERLAP
    host = np.zeros(64 * 64, dtype=np.uint16)
    assert call("c3_gemm", host.ctypes.data, ptr(dB), ptr(dC), 64, 64, 64,
                None) == c3gpu.C3_E_INVALID
    assert call("c3_gemm", ptr(dA) + (1 << 40), ptr(dB), ptr(dC), 64, 64, 64,
                None) == c3gpu.C3_E_INVALID
    torch.cuda.synchronize()
