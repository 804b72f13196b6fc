"""GPU parity of the reduce-scatter kernel and the all-reduce local share (reduce-scatter on the
CUs, then the all-gather by either mover) through the C ABI: bit-exact against the oracle on
seeded bf16 inputs, for 1..64 ranks, ragged element counts (vector body + per-element tail),
misaligned pointers, empty chunks, and argument errors."""
import ctypes

import numpy as np
import pytest

import oracle
from concurrent_gemm_dma_amd import workloads as wl
from gpu_util import bf16_from_dev, bytes_from_dev, empty_bf16, empty_bytes, to_dev

pytestmark = pytest.mark.gpu
MiB = 1 << 20


def sync():
    import torch

    torch.cuda.synchronize()


def contributions(world, n, seed, dist=("normal", 0.0, 1.0)):
    return [wl.gen_bf16((n,), dist, seed + r) for r in range(world)]


@pytest.mark.parametrize("world,n", [(1, 4097), (2, 8), (3, 1), (8, 7), (8, 4096 * 33 + 5),
                                     (16, 100003), (64, 2053)])
def test_reduce_scatter_parity(c3gpu, world, n):
    cs = contributions(world, n, 10000 + 97 * world)
    d = [to_dev(c) for c in cs]
    out = empty_bf16((n + 8,))
    c3gpu.c3_reduce_scatter(out, d, 2 * n)
    sync()
    got = bf16_from_dev(out)
    want = oracle.reduce_sum_bf16(cs)
    np.testing.assert_array_equal(got[:n], want)
    assert np.all(got[n:] == 0xFFFF)  # nothing written past the chunk


def test_reduce_scatter_integer_exact_and_cancellation(c3gpu):
    # integer-valued inputs: every partial sum is exact, so the result is the integer sum
    rng = np.random.default_rng(7)
    ints = rng.integers(-16, 17, size=(8, 20001))
    cs = [((ints[r].astype(np.float32).view(np.uint32)) >> np.uint32(16)).astype(np.uint16)
          for r in range(8)]
    out = empty_bf16((20001,))
    c3gpu.c3_reduce_scatter(out, [to_dev(c) for c in cs], 2 * 20001)
    sync()
    want = (ints.sum(axis=0).astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    np.testing.assert_array_equal(bf16_from_dev(out), want)
    # rank order, single rounding and signed zero (the oracle's hand-worked cases), 8 lanes each
    cases = [([0x3F80, 0x4B80, 0xCB80], 0x0000), ([0x3F80, 0x3B80, 0x3B80], 0x3F81),
             ([0x8000, 0x8000, 0x8000], 0x8000)]
    for vals, want_bits in cases:
        cs = [np.full(16, v, np.uint16) for v in vals]
        out = empty_bf16((16,))
        c3gpu.c3_reduce_scatter(out, [to_dev(c) for c in cs], 32)
        sync()
        assert np.all(bf16_from_dev(out) == want_bits), (vals, bf16_from_dev(out))


def test_reduce_scatter_misaligned(c3gpu):
    import torch

    world, n = 4, 5000
    cs = contributions(world, n, 10500)
    # contributions at odd element offsets (2-byte aligned, not 16): the per-element path
    bases = [to_dev(np.concatenate([np.zeros(r + 1, np.uint16), c])) for r, c in enumerate(cs)]
    ptrs = [b.data_ptr() + 2 * (r + 1) for r, b in enumerate(bases)]
    out = torch.full((n + 3,), -1, dtype=torch.int16, device="cuda:0")
    c3gpu.c3_reduce_scatter(out.data_ptr() + 2, ptrs, 2 * n)
    sync()
    got = bf16_from_dev(out)
    np.testing.assert_array_equal(got[1:n + 1], oracle.reduce_sum_bf16(cs))
    assert got[0] == 0xFFFF and np.all(got[n + 1:] == 0xFFFF)


def test_reduce_scatter_empty_and_errors(c3gpu):
    cs = contributions(2, 64, 10600)
    d = [to_dev(c) for c in cs]
    out = empty_bf16((64,))
    c3gpu.c3_reduce_scatter(out, d, 0)  # no-op
    sync()
    assert np.all(bf16_from_dev(out) == 0xFFFF)
    call = c3gpu.call
    P = lambda xs: (ctypes.c_void_p * len(xs))(*[x.data_ptr() for x in xs])  # noqa: E731
    assert call("c3_reduce_scatter", out.data_ptr(), P(d), 2, 127, None, None) == c3gpu.C3_E_INVALID
    assert call("c3_reduce_scatter", out.data_ptr(), P(d), 0, 128, None, None) == c3gpu.C3_E_INVALID
    assert call("c3_reduce_scatter", out.data_ptr(), P(d * 33), 66, 128, None,
                None) == c3gpu.C3_E_INVALID
    assert call("c3_reduce_scatter", d[1].data_ptr(), P(d), 2, 128, None,
                None) == c3gpu.C3_E_OVERLAP
    assert call("c3_reduce_scatter", out.data_ptr() + (1 << 40), P(d), 2, 128, None,
                None) == c3gpu.C3_E_INVALID  # not device memory
    sync()


def run_allreduce(c3, world, rank, chunk_bytes, mover, seed, opts=None):
    n = chunk_bytes // 2
    cs = contributions(world, n, seed)
    peers = [None if i == rank else wl.gen_bf16((n,), ("normal", 0.0, 1.0), seed + 500 + i)
             for i in range(world)]
    dc = [to_dev(c) for c in cs]
    dp = [None if p is None else to_dev(p) for p in peers]
    reduced = empty_bytes(chunk_bytes + 1)
    dst = empty_bytes(world * chunk_bytes + 1)
    c3.c3_allreduce_local(dst, reduced, dc, dp, rank, chunk_bytes, mover, opts)
    sync()
    want_red, want = oracle.allreduce_local(cs, peers, rank)
    got_red, got = bytes_from_dev(reduced), bytes_from_dev(dst)
    assert oracle.first_diff(want_red.view(np.uint8), got_red[:chunk_bytes]) == -1
    assert oracle.first_diff(want.view(np.uint8), got[:world * chunk_bytes]) == -1
    assert got_red[-1] == 0xA5 and got[-1] == 0xA5


@pytest.mark.parametrize("mover", ["cu", "sdma"])
@pytest.mark.parametrize("world,rank,chunk_bytes", [(8, 0, MiB), (8, 5, MiB + 6), (1, 0, 4096),
                                                    (3, 2, 2), (16, 15, 64 * 1024)])
def test_allreduce_local(c3gpu, mover, world, rank, chunk_bytes):
    m = c3gpu.C3_MOVER_CU if mover == "cu" else c3gpu.C3_MOVER_SDMA
    run_allreduce(c3gpu, world, rank, chunk_bytes, m, 11000 + world * 31 + rank)


def test_allreduce_sdma_chunked(c3gpu):
    run_allreduce(c3gpu, 8, 3, 4 * MiB, c3gpu.C3_MOVER_SDMA, 11500,
                  c3gpu.move_opts(chunk_bytes=256 * 1024))


@pytest.mark.parametrize("mover", ["cu", "sdma"])
def test_allreduce_errors(c3gpu, mover):
    m = c3gpu.C3_MOVER_CU if mover == "cu" else c3gpu.C3_MOVER_SDMA
    n = 256
    cs = [to_dev(c) for c in contributions(2, n, 11600)]
    peer = to_dev(wl.gen_bf16((n,), ("normal", 0.0, 1.0), 11610))
    reduced = empty_bytes(2 * n)
    dst = empty_bytes(4 * n)
    call = c3gpu.call
    P = lambda xs: (ctypes.c_void_p * len(xs))(*[None if x is None else x.data_ptr() for x in xs])  # noqa: E731
    args = lambda d, r, c, p, rank, nb: (d.data_ptr(), r.data_ptr(), P(c), P(p), len(c), rank, nb, m,  # noqa: E731
                                         None, None)
    assert call("c3_allreduce_local", *args(dst, reduced, cs, [None, peer], 0, 2 * n)) == c3gpu.C3_OK
    sync()
    # rank out of range, odd chunk, NULL peer for another rank, reduced inside dst, peer = dst
    assert call("c3_allreduce_local", *args(dst, reduced, cs, [None, peer], 2, 2 * n)) == c3gpu.C3_E_INVALID
    assert call("c3_allreduce_local", *args(dst, reduced, cs, [None, peer], 0, 2 * n - 1)) == c3gpu.C3_E_INVALID
    assert call("c3_allreduce_local", *args(dst, reduced, cs, [None, None], 0, 2 * n)) == c3gpu.C3_E_INVALID
    assert call("c3_allreduce_local", *args(dst, dst, cs, [None, peer], 0, 2 * n)) == c3gpu.C3_E_OVERLAP
    assert call("c3_allreduce_local", *args(dst, reduced, cs, [None, dst], 0, 2 * n)) == c3gpu.C3_E_OVERLAP
    assert call("c3_allreduce_local", *args(dst, reduced, [cs[0], reduced], [None, peer], 0,
                                            2 * n)) == c3gpu.C3_E_OVERLAP
    sync()
