"""GPU parity of the two movers (CU kernel, SDMA engines) for the collective-shaped copies, through
the C ABI: byte-exact against the oracle's memcpy definitions, including ragged sizes, misaligned
pointers, empty and single-element cases, chunked SDMA transfers, and the host-forced fault
hooks (dropped, stuck and failed transfers), which must be caught."""
import numpy as np
import pytest

import oracle
from concurrent_gemm_dma_amd import workloads as wl
from gpu_util import bytes_from_dev, empty_bytes, to_dev

pytestmark = pytest.mark.gpu

MOVERS = ["cu", "sdma"]
KiB = 1 << 10
MiB = 1 << 20


def mover_id(c3, name):
    return {"cu": c3.C3_MOVER_CU, "sdma": c3.C3_MOVER_SDMA, "hybrid": c3.C3_MOVER_HYBRID}[name]


def sync():
    import torch

    torch.cuda.synchronize()


def do_gather(c3, shards_np, mover, opts=None, dst_offset=0, src_offset=0):
    import torch

    sb = shards_np[0].size if shards_np else 0
    n = len(shards_np)
    bases = [to_dev(np.concatenate([np.zeros(src_offset, np.uint8), s])) for s in shards_np]
    shards = [b.data_ptr() + src_offset for b in bases]
    dst_base = empty_bytes(n * sb + dst_offset + 1)
    c3.c3_gather(dst_base.data_ptr() + dst_offset, shards, sb, mover_id(c3, mover), opts)
    sync()
    out = bytes_from_dev(dst_base)
    return out[dst_offset:dst_offset + n * sb], out


@pytest.mark.parametrize("mover", MOVERS)
@pytest.mark.parametrize("n,sb", [(8, MiB), (8, MiB + 5), (1, 1), (3, 16), (8, 4 * KiB + 1), (2, 3)])
def test_gather(c3gpu, mover, n, sb):
    shards = [wl.gen_bytes(sb, 8000 + i + 16 * n) for i in range(n)]
    got, whole = do_gather(c3gpu, shards, mover)
    assert oracle.first_diff(oracle.gather(shards), got) == -1
    assert whole[-1] == 0xA5  # nothing written past the end


@pytest.mark.parametrize("mover,kw", [("cu", {}), ("sdma", {}), ("sdma", {"chunk_bytes": 40 * KiB}),
                                       ("hybrid", {"sdma_permille": 500}),
                                       ("hybrid", {"sdma_permille": 137, "chunk_bytes": 64 * KiB})])
@pytest.mark.parametrize("n,sb", [(8, 2 * MiB + 8), (5, 24 * KiB)])
def test_gather_tagged(c3gpu, mover, kw, n, sb):
    """The diagnostic pattern: each 8-byte word carries its shard and its destination offset, so
    a misplaced, swapped or missing word is reported by name."""
    print(f"tagged gather mover={mover} opts={kw} n={n} shard={sb}", flush=True)
    shards = wl.gen_tagged_shards(n, sb)
    got, whole = do_gather(c3gpu, shards, mover, c3gpu.move_opts(**kw) if kw else None)
    assert oracle.explain_tagged_gather(got, n, sb) == []
    assert oracle.first_diff(oracle.gather(shards), got) == -1
    assert whole[-1] == 0xA5


@pytest.mark.parametrize("mover", MOVERS)
def test_gather_misaligned(c3gpu, mover):
    shards = [wl.gen_bytes(64 * KiB + 3, 8100 + i) for i in range(8)]
    got, _ = do_gather(c3gpu, shards, mover, dst_offset=1, src_offset=3)
    assert oracle.first_diff(oracle.gather(shards), got) == -1


@pytest.mark.parametrize("mover", MOVERS)
def test_gather_empty(c3gpu, mover):
    dst = empty_bytes(16)
    c3gpu.c3_gather(dst, [], 0, mover_id(c3gpu, mover))
    s = to_dev(wl.gen_bytes(16, 1))
    c3gpu.c3_gather(dst, [s, s], 0, mover_id(c3gpu, mover))
    sync()
    assert np.all(bytes_from_dev(dst) == 0xA5)


@pytest.mark.parametrize("mover", MOVERS)
@pytest.mark.parametrize("grid,bb", [(8, 64 * KiB), (8, MiB), (3, 1000), (1, 4096), (2, 17)])
def test_all2all(c3gpu, mover, grid, bb):
    src_np = wl.gen_bytes(grid * grid * bb, 8200 + grid)
    src = to_dev(src_np)
    dst = empty_bytes(grid * grid * bb)
    c3gpu.c3_all2all_block(dst, src, grid, bb, mover_id(c3gpu, mover))
    sync()
    want = oracle.all2all_block(src_np, grid, bb)
    assert oracle.first_diff(want, bytes_from_dev(dst)) == -1
    # involution: transposing back restores the source
    back = empty_bytes(grid * grid * bb)
    c3gpu.c3_all2all_block(back, dst, grid, bb, mover_id(c3gpu, mover))
    sync()
    assert oracle.first_diff(src_np, bytes_from_dev(back)) == -1


def test_sdma_chunks_and_engines(c3gpu):
    info = c3gpu.c3_device_info()
    assert info["sdma_engine_mask"] != 0, info
    shards = [wl.gen_bytes(MiB + 48, 8300 + i) for i in range(8)]
    want = oracle.gather(shards)
    # many chunks over all engines
    got, _ = do_gather(c3gpu, shards, "sdma", c3gpu.move_opts(chunk_bytes=96 * KiB))
    assert oracle.first_diff(want, got) == -1
    # each single engine on its own
    mask = info["sdma_engine_mask"]
    for b in range(32):
        if mask & (1 << b):
            got, _ = do_gather(c3gpu, shards, "sdma", c3gpu.move_opts(engine_mask=1 << b))
            assert oracle.first_diff(want, got) == -1, f"engine bit {b}"


@pytest.mark.parametrize("n,sb", [(8, 40 * MiB + 256), (8, MiB), (8, 128 * KiB + 5), (3, 20 * MiB),
                                  (1, 1000)])
def test_sdma_default_split(c3gpu, n, sb):
    """Default split: per segment p = max(1, min(ceil(E / segments), bytes // 128 KiB),
    ceil(bytes / 16 MiB)) equal 256-byte-multiple pieces, E = engines available."""
    info = c3gpu.c3_device_info()
    engines = bin(info["sdma_engine_mask"]).count("1")
    shards_np = [wl.gen_bytes(sb, 8400 + i) for i in range(n)]
    shards = [to_dev(s) for s in shards_np]
    dst = empty_bytes(n * sb)
    cargs, _keep = c3gpu.gather_args(dst, shards, sb, c3gpu.C3_MOVER_SDMA)
    t = c3gpu.c3_run_concurrent(None, cargs)
    assert oracle.first_diff(oracle.gather(shards_np), bytes_from_dev(dst)) == -1
    p = max(1, min(-(-engines // n), sb // (128 * KiB)), -(-sb // (16 * MiB)))
    step = -(-sb // p)
    step = (step + 255) // 256 * 256
    assert t["n_chunks"] == n * -(-sb // step), (t["n_chunks"], p, step)


def test_cu_nontemporal_and_block_count(c3gpu):
    shards = [wl.gen_bytes(MiB, 8400 + i) for i in range(8)]
    want = oracle.gather(shards)
    for opts in (c3gpu.move_opts(nontemporal=1), c3gpu.move_opts(cu_blocks=7),
                 c3gpu.move_opts(cu_blocks=100000)):
        got, _ = do_gather(c3gpu, shards, "cu", opts)
        assert oracle.first_diff(want, got) == -1


def test_sdma_fault_hooks(c3gpu):
    sb = 256 * KiB
    shards = [wl.gen_bytes(sb, 8500 + i) for i in range(8)]
    want = oracle.gather(shards)
    # one chunk per shard (chunk_bytes = shard size), so chunk i is shard i
    # dropped transfer: call succeeds, the byte-exact check must catch the stale chunk 3
    got, _ = do_gather(c3gpu, shards, "sdma",
                       c3gpu.move_opts(chunk_bytes=sb, fault_mode=c3gpu.C3_FAULT_DROP_CHUNK,
                                       fault_chunk=3))
    off = oracle.first_diff(want, got)
    assert 3 * sb <= off < 4 * sb
    assert oracle.first_diff(want[4 * sb:], got[4 * sb:]) == -1
    # default split (16 transfers over 16 engines): dropping transfer 7 loses the second half
    # of shard 3
    got, _ = do_gather(c3gpu, shards, "sdma",
                       c3gpu.move_opts(fault_mode=c3gpu.C3_FAULT_DROP_CHUNK, fault_chunk=7))
    off = oracle.first_diff(want, got)
    n_eng = bin(c3gpu.c3_device_info()["sdma_engine_mask"]).count("1")
    if n_eng == 16:
        assert 3 * sb + sb // 2 <= off < 4 * sb
    else:
        assert off != -1
    # stuck transfer: timeout, after every real chunk completed
    with pytest.raises(c3gpu.C3Error) as e:
        do_gather(c3gpu, shards, "sdma", c3gpu.move_opts(chunk_bytes=sb,
                                                         fault_mode=c3gpu.C3_FAULT_STUCK_CHUNK,
                                                         fault_chunk=5, timeout_ms=300))
    assert e.value.status == c3gpu.C3_E_TIMEOUT
    # failed transfer (negative completion signal): reported as an HSA error
    with pytest.raises(c3gpu.C3Error) as e:
        do_gather(c3gpu, shards, "sdma", c3gpu.move_opts(chunk_bytes=sb,
                                                         fault_mode=c3gpu.C3_FAULT_ERROR_CHUNK,
                                                         fault_chunk=0))
    assert e.value.status == c3gpu.C3_E_HSA
    # the library is still usable afterwards
    got, _ = do_gather(c3gpu, shards, "sdma")
    assert oracle.first_diff(want, got) == -1


@pytest.mark.parametrize("mover", MOVERS)
def test_copy_argument_errors(c3gpu, mover):
    import ctypes

    m = mover_id(c3gpu, mover)
    buf = empty_bytes(8 * 4096)
    src = to_dev(wl.gen_bytes(4096, 3))
    call = c3gpu.call
    ptrs = (ctypes.c_void_p * 2)(buf.data_ptr(), src.data_ptr())
    # a shard inside dst
    assert call("c3_gather", buf.data_ptr(), ptrs, 2, 4096, m, None, None) == c3gpu.C3_E_OVERLAP
    # all2all in place
    assert call("c3_all2all_block", buf.data_ptr(), buf.data_ptr(), 2, 4096, m, None,
                None) == c3gpu.C3_E_OVERLAP
    # pointers the runtime does not know
    host = np.zeros(4096, np.uint8)
    ptrs = (ctypes.c_void_p * 1)(host.ctypes.data)
    assert call("c3_gather", buf.data_ptr(), ptrs, 1, 4096, m, None, None) == c3gpu.C3_E_INVALID
    ptrs = (ctypes.c_void_p * 1)(src.data_ptr())
    assert call("c3_gather", buf.data_ptr() + (1 << 40), ptrs, 1, 4096, m, None,
                None) == c3gpu.C3_E_INVALID
    assert call("c3_all2all_block", buf.data_ptr(), src.data_ptr(), 0, 16, m, None,
                None) == c3gpu.C3_E_INVALID
    assert call("c3_all2all_block", buf.data_ptr(), src.data_ptr(), 65, 16, m, None,
                None) == c3gpu.C3_E_INVALID
    sync()
