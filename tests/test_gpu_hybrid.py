"""GPU parity of the hybrid mover (each copy segment split between the SDMA engines and the CU
copy kernel, both running at once), through the C ABI: byte-exact against the oracle's memcpy
definitions for every collective shape, at shares from all-CU to all-engine, ragged and
misaligned sizes, isolated and beside a GEMM (C still bit-identical to its isolated run)."""
import ctypes

import numpy as np
import pytest

import oracle
from concurrent_gemm_dma_amd import workloads as wl
from gpu_util import bf16_from_dev, bytes_from_dev, empty_bytes, to_dev
from test_gpu_concurrent import Case

pytestmark = pytest.mark.gpu
KiB = 1 << 10
MiB = 1 << 20


def sync():
    import torch

    torch.cuda.synchronize()


def hybrid(c3, pm, **kw):
    return c3.move_opts(sdma_permille=pm, **kw)


def gather(c3, shards_np, opts, dst_offset=0, src_offset=0):
    sb = shards_np[0].size
    n = len(shards_np)
    bases = [to_dev(np.concatenate([np.zeros(src_offset, np.uint8), s])) for s in shards_np]
    dst_base = empty_bytes(n * sb + dst_offset + 1)
    c3.c3_gather(dst_base.data_ptr() + dst_offset, [b.data_ptr() + src_offset for b in bases], sb,
                 c3.C3_MOVER_HYBRID, opts)
    sync()
    out = bytes_from_dev(dst_base)
    return out[dst_offset:dst_offset + n * sb], out


@pytest.mark.parametrize("pm", [0, 1, 300, 500, 999, 1000])
@pytest.mark.parametrize("n,sb", [(8, MiB + 5), (8, 4 * KiB + 1), (1, 1), (3, 16), (2, 300),
                                  (8, 256)])
def test_hybrid_gather(c3gpu, pm, n, sb):
    print(f"hybrid gather n={n} shard={sb} permille={pm}", flush=True)
    shards = [wl.gen_bytes(sb, 12000 + i + 16 * n) for i in range(n)]
    got, whole = gather(c3gpu, shards, hybrid(c3gpu, pm))
    assert oracle.first_diff(oracle.gather(shards), got) == -1
    assert whole[-1] == 0xA5  # nothing written past the end


def test_hybrid_gather_misaligned_and_chunked(c3gpu):
    shards = [wl.gen_bytes(256 * KiB + 3, 12100 + i) for i in range(8)]
    got, _ = gather(c3gpu, shards, hybrid(c3gpu, 500), dst_offset=1, src_offset=3)
    assert oracle.first_diff(oracle.gather(shards), got) == -1
    info = c3gpu.c3_device_info()
    two = [1 << b for b in range(32) if info["sdma_engine_mask"] >> b & 1][:2]
    got, _ = gather(c3gpu, shards, hybrid(c3gpu, 640, chunk_bytes=40 * KiB, engine_mask=sum(two)))
    assert oracle.first_diff(oracle.gather(shards), got) == -1


@pytest.mark.parametrize("grid,bb,pm", [(8, 64 * KiB + 3, 700), (3, 1000, 500), (8, MiB, 250),
                                        (2, 17, 999)])
def test_hybrid_all2all(c3gpu, grid, bb, pm):
    print(f"hybrid all2all grid={grid} block={bb} permille={pm}", flush=True)
    src_np = wl.gen_bytes(grid * grid * bb, 12200 + grid)
    src = to_dev(src_np)
    dst = empty_bytes(src_np.size + 1)
    c3gpu.c3_all2all_block(dst.data_ptr(), src, grid, bb, c3gpu.C3_MOVER_HYBRID, hybrid(c3gpu, pm))
    sync()
    out = bytes_from_dev(dst)
    assert oracle.first_diff(oracle.all2all_block(src_np, grid, bb), out[:-1]) == -1
    assert out[-1] == 0xA5


@pytest.mark.parametrize("pm", [0, 450, 1000])
def test_hybrid_allreduce_isolated(c3gpu, pm):
    world, rank, chunk = 8, 3, 64 * KiB + 6
    n = chunk // 2
    contribs_np = [wl.gen_bf16((n,), ("normal", 0.0, 1.0), 12300 + r) for r in range(world)]
    peers_np = [None if i == rank else wl.gen_bf16((n,), ("normal", 0.0, 1.0), 12400 + i)
                for i in range(world)]
    want_red, want = oracle.allreduce_local(contribs_np, peers_np, rank)
    contribs = [to_dev(c) for c in contribs_np]
    peers = [None if p is None else to_dev(p) for p in peers_np]
    red = empty_bytes(chunk)
    dst = empty_bytes(world * chunk)
    c3gpu.c3_allreduce_local(dst, red, contribs, peers, rank, chunk, c3gpu.C3_MOVER_HYBRID,
                             hybrid(c3gpu, pm))
    sync()
    assert oracle.first_diff(want_red.view(np.uint8), bytes_from_dev(red)) == -1
    assert oracle.first_diff(want.view(np.uint8), bytes_from_dev(dst)) == -1


def test_hybrid_share_out_of_range(c3gpu):
    src = to_dev(wl.gen_bytes(4096, 3))
    dst = empty_bytes(2 * 4096)
    ptrs = (ctypes.c_void_p * 2)(src.data_ptr(), src.data_ptr())
    for pm in (-1, 1001):
        o = hybrid(c3gpu, pm)
        st = c3gpu.call("c3_gather", dst.data_ptr(), ptrs, 2, 4096, c3gpu.C3_MOVER_HYBRID,
                        ctypes.byref(o), None)
        assert st == c3gpu.C3_E_INVALID
    st = c3gpu.call("c3_gather", dst.data_ptr(), ptrs, 2, 4096, 3, None, None)
    assert st == c3gpu.C3_E_INVALID
    sync()


def run_hybrid_cells(c3, case, cells):
    case.poison(0)
    c3.c3_run_concurrent(case.gargs(c3), None)
    iso_c = bf16_from_dev(case.dC)
    rep = oracle.gemm_compare(case.ref, iso_c)
    assert oracle.gemm_within_tolerance(rep), rep
    info = c3.c3_device_info()
    per = info["n_cu"] // info["n_xcc"]
    for r, (pm, keep, comm_first) in enumerate(cells, start=1):
        case.poison(r)
        gm = None if keep == per else c3.c3_cu_mask_balanced(keep)
        cm = None if keep == per else c3.c3_cu_mask_balanced(keep, True)
        cargs, _keep = case.cargs(c3, c3.C3_MOVER_HYBRID, hybrid(c3, pm))
        label = f"hybrid {case.copy} permille={pm} keep={keep} comm_first={comm_first}"
        print(label, flush=True)
        t = c3.c3_run_concurrent(case.gargs(c3), cargs,
                                 c3.conc_opts(gemm_mask=gm, comm_mask=cm, comm_first=comm_first))
        case.check_comm(label)
        np.testing.assert_array_equal(bf16_from_dev(case.dC), iso_c, err_msg=label)
        assert t["t_conc_ns"] >= max(t["t_gemm_done_ns"], t["t_copy_done_ns"]) > 0
        assert t["copy_gpu_ms"] > 0
        if 0 < pm:
            assert t["engines_used"] != 0
        if 0 < pm < 1000:
            assert t["n_chunks"] > case.units  # engine transfers plus CU segments
        if case.copy == "allreduce":
            assert t["reduce_gpu_ms"] > 0 and 0 < t["t_reduce_done_ns"] <= t["t_conc_ns"]
            if pm > 0:
                assert t["t_copy_done_ns"] >= t["t_reduce_done_ns"]
        print(label, {k: t[k] for k in ("t_conc_ns", "t_gemm_done_ns", "t_copy_done_ns",
                                        "gemm_gpu_ms", "copy_gpu_ms", "n_chunks")}, flush=True)


def test_hybrid_concurrent_gather(c3gpu):
    case = Case(c3gpu, 512, 512, 512, "gather", 8, MiB + 16, 12500)
    run_hybrid_cells(c3gpu, case, [(0, 32, True), (250, 32, True), (600, 32, False),
                                   (1000, 32, True), (500, 28, True), (800, 24, False)])


def test_hybrid_concurrent_all2all_and_skinny(c3gpu):
    case = Case(c3gpu, 1024, 1032, 1024, "all2all", 8, 256 * KiB, 12600)
    run_hybrid_cells(c3gpu, case, [(500, 32, True), (700, 28, False)])
    case = Case(c3gpu, 16, 4096, 2048, "gather", 8, 2 * MiB + 16, 12700)
    run_hybrid_cells(c3gpu, case, [(400, 32, True), (900, 32, False)])


def test_hybrid_concurrent_allreduce(c3gpu):
    case = Case(c3gpu, 512, 768, 1024, "allreduce", 8, MiB, 12800)
    run_hybrid_cells(c3gpu, case, [(500, 32, True), (900, 32, False), (300, 28, True)])
    case.poison(9)
    cargs, _keep = case.cargs(c3gpu, c3gpu.C3_MOVER_HYBRID, hybrid(c3gpu, 600))
    t = c3gpu.c3_run_concurrent(None, cargs, c3gpu.conc_opts(flush_bytes=64 * MiB))
    case.check_comm("isolated hybrid all-reduce")
    assert t["t_gemm_done_ns"] == 0 and t["t_copy_done_ns"] > 0 and t["reduce_gpu_ms"] > 0


def test_hybrid_fault_hooks(c3gpu):
    """Host-forced SDMA faults in the engines' share: a dropped transfer leaves exactly its bytes
    stale (the CU share is intact, the byte check catches it); a stuck or failed transfer is
    reported, alone and beside a GEMM, after the CU share finished; the library stays usable."""
    sb = 256 * KiB
    shards = [wl.gen_bytes(sb, 12900 + i) for i in range(8)]
    want = oracle.gather(shards)
    # 500 per mille with 128 KiB chunks: engine chunk i is the first half of shard i
    got, _ = gather(c3gpu, shards, hybrid(c3gpu, 500, chunk_bytes=128 * KiB,
                                          fault_mode=c3gpu.C3_FAULT_DROP_CHUNK, fault_chunk=3))
    off = oracle.first_diff(want, got)
    assert 3 * sb <= off < 3 * sb + sb // 2
    assert oracle.first_diff(want[3 * sb + sb // 2:], got[3 * sb + sb // 2:]) == -1
    with pytest.raises(c3gpu.C3Error) as e:
        gather(c3gpu, shards, hybrid(c3gpu, 500, chunk_bytes=128 * KiB, timeout_ms=300,
                                     fault_mode=c3gpu.C3_FAULT_STUCK_CHUNK, fault_chunk=5))
    assert e.value.status == c3gpu.C3_E_TIMEOUT
    # beside a GEMM: the error comes back after both operations finished, C is still right
    case = Case(c3gpu, 512, 512, 512, "gather", 8, sb, 12950)
    case.poison(0)
    c3gpu.c3_run_concurrent(case.gargs(c3gpu), None)
    iso_c = bf16_from_dev(case.dC)
    case.poison(1)
    cargs, _keep = case.cargs(c3gpu, c3gpu.C3_MOVER_HYBRID,
                              hybrid(c3gpu, 500, chunk_bytes=128 * KiB,
                                     fault_mode=c3gpu.C3_FAULT_ERROR_CHUNK, fault_chunk=0))
    with pytest.raises(c3gpu.C3Error) as e:
        c3gpu.c3_run_concurrent(case.gargs(c3gpu), cargs, c3gpu.conc_opts(comm_first=True))
    assert e.value.status == c3gpu.C3_E_HSA
    np.testing.assert_array_equal(bf16_from_dev(case.dC), iso_c)
    got = bytes_from_dev(case.dst)
    for i in range(8):  # every CU share (second halves) landed
        lo = i * sb + sb // 2
        assert oracle.first_diff(case.want[lo:lo + sb // 2], got[lo:lo + sb // 2]) == -1, i
    got, _ = gather(c3gpu, shards, hybrid(c3gpu, 500))
    assert oracle.first_diff(want, got) == -1
