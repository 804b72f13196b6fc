"""The seeded input generators: deterministic, distinct per buffer, right shapes and moments."""
import numpy as np

from concurrent_gemm_dma_amd import workloads as wl


def test_table_shapes():
    w = wl.WORKLOADS
    assert (w[1].M, w[1].N, w[1].K, w[1].copy_bytes) == (512, 512, 512, 8 * wl.MiB)
    assert (w[2].M, w[2].N, w[2].K, w[2].copy_bytes) == (8192, 28672, 8192, 128 * wl.MiB)
    assert (w[3].M, w[3].N, w[3].K, w[3].copy_bytes) == (16, 28672, 8192, 256 * wl.MiB)
    assert (w[4].M, w[4].N, w[4].K, w[4].copy_bytes) == (8192, 53248, 16384, 512 * wl.MiB)
    assert (w[6].M, w[6].N, w[6].K, w[6].copy_bytes) == (8192, 28672, 8192, 256 * wl.MiB)
    # all-reduce local share: reduce-scatter reads 8 chunks, writes 1; all-gather reads and
    # writes 8 chunks (32 MiB each)
    assert w[6].comm_hbm_bytes == (8 + 1 + 16) * 32 * wl.MiB
    assert w[2].comm_hbm_bytes == 2 * w[2].copy_bytes
    assert (w[5].M, w[5].N, w[5].K) == (4096, 16384, 8192)
    assert w[5].sweep_total_bytes[0] == 32 * wl.MiB and w[5].sweep_total_bytes[-1] == wl.MiB * 1024
    assert w[5].with_gather_total(64 * wl.MiB).unit_bytes == 8 * wl.MiB
    assert w[2].gemm_flops == 2 * 8192 * 28672 * 8192


def test_deterministic_and_distinct():
    a1 = wl.gen_bf16((64, 33), ("normal", 0.0, 1.0), wl.seed_for(2, wl.BUF_A))
    a2 = wl.gen_bf16((64, 33), ("normal", 0.0, 1.0), wl.seed_for(2, wl.BUF_A))
    b = wl.gen_bf16((64, 33), ("normal", 0.0, 1.0), wl.seed_for(2, wl.BUF_B))
    np.testing.assert_array_equal(a1, a2)
    assert not np.array_equal(a1, b)
    x = wl.gen_bytes(1000, 3)
    np.testing.assert_array_equal(x, wl.gen_bytes(1000, 3))
    assert x.dtype == np.uint8


def test_moments():
    f = (wl.gen_bf16((1 << 18,), ("normal", 0.0, 0.02), 9).astype(np.uint32) << 16).view(np.float32)
    assert abs(f.mean()) < 1e-3 and abs(f.std() - 0.02) < 1e-3
    u = (wl.gen_bf16((1 << 18,), ("uniform", -1.0, 1.0), 10).astype(np.uint32) << 16).view(np.float32)
    assert u.min() >= -1.0 and u.max() <= 1.0 and abs(u.mean()) < 1e-2
    i = (wl.gen_small_int_bf16((1 << 16,), 11).astype(np.uint32) << 16).view(np.float32)
    assert set(np.unique(i).tolist()) == {-2.0, -1.0, 0.0, 1.0, 2.0}


def test_payloads():
    w = wl.WORKLOADS[2]
    s = wl.gen_shards(w, shard_bytes=4096)
    assert len(s) == 8 and all(x.size == 4096 and x.dtype == np.uint8 for x in s)
    w4 = wl.WORKLOADS[4]
    src = wl.gen_a2a_source(w4, block_bytes=128)
    assert src.size == 64 * 128


def test_sample_indices():
    r, c = wl.sample_indices(10, 20, 30, seed=1, full_rows=(2,), full_cols=(19,))
    assert r.size == 30 + 4 + 20 + 10
    assert r.max() < 10 and c.max() < 20


def test_allreduce_generator_is_seeded_and_leaves_rank_slot_empty():
    w = wl.WORKLOADS[6]
    c1, p1 = wl.gen_allreduce(w, 4096, rank=2)
    c2, p2 = wl.gen_allreduce(w, 4096, rank=2)
    assert len(c1) == 8 and all(x.size == 2048 for x in c1)
    assert p1[2] is None and all(p is not None for i, p in enumerate(p1) if i != 2)
    assert all((a == b).all() for a, b in zip(c1, c2))
    assert not (c1[0] == c1[1]).all()
