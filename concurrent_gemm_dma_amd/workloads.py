"""Workload table and seeded synthetic inputs for the C3 hot path.

This module is shared by the tests (oracle side and device side) and the benchmark. It holds
shapes, seeds and random draws only -- none of the method's arithmetic. bf16 operands are made
by drawing fp32 samples with numpy's PCG64 and converting them with torch's CPU bf16 cast (a
library routine), then viewing the result as uint16 bit patterns.

The workloads stand in for the C3 scenarios of "Optimizing ML Concurrent Computation and
Communication with GPU DMA Engines" (arXiv 2412.14335): GEMMs from LLaMA-70B/405B-class
training concurrent with FSDP-style all-gathers or MoE-style all-to-alls (Section III, Fig. 4;
the paper's scenario table itself is not available, so these shapes are synthetic stand-ins).

Seeds: seed = 0xC3000000 + 256 * workload_id + buffer_id, buffer ids A = 1, B = 2, shard i =
16 + i (all-reduce: rank r's contribution = 16 + r), all-to-all source = 32, all-reduce peer
chunk i = 48 + i; the small-integer variant adds 64.

Workload 6 widens the collective to an all-reduce, split into a reduce-scatter (arithmetic, on
the CUs) and an all-gather of the reduced chunks (a copy either mover can take), the split the
pages propose because DMA engines do no arithmetic (L3 Synthesis page on 2412.14335, section 3,
Attack 1): a 256 MiB bf16 gradient bucket over 8 ranks, as data-parallel training all-reduces
gradients while the next GEMM runs.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

MiB = 1 << 20

BUF_A = 1
BUF_B = 2
BUF_SHARD0 = 16
BUF_A2A_SRC = 32
BUF_PEER0 = 48
INT_VARIANT = 64

_CHUNK = 1 << 24  # elements per generation chunk (fixed so the streams never depend on size)


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    M: int
    N: int
    K: int
    a_dist: tuple          # ("uniform", lo, hi) or ("normal", mean, std)
    b_dist: tuple
    copy: str              # "gather", "all2all" or "allreduce"
    units: int             # gather: shards; all2all: grid (grid x grid blocks); allreduce: ranks
    unit_bytes: int        # gather: bytes per shard; all2all: bytes per block; allreduce: chunk
    payload: str           # "bytes" (uniform random bytes) or "bf16_normal"
    sweep_total_bytes: tuple = ()  # gather totals swept by the GC-equal workload

    @property
    def copy_bytes(self) -> int:
        """Bytes the collective delivers: the gathered / transposed / all-reduced buffer."""
        n = self.units * self.units if self.copy == "all2all" else self.units
        return n * self.unit_bytes

    @property
    def comm_hbm_bytes(self) -> int:
        """Algorithmic HBM bytes of the local share: copies read and write every byte once;
        an all-reduce's reduce-scatter reads `units` chunks and writes one, then its all-gather
        reads and writes `units` chunks."""
        if self.copy == "allreduce":
            return (3 * self.units + 1) * self.unit_bytes
        return 2 * self.copy_bytes

    @property
    def gemm_flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def gemm_bytes(self) -> int:
        """Algorithmic GEMM bytes: A, B read once, C written once (bf16)."""
        return 2 * (self.M * self.K + self.K * self.N + self.M * self.N)

    def with_gather_total(self, total_bytes: int) -> "Workload":
        if self.copy != "gather" or total_bytes % self.units:
            raise ValueError("gather total must split into equal shards")
        return dataclasses.replace(self, unit_bytes=total_bytes // self.units)


WORKLOADS = {
    1: Workload(1, "tiny_c3", 512, 512, 512, ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0),
                "gather", 8, 1 * MiB, "bytes"),
    2: Workload(2, "g_long_70b_ffn", 8192, 28672, 8192, ("normal", 0.0, 1.0),
                ("normal", 0.0, 0.02), "gather", 8, 16 * MiB, "bf16_normal"),
    3: Workload(3, "memory_bound_skinny", 16, 28672, 8192, ("normal", 0.0, 1.0),
                ("normal", 0.0, 0.02), "gather", 8, 32 * MiB, "bytes"),
    4: Workload(4, "405b_all2all", 8192, 53248, 16384, ("normal", 0.0, 1.0),
                ("normal", 0.0, 0.02), "all2all", 8, 8 * MiB, "bytes"),
    5: Workload(5, "gc_equal_sweep", 4096, 16384, 8192, ("normal", 0.0, 1.0),
                ("normal", 0.0, 0.02), "gather", 8, 32 * MiB, "bytes",
                sweep_total_bytes=tuple(s * MiB for s in (32, 64, 128, 256, 384, 512, 768, 1024))),
    6: Workload(6, "dp_allreduce_70b_ffn", 8192, 28672, 8192, ("normal", 0.0, 1.0),
                ("normal", 0.0, 0.02), "allreduce", 8, 32 * MiB, "bf16_normal"),
}

ALLREDUCE_RANK = 0  # the local rank of the all-reduce workloads


def seed_for(wid: int, buf: int) -> int:
    return 0xC3000000 + 256 * wid + buf


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def gen_bf16(shape, dist: tuple, seed: int) -> np.ndarray:
    """bf16 bit patterns of fp32 draws from `dist` (uniform or normal), PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    kind = dist[0]
    for start in range(0, n, _CHUNK):
        m = min(_CHUNK, n - start)
        if kind == "uniform":
            x = rng.uniform(dist[1], dist[2], size=m).astype(np.float32)
        elif kind == "normal":
            x = rng.standard_normal(size=m, dtype=np.float32)
            x = x * np.float32(dist[2]) + np.float32(dist[1])
        else:
            raise ValueError(f"unknown distribution {dist}")
        out[start:start + m] = _to_bf16_bits(x)
    return out.reshape(shape)


def gen_small_int_bf16(shape, seed: int, lo: int = -2, hi: int = 2) -> np.ndarray:
    """bf16 bit patterns of integers drawn uniformly from [lo, hi] (exact in bf16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for start in range(0, n, _CHUNK):
        m = min(_CHUNK, n - start)
        v = rng.integers(lo, hi + 1, size=m).astype(np.float32)
        out[start:start + m] = _to_bf16_bits(v)
    return out.reshape(shape)


def gen_bytes(nbytes: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, 256, size=nbytes, dtype=np.uint8)


def gen_tagged_shards(n_shards: int, shard_bytes: int) -> list:
    """Gather sources in the diagnostic pattern: every little-endian 8-byte word of shard i holds
    (i << 56) | d, d = the byte offset where that word belongs in the gathered buffer
    (i * shard_bytes + its offset in the shard). A word found anywhere else names its shard and
    its place. shard_bytes must be a multiple of 8; n_shards at most 256."""
    if shard_bytes % 8 or not 0 <= n_shards <= 256:
        raise ValueError("tagged shards need shard_bytes % 8 == 0 and 0 <= n_shards <= 256")
    words = shard_bytes // 8
    out = []
    for i in range(n_shards):
        d = np.arange(words, dtype=np.uint64) * np.uint64(8) + np.uint64(i * shard_bytes)
        out.append((d | (np.uint64(i) << np.uint64(56))).astype("<u8").view(np.uint8))
    return out


def gen_gemm_operands(w: Workload, int_exact: bool = False):
    """(A [M,K], B [K,N]) as uint16 bf16 bit patterns."""
    if int_exact:
        A = gen_small_int_bf16((w.M, w.K), seed_for(w.wid, BUF_A + INT_VARIANT))
        B = gen_small_int_bf16((w.K, w.N), seed_for(w.wid, BUF_B + INT_VARIANT))
    else:
        A = gen_bf16((w.M, w.K), w.a_dist, seed_for(w.wid, BUF_A))
        B = gen_bf16((w.K, w.N), w.b_dist, seed_for(w.wid, BUF_B))
    return A, B


def gen_payload(w: Workload, nbytes: int, buf: int) -> np.ndarray:
    """Copy payload as uint8: random bytes, or bf16 bit patterns of N(0, 1) draws."""
    seed = seed_for(w.wid, buf)
    if w.payload == "bytes":
        return gen_bytes(nbytes, seed)
    if w.payload == "bf16_normal":
        if nbytes % 2:
            raise ValueError("bf16 payload needs an even byte count")
        return gen_bf16((nbytes // 2,), ("normal", 0.0, 1.0), seed).view(np.uint8)
    raise ValueError(w.payload)


def gen_shards(w: Workload, shard_bytes: Optional[int] = None):
    """Gather sources: list of `units` arrays of `shard_bytes` bytes each."""
    sb = w.unit_bytes if shard_bytes is None else shard_bytes
    return [gen_payload(w, sb, BUF_SHARD0 + i) for i in range(w.units)]


def gen_allreduce(w: Workload, chunk_bytes: Optional[int] = None, rank: int = ALLREDUCE_RANK):
    """All-reduce inputs as uint16 bf16 arrays: (contributions of the `units` ranks to this
    rank's chunk, the other ranks' reduced chunks with None at `rank`)."""
    cb = w.unit_bytes if chunk_bytes is None else chunk_bytes
    if cb % 2:
        raise ValueError("all-reduce chunks hold bf16: even byte count")
    n = cb // 2
    contribs = [gen_bf16((n,), ("normal", 0.0, 1.0), seed_for(w.wid, BUF_SHARD0 + r))
                for r in range(w.units)]
    peers = [None if i == rank else gen_bf16((n,), ("normal", 0.0, 1.0), seed_for(w.wid, BUF_PEER0 + i))
             for i in range(w.units)]
    return contribs, peers


def gen_a2a_source(w: Workload, block_bytes: Optional[int] = None) -> np.ndarray:
    bb = w.unit_bytes if block_bytes is None else block_bytes
    return gen_payload(w, w.units * w.units * bb, BUF_A2A_SRC)


def sample_indices(M: int, N: int, n: int, seed: int, full_rows=(), full_cols=()):
    """Output coordinates to check at full size: random (m, n) pairs, plus the corners, plus
    any requested full rows and columns."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = [rng.integers(0, M, size=n)]
    cols = [rng.integers(0, N, size=n)]
    corners_r = np.array([0, 0, M - 1, M - 1], dtype=np.int64)
    corners_c = np.array([0, N - 1, 0, N - 1], dtype=np.int64)
    rows.append(corners_r)
    cols.append(corners_c)
    for r in full_rows:
        rows.append(np.full(N, r, dtype=np.int64))
        cols.append(np.arange(N, dtype=np.int64))
    for c in full_cols:
        rows.append(np.arange(M, dtype=np.int64))
        cols.append(np.full(M, c, dtype=np.int64))
    return np.concatenate(rows).astype(np.int64), np.concatenate(cols).astype(np.int64)
