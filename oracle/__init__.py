"""CPU oracle for the C3 hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
import this package. The product library never imports, links or calls it, and it shares no
code with the product. See ``oracle.h`` for what each routine computes and which passage of
"Optimizing ML Concurrent Computation and Communication with GPU DMA Engines" (arXiv 2412.14335)
it follows.

Arrays are numpy: bf16 values travel as their uint16 bit patterns; A is [M, K], B is [K, N],
C is [M, N], all row-major (C-contiguous).

Parity status of each routine (pins are in the CPU test suite):
  bf16_from_f32_bits  pinned: independent nearest-of-two-neighbours formulation, hand-derived
                      format cases, a structured 2M-pattern sweep over every rounding edge
                      (full 2^32 sweep behind C3_EXHAUSTIVE=1)
  bf16_from_f64       pinned: same independent formulation, double-rounding cases
  gemm_f32acc         pinned: numpy step-by-step fp32 accumulation (bitwise), fp64 brute force
                      within the recursive-summation bound, identity / zero / integer-exact
  gemm_f64acc         pinned: exact integer products (numpy int64), fp64 brute force
  gather / all2all    pinned: per-byte Python loops, involution, diagonal invariance
  reduce_sum_bf16     pinned: exact integer sums, exhaustive two-rank sums against exact rational
                      sums rounded by the independent bf16 formulation, hand-worked order /
                      single-rounding / signed-zero cases, the fp32 summation error bound
  allreduce_local     pinned: slot placement by per-element loops, rank variation
  checkers            pinned: planted mistakes (dropped chunk, flipped byte, swapped shards)
  (mutants)           mistakes planted in a scratch copy of oracle.c fail the pins above
  metrics             pinned: closed forms (S_ideal in [1, 2], = 2 iff equal times)
  partition           pinned: hand-worked roofline values and machine balance, hand-worked
                      predictions with the tie rule, limiting tables, scoring
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import numpy as np

from . import metrics  # noqa: F401  (re-export)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")


class GemmReport(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int64),
        ("n_diff", ctypes.c_int64),
        ("n_violations", ctypes.c_int64),
        ("first_violation", ctypes.c_int64),
        ("max_scaled_err", ctypes.c_double),
        ("frob_rel", ctypes.c_double),
        ("n_nonfinite", ctypes.c_int64),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


def lib():
    """Load liboracle.so, building it with gcc first if it is not there yet."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from .build import build

        build()
    _lib = load_library(_LIB_PATH)
    return _lib


def load_library(path: str):
    """Open a build of oracle.c at `path` and declare its signatures."""
    L = ctypes.CDLL(path)
    L.orc_bf16_from_f32_bits.restype = ctypes.c_uint16
    L.orc_bf16_from_f32_bits.argtypes = [ctypes.c_uint32]
    L.orc_bf16_from_f64.restype = ctypes.c_uint16
    L.orc_bf16_from_f64.argtypes = [ctypes.c_double]
    L.orc_bf16_from_f32_bits_array.restype = None
    L.orc_bf16_from_f32_bits_array.argtypes = [_u32p, _u16p, ctypes.c_size_t]
    L.orc_bf16_from_f64_array.restype = None
    L.orc_bf16_from_f64_array.argtypes = [_f64p, _u16p, ctypes.c_size_t]
    L.orc_gemm_f32acc_rows.restype = None
    L.orc_gemm_f32acc_rows.argtypes = [
        _u16p, _u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, _u16p, ctypes.c_void_p, ctypes.c_int,
    ]
    L.orc_gemm_f64acc_rows.restype = None
    L.orc_gemm_f64acc_rows.argtypes = [
        _u16p, _u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
    ]
    L.orc_gemm_elems.restype = ctypes.c_int
    L.orc_gemm_elems.argtypes = [
        _u16p, _u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _i64p, _i64p,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
    ]
    L.orc_gather.restype = None
    L.orc_gather.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                             ctypes.c_size_t]
    L.orc_all2all_block.restype = None
    L.orc_all2all_block.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_size_t]
    L.orc_reduce_sum_bf16.restype = None
    L.orc_reduce_sum_bf16.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                      ctypes.c_size_t, _u16p]
    L.orc_allreduce_local.restype = None
    L.orc_allreduce_local.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                      ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int,
                                      ctypes.c_size_t, _u16p, _u16p]
    L.orc_first_diff.restype = ctypes.c_int64
    L.orc_first_diff.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
    L.orc_gemm_compare.restype = None
    L.orc_gemm_compare.argtypes = [_u16p, _u16p, ctypes.c_int64, ctypes.c_double,
                                   ctypes.POINTER(GemmReport)]
    L.orc_threads.restype = ctypes.c_int
    L.orc_threads.argtypes = [ctypes.c_int]
    return L


def threads(nthreads: int = 0) -> int:
    return lib().orc_threads(nthreads)


# ---------------------------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------------------------

def bf16_from_f32_bits(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint32)
    out = np.empty(bits.shape, dtype=np.uint16)
    lib().orc_bf16_from_f32_bits_array(bits.reshape(-1), out.reshape(-1), bits.size)
    return out


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    return bf16_from_f32_bits(np.ascontiguousarray(x, dtype=np.float32).view(np.uint32))


def bf16_from_f64(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_bf16_from_f64_array(x.reshape(-1), out.reshape(-1), x.size)
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact decode: the bf16 bits become the top half of an fp32."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------------------------

def _check_ab(A: np.ndarray, B: np.ndarray):
    if A.dtype != np.uint16 or B.dtype != np.uint16 or A.ndim != 2 or B.ndim != 2:
        raise TypeError("A and B must be 2-D uint16 (bf16 bit pattern) arrays")
    if A.shape[1] != B.shape[0]:
        raise ValueError(f"inner dimensions differ: {A.shape} x {B.shape}")
    return np.ascontiguousarray(A), np.ascontiguousarray(B)


def gemm_f32acc(A: np.ndarray, B: np.ndarray, rows: tuple[int, int] | None = None,
                want_acc: bool = False, nthreads: int = 0):
    """bf16(sum_k fp32 products, fp32 accumulation, k ascending) for rows [r0, r1) of C."""
    A, B = _check_ab(A, B)
    M, K = A.shape
    N = B.shape[1]
    r0, r1 = rows if rows is not None else (0, M)
    if not (0 <= r0 <= r1 <= M):
        raise ValueError("row range out of bounds")
    C = np.empty((r1 - r0, N), dtype=np.uint16)
    acc = np.empty((r1 - r0, N), dtype=np.float32) if want_acc else None
    lib().orc_gemm_f32acc_rows(A, B, M, N, K, r0, r1, C,
                               acc.ctypes.data if acc is not None else None, nthreads)
    return (C, acc) if want_acc else C


def gemm_f64acc(A: np.ndarray, B: np.ndarray, rows: tuple[int, int] | None = None,
                want_sum: bool = False, nthreads: int = 0):
    """bf16 of the fp64 sum of products (single rounding) for rows [r0, r1) of C."""
    A, B = _check_ab(A, B)
    M, K = A.shape
    N = B.shape[1]
    r0, r1 = rows if rows is not None else (0, M)
    if not (0 <= r0 <= r1 <= M):
        raise ValueError("row range out of bounds")
    C = np.empty((r1 - r0, N), dtype=np.uint16)
    s = np.empty((r1 - r0, N), dtype=np.float64) if want_sum else None
    lib().orc_gemm_f64acc_rows(A, B, M, N, K, r0, r1, C.ctypes.data,
                               s.ctypes.data if s is not None else None, nthreads)
    return (C, s) if want_sum else C


def gemm_elems(A: np.ndarray, B: np.ndarray, rows: Sequence[int], cols: Sequence[int],
               nthreads: int = 0):
    """Selected elements of C: returns (bf16 fp32-acc, bf16 fp64-acc, fp64 sums)."""
    A, B = _check_ab(A, B)
    M, K = A.shape
    N = B.shape[1]
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    if r.shape != c.shape:
        raise ValueError("rows and cols differ in length")
    n = r.size
    c32 = np.empty(n, dtype=np.uint16)
    c64 = np.empty(n, dtype=np.uint16)
    s64 = np.empty(n, dtype=np.float64)
    rc = lib().orc_gemm_elems(A, B, M, N, K, r, c, n, c32.ctypes.data, c64.ctypes.data,
                              s64.ctypes.data, nthreads)
    if rc != 0:
        raise IndexError("element index out of range")
    return c32, c64, s64


# ---------------------------------------------------------------------------------------------
# Copies
# ---------------------------------------------------------------------------------------------

def gather(shards: Sequence[np.ndarray]) -> np.ndarray:
    """All-gather local share: concatenation of equally sized shards, as uint8."""
    views = [np.ascontiguousarray(s).view(np.uint8).reshape(-1) for s in shards]
    if not views:
        return np.empty(0, dtype=np.uint8)
    shard_bytes = views[0].size
    if any(v.size != shard_bytes for v in views):
        raise ValueError("shards must all have the same size")
    dst = np.empty(len(views) * shard_bytes, dtype=np.uint8)
    ptrs = (ctypes.c_void_p * len(views))(*[v.ctypes.data for v in views])
    lib().orc_gather(dst.ctypes.data, ptrs, len(views), shard_bytes)
    return dst


def all2all_block(src: np.ndarray, grid: int, block_bytes: int) -> np.ndarray:
    """Block transpose of a grid x grid array of blocks, as uint8."""
    s = np.ascontiguousarray(src).view(np.uint8).reshape(-1)
    if s.size != grid * grid * block_bytes:
        raise ValueError("src size must be grid*grid*block_bytes")
    dst = np.empty_like(s)
    lib().orc_all2all_block(dst.ctypes.data, s.ctypes.data, grid, block_bytes)
    return dst


# ---------------------------------------------------------------------------------------------
# All-reduce local share
# ---------------------------------------------------------------------------------------------

def _u16_views(arrays: Sequence[np.ndarray], n: int, what: str) -> list:
    views = [np.ascontiguousarray(a).view(np.uint16).reshape(-1) for a in arrays]
    if any(v.size != n for v in views):
        raise ValueError(f"{what}: every array must hold {n} bf16 elements")
    return views


def reduce_sum_bf16(contribs: Sequence[np.ndarray]) -> np.ndarray:
    """Reduce-scatter local share: elementwise fp32 sum of the ranks' bf16 contributions in rank
    order, rounded once to bf16 (uint16 bit patterns)."""
    if not contribs:
        raise ValueError("reduce_sum_bf16 needs at least one contribution")
    n = np.asarray(contribs[0]).view(np.uint16).size
    views = _u16_views(contribs, n, "reduce_sum_bf16")
    out = np.empty(n, dtype=np.uint16)
    ptrs = (ctypes.c_void_p * len(views))(*[v.ctypes.data for v in views])
    lib().orc_reduce_sum_bf16(ptrs, len(views), n, out)
    return out


def allreduce_local(contribs: Sequence[np.ndarray], peers: Sequence[np.ndarray | None],
                    rank: int) -> tuple[np.ndarray, np.ndarray]:
    """All-reduce local share: (reduced chunk, gathered result). peers[i] is rank i's reduced
    chunk for i != rank; peers[rank] is ignored (may be None)."""
    world = len(contribs)
    if world < 1 or len(peers) != world or not 0 <= rank < world:
        raise ValueError("allreduce_local: need world >= 1 contributions, world peers, 0 <= rank < world")
    n = np.asarray(contribs[0]).view(np.uint16).size
    cv = _u16_views(contribs, n, "allreduce_local contribs")
    if any(peers[i] is None for i in range(world) if i != rank):
        raise ValueError("allreduce_local: every peer other than rank needs a chunk")
    pv = [None if peers[i] is None else _u16_views([peers[i]], n, "allreduce_local peers")[0]
          for i in range(world)]
    reduced = np.empty(n, dtype=np.uint16)
    dst = np.empty(world * n, dtype=np.uint16)
    cp = (ctypes.c_void_p * world)(*[v.ctypes.data for v in cv])
    pp = (ctypes.c_void_p * world)(*[None if v is None else v.ctypes.data for v in pv])
    lib().orc_allreduce_local(cp, pp, world, rank, n, reduced, dst)
    return reduced, dst


# ---------------------------------------------------------------------------------------------
# Checkers
# ---------------------------------------------------------------------------------------------

def first_diff(a: np.ndarray, b: np.ndarray) -> int:
    """Offset of the first differing byte (-1 if equal); sizes must match."""
    va = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
    vb = np.ascontiguousarray(b).view(np.uint8).reshape(-1)
    if va.size != vb.size:
        raise ValueError(f"sizes differ: {va.size} vs {vb.size}")
    return int(lib().orc_first_diff(va.ctypes.data, vb.ctypes.data, va.size))


def explain_tagged_gather(got: np.ndarray, n_shards: int, shard_bytes: int,
                          limit: int = 16) -> list:
    """For a gather of shards in the tagged pattern (each 8-byte word = shard << 56 | the byte
    offset where it belongs): the misplaced words of `got`, as (offset in got, shard found,
    offset the found word belongs at), at most `limit` of them; [] when every word is in place.
    Offset -1 / shard -1 mark a word that carries no valid tag (never written, or torn)."""
    g = np.ascontiguousarray(got).view(np.uint8).reshape(-1)
    if shard_bytes % 8 or g.size != n_shards * shard_bytes:
        raise ValueError("explain_tagged_gather: size must be n_shards * shard_bytes, "
                         "shard_bytes a multiple of 8")
    words = g.view("<u8")
    want = np.arange(words.size, dtype=np.uint64) * np.uint64(8)
    want |= (want // np.uint64(max(shard_bytes, 1))) << np.uint64(56)
    bad = np.flatnonzero(words != want)[:limit]
    out = []
    for w in bad:
        v = int(words[w])
        shard, off = v >> 56, v & ((1 << 56) - 1)
        valid = (shard < n_shards and off % 8 == 0 and off < g.size
                 and off // shard_bytes == shard)
        out.append((int(w) * 8, shard if valid else -1, off if valid else -1))
    return out


def gemm_compare(ref: np.ndarray, got: np.ndarray, tol: float = 1e-2) -> dict:
    r = np.ascontiguousarray(ref, dtype=np.uint16).reshape(-1)
    g = np.ascontiguousarray(got, dtype=np.uint16).reshape(-1)
    if r.size != g.size:
        raise ValueError("sizes differ")
    rep = GemmReport()
    lib().orc_gemm_compare(r, g, r.size, tol, ctypes.byref(rep))
    return rep.as_dict()


# Tolerances for GEMM parity: elementwise |got - ref| <= ELEM_TOL * max(1, |ref|) and
# ||got - ref||_F / ||ref||_F <= FROB_TOL.
ELEM_TOL = 1e-2
FROB_TOL = 1e-3


def gemm_within_tolerance(report: dict) -> bool:
    return (report["n_violations"] == 0 and report["n_nonfinite"] == 0
            and report["frob_rel"] <= FROB_TOL)
