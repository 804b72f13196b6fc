"""ctypes binding of libc3 (include/c3.h): same names, argument marshalling only.

Every step of the hot path runs in libc3's kernels and movers; this module only converts Python
arguments (ints, torch tensors) into the C ABI's pointers, sizes and structs. torch is imported
before the library is opened so that libc3 binds to the HIP/ROCr runtime torch already loaded
(one runtime per process). If libc3.so is missing, loading raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libc3.so")

C3_OK = 0
C3_E_INVALID = 1
C3_E_HIP = 2
C3_E_HSA = 3
C3_E_NO_SDMA = 4
C3_E_TIMEOUT = 5
C3_E_OVERLAP = 6
C3_E_UNSUPPORTED = 7
C3_E_NOT_INIT = 8
STATUS_NAMES = {0: "C3_OK", 1: "C3_E_INVALID", 2: "C3_E_HIP", 3: "C3_E_HSA", 4: "C3_E_NO_SDMA",
                5: "C3_E_TIMEOUT", 6: "C3_E_OVERLAP", 7: "C3_E_UNSUPPORTED", 8: "C3_E_NOT_INIT"}

C3_MOVER_CU = 0
C3_MOVER_SDMA = 1
C3_MOVER_HYBRID = 2
C3_COPY_GATHER = 0
C3_COPY_ALL2ALL = 1
C3_COPY_ALLREDUCE = 2
C3_FAULT_NONE = 0
C3_FAULT_DROP_CHUNK = 1
C3_FAULT_STUCK_CHUNK = 2
C3_FAULT_ERROR_CHUNK = 3
C3_MAX_MASK_WORDS = 8
C3_MAX_WORLD = 64
C3_MAX_CURVE = 16
C3_NOALLOC_SCRATCH_BYTES = 16 << 20  # c3_gemm_noalloc: fixed split-K partials per device
C3_ABI_VERSION = 5
TAXONOMY = {0: "GC-equal", 1: "G-long", 2: "C-long"}

# Every symbol include/c3.h declares.
EXPORTS = ("c3_init", "c3_finalize", "c3_last_error", "c3_device_info", "c3_stream_create",
           "c3_stream_destroy", "c3_cu_mask_balanced", "c3_probe_placement", "c3_gemm",
           "c3_gemm_noalloc", "c3_probe_mfma_rate",
           "c3_gather", "c3_all2all_block", "c3_reduce_scatter", "c3_allreduce_local",
           "c3_flush_llc", "c3_run_concurrent", "c3_derive_metrics", "c3_roofline_time",
           "c3_predict_partition", "c3_hybrid_share")


class C3Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class c3_info(ctypes.Structure):
    _fields_ = [("hip_device", ctypes.c_int32), ("n_cu", ctypes.c_int32),
                ("n_xcc", ctypes.c_int32), ("n_sdma", ctypes.c_int32),
                ("n_sdma_xgmi", ctypes.c_int32), ("sdma_engine_mask", ctypes.c_uint32),
                ("sdma_status_mask", ctypes.c_uint32),
                ("sdma_preferred_mask", ctypes.c_uint32), ("max_clock_mhz", ctypes.c_int32),
                ("lds_bytes_per_cu", ctypes.c_int32), ("l2_bytes", ctypes.c_int32),
                ("reserved", ctypes.c_int32),
                ("hbm_bytes", ctypes.c_uint64), ("arch", ctypes.c_char * 64)]

    def as_dict(self):
        d = {n: getattr(self, n) for n, _ in self._fields_}
        d["arch"] = self.arch.decode(errors="replace")
        return d


class c3_move_opts(ctypes.Structure):
    _fields_ = [("chunk_bytes", ctypes.c_uint64), ("engine_mask", ctypes.c_uint32),
                ("nontemporal", ctypes.c_int32), ("cu_blocks", ctypes.c_int32),
                ("timeout_ms", ctypes.c_int32), ("fault_mode", ctypes.c_int32),
                ("fault_chunk", ctypes.c_int32), ("sdma_permille", ctypes.c_int32)]


class c3_gemm_args(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class c3_copy_args(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("mover", ctypes.c_int32), ("dst", ctypes.c_void_p),
                ("shards", ctypes.POINTER(ctypes.c_void_p)), ("n_shards", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("shard_bytes", ctypes.c_uint64),
                ("src", ctypes.c_void_p), ("block_bytes", ctypes.c_uint64),
                ("opts", c3_move_opts), ("peers", ctypes.POINTER(ctypes.c_void_p)),
                ("reduced", ctypes.c_void_p), ("rank", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class c3_conc_opts(ctypes.Structure):
    _fields_ = [("gemm_cu_mask", ctypes.c_uint32 * C3_MAX_MASK_WORDS),
                ("comm_cu_mask", ctypes.c_uint32 * C3_MAX_MASK_WORDS),
                ("comm_first", ctypes.c_int32), ("use_priority", ctypes.c_int32),
                ("flush_bytes", ctypes.c_uint64)]


class c3_timing(ctypes.Structure):
    _fields_ = [("t_conc_ns", ctypes.c_int64), ("t_gemm_done_ns", ctypes.c_int64),
                ("t_copy_done_ns", ctypes.c_int64), ("t_issue_ns", ctypes.c_int64),
                ("gemm_gpu_ms", ctypes.c_double), ("copy_gpu_ms", ctypes.c_double),
                ("sdma_first_start_ns", ctypes.c_int64), ("sdma_last_end_ns", ctypes.c_int64),
                ("n_chunks", ctypes.c_int32), ("engines_used", ctypes.c_uint32),
                ("applied_priority", ctypes.c_int32), ("comm_issued_first", ctypes.c_int32),
                ("t_reduce_done_ns", ctypes.c_int64), ("reduce_gpu_ms", ctypes.c_double),
                ("gemm_applied_mask", ctypes.c_uint32 * C3_MAX_MASK_WORDS),
                ("comm_applied_mask", ctypes.c_uint32 * C3_MAX_MASK_WORDS)]

    def as_dict(self):
        d = {n: getattr(self, n) for n, _ in self._fields_}
        for n in ("gemm_applied_mask", "comm_applied_mask"):
            d[n] = list(d[n])
        return d


class c3_metrics(ctypes.Structure):
    _fields_ = [("ideal_speedup", ctypes.c_double), ("speedup", ctypes.c_double),
                ("uplift_fraction", ctypes.c_double), ("ratio_of_ideal", ctypes.c_double),
                ("gemm_slowdown", ctypes.c_double), ("hbm_ceiling", ctypes.c_double),
                ("taxonomy", ctypes.c_int32), ("reserved", ctypes.c_int32)]

    def as_dict(self):
        d = {n: getattr(self, n) for n, _ in self._fields_ if n != "reserved"}
        d["taxonomy"] = TAXONOMY.get(self.taxonomy, str(self.taxonomy))
        return d


_lib = None


class c3_slowdown_curve(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("cus_per_xcc", ctypes.c_int32 * C3_MAX_CURVE),
                ("slowdown", ctypes.c_double * C3_MAX_CURVE)]


def load(path: Optional[str] = None):
    """Open libc3.so (after importing torch so both share one HIP runtime). The path defaults
    to the in-tree build; the C3_LIB environment variable names another build of it."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads the HIP/ROCr runtime libc3 binds to)

    if path is None:
        path = os.environ.get("C3_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is not built; run __graft_entry__.build() "
                                "(python -m concurrent_gemm_dma_amd.build)")
    L = ctypes.CDLL(path)
    st = ctypes.c_int
    vp = ctypes.c_void_p
    L.c3_init.argtypes = [ctypes.c_int]
    L.c3_finalize.argtypes = []
    L.c3_last_error.argtypes = []
    L.c3_last_error.restype = ctypes.c_char_p
    L.c3_device_info.argtypes = [ctypes.POINTER(c3_info)]
    L.c3_stream_create.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(vp)]
    L.c3_stream_destroy.argtypes = [vp]
    L.c3_cu_mask_balanced.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_uint32)]
    L.c3_probe_placement.argtypes = [vp, ctypes.c_int, vp]
    L.c3_probe_mfma_rate.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    L.c3_gemm.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, vp]
    L.c3_gemm_noalloc.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, vp]
    L.c3_gather.argtypes = [vp, ctypes.POINTER(vp), ctypes.c_int, ctypes.c_size_t, ctypes.c_int,
                            ctypes.POINTER(c3_move_opts), vp]
    L.c3_all2all_block.argtypes = [vp, vp, ctypes.c_int, ctypes.c_size_t, ctypes.c_int,
                                   ctypes.POINTER(c3_move_opts), vp]
    L.c3_reduce_scatter.argtypes = [vp, ctypes.POINTER(vp), ctypes.c_int, ctypes.c_size_t,
                                    ctypes.POINTER(c3_move_opts), vp]
    L.c3_allreduce_local.argtypes = [vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int,
                                     ctypes.c_int, ctypes.c_size_t, ctypes.c_int,
                                     ctypes.POINTER(c3_move_opts), vp]
    L.c3_flush_llc.argtypes = [ctypes.c_size_t, vp]
    L.c3_run_concurrent.argtypes = [ctypes.POINTER(c3_gemm_args), ctypes.POINTER(c3_copy_args),
                                    ctypes.POINTER(c3_conc_opts), ctypes.POINTER(c3_timing)]
    L.c3_derive_metrics.argtypes = [ctypes.c_double] * 5 + [ctypes.POINTER(c3_metrics)]
    L.c3_roofline_time.argtypes = [ctypes.c_double] * 5 + [ctypes.POINTER(ctypes.c_double)]
    L.c3_predict_partition.argtypes = [ctypes.POINTER(c3_slowdown_curve),
                                       ctypes.POINTER(c3_slowdown_curve), ctypes.c_double,
                                       ctypes.c_double, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_int32), ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_int32),
                                       ctypes.POINTER(ctypes.c_double)]
    L.c3_hybrid_share.argtypes = [ctypes.c_double] * 3 + [ctypes.POINTER(ctypes.c_int32)]
    for name in EXPORTS:
        if name != "c3_last_error":
            getattr(L, name).restype = st
    _lib = L
    return L


def _ptr(x) -> Optional[int]:
    """Device pointer of a torch tensor, or an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream  # torch.cuda.Stream


def check(status: int) -> None:
    if status != C3_OK:
        raise C3Error(status, load().c3_last_error().decode(errors="replace"))


def call(name: str, *args) -> int:
    """Raw call returning the status (no raise)."""
    return getattr(load(), name)(*args)


# ---- thin wrappers with the ABI's names ---------------------------------------------------------

def c3_init(hip_device: int = 0) -> None:
    check(load().c3_init(hip_device))


def c3_finalize() -> None:
    check(load().c3_finalize())


def c3_last_error() -> str:
    return load().c3_last_error().decode(errors="replace")


def c3_device_info() -> dict:
    info = c3_info()
    check(load().c3_device_info(ctypes.byref(info)))
    return info.as_dict()


def _mask_array(mask: Optional[Sequence[int]]):
    arr = (ctypes.c_uint32 * C3_MAX_MASK_WORDS)()
    if mask is not None:
        for i, w in enumerate(mask[:C3_MAX_MASK_WORDS]):
            arr[i] = int(w) & 0xFFFFFFFF
    return arr


def c3_stream_create(cu_mask: Optional[Sequence[int]] = None, priority: int = 0) -> int:
    out = ctypes.c_void_p()
    n = 0 if cu_mask is None else min(len(cu_mask), C3_MAX_MASK_WORDS)
    check(load().c3_stream_create(_mask_array(cu_mask), n, priority, ctypes.byref(out)))
    return out.value


def c3_stream_destroy(stream: int) -> None:
    check(load().c3_stream_destroy(stream))


def c3_cu_mask_balanced(keep_per_xcc: int, complement: bool = False) -> list:
    arr = (ctypes.c_uint32 * C3_MAX_MASK_WORDS)()
    check(load().c3_cu_mask_balanced(keep_per_xcc, int(bool(complement)), arr))
    return list(arr)


def c3_probe_placement(out_dev, n_blocks: int, stream=None) -> None:
    check(load().c3_probe_placement(_stream(stream), n_blocks, _ptr(out_dev)))


def c3_probe_mfma_rate(out_dev, n_workgroups: int, iterations: int, random: int = 1,
                       stream=None) -> None:
    check(load().c3_probe_mfma_rate(_stream(stream), n_workgroups, iterations, random,
                                    _ptr(out_dev)))


def c3_gemm(A, B, C, M: int, N: int, K: int, stream=None) -> None:
    check(load().c3_gemm(_ptr(A), _ptr(B), _ptr(C), M, N, K, _stream(stream)))


def c3_gemm_noalloc(A, B, C, M: int, N: int, K: int, stream=None) -> None:
    check(load().c3_gemm_noalloc(_ptr(A), _ptr(B), _ptr(C), M, N, K, _stream(stream)))


def move_opts(**kw) -> c3_move_opts:
    o = c3_move_opts()
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def c3_gather(dst, shards, shard_bytes: int, mover: int = C3_MOVER_CU, opts=None,
              stream=None) -> None:
    ptrs = (ctypes.c_void_p * max(1, len(shards)))(*[_ptr(s) for s in shards])
    o = ctypes.byref(opts) if opts is not None else None
    check(load().c3_gather(_ptr(dst), ptrs, len(shards), shard_bytes, mover, o, _stream(stream)))


def c3_all2all_block(dst, src, grid: int, block_bytes: int, mover: int = C3_MOVER_CU, opts=None,
                     stream=None) -> None:
    o = ctypes.byref(opts) if opts is not None else None
    check(load().c3_all2all_block(_ptr(dst), _ptr(src), grid, block_bytes, mover, o,
                                  _stream(stream)))


def _ptr_array(xs):
    return (ctypes.c_void_p * max(1, len(xs)))(*[_ptr(x) for x in xs])


def c3_reduce_scatter(out, contribs, chunk_bytes: int, opts=None, stream=None) -> None:
    o = ctypes.byref(opts) if opts is not None else None
    check(load().c3_reduce_scatter(_ptr(out), _ptr_array(contribs), len(contribs), chunk_bytes, o,
                                   _stream(stream)))


def c3_allreduce_local(dst, reduced, contribs, peers, rank: int, chunk_bytes: int,
                       mover: int = C3_MOVER_CU, opts=None, stream=None) -> None:
    """peers[i] is rank i's reduced chunk for i != rank (peers[rank] may be None)."""
    o = ctypes.byref(opts) if opts is not None else None
    check(load().c3_allreduce_local(_ptr(dst), _ptr(reduced), _ptr_array(contribs),
                                    _ptr_array(peers), len(contribs), rank, chunk_bytes, mover, o,
                                    _stream(stream)))


def c3_flush_llc(nbytes: int, stream=None) -> None:
    check(load().c3_flush_llc(nbytes, _stream(stream)))


def gemm_args(A, B, C, M, N, K) -> c3_gemm_args:
    return c3_gemm_args(_ptr(A), _ptr(B), _ptr(C), M, N, K)


def gather_args(dst, shards, shard_bytes, mover, opts=None):
    """A c3_copy_args for a gather; the returned tuple keeps the pointer array alive."""
    ptrs = (ctypes.c_void_p * max(1, len(shards)))(*[_ptr(s) for s in shards])
    a = c3_copy_args()
    a.kind = C3_COPY_GATHER
    a.mover = mover
    a.dst = _ptr(dst)
    a.shards = ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p))
    a.n_shards = len(shards)
    a.shard_bytes = shard_bytes
    if opts is not None:
        a.opts = opts
    return a, ptrs


def all2all_args(dst, src, grid, block_bytes, mover, opts=None):
    a = c3_copy_args()
    a.kind = C3_COPY_ALL2ALL
    a.mover = mover
    a.dst = _ptr(dst)
    a.src = _ptr(src)
    a.grid = grid
    a.block_bytes = block_bytes
    if opts is not None:
        a.opts = opts
    return a, None


def allreduce_args(dst, reduced, contribs, peers, rank, chunk_bytes, mover, opts=None):
    """A c3_copy_args for an all-reduce local share; the returned tuple keeps the pointer arrays
    alive."""
    cp, pp = _ptr_array(contribs), _ptr_array(peers)
    a = c3_copy_args()
    a.kind = C3_COPY_ALLREDUCE
    a.mover = mover
    a.dst = _ptr(dst)
    a.shards = ctypes.cast(cp, ctypes.POINTER(ctypes.c_void_p))
    a.n_shards = len(contribs)
    a.shard_bytes = chunk_bytes
    a.peers = ctypes.cast(pp, ctypes.POINTER(ctypes.c_void_p))
    a.reduced = _ptr(reduced)
    a.rank = rank
    if opts is not None:
        a.opts = opts
    return a, (cp, pp)


def conc_opts(gemm_mask=None, comm_mask=None, comm_first=False, flush_bytes=0,
              use_priority=0) -> c3_conc_opts:
    o = c3_conc_opts()
    o.gemm_cu_mask = _mask_array(gemm_mask)
    o.comm_cu_mask = _mask_array(comm_mask)
    o.comm_first = int(bool(comm_first))
    o.use_priority = use_priority
    o.flush_bytes = flush_bytes
    return o


def c3_run_concurrent(g: Optional[c3_gemm_args], c: Optional[c3_copy_args],
                      o: Optional[c3_conc_opts] = None) -> dict:
    t = c3_timing()
    check(load().c3_run_concurrent(ctypes.byref(g) if g is not None else None,
                                   ctypes.byref(c) if c is not None else None,
                                   ctypes.byref(o) if o is not None else None, ctypes.byref(t)))
    return t.as_dict()


def c3_derive_metrics(t_gemm: float, t_copy: float, t_conc: float, bytes_total: float = 0.0,
                      bandwidth: float = 0.0) -> dict:
    m = c3_metrics()
    check(load().c3_derive_metrics(t_gemm, t_copy, t_conc, bytes_total, bandwidth,
                                   ctypes.byref(m)))
    return m.as_dict()


def slowdown_curve(table) -> c3_slowdown_curve:
    """A c3_slowdown_curve from {cus_per_xcc: slowdown}."""
    items = sorted(table.items())
    if not 1 <= len(items) <= C3_MAX_CURVE:
        raise ValueError(f"a slowdown curve holds 1..{C3_MAX_CURVE} entries")
    c = c3_slowdown_curve()
    c.n = len(items)
    for i, (k, v) in enumerate(items):
        c.cus_per_xcc[i] = k
        c.slowdown[i] = v
    return c


def c3_roofline_time(flops: float, nbytes: float, peak_flops: float, peak_bw: float,
                     efficiency: float = 0.70) -> float:
    t = ctypes.c_double()
    check(load().c3_roofline_time(flops, nbytes, peak_flops, peak_bw, efficiency, ctypes.byref(t)))
    return t.value


def c3_predict_partition(gemm_table, comm_table, t_gemm: float, t_comm: float, cus_per_xcc: int,
                         options) -> tuple:
    """(chosen CUs per XCC for the collective, predictions per option) from {k: slowdown}
    tables."""
    g, c = slowdown_curve(gemm_table), slowdown_curve(comm_table)
    opts = (ctypes.c_int32 * len(options))(*options)
    preds = (ctypes.c_double * len(options))()
    chosen = ctypes.c_int32()
    check(load().c3_predict_partition(ctypes.byref(g), ctypes.byref(c), t_gemm, t_comm,
                                      cus_per_xcc, opts, len(options), ctypes.byref(chosen), preds))
    return chosen.value, list(preds)


def c3_hybrid_share(t_gemm: float, t_sdma: float, t_cu: float) -> int:
    """Thousandths of every copy segment the hybrid mover gives the SDMA engines."""
    out = ctypes.c_int32()
    check(load().c3_hybrid_share(t_gemm, t_sdma, t_cu, ctypes.byref(out)))
    return out.value
