"""Parity at the workloads' full sizes, in the launch configuration the benchmark times
(c3_run_concurrent; SDMA, CU and hybrid movers): the whole copy destination byte-exact (for the
all-reduce: the whole reduced chunk and the whole gathered output bit-exact), the GEMM checked on
sampled outputs (random elements, corners, a full row and a full column) against the oracle,
and bit-exact at full shape with small-integer operands (where the result is unique).

Every concurrent cell's C must also be bit-identical to the GEMM's isolated run. The GC-equal
workload (4096x16384x8192 beside an 8-shard gather) runs its whole grid at full size: mover
{CU, SDMA} x GEMM CUs per XCC {all, 7/8, 3/4} (a CU-mover copy gets the complement, the SDMA
mover leaves it idle) x {communication first, GEMM first} (Section V-B and Fig. 8 of the paper
for the two controls; the Pith review's referee comment on Section V-B and its suggested test
of checking every buffer after each concurrent run)."""
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


def run_workload(c3, w, int_exact=False, movers=("sdma", "cu"), n_samples=1024, cells=None):
    """cells: (mover, GEMM CUs per XCC or None for all, comm_first) tuples; by default every
    mover of `movers` on all CUs, communication first."""
    if cells is None:
        cells = [(m, None, True) for m in movers]
    A, B = wl.gen_gemm_operands(w, int_exact=int_exact)
    dA, dB = to_dev(A), to_dev(B)
    dC = empty_bf16((w.M, w.N))
    reduced = want_red = None
    if w.copy == "gather":
        src_np = wl.gen_shards(w)
        src = [to_dev(s) for s in src_np]
        want = oracle.gather(src_np)
    elif w.copy == "allreduce":
        contribs, peers = wl.gen_allreduce(w)
        src = [to_dev(c) for c in contribs]
        dpeers = [None if p is None else to_dev(p) for p in peers]
        want_red, want = oracle.allreduce_local(contribs, peers, wl.ALLREDUCE_RANK)
        want_red, want = want_red.view(np.uint8), want.view(np.uint8)
        reduced = empty_bytes(want_red.size)
        src_np = contribs
    else:
        src_np = wl.gen_a2a_source(w)
        src = to_dev(src_np)
        want = oracle.all2all_block(src_np, w.units, w.unit_bytes)
    del src_np
    dst = empty_bytes(want.size)
    rows, cols = wl.sample_indices(w.M, w.N, n_samples, seed=w.wid, full_rows=(w.M // 3,),
                                   full_cols=(w.N - 1,))
    c32, c64, _ = oracle.gemm_elems(A, B, rows, cols)

    def check_sampled(got, label):
        sampled = got[rows, cols]
        if int_exact:
            np.testing.assert_array_equal(sampled, c32, err_msg=label)
        else:
            for ref in (c64, c32):
                rep = oracle.gemm_compare(ref, sampled)
                assert oracle.gemm_within_tolerance(rep), (label, rep)

    # the isolated GEMM: the bits every concurrent cell must reproduce
    dC.fill_(-1)
    sync()
    c3.c3_run_concurrent(c3.gemm_args(dA, dB, dC, w.M, w.N, w.K), None)
    iso_c = bf16_from_dev(dC)
    check_sampled(iso_c, "isolated")
    info = c3.c3_device_info()
    for r, (mover, keep, comm_first) in enumerate(cells, start=1):
        dC.fill_(-1 - r)
        dst.fill_(0x5A + r)
        if reduced is not None:
            reduced.fill_(0x3C + r)
        sync()
        opts = None
        if mover.startswith("hybrid:"):  # "hybrid:<engines' share in thousandths>"
            m, opts = c3.C3_MOVER_HYBRID, c3.move_opts(sdma_permille=int(mover.split(":")[1]))
        else:
            m = c3.C3_MOVER_SDMA if mover == "sdma" else c3.C3_MOVER_CU
        if w.copy == "gather":
            cargs, _keep = c3.gather_args(dst, src, w.unit_bytes, m, opts)
        elif w.copy == "allreduce":
            cargs, _keep = c3.allreduce_args(dst, reduced, src, dpeers, wl.ALLREDUCE_RANK,
                                             w.unit_bytes, m, opts)
        else:
            cargs, _keep = c3.all2all_args(dst, src, w.units, w.unit_bytes, m, opts)
        gm = cm = None
        if keep is not None:
            gm = c3.c3_cu_mask_balanced(keep)
            if m != c3.C3_MOVER_SDMA:
                cm = c3.c3_cu_mask_balanced(keep, complement=True)
        label = (f"workload {w.wid} ({w.name}, copy {w.copy_bytes // MiB} MiB) mover={mover} "
                 f"gemm_cus_per_xcc={keep or 'all'} "
                 f"{'comm-first' if comm_first else 'gemm-first'} int_exact={int_exact}")
        print(label, flush=True)
        t = c3.c3_run_concurrent(c3.gemm_args(dA, dB, dC, w.M, w.N, w.K), cargs,
                                 c3.conc_opts(gemm_mask=gm, comm_mask=cm, comm_first=comm_first))
        print(f"  t_conc={t['t_conc_ns'] / 1e6:.3f} ms", flush=True)
        assert t["comm_issued_first"] == int(comm_first)
        if gm is not None:
            assert t["gemm_applied_mask"] == list(gm), label
            assert sum(bin(x).count("1") for x in t["gemm_applied_mask"]) == keep * info["n_xcc"]
        assert oracle.first_diff(want, bytes_from_dev(dst)) == -1, f"copy mismatch ({label})"
        if reduced is not None:
            assert oracle.first_diff(want_red, bytes_from_dev(reduced)) == -1, \
                f"reduce-scatter mismatch ({label})"
        got = bf16_from_dev(dC)
        check_sampled(got, label)
        np.testing.assert_array_equal(got, iso_c, err_msg=label)
    return iso_c


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 6])
def test_full_workload(c3gpu, wid):
    run_workload(c3gpu, wl.WORKLOADS[wid], movers=("sdma", "cu", "hybrid:500"))


@pytest.mark.parametrize("total_mib", [32, 1024])
def test_full_gc_equal_sweep_ends(c3gpu, total_mib):
    run_workload(c3gpu, wl.WORKLOADS[5].with_gather_total(total_mib * MiB),
                 movers=("sdma", "hybrid:679"))


@pytest.mark.parametrize("total_mib", [256, 1024])
@pytest.mark.parametrize("mover", ["cu", "sdma"])
def test_full_gc_equal_grid(c3gpu, mover, total_mib):
    """The GC-equal workload's grid at full size: for one mover and gather size, GEMM CUs per
    XCC {all, 7/8, 3/4} x {communication first, GEMM first}."""
    info = c3gpu.c3_device_info()
    per = info["n_cu"] // info["n_xcc"]
    cells = [(mover, keep, cf) for keep in (None, per * 7 // 8, per * 3 // 4)
             for cf in (True, False)]
    run_workload(c3gpu, wl.WORKLOADS[5].with_gather_total(total_mib * MiB), cells=cells)


@pytest.mark.parametrize("wid", [2, 3])
def test_full_integer_exact(c3gpu, wid):
    run_workload(c3gpu, wl.WORKLOADS[wid], int_exact=True, movers=("sdma",), n_samples=2048)
