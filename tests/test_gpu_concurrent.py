"""GPU tests of the concurrent run (c3_run_concurrent) and the C3 controls, through the C ABI.

After every run: the copy destination is byte-exact against the oracle, C is bit-identical to
the GEMM's isolated run and within tolerance of the oracle. Also: CU-mask placement on the
hardware (workgroups only land on the CUs a mask keeps, evenly per XCC), the comm-first issue
order, and refusal of stream priorities."""
import numpy as np
import pytest

import oracle
from concurrent_gemm_dma_amd import workloads as wl
from gpu_util import bf16_from_dev, bytes_from_dev, empty_bf16, empty_bytes, to_dev

pytestmark = pytest.mark.gpu
KiB = 1 << 10
MiB = 1 << 20


def sync():
    import torch

    torch.cuda.synchronize()


def decode_placement(raw):
    """(xcc, se, sh, cu) of each probed workgroup from raw HW_ID / XCC_ID register values."""
    hw = raw[0::2].astype(np.int64)
    xcc = raw[1::2].astype(np.int64) & 0xF
    cu = (hw >> 8) & 0xF
    sh = (hw >> 12) & 0x1
    se = (hw >> 13) & 0x7
    return np.stack([xcc, se, sh, cu], axis=1)


def probe(c3, stream, n_blocks=4096):
    import torch

    out = torch.zeros(2 * n_blocks, dtype=torch.int32, device="cuda:0")
    c3.c3_probe_placement(out, n_blocks, stream)
    return decode_placement(out.cpu().numpy().view(np.uint32))


def cu_sets(places):
    per = {}
    for x, se, sh, cu in places:
        per.setdefault(int(x), set()).add((int(se), int(sh), int(cu)))
    return per


def test_cu_mask_placement(c3gpu):
    info = c3gpu.c3_device_info()
    n_xcc = info["n_xcc"]
    per_xcc = info["n_cu"] // n_xcc
    full = c3gpu.c3_stream_create(None)
    try:
        all_sets = cu_sets(probe(c3gpu, full))
    finally:
        sync()
        c3gpu.c3_stream_destroy(full)
    print("CUs seen per XCC (all):", {k: len(v) for k, v in sorted(all_sets.items())}, flush=True)
    assert len(all_sets) == n_xcc
    assert all(len(v) == per_xcc for v in all_sets.values())
    for keep in (28, 24, 4):
        kept_mask = c3gpu.c3_cu_mask_balanced(keep)
        comp_mask = c3gpu.c3_cu_mask_balanced(keep, complement=True)
        assert sum(bin(w).count("1") for w in kept_mask) == keep * n_xcc
        s_keep = c3gpu.c3_stream_create(kept_mask)
        s_comp = c3gpu.c3_stream_create(comp_mask)
        try:
            kept = cu_sets(probe(c3gpu, s_keep))
            comp = cu_sets(probe(c3gpu, s_comp))
        finally:
            sync()
            c3gpu.c3_stream_destroy(s_keep)
            c3gpu.c3_stream_destroy(s_comp)
        print(f"keep={keep}:", {k: len(v) for k, v in sorted(kept.items())},
              "complement:", {k: len(v) for k, v in sorted(comp.items())}, flush=True)
        assert sorted(kept) == list(range(n_xcc)), "a balanced mask must keep CUs on every XCC"
        for x in range(n_xcc):
            assert len(kept[x]) == keep
            assert len(comp.get(x, set())) == per_xcc - keep
            assert not (kept[x] & comp.get(x, set())), "mask and complement share a CU"


@pytest.mark.parametrize("keep", [None, 32, 28, 4])
def test_workgroups_of_one_residue_share_an_xcc(c3gpu, keep):
    """The tile GEMM groups its tiles per XCD by workgroup id mod 8 (the dispatcher deals
    workgroups to the XCDs in turn, from a start that moves between dispatches): every workgroup
    of one residue b mod n_xcc must land on one XCC, on a plain stream and under balanced CU
    masks, so that the grouping holds whatever mask the GEMM runs under."""
    info = c3gpu.c3_device_info()
    n_xcc = info["n_xcc"]
    per_xcc = info["n_cu"] // n_xcc
    if keep is not None and keep > per_xcc:
        pytest.skip(f"{keep} CUs per XCC exceed the device's {per_xcc}")
    mask = None if keep is None else c3gpu.c3_cu_mask_balanced(keep)
    st = c3gpu.c3_stream_create(mask)
    try:
        places = probe(c3gpu, st, n_blocks=2048)
    finally:
        sync()
        c3gpu.c3_stream_destroy(st)
    xcc = places[:, 0]
    b = np.arange(len(xcc))
    first = xcc[:n_xcc]
    print(f"keep={keep}: first workgroups on XCCs {first.tolist()}", flush=True)
    assert sorted(first.tolist()) == list(range(n_xcc))
    assert np.array_equal(xcc, first[b % n_xcc])


def test_priority_is_refused(c3gpu):
    with pytest.raises(c3gpu.C3Error) as e:
        c3gpu.c3_stream_create(None, priority=-1)
    assert e.value.status == c3gpu.C3_E_UNSUPPORTED
    A = to_dev(wl.gen_bf16((64, 64), ("normal", 0.0, 1.0), 1))
    C = empty_bf16((64, 64))
    with pytest.raises(c3gpu.C3Error) as e:
        c3gpu.c3_run_concurrent(c3gpu.gemm_args(A, A, C, 64, 64, 64), None,
                                c3gpu.conc_opts(use_priority=1))
    assert e.value.status == c3gpu.C3_E_UNSUPPORTED


class Case:
    """GEMM operands + copy payload on the device, with oracle expectations."""

    def __init__(self, c3, M, N, K, copy, units, unit_bytes, seed):
        self.M, self.N, self.K = M, N, K
        self.A = wl.gen_bf16((M, K), ("normal", 0.0, 1.0), seed)
        self.B = wl.gen_bf16((K, N), ("normal", 0.0, 0.02), seed + 1)
        self.dA, self.dB = to_dev(self.A), to_dev(self.B)
        self.dC = empty_bf16((M, N))
        self.copy, self.units, self.unit_bytes = copy, units, unit_bytes
        self.reduced = None
        if copy == "gather":
            self.src_np = [wl.gen_bytes(unit_bytes, seed + 10 + i) for i in range(units)]
            self.src = [to_dev(s) for s in self.src_np]
            self.want = oracle.gather(self.src_np)
        elif copy == "allreduce":
            # units = world, unit_bytes = chunk bytes; this rank is 1
            n = unit_bytes // 2
            self.rank = 1
            self.contribs_np = [wl.gen_bf16((n,), ("normal", 0.0, 1.0), seed + 10 + r)
                                for r in range(units)]
            self.peers_np = [None if i == self.rank else
                             wl.gen_bf16((n,), ("normal", 0.0, 1.0), seed + 100 + i)
                             for i in range(units)]
            self.contribs = [to_dev(c) for c in self.contribs_np]
            self.peers = [None if p is None else to_dev(p) for p in self.peers_np]
            want_red, want = oracle.allreduce_local(self.contribs_np, self.peers_np, self.rank)
            self.want_reduced = want_red.view(np.uint8)
            self.want = want.view(np.uint8)
            self.reduced = empty_bytes(unit_bytes)
        else:
            self.src_np = wl.gen_bytes(units * units * unit_bytes, seed + 10)
            self.src = to_dev(self.src_np)
            self.want = oracle.all2all_block(self.src_np, units, unit_bytes)
        self.dst = empty_bytes(self.want.size)
        self.ref = oracle.gemm_f64acc(self.A, self.B)

    def gargs(self, c3):
        return c3.gemm_args(self.dA, self.dB, self.dC, self.M, self.N, self.K)

    def cargs(self, c3, mover, opts=None):
        if self.copy == "gather":
            return c3.gather_args(self.dst, self.src, self.unit_bytes, mover, opts)
        if self.copy == "allreduce":
            return c3.allreduce_args(self.dst, self.reduced, self.contribs, self.peers, self.rank,
                                     self.unit_bytes, mover, opts)
        return c3.all2all_args(self.dst, self.src, self.units, self.unit_bytes, mover, opts)

    def poison(self, rep):
        self.dC.fill_(-1 - rep)
        self.dst.fill_((0xA5 + rep) & 0xFF)
        if self.reduced is not None:
            self.reduced.fill_((0x5A + rep) & 0xFF)
        sync()

    def check_comm(self, label):
        assert oracle.first_diff(self.want, bytes_from_dev(self.dst)) == -1, label
        if self.reduced is not None:
            assert oracle.first_diff(self.want_reduced, bytes_from_dev(self.reduced)) == -1, label


def applied(mask, n_cu):
    """The mask a run applies for a requested one: None means every CU of the device."""
    if mask is None:
        words = [0] * 8
        for b in range(n_cu):
            words[b // 32] |= 1 << (b % 32)
        return words
    return [int(w) for w in mask]


def run_cells(c3, case, cells):
    # isolated GEMM (the reference bits for every concurrent cell)
    case.poison(0)
    c3.c3_run_concurrent(case.gargs(c3), None)
    iso_c = bf16_from_dev(case.dC)
    rep = oracle.gemm_compare(case.ref, iso_c)
    assert oracle.gemm_within_tolerance(rep), rep
    info = c3.c3_device_info()
    per_xcc = info["n_cu"] // info["n_xcc"]
    for r, (mover, keep, comm_first) in enumerate(cells, start=1):
        case.poison(r)
        m = c3.C3_MOVER_CU if mover == "cu" else c3.C3_MOVER_SDMA
        gm = None if keep == per_xcc else c3.c3_cu_mask_balanced(keep)
        cm = None if (keep == per_xcc or mover == "sdma") else c3.c3_cu_mask_balanced(keep, True)
        cargs, _keep = case.cargs(c3, m)
        t = c3.c3_run_concurrent(case.gargs(c3), cargs,
                                 c3.conc_opts(gemm_mask=gm, comm_mask=cm, comm_first=comm_first))
        label = f"cell {mover}/{keep}/{'comm-first' if comm_first else 'gemm-first'}"
        case.check_comm(label)
        got_c = bf16_from_dev(case.dC)
        np.testing.assert_array_equal(got_c, iso_c, err_msg=label)
        assert t["t_conc_ns"] > 0 and t["t_conc_ns"] >= max(t["t_gemm_done_ns"], t["t_copy_done_ns"])
        assert t["comm_issued_first"] == int(comm_first)
        assert t["applied_priority"] == 0
        # the masks the run reports are the ones it was given (all CUs for "no mask"); a pure
        # SDMA gather or all-to-all runs no kernel on the communication stream
        assert t["gemm_applied_mask"] == applied(gm, info["n_cu"]), label
        comm_on_cus = mover == "cu" or case.copy == "allreduce"
        assert t["comm_applied_mask"] == (applied(cm, info["n_cu"]) if comm_on_cus
                                          else [0] * c3.C3_MAX_MASK_WORDS), label
        if mover == "sdma":
            assert t["engines_used"] != 0 and t["n_chunks"] >= 1
        if case.copy == "allreduce":
            assert t["reduce_gpu_ms"] > 0 and 0 < t["t_reduce_done_ns"] <= t["t_conc_ns"]
            if mover == "sdma":
                # the engines' all-gather is issued after the reduce-scatter was seen complete
                assert t["t_copy_done_ns"] >= t["t_reduce_done_ns"]
                assert t["copy_gpu_ms"] >= t["reduce_gpu_ms"]
        print(label, {k: t[k] for k in ("t_conc_ns", "t_gemm_done_ns", "t_copy_done_ns",
                                        "gemm_gpu_ms", "copy_gpu_ms", "engines_used")}, flush=True)


def all_cells(c3):
    info = c3.c3_device_info()
    per = info["n_cu"] // info["n_xcc"]
    return [(mv, keep, cf) for mv in ("cu", "sdma") for keep in (per, per * 7 // 8, per * 3 // 4)
            for cf in (False, True)]


def test_concurrent_tiny_all_cells(c3gpu):
    """512^3 GEMM with an 8 x 1 MiB gather, every mover x mask x order cell."""
    case = Case(c3gpu, 512, 512, 512, "gather", 8, MiB, 9000)
    run_cells(c3gpu, case, all_cells(c3gpu))


def test_concurrent_all2all(c3gpu):
    case = Case(c3gpu, 1024, 1032, 1024, "all2all", 8, 256 * 1024, 9100)
    run_cells(c3gpu, case, [("cu", 32, False), ("sdma", 32, True), ("cu", 28, True),
                            ("sdma", 28, False)])


def test_comm_first_issues_later_transfers_after_the_gemm(c3gpu):
    """Communication first beside a GEMM with more transfers than engines (an 8 x 8 all-to-all of
    256 KiB blocks, one transfer per block): each engine's first transfer goes before the GEMM
    launch and the others right after it. All 64 are issued and land byte-exact; a dropped,
    failed or stuck transfer among the later ones is caught or reported like one among the
    first, after both operations finished, with C unchanged; the library stays usable."""
    n_eng = bin(c3gpu.c3_device_info()["sdma_engine_mask"]).count("1")
    ub = 256 * KiB
    case = Case(c3gpu, 1024, 1032, 1024, "all2all", 8, ub, 9150)
    case.poison(0)
    c3gpu.c3_run_concurrent(case.gargs(c3gpu), None)
    iso_c = bf16_from_dev(case.dC)
    first = c3gpu.conc_opts(comm_first=True)

    def run(rep, **fault):
        case.poison(rep)
        cargs, _keep = case.cargs(c3gpu, c3gpu.C3_MOVER_SDMA,
                                  c3gpu.move_opts(chunk_bytes=ub, **fault))
        try:
            return c3gpu.c3_run_concurrent(case.gargs(c3gpu), cargs, first)
        finally:
            np.testing.assert_array_equal(bf16_from_dev(case.dC), iso_c, err_msg=str(fault))

    t = run(1)
    case.check_comm("comm-first, 64 transfers")
    assert t["n_chunks"] == 64 and t["comm_issued_first"] == 1
    late = min(n_eng + 3, 63)  # issued after the GEMM launch
    print(f"engines {n_eng}, faulted transfer {late}", flush=True)
    # dropped: the call succeeds and exactly that transfer's block is stale
    run(2, fault_mode=c3gpu.C3_FAULT_DROP_CHUNK, fault_chunk=late)
    got = bytes_from_dev(case.dst)
    d = (late % 8) * 8 + late // 8  # source block (late // 8, late % 8) lands at block d
    assert oracle.first_diff(case.want[d * ub:(d + 1) * ub], got[d * ub:(d + 1) * ub]) != -1
    assert oracle.first_diff(case.want[:d * ub], got[:d * ub]) == -1
    assert oracle.first_diff(case.want[(d + 1) * ub:], got[(d + 1) * ub:]) == -1
    with pytest.raises(c3gpu.C3Error) as e:
        run(3, fault_mode=c3gpu.C3_FAULT_ERROR_CHUNK, fault_chunk=late)
    assert e.value.status == c3gpu.C3_E_HSA
    with pytest.raises(c3gpu.C3Error) as e:
        run(4, fault_mode=c3gpu.C3_FAULT_STUCK_CHUNK, fault_chunk=63, timeout_ms=300)
    assert e.value.status == c3gpu.C3_E_TIMEOUT
    run(5)
    case.check_comm("comm-first after the faults")


def test_concurrent_skinny_gemm(c3gpu):
    case = Case(c3gpu, 16, 4096, 2048, "gather", 8, 2 * MiB + 16, 9200)
    run_cells(c3gpu, case, [("cu", 32, True), ("sdma", 32, True), ("sdma", 28, False)])


def test_concurrent_allreduce(c3gpu):
    """All-reduce local share (8 ranks x 1 MiB chunk): reduce-scatter on CUs + all-gather by
    either mover, concurrent with a GEMM, every mask / order cell."""
    case = Case(c3gpu, 512, 768, 1024, "allreduce", 8, MiB, 9500)
    run_cells(c3gpu, case, all_cells(c3gpu))


def test_concurrent_allreduce_isolated_and_skinny(c3gpu):
    case = Case(c3gpu, 16, 2048, 1024, "allreduce", 8, 2 * MiB + 6, 9600)
    run_cells(c3gpu, case, [("cu", 32, True), ("sdma", 32, True), ("sdma", 28, False)])
    for mover in (c3gpu.C3_MOVER_CU, c3gpu.C3_MOVER_SDMA):
        case.poison(7)
        cargs, _keep = case.cargs(c3gpu, mover)
        t = c3gpu.c3_run_concurrent(None, cargs, c3gpu.conc_opts(flush_bytes=64 * MiB))
        case.check_comm(f"isolated all-reduce, mover {mover}")
        assert t["t_gemm_done_ns"] == 0 and t["t_copy_done_ns"] > 0 and t["reduce_gpu_ms"] > 0


def test_concurrent_tagged_gather(c3gpu):
    """A gather in the diagnostic pattern (each 8-byte word = shard << 56 | its destination
    offset) overlapped with a GEMM, for every mover: any word out of place is named."""
    c3 = c3gpu
    n, sb = 8, MiB
    case = Case(c3, 1000, 2000, 1000, "gather", n, sb, 7100)
    case.src_np = wl.gen_tagged_shards(n, sb)
    case.src = [to_dev(s) for s in case.src_np]
    case.want = oracle.gather(case.src_np)
    cells = [(c3.C3_MOVER_CU, None), (c3.C3_MOVER_SDMA, c3.move_opts(chunk_bytes=96 * KiB)),
             (c3.C3_MOVER_HYBRID, c3.move_opts(sdma_permille=400))]
    for r, (m, opts) in enumerate(cells, start=1):
        for comm_first in (False, True):
            case.poison(2 * r + comm_first)
            cargs, _keep = case.cargs(c3, m, opts)
            c3.c3_run_concurrent(case.gargs(c3), cargs, c3.conc_opts(comm_first=comm_first))
            label = f"tagged gather mover={m} comm_first={comm_first}"
            print(label, flush=True)
            assert oracle.explain_tagged_gather(bytes_from_dev(case.dst), n, sb) == [], label
            case.check_comm(label)
            rep = oracle.gemm_compare(case.ref, bf16_from_dev(case.dC))
            assert oracle.gemm_within_tolerance(rep), (label, rep)


def test_isolated_copy_via_run_concurrent(c3gpu):
    case = Case(c3gpu, 64, 64, 64, "gather", 8, MiB, 9300)
    for mover in (c3gpu.C3_MOVER_CU, c3gpu.C3_MOVER_SDMA):
        case.poison(3)
        cargs, _keep = case.cargs(c3gpu, mover)
        t = c3gpu.c3_run_concurrent(None, cargs, c3gpu.conc_opts(flush_bytes=64 * MiB))
        assert oracle.first_diff(case.want, bytes_from_dev(case.dst)) == -1
        assert t["t_gemm_done_ns"] == 0 and t["t_copy_done_ns"] > 0


def test_concurrent_overlap_rejected(c3gpu):
    case = Case(c3gpu, 64, 64, 64, "gather", 2, 4096, 9400)
    import ctypes

    g = c3gpu.c3_gemm_args(case.dA.data_ptr(), case.dB.data_ptr(), case.src[0].data_ptr(), 64, 64, 64)
    cargs, _keep = case.cargs(c3gpu, c3gpu.C3_MOVER_CU)
    st = c3gpu.call("c3_run_concurrent", ctypes.byref(g), ctypes.byref(cargs), None, None)
    assert st == c3gpu.C3_E_OVERLAP
    sync()
