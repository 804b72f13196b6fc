#!/usr/bin/env python3
"""Benchmark of the C3 hot path on one MI355X: a bf16 GEMM concurrent with a collective-shaped
copy, moved by the SDMA engines (headline) and by a CU kernel (baseline).

Default mode (`--mode c3`, the contract): a step is one concurrent run (c3_run_concurrent) of
the whole path over the workload: GEMM and copy issued (communication first), both completed.
The default workload is the largest one: the 405B-class GEMM 8192x53248x16384 beside the
all-to-all block transpose of 8x8 blocks of 8 MiB (`--workload` picks another).
Every round runs the isolated GEMM and, per mover, the isolated copy then the concurrent step,
in an order shuffled per round (fixed seeds), so clock and thermal drift hit isolated and
concurrent times, and every mover, alike. Before
every run, untimed: outputs poisoned, then the library reads 512 MiB of scratch (Infinity Cache
flush) before its clock starts. After every run, untimed: each destination range is compared
byte for byte with its source on the device (the copy's definition) and C bit for bit with the
isolated GEMM's C. The CPU oracle runs only in the cpu_baseline leg: it computes a bounded
sample of C's rows (timed), which are then compared with the GPU's rows (untimed).

`--workload 6` runs the same protocol on the all-reduce workload (reduce-scatter on the CUs,
all-gather by the mover under test).

A third cell, the hybrid mover (every copy segment split between the SDMA engines and the CU
kernel, the engines' share chosen by c3_hybrid_share from isolated times measured in untimed
runs before the timed rounds), runs beside the two; `--hybrid-permille` fixes the share, -2
drops the cell. The headline value stays the SDMA mover's.

Other modes print one JSON line per measured cell:
  --mode movers    isolated copy GB/s vs size, CU mover variants, SDMA engine/chunk counts and
                   hybrid shares
  --mode grid      the GC-equal workload's gather-size sweep: mover (CU, SDMA, hybrid) x GEMM
                   CU mask x order
  --mode cus       isolated GEMM time and CU-copy GB/s under balanced CU masks
  --mode partition CU-partitioning sweep (c3_rp) over 30 GEMM x collective scenarios and the
                   slowdown-lookup-table heuristic (paired and isolated calibration tables)
                   scored against it
  --mode hybrid    the hybrid mover's concurrent time against its engine share on 8 workloads,
                   and the share c3_hybrid_share picks scored against the best of the sweep
  --mode ksteps    the tile GEMM at 8192 x 28672 x K for K = 1024 ... 16384 (per-tile start/end
                   cost against per-K-step cost)
  --mode mfma_ceiling  the matrix cores' sustained bf16 rate with nothing but MFMAs in flight
                   (the power-limited ceiling for any GEMM kernel on this chip)
  --mode gemm_data the tile GEMM of workloads 2 and 4 on the workloads' operand distributions,
                   small integers and zeros (same cycles, clock set by the operands' power)
  --mode gemm_vs_vendor  the library's GEMM against torch.matmul (hipBLASLt) on the same
                   operands, alternating single launches and back-to-back batches (a reference
                   point for kernel quality; torch's result is not used for anything else)

Prints ONE JSON line on stdout in the default mode. Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import random
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MiB = 1 << 20
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
METRIC = "concurrent GEMM TFLOP/s + copy GB/s; realized % of ideal C3 speedup"
FLUSH_BYTES = 512 * MiB
# Rounds of the MFMA rate probe run before every run of the C3 mode (about 2.6 ms on 256 CUs): a
# fixed MFMA load that puts the chip in the same power state before every cell.
PRECOND_ITERS = 8400


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    path = os.path.join(ROOT, "concurrent_gemm_dma_amd", "csrc", "gemm.hip")
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def measured_traffic(kernel: str, w):
    """HBM-side bytes per launch of `kernel` on workload `w`, from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE record (each scaled by its calibration against a copy kernel of
    known size), or None when there is no record or the kernel source changed since it was
    taken."""
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kernel}@{w.name}")
    if not rec or rec.get("source_sha256") != kernel_source_hash():
        return None
    return int(rec["fetch_kib"] * 1024 * rec["fetch_scale"] + rec["write_kib"] * 1024 * rec["write_scale"])


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed rounds (default 50 in the c3 mode, whose headline uplift divides by "
                        "an ideal of only 7%% on workload 4, so its medians need the rounds; 20 in "
                        "the other modes)")
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--mode", default="c3",
                   choices=["c3", "movers", "grid", "cus", "partition", "gemm_vs_vendor",
                            "hybrid", "ksteps", "mfma_ceiling", "gemm_data"])
    p.add_argument("--workload", type=int, default=4,
                   help="workload id (1..6); 4 = the 405B-class GEMM beside the 512 MiB all-to-all")
    p.add_argument("--gather-mib", type=int, default=0, help="workload 5: total gather MiB")
    p.add_argument("--keep-per-xcc", type=int, default=0,
                   help="GEMM CU mask: CUs kept per XCC (0 = all)")
    p.add_argument("--gemm-first", action="store_true", help="issue the GEMM first")
    p.add_argument("--sdma-engines", type=int, default=0,
                   help="SDMA mover: use only the first N engines found (0 = all)")
    p.add_argument("--cu-nontemporal", action="store_true",
                   help="CU mover: streaming (non-temporal) loads and stores")
    p.add_argument("--hybrid-permille", type=int, default=-1,
                   help="hybrid mover: thousandths of the copy on the SDMA engines (-1 = chosen "
                        "by c3_hybrid_share from isolated times measured before the timed runs; "
                        "-2 = no hybrid cell)")
    p.add_argument("--shapes", default="",
                   help="gemm_vs_vendor: comma-separated MxNxK list instead of the workloads' shapes")
    p.add_argument("--no-precondition", action="store_true",
                   help="c3 and grid modes: no fixed MFMA load before each run (the earlier protocol)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--profile", action="store_true",
                   help="no verification or CPU baseline (for rocprofv3 runs)")
    a = p.parse_args()
    if a.steps is None:
        a.steps = 50 if a.mode == "c3" else 20
    return a


def make_preconditioner(c3, info, args):
    """Every run of the C3 and grid modes starts from the same power state. The chip's clock
    follows its recent load: it falls during light or memory-bound work (a lone copy, the checks)
    and climbs back under MFMA load, so a GEMM launched after a light run starts slower than one
    launched after a heavy run. Before each run, timed or not, a fixed MFMA load of about 2.6 ms
    (c3_probe_mfma_rate) brings the chip to the state a GEMM in a busy training step starts from;
    then come the poison and the flush, the same for every cell. Without it a concurrent step that
    always follows its mover's lone copy started from a lower clock than the isolated GEMM.
    `--no-precondition` turns it off (the earlier protocol)."""
    import torch

    probe_out = torch.empty(info["n_cu"] * 256, dtype=torch.float64, device="cuda:0")

    def precondition():
        if not args.no_precondition:
            c3.c3_probe_mfma_rate(probe_out, info["n_cu"], PRECOND_ITERS, 1, None)

    return precondition


class Setup:
    """Seeded inputs of one workload resident in HBM, plus the per-run checks."""

    def __init__(self, c3, w, with_gemm=True, check=True, with_comm=True):
        import numpy as np
        import torch

        from concurrent_gemm_dma_amd import workloads as wl

        self.c3, self.w, self.torch, self.np, self.check = c3, w, torch, np, check
        dev = torch.device("cuda:0")
        t0 = time.time()
        if with_gemm:
            self.A, self.B = wl.gen_gemm_operands(w)
            self.dA = torch.from_numpy(self.A.view(np.int16)).to(dev)
            self.dB = torch.from_numpy(self.B.view(np.int16)).to(dev)
            self.dC = torch.empty((w.M, w.N), dtype=torch.int16, device=dev)
            self.gargs = c3.gemm_args(self.dA, self.dB, self.dC, w.M, w.N, w.K)
        self.iso_c = None
        self.dred = None
        if not with_comm:
            self.ddst = torch.empty(0, dtype=torch.uint8, device=dev)
        elif w.copy == "gather":
            self.dsrc = [torch.from_numpy(s).to(dev) for s in wl.gen_shards(w)]
            total = w.units * w.unit_bytes
        elif w.copy == "allreduce":
            contribs, peers = wl.gen_allreduce(w)
            self.rank = wl.ALLREDUCE_RANK
            self.dsrc = [torch.from_numpy(c.view(np.int16)).to(dev) for c in contribs]
            self.dpeers = [None if p is None else torch.from_numpy(p.view(np.int16)).to(dev)
                           for p in peers]
            self.dred = torch.empty(w.unit_bytes // 2, dtype=torch.int16, device=dev)
            # the reduced chunk by its definition, with plain torch ops on the device: fp32 sum
            # in rank order starting from rank 0, one rounding to bf16
            acc = self.dsrc[0].view(torch.bfloat16).float()
            for c in self.dsrc[1:]:
                acc = acc + c.view(torch.bfloat16).float()
            self.want_red = acc.to(torch.bfloat16).view(torch.int16)
            del acc
            total = w.units * w.unit_bytes
        else:
            self.dsrc = torch.from_numpy(wl.gen_a2a_source(w)).to(dev)
            total = w.units * w.units * w.unit_bytes
        if with_comm:
            self.ddst = torch.empty(total, dtype=torch.uint8, device=dev)
        self.poison_i = 0
        torch.cuda.synchronize()
        log(f"{w.name}: inputs resident in HBM in {time.time() - t0:.1f} s")

    def cargs(self, mover, opts=None):
        w = self.w
        if w.copy == "gather":
            return self.c3.gather_args(self.ddst, self.dsrc, w.unit_bytes, mover, opts)
        if w.copy == "allreduce":
            return self.c3.allreduce_args(self.ddst, self.dred, self.dsrc, self.dpeers, self.rank,
                                          w.unit_bytes, mover, opts)
        return self.c3.all2all_args(self.ddst, self.dsrc, w.units, w.unit_bytes, mover, opts)

    def poison(self):
        self.poison_i += 1
        if hasattr(self, "dC"):
            self.dC.fill_(-1 - (self.poison_i % 7))
        self.ddst.fill_((0xA5 + self.poison_i) & 0xFF)
        if self.dred is not None:
            self.dred.fill_(-2 - (self.poison_i % 5))
        self.torch.cuda.synchronize()

    def verify_copy(self, label):
        """Every destination range equals its source range, byte for byte (on the device)."""
        if not self.check:
            return
        w, teq = self.w, self.torch.equal
        if w.copy == "gather":
            sb = w.unit_bytes
            for i, s in enumerate(self.dsrc):
                if not teq(self.ddst[i * sb:(i + 1) * sb], s):
                    raise SystemExit(f"{label}: gather shard {i} differs from its destination range")
        elif w.copy == "allreduce":
            cb = w.unit_bytes
            if not teq(self.dred, self.want_red):
                raise SystemExit(f"{label}: reduced chunk differs from the fp32 rank-order sum")
            for i in range(w.units):
                src = self.dred if i == self.rank else self.dpeers[i]
                if not teq(self.ddst[i * cb:(i + 1) * cb], src.view(self.torch.uint8)):
                    raise SystemExit(f"{label}: all-gather slot {i} differs from its chunk")
        else:
            g, bb = w.units, w.unit_bytes
            for i in range(g):
                for j in range(g):
                    src = self.dsrc[(i * g + j) * bb:(i * g + j + 1) * bb]
                    dst = self.ddst[(j * g + i) * bb:(j * g + i + 1) * bb]
                    if not teq(src, dst):
                        raise SystemExit(f"{label}: all-to-all block ({i},{j}) misplaced")

    def verify_c(self, label):
        """C is bit-identical to the first isolated GEMM's C (deterministic kernel)."""
        if self.iso_c is None:
            self.iso_c = self.dC.clone()
        elif self.check and not self.torch.equal(self.dC, self.iso_c):
            raise SystemExit(f"{label}: C differs from the isolated GEMM")


def gpu_state() -> dict | None:
    """Current shader / memory clock levels, power and temperatures of the AMD GPUs, read from the
    driver's sysfs files (no child process), or None when they are not readable."""
    import glob

    def read(path):
        try:
            with open(path) as f:
                return f.read().strip()
        except OSError:
            return None

    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card[0-9]*/device")):
        if read(os.path.join(dev, "vendor")) != "0x1002":
            continue
        st = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            txt = read(os.path.join(dev, name))
            if txt:
                cur = [ln for ln in txt.splitlines() if ln.rstrip().endswith("*")]
                st[name] = cur[0].split(":", 1)[-1].strip(" *") if cur else txt.splitlines()[-1]
        for hw in glob.glob(os.path.join(dev, "hwmon", "hwmon*")):
            for fname, key, scale in (("power1_average", "power_w", 1e-6), ("power1_input", "power_w", 1e-6),
                                      ("temp1_input", "temp_edge_c", 1e-3), ("temp2_input", "temp_junction_c", 1e-3),
                                      ("temp3_input", "temp_mem_c", 1e-3), ("freq1_input", "sclk_mhz", 1e-6)):
                v = read(os.path.join(hw, fname))
                if v is not None and key not in st:
                    try:
                        st[key] = round(int(v) * scale, 1)
                    except ValueError:
                        pass
        if st:
            out[os.path.basename(os.path.dirname(dev))] = st
    return out or None


def cpu_baseline_and_parity(args, s, w, oracle_seconds):
    """The oracle as it stands, on a bounded sample of the workload (rows 0..r-1 of C, sized to
    take about `oracle_seconds` on the host cores), timed; then those rows are compared with the
    GPU's C (|d| <= 1e-2 max(1,|ref|) elementwise, relative Frobenius <= 1e-3)."""
    import numpy as np

    import oracle

    nthreads = oracle.threads(0)
    t1 = time.time()
    oracle.gemm_f32acc(s.A, s.B, rows=(0, 1))
    dt = max(time.time() - t1, 1e-3)
    r = int(max(1, min(w.M, oracle_seconds / dt)))
    t1 = time.time()
    ref = oracle.gemm_f32acc(s.A, s.B, rows=(0, r))
    dt = time.time() - t1
    got = s.iso_c[:r].cpu().numpy().view(np.uint16)
    rep = oracle.gemm_compare(ref, got)
    if not oracle.gemm_within_tolerance(rep):
        raise SystemExit(f"GEMM parity failure vs oracle on rows 0..{r - 1}: {rep}")
    log(f"oracle rows 0..{r - 1}: GPU C within tolerance ({rep['n_diff']} of {rep['n']} elements "
        f"differ by rounding, max scaled err {rep['max_scaled_err']:.2e})")
    cpu_model = "?"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    cpu = {"value": round(2.0 * r * w.N * w.K / dt / 1e12, 6), "unit": "TFLOP/s",
           "cores": nthreads, "kind": "oracle",
           "sample": f"fp32-accumulate triple-loop GEMM oracle, rows 0..{r - 1} of C "
                     f"({r}x{w.N}x{w.K}, {2.0 * r * w.N * w.K / 1e9:.1f} GFLOP) in {dt:.1f} s "
                     f"on {nthreads} threads of {os.cpu_count()} logical CPUs ({cpu_model})"}
    parity = {"rows": r, "elements": rep["n"], "differ_by_rounding": rep["n_diff"],
              "max_scaled_err": rep["max_scaled_err"], "frob_rel": rep["frob_rel"]}
    # the oracle's collective on the whole workload (inputs regenerated from the same seeds,
    # untimed; single host thread), for the copy half of the path
    from concurrent_gemm_dma_amd import workloads as wl
    if w.copy == "gather":
        shards = wl.gen_shards(w)
        t1 = time.time()
        oracle.gather(shards)
    elif w.copy == "all2all":
        src = wl.gen_a2a_source(w)
        t1 = time.time()
        oracle.all2all_block(src, w.units, w.unit_bytes)
    else:
        contribs, peers = wl.gen_allreduce(w)
        t1 = time.time()
        oracle.allreduce_local(contribs, peers, wl.ALLREDUCE_RANK)
    dtc = max(time.time() - t1, 1e-6)
    cpu["copy"] = {"value": round(w.comm_hbm_bytes / dtc / 1e9, 2), "unit": "GB/s", "cores": 1,
                   "sample": f"oracle {w.copy} of the whole workload ({w.comm_hbm_bytes / MiB:.0f} "
                             f"MiB of algorithmic traffic) in {dtc * 1e3:.1f} ms on one thread"}
    return cpu, parity


def mover_cell(c3, t_gemm, r, *, comm_bytes, flops, hbm_total, best_copy):
    """One mover's cell of the c3 mode from its timed rounds. t_gemm: the isolated GEMM's host
    times (s), one per round; r: the mover's per-round lists "t_copy", "t_conc" (host, s),
    "c_gpu" (the copy's GPU time, s), "gk" (the GEMM kernel's event time in the concurrent run,
    s) and "done" ((GEMM, copy) completion seen by the library, ms from the first issue).
    The speedup metrics take the median of each of the three times. Each round's own three times
    (run close together, in the same power state) also give an uplift per round: their median is
    the paired estimate, and their quartiles the dispersion."""
    T_gemm = statistics.median(t_gemm)
    T_copy = statistics.median(r["t_copy"])
    T_conc_med = statistics.median(r["t_conc"])
    T_conc_mean = statistics.mean(r["t_conc"])
    c_gpu_med = statistics.median(r["c_gpu"])
    m = c3.c3_derive_metrics(T_gemm, T_copy, T_conc_med, hbm_total, PEAK_HBM_GBPS * 1e9)
    per_round = sorted(c3.c3_derive_metrics(tg, tc, tx, hbm_total, PEAK_HBM_GBPS * 1e9)
                       ["uplift_fraction"] for tg, tc, tx in zip(t_gemm, r["t_copy"], r["t_conc"]))
    copy_done_s = statistics.median(d[1] for d in r["done"]) * 1e-3
    return {
        "t_copy_ms": T_copy * 1e3, "t_conc_ms": T_conc_med * 1e3,
        "t_conc_ms_mean": T_conc_mean * 1e3,
        "t_conc_ms_min": min(r["t_conc"]) * 1e3, "t_conc_ms_max": max(r["t_conc"]) * 1e3,
        "t_conc_ms_std": (statistics.pstdev(r["t_conc"]) * 1e3) if len(r["t_conc"]) > 1 else 0.0,
        "copy_gbps_isolated": comm_bytes / T_copy / 1e9,
        "copy_gbps_isolated_engine_clock": (comm_bytes / c_gpu_med / 1e9 if c_gpu_med > 0 else None),
        "gemm_tflops_concurrent": flops / T_conc_mean / 1e12,
        # the copy's own rate beside the GEMM: its bytes over the time from the first issue to the
        # copy's observed completion (not over the whole concurrent run)
        "copy_gbps_concurrent": comm_bytes / copy_done_s / 1e9 if copy_done_s > 0 else None,
        "uplift_paired_median": statistics.median(per_round),
        "uplift_per_round_p25_median_p75": [per_round[len(per_round) // 4],
                                            statistics.median(per_round),
                                            per_round[(3 * len(per_round)) // 4]],
        "gemm_kernel_ms_concurrent": statistics.mean(r["gk"]) * 1e3,
        # overlap evidence on the library's clock: when each operation was seen complete
        "gemm_done_ms_median": statistics.median(d[0] for d in r["done"]),
        "copy_done_ms_median": statistics.median(d[1] for d in r["done"]),
        "speedup_vs_best_serial": (T_gemm + best_copy) / T_conc_med,
        **{k: m[k] for k in ("ideal_speedup", "speedup", "uplift_fraction", "ratio_of_ideal",
                             "gemm_slowdown", "hbm_ceiling", "taxonomy")},
        # overlap cannot beat running both at their isolated speeds: a realized speedup above the
        # ideal means the isolated times were measured slow (a measurement anomaly)
        "anomaly_speedup_above_ideal": bool(m["speedup"] > m["ideal_speedup"] * 1.001),
    }


def run_c3(args, c3, info):
    from concurrent_gemm_dma_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    if args.gather_mib:
        w = w.with_gather_total(args.gather_mib * MiB)
    M, N, K = w.M, w.N, w.K
    flops = w.gemm_flops
    copy_bytes = w.copy_bytes  # payload S
    comm_bytes = w.comm_hbm_bytes  # algorithmic HBM bytes of the local share (2S for copies)
    s = Setup(c3, w, check=not args.profile)

    gmask = c3.c3_cu_mask_balanced(args.keep_per_xcc) if args.keep_per_xcc else None
    comm_first = not args.gemm_first
    movers = (("sdma", c3.C3_MOVER_SDMA), ("cu", c3.C3_MOVER_CU))
    sdma_opts = None
    if args.sdma_engines:
        engines = [1 << b for b in range(32) if info["sdma_engine_mask"] >> b & 1][:args.sdma_engines]
        sdma_opts = c3.move_opts(engine_mask=sum(engines))
    cu_opts = c3.move_opts(nontemporal=1) if args.cu_nontemporal else None
    copy_args = {name: s.cargs(mv, sdma_opts if mv == c3.C3_MOVER_SDMA else cu_opts)
                 for name, mv in movers}
    iso_g_opts = c3.conc_opts(gemm_mask=gmask, flush_bytes=FLUSH_BYTES)
    iso_c_opts = c3.conc_opts(flush_bytes=FLUSH_BYTES)
    torch = s.torch
    precondition = make_preconditioner(c3, info, args)
    hybrid_pm = None
    if args.hybrid_permille != -2:
        hybrid_pm = args.hybrid_permille
        if hybrid_pm < 0:
            # the engines' share from isolated times (best of two untimed runs of each)
            cal = {"gemm": [], "sdma": [], "cu": []}
            for _ in range(2):
                precondition()
                s.poison()
                cal["gemm"].append(c3.c3_run_concurrent(s.gargs, None, iso_g_opts)["t_conc_ns"])
                s.verify_c("calibration GEMM")
                for name in ("sdma", "cu"):
                    precondition()
                    s.poison()
                    cal[name].append(c3.c3_run_concurrent(None, copy_args[name][0],
                                                          iso_c_opts)["t_conc_ns"])
                    s.verify_copy(f"calibration {name} copy")
            hybrid_pm = c3.c3_hybrid_share(min(cal["gemm"]) * 1e-9, min(cal["sdma"]) * 1e-9,
                                           min(cal["cu"]) * 1e-9)
        log(f"hybrid mover: {hybrid_pm / 10:.1f}% of every segment on the SDMA engines")
        movers += (("hybrid", c3.C3_MOVER_HYBRID),)
        hy = c3.move_opts(sdma_permille=hybrid_pm, nontemporal=int(args.cu_nontemporal))
        if sdma_opts is not None:
            hy.engine_mask = sdma_opts.engine_mask
        copy_args["hybrid"] = s.cargs(c3.C3_MOVER_HYBRID, hy)
    conc = {}
    for name, mv in movers:
        cmask = None
        if gmask is not None and (mv != c3.C3_MOVER_SDMA or w.copy == "allreduce"):
            cmask = c3.c3_cu_mask_balanced(args.keep_per_xcc, complement=True)
        conc[name] = c3.conc_opts(gemm_mask=gmask, comm_mask=cmask, comm_first=comm_first,
                                  flush_bytes=FLUSH_BYTES)

    t_gemm, g_gpu = [], []
    rec = {name: {"t_copy": [], "c_gpu": [], "t_conc": [], "gk": [], "rs": [], "done": []}
           for name, _ in movers}
    torch.cuda.synchronize()
    state_before = gpu_state()
    wall0 = time.time()
    # One round runs the isolated GEMM and, per mover, its isolated copy then its concurrent
    # step, in an order shuffled per round (seeded by the round number), so that no cell always
    # takes the same position or follows the same neighbour: the state a long GEMM leaves the
    # chip in (clock, temperature) then biases no cell.
    units = ["gemm"] + [name for name, _ in movers]
    for i in range(args.warmup + args.steps):
        if i == args.warmup:
            torch.cuda.synchronize()
            wall0 = time.time()
        timed = i >= args.warmup
        order = list(units)
        random.Random(1000 + i).shuffle(order)
        for name in order:
            if name == "gemm":
                precondition()
                s.poison()
                t = c3.c3_run_concurrent(s.gargs, None, iso_g_opts)
                s.verify_c(f"isolated GEMM {i}")
                if timed:
                    t_gemm.append(t["t_conc_ns"] * 1e-9)
                    g_gpu.append(t["gemm_gpu_ms"] * 1e-3)
                continue
            ca = copy_args[name][0]
            r = rec[name]
            precondition()
            s.poison()
            t = c3.c3_run_concurrent(None, ca, iso_c_opts)
            s.verify_copy(f"isolated {name} copy {i}")
            if timed:
                r["t_copy"].append(t["t_conc_ns"] * 1e-9)
                r["c_gpu"].append(t["copy_gpu_ms"] * 1e-3)
                r["rs"].append(t["reduce_gpu_ms"] * 1e-3)
            precondition()
            s.poison()
            t = c3.c3_run_concurrent(s.gargs, ca, conc[name])
            s.verify_copy(f"{name} step {i}")
            s.verify_c(f"{name} step {i}")
            if timed:
                r["t_conc"].append(t["t_conc_ns"] * 1e-9)
                r["gk"].append(t["gemm_gpu_ms"] * 1e-3)
                r["done"].append((t["t_gemm_done_ns"] * 1e-6, t["t_copy_done_ns"] * 1e-6))
    torch.cuda.synchronize()
    wall = time.time() - wall0
    state_after = gpu_state()
    T_gemm = statistics.median(t_gemm)
    log(f"isolated GEMM: median {T_gemm * 1e3:.3f} ms  ({flops / T_gemm / 1e12:.1f} TFLOP/s host, "
        f"{flops / statistics.median(g_gpu) / 1e12:.1f} TFLOP/s events)")

    results = {}
    # the faster of the paper's two movers: a cell cannot look good against its own slow serial time
    best_copy = min(statistics.median(rec[name]["t_copy"]) for name in ("sdma", "cu"))
    for name, _ in movers:
        r = rec[name]
        res = mover_cell(c3, t_gemm, r, comm_bytes=comm_bytes, flops=flops,
                         hbm_total=float(w.gemm_bytes + comm_bytes), best_copy=best_copy)
        if name == "hybrid":
            res["sdma_permille"] = hybrid_pm
        if w.copy == "allreduce":
            res["reduce_scatter_ms_isolated"] = statistics.median(r["rs"]) * 1e3
            res["reduce_scatter_gbps_isolated"] = ((w.units + 1) * w.unit_bytes
                                                   / statistics.median(r["rs"]) / 1e9)
        results[name] = res
        if res["anomaly_speedup_above_ideal"]:
            log(f"{name}: WARNING realized speedup {res['speedup']:.4f} above the ideal "
                f"{res['ideal_speedup']:.4f}: isolated timings suspect")
        q = res["uplift_per_round_p25_median_p75"]
        log(f"{name}: T_copy {res['t_copy_ms']:.3f} ms ({res['copy_gbps_isolated']:.0f} GB/s), "
            f"T_conc median {res['t_conc_ms']:.3f} ms (mean {res['t_conc_ms_mean']:.3f}), "
            f"S {res['speedup']:.4f} / ideal {res['ideal_speedup']:.4f}, "
            f"uplift {q[1] * 100:.1f}% paired (per-round quartiles {q[0] * 100:.1f}.."
            f"{q[2] * 100:.1f}%; {res['uplift_fraction'] * 100:.1f}% from the medians)")

    # ---- roofline of the dominant kernel (the GEMM): HIP events recorded by the library on the
    # GEMM's own stream around every launch of the timed SDMA-concurrent steps ----
    gemm_kernel_s = statistics.mean(rec["sdma"]["gk"])
    roofline = {"bound": "mfma" if M > 64 else "hbm"}
    if M > 64:
        a = flops / gemm_kernel_s / 1e12
        roofline.update(achieved=round(a, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                        frac=round(a / PEAK_BF16_TFLOPS, 4))
    else:
        a = w.gemm_bytes / gemm_kernel_s / 1e9
        roofline.update(achieved=round(a, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                        frac=round(a / PEAK_HBM_GBPS, 4))
    roofline["kernel"] = "gemm_bf16_tile256_dma" if M > 64 else "gemm_bf16_skinny (+splitk_reduce)"
    roofline["traffic"] = measured_traffic(roofline["kernel"], w)
    roofline["kernel_ms"] = round(gemm_kernel_s * 1e3, 4)

    cpu, parity = None, None
    if not args.no_cpu_baseline and not args.profile:
        cpu, parity = cpu_baseline_and_parity(args, s, w, args.cpu_seconds)
        log("cpu baseline:", cpu)

    head = results["sdma"]
    out = {
        "metric": METRIC,
        "value": round(head["gemm_tflops_concurrent"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["t_conc_ms_mean"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; bf16 N(0,1) activations, N(0,0.02) weights; copy payload as "
                "the workload states)",
        "config": {
            "workload": f"{w.name}: bf16 GEMM {M}x{N}x{K} || {w.copy} "
                        f"{w.units}{'x' + str(w.units) if w.copy == 'all2all' else ''} x "
                        f"{w.unit_bytes / MiB:g} MiB; value = SDMA mover, "
                        f"{'comm-first' if comm_first else 'GEMM-first'}, "
                        f"GEMM CUs {'all' if not gmask else str(args.keep_per_xcc) + '/XCC'}"
                        f"{', SDMA engines ' + str(args.sdma_engines) if args.sdma_engines else ''}"
                        f"{', CU copy non-temporal' if args.cu_nontemporal else ''}",
            "M": M, "N": N, "K": K, "copy_bytes": copy_bytes, "comm_hbm_bytes": comm_bytes,
        },
        "copy_gbps_concurrent": (round(head["copy_gbps_concurrent"], 1)
                                 if head["copy_gbps_concurrent"] else None),
        "pct_of_ideal_uplift": round(head["uplift_paired_median"] * 100, 2),
        "pct_of_ideal_uplift_from_medians": round(head["uplift_fraction"] * 100, 2),
        "pct_of_ideal_uplift_per_round_p25_median_p75": [
            round(x * 100, 2) for x in head["uplift_per_round_p25_median_p75"]],
        "pct_of_ideal_ratio": round(head["ratio_of_ideal"] * 100, 2),
        "speedup": round(head["speedup"], 5),
        "ideal_speedup": round(head["ideal_speedup"], 5),
        "gemm_tflops_isolated": round(flops / T_gemm / 1e12, 2),
        "gemm_frac_of_peak_isolated": round(flops / T_gemm / 1e12 / PEAK_BF16_TFLOPS, 4),
        "t_gemm_ms": round(T_gemm * 1e3, 4),
        "movers": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                   for k, v in results.items()},
        "timing": "ms_per_step (and value) = mean over the timed steps of the library's host "
                  "clock from the first issue to both operations complete (SDMA cell); "
                  "pct_of_ideal_uplift = the median over the timed rounds of each round's own "
                  "uplift (its isolated GEMM, isolated copy and concurrent run, paired in time), "
                  "with the quartiles beside it; speedup, ideal_speedup and "
                  "pct_of_ideal_uplift_from_medians use the median of each of T_gemm, T_copy and "
                  "T_conc; copy_gbps_concurrent = the copy's bytes over the "
                  "median time from the first issue to its own completion; isolated and concurrent "
                  "runs interleaved per step, each after a fixed MFMA load of about 2.6 ms (the "
                  "same power state for every cell; off with --no-precondition), a poison and a "
                  "512 MiB read flush",
        "wall_s_timed_rounds": round(wall, 3),
        "verified": "every run: each copy destination range equal to its source (device compare; "
                    "all-reduce: the reduced chunk equal to the fp32 rank-order sum done with "
                    "torch on the device), "
                    "C bit-identical to the isolated C; isolated C vs the CPU oracle on the "
                    "cpu_baseline rows",
        "gemm_parity_vs_oracle": parity,
        "gpu_state": {"before": state_before, "after": state_after},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def time_copy(c3, s, mover, opts, reps, conc_opts=None):
    ca, _keep = s.cargs(mover, opts)
    ts, gs, eng = [], [], 0
    o = conc_opts if conc_opts is not None else c3.conc_opts(flush_bytes=FLUSH_BYTES)
    for i in range(reps + 1):
        s.poison()
        t = c3.c3_run_concurrent(None, ca, o)
        s.verify_copy("mover sweep")
        if i:
            ts.append(t["t_conc_ns"] * 1e-9)
            gs.append(t["copy_gpu_ms"] * 1e-3)
            eng = t["engines_used"]
    return statistics.median(ts), statistics.median(gs), eng, t["n_chunks"]


def run_movers(args, c3, info):
    """Isolated copy throughput against size (the paper's Fig. 9 question on one GPU)."""
    from concurrent_gemm_dma_amd import workloads as wl

    base = wl.WORKLOADS[5]
    engines = [1 << b for b in range(32) if info["sdma_engine_mask"] >> b & 1]
    reps = max(3, args.steps)
    for total_mib in (1, 4, 16, 64, 128, 256, 512, 1024):
        w = base.with_gather_total(total_mib * MiB)
        s = Setup(c3, w, with_gemm=False, check=not args.profile)
        S = w.copy_bytes
        cells = [("cu", "default", c3.C3_MOVER_CU, c3.move_opts()),
                 ("cu", "nontemporal", c3.C3_MOVER_CU, c3.move_opts(nontemporal=1))]
        for n in (1, 2, 4, 8, 16):
            if n <= len(engines):
                mask = sum(engines[:n])
                cells.append(("sdma", f"{n} engines, default split", c3.C3_MOVER_SDMA,
                              c3.move_opts(engine_mask=mask)))
        for chunks in (16, 32, 64):
            cells.append(("sdma", f"{len(engines)} engines, {chunks} chunks", c3.C3_MOVER_SDMA,
                          c3.move_opts(chunk_bytes=max(4096, S // chunks))))
        # both at once: the engines' bandwidth on top of the CUs' (balanced near 200 per mille)
        for pm in (100, 150, 200, 250, 300):
            cells.append(("hybrid", f"{pm} per mille on the engines", c3.C3_MOVER_HYBRID,
                          c3.move_opts(sdma_permille=pm)))
        for mover, label, mv, opts in cells:
            T, G, eng, nch = time_copy(c3, s, mv, opts, reps)
            print(json.dumps({"mode": "movers", "total_mib": total_mib, "mover": mover,
                              "variant": label, "chunks": nch, "engines_used": eng,
                              "t_ms_host": round(T * 1e3, 4), "t_ms_device": round(G * 1e3, 4),
                              "gbps_2S_host": round(2 * S / T / 1e9, 1),
                              "gbps_2S_device": round(2 * S / G / 1e9, 1) if G > 0 else None}),
                  flush=True)
        del s


def run_grid(args, c3, info):
    """The GC-equal workload's sweep: gather size x mover x GEMM CU mask x issue order."""
    from concurrent_gemm_dma_amd import workloads as wl

    base = wl.WORKLOADS[5]
    per = info["n_cu"] // info["n_xcc"]
    keeps = (per, per * 7 // 8, per * 3 // 4)
    reps = max(3, args.steps)
    precondition = make_preconditioner(c3, info, args)
    for total in base.sweep_total_bytes:
        w = base.with_gather_total(total)
        s = Setup(c3, w, check=not args.profile)
        copy_bytes = w.copy_bytes
        rounds = []
        names = ("cu", "sdma") + (("hybrid",) if args.hybrid_permille != -2 else ())
        pm = args.hybrid_permille
        for i in range(reps + 1):
            rnd = {}
            precondition()
            s.poison()
            rnd["gemm"] = c3.c3_run_concurrent(s.gargs, None, c3.conc_opts(flush_bytes=FLUSH_BYTES))["t_conc_ns"]
            s.verify_c("grid isolated GEMM")
            # movers in an order shuffled per round (round 0 in list order: the hybrid's share
            # needs the other two movers' isolated times first)
            order = list(names)
            if i:
                random.Random(2000 + i).shuffle(order)
            for mname in order:
                if mname == "hybrid":
                    if pm < 0:  # chosen once, from the untimed first round's isolated times
                        pm = c3.c3_hybrid_share(rnd["gemm"] * 1e-9, rnd[("copy", "sdma")] * 1e-9,
                                                rnd[("copy", "cu")] * 1e-9)
                    mv = c3.C3_MOVER_HYBRID
                    ca, _keep = s.cargs(mv, c3.move_opts(sdma_permille=pm))
                else:
                    mv = c3.C3_MOVER_CU if mname == "cu" else c3.C3_MOVER_SDMA
                    ca, _keep = s.cargs(mv)
                precondition()
                s.poison()
                rnd[("copy", mname)] = c3.c3_run_concurrent(None, ca, c3.conc_opts(flush_bytes=FLUSH_BYTES))["t_conc_ns"]
                s.verify_copy("grid isolated copy")
                for keep in keeps:
                    gm = None if keep == per else c3.c3_cu_mask_balanced(keep)
                    cm = None if (keep == per or mv == c3.C3_MOVER_SDMA) else c3.c3_cu_mask_balanced(keep, True)
                    for cf in (False, True):
                        precondition()
                        s.poison()
                        t = c3.c3_run_concurrent(s.gargs, ca, c3.conc_opts(
                            gemm_mask=gm, comm_mask=cm, comm_first=cf, flush_bytes=FLUSH_BYTES))
                        s.verify_copy("grid step")
                        s.verify_c("grid step")
                        rnd[("conc", mname, keep, cf)] = t["t_conc_ns"]
            if i:
                rounds.append(rnd)
        Tg = statistics.median(r["gemm"] for r in rounds) * 1e-9
        best_copy = min(statistics.median(r[("copy", m)] for r in rounds) for m in ("cu", "sdma")) * 1e-9
        for mname in names:
            Tc = statistics.median(r[("copy", mname)] for r in rounds) * 1e-9
            for keep in keeps:
                for cf in (False, True):
                    Tconc = statistics.median(r[("conc", mname, keep, cf)] for r in rounds) * 1e-9
                    m = c3.c3_derive_metrics(Tg, Tc, Tconc, float(w.gemm_bytes + 2 * copy_bytes),
                                             PEAK_HBM_GBPS * 1e9)
                    print(json.dumps({
                        "mode": "grid", "gather_mib": total // MiB, "mover": mname,
                        **({"sdma_permille": pm} if mname == "hybrid" else {}),
                        "gemm_cus_per_xcc": keep, "comm_first": cf,
                        "t_gemm_ms": round(Tg * 1e3, 4), "t_copy_ms": round(Tc * 1e3, 4),
                        "t_conc_ms": round(Tconc * 1e3, 4),
                        # against the faster mover's serial time, so that a slow mover cannot
                        # look good by inflating its own serial baseline
                        "speedup_vs_best_serial": round((Tg + best_copy) / Tconc, 4),
                        "gemm_tflops_concurrent": round(w.gemm_flops / Tconc / 1e12, 1),
                        **{k: (round(v, 4) if isinstance(v, float) else v) for k, v in m.items()}}),
                        flush=True)
        del s


def run_cus(args, c3, info):
    """Isolated GEMM time and CU-copy throughput with only k CUs per XCC (Fig. 5 analog)."""
    from concurrent_gemm_dma_amd import workloads as wl

    per = info["n_cu"] // info["n_xcc"]
    reps = max(3, args.steps)
    for wid in (2, 3, 5):
        w = wl.WORKLOADS[wid]
        s = Setup(c3, w, check=not args.profile)
        for keep in (per, per * 7 // 8, per * 3 // 4, per // 2, per // 4, per // 8):
            gm = None if keep == per else c3.c3_cu_mask_balanced(keep)
            ts = []
            for i in range(reps + 1):
                s.poison()
                t = c3.c3_run_concurrent(s.gargs, None, c3.conc_opts(gemm_mask=gm, flush_bytes=FLUSH_BYTES))
                s.verify_c("cus GEMM")
                if i:
                    ts.append(t["gemm_gpu_ms"] * 1e-3)
            T = statistics.median(ts)
            ca, _keep = s.cargs(c3.C3_MOVER_CU)
            tc = []
            for i in range(reps + 1):
                s.poison()
                t = c3.c3_run_concurrent(None, ca, c3.conc_opts(comm_mask=gm, flush_bytes=FLUSH_BYTES))
                s.verify_copy("cus copy")
                if i:
                    tc.append(t["copy_gpu_ms"] * 1e-3)
            Tc = statistics.median(tc)
            print(json.dumps({"mode": "cus", "workload": w.name, "cus_per_xcc": keep,
                              "gemm_ms": round(T * 1e3, 4),
                              "gemm_tflops": round(w.gemm_flops / T / 1e12, 1),
                              "gemm_gbps": round(w.gemm_bytes / T / 1e9, 1),
                              "cu_copy_ms": round(Tc * 1e3, 4),
                              "cu_copy_gbps_2S": round(2 * w.copy_bytes / Tc / 1e9, 1)}), flush=True)
        del s


def run_partition(args, c3, info):
    """Resource partitioning (c3_rp): the GEMM keeps N - c CUs per XCC and a CU-mover collective
    gets the other c, for c in powers of two; the best split is the sweep's upper bound. The
    heuristic predicts the split from a one-time slowdown lookup table (calibration kernels run
    side by side on complementary CUs, each timed to its own completion; or, the first reading,
    each alone under each mask) and isolated times estimated by a 0.70-efficiency roofline (or
    measured), and every combination is scored against the sweep: hit = same split, loss =
    T_conc(chosen) / T_conc(best) - 1. Every configuration of a table or a scenario is run once
    per round and rounds repeat, so clock drift hits all of them alike; medians over rounds."""
    import dataclasses

    from concurrent_gemm_dma_amd import workloads as wl

    per = info["n_cu"] // info["n_xcc"]
    opts = [c for c in (1, 2, 4, 8, 16) if c < per]
    # at least the paper's nine measured runs per configuration (the default --steps gives 20 here)
    reps = max(9, args.steps)
    eff = 0.70
    base = wl.WORKLOADS[2]
    peak_f, peak_b = PEAK_BF16_TFLOPS * 1e12, PEAK_HBM_GBPS * 1e9

    def gemm_w(wid, M, N, K):
        return dataclasses.replace(base, wid=wid, name=f"gemm_{M}x{N}x{K}", M=M, N=N, K=K)

    def comm_w(wid, kind, units, unit_mib):
        return dataclasses.replace(base, wid=wid, name=f"{kind}_{units}x{unit_mib}MiB", copy=kind,
                                   units=units, unit_bytes=int(unit_mib * MiB), payload="bytes")

    def mask(keep):
        return None if keep == per else c3.c3_cu_mask_balanced(keep)

    def run(g, cm, gkeep=per, ckeep=per, done=False):
        """One verified run: GEMM alone (cm None), collective alone (g None), or both with the
        GEMM on gkeep CUs per XCC and the collective on the complementary ckeep. Returns the
        run's time, or with done=True (both kernels) when each of the two completed."""
        for x in (g, cm):
            if x is not None:
                x.poison()
        ca = cm.cargs(c3.C3_MOVER_CU)[0] if cm is not None else None
        if g is not None and cm is not None:
            o = c3.conc_opts(gemm_mask=mask(gkeep),
                             comm_mask=None if gkeep == per else c3.c3_cu_mask_balanced(gkeep, True),
                             comm_first=True, flush_bytes=FLUSH_BYTES)
        else:
            o = c3.conc_opts(gemm_mask=mask(gkeep), comm_mask=mask(ckeep), flush_bytes=FLUSH_BYTES)
        t = c3.c3_run_concurrent(g.gargs if g is not None else None, ca, o)
        if cm is not None:
            cm.verify_copy("partition run")
        if g is not None:
            g.verify_c("partition run")
        if done:
            return t["t_gemm_done_ns"] * 1e-9, t["t_copy_done_ns"] * 1e-9
        return t["t_conc_ns"] * 1e-9

    def medians(cells):
        """cells: {key: thunk}; one untimed round, then `reps` rounds of every cell."""
        out = {k: [] for k in cells}
        for i in range(reps + 1):
            for k, f in cells.items():
                t = f()
                if i:
                    out[k].append(t)
        return {k: statistics.median(v) for k, v in out.items()}

    def median_pairs(cells):
        """cells: {key: thunk returning (a, b)}; medians of a and of b per key."""
        out = {k: [] for k in cells}
        for i in range(reps + 1):
            for k, f in cells.items():
                t = f()
                if i:
                    out[k].append(t)
        return {k: (statistics.median(a for a, _ in v), statistics.median(b for _, b in v))
                for k, v in out.items()}

    # ---- one-time lookup tables from calibration kernels (shapes not among the scenarios) ----
    # "isolated": each calibration kernel alone under each mask (the first reading of the
    # table). "paired": each calibration GEMM and collective side by side on complementary CUs,
    # each slowed-down time taken at its own completion, relative to the kernel alone on all CUs:
    # a collective on few CUs beside a compute-bound GEMM runs at the clock the GEMM leaves it
    # (the chip is power-limited), which an isolated table cannot see. Tables are per GEMM class
    # and collective kind, so a scenario looks its pair up.
    calib_gemm = {"compute": gemm_w(20, 8192, 16384, 8192), "memory": gemm_w(21, 32, 28672, 8192)}
    calib_comm = {"gather": comm_w(22, "gather", 8, 16), "all2all": comm_w(23, "all2all", 8, 2)}
    tables = {}
    calib_g = {cls: Setup(c3, w, check=not args.profile, with_comm=False)
               for cls, w in calib_gemm.items()}
    calib_c = {kind: Setup(c3, w, with_gemm=False, check=not args.profile)
               for kind, w in calib_comm.items()}
    alone = {}
    for cls, g in calib_g.items():
        for _ in range(5):  # clocks up before anything is timed
            run(g, None)
        m = medians({k: (lambda k=k: run(g, None, gkeep=k)) for k in [per] + [per - c for c in opts]})
        tables[("gemm", cls)] = {k: m[k] / m[per] for k in m if k != per}
        alone[cls] = m[per]
    for kind, cm in calib_c.items():
        m = medians({k: (lambda k=k: run(None, cm, ckeep=k)) for k in [per] + opts})
        tables[("comm", kind)] = {k: m[k] / m[per] for k in m if k != per}
        alone[kind] = m[per]
    for cls, g in calib_g.items():
        for kind, cm in calib_c.items():
            m = median_pairs({c: (lambda c=c: run(g, cm, gkeep=per - c, done=True)) for c in opts})
            tables[("gemm", cls, kind)] = {per - c: m[c][0] / alone[cls] for c in opts}
            tables[("comm", kind, cls)] = {c: m[c][1] / alone[kind] for c in opts}
    del calib_g, calib_c
    for key, tab in tables.items():
        print(json.dumps({"mode": "partition", "table": ":".join(key),
                          "slowdown_by_cus_per_xcc": {str(k): round(v, 4) for k, v in sorted(tab.items())}}),
              flush=True)

    # ---- scenarios: GEMMs x CU-mover collectives ----
    gemms = [(8192, 28672, 8192), (4096, 16384, 8192), (2048, 28672, 8192), (8192, 8192, 8192),
             (16, 28672, 8192), (32, 53248, 8192)]
    comms = [("gather", 8, 8), ("gather", 8, 32), ("gather", 8, 128), ("all2all", 8, 1),
             ("all2all", 8, 4)]
    comm_setups = [Setup(c3, comm_w(40 + i, *cdef), with_gemm=False, check=not args.profile)
                   for i, cdef in enumerate(comms)]
    variants = [(t, tv) for tv in ("paired", "isolated") for t in ("measured", "roofline")]
    hits = {v: 0 for v in variants}
    losses = {v: [] for v in variants}
    gain_rp_over_sp = []
    n = 0
    for gi, (M, N, K) in enumerate(gemms):
        w = gemm_w(30 + gi, M, N, K)
        g = Setup(c3, w, check=not args.profile, with_comm=False)
        gcls = "compute" if w.gemm_flops / peak_f >= w.gemm_bytes / peak_b else "memory"
        for _ in range(3):
            run(g, None)
        for cm, (kind, units, unit_mib) in zip(comm_setups, comms):
            cw = cm.w
            cells = {"gemm": lambda: run(g, None), "comm": lambda: run(None, cm),
                     "shared": lambda: run(g, cm)}
            cells.update({c: (lambda c=c: run(g, cm, gkeep=per - c)) for c in opts})
            m = medians(cells)
            T_g, T_c = m["gemm"], m["comm"]
            measured = {c: m[c] for c in opts}
            best_c = min(opts, key=lambda c: (measured[c], c))
            est_g = c3.c3_roofline_time(w.gemm_flops, w.gemm_bytes, peak_f, peak_b, eff)
            est_c = c3.c3_roofline_time(0.0, cw.comm_hbm_bytes, peak_f, peak_b, eff)
            picks = {}
            for variant in variants:
                tg, tc = (T_g, T_c) if variant[0] == "measured" else (est_g, est_c)
                if variant[1] == "paired":
                    gt, ct = tables[("gemm", gcls, kind)], tables[("comm", kind, gcls)]
                else:
                    gt, ct = tables[("gemm", gcls)], tables[("comm", kind)]
                chosen, preds = c3.c3_predict_partition(gt, ct, tg, tc, per, opts)
                hit = chosen == best_c
                loss = measured[chosen] / measured[best_c] - 1.0
                hits[variant] += hit
                losses[variant].append(loss)
                picks[f"{variant[0]}_times_{variant[1]}_table"] = {
                    "chosen_cus_per_xcc": chosen, "hit": hit, "loss": round(loss, 5),
                    "predicted_ms": [round(p * 1e3, 4) for p in preds]}
            T_sp = m["shared"]
            mt = c3.c3_derive_metrics(T_g, T_c, measured[best_c])
            gain_rp_over_sp.append(T_sp / measured[best_c])
            n += 1
            print(json.dumps({
                "mode": "partition", "scenario": n, "gemm": f"{M}x{N}x{K}", "gemm_class": gcls,
                "collective": cw.name, "t_gemm_ms": round(T_g * 1e3, 4),
                "t_comm_ms": round(T_c * 1e3, 4), "taxonomy": mt["taxonomy"],
                "t_conc_ms_by_comm_cus_per_xcc": {str(c): round(v * 1e3, 4) for c, v in measured.items()},
                "best_comm_cus_per_xcc": best_c, "t_conc_ms_shared_cus": round(T_sp * 1e3, 4),
                "speedup_best_split": round((T_g + T_c) / measured[best_c], 4),
                "speedup_shared_cus": round((T_g + T_c) / T_sp, 4),
                "heuristic": picks}), flush=True)
        del g
    print(json.dumps({
        "mode": "partition", "summary": True, "scenarios": n, "rounds": reps,
        "heuristic": {f"{'roofline_0.70' if v[0] == 'roofline' else 'measured'}_times_{v[1]}_table":
                      {"hits": hits[v], "within_1.5pct": sum(x <= 0.015 for x in losses[v]),
                       "max_loss": round(max(losses[v]), 5),
                       "mean_loss": round(statistics.mean(losses[v]), 5)} for v in variants},
        "best_split_vs_shared_cus_geomean": round(statistics.geometric_mean(gain_rp_over_sp), 4),
        "scenarios_where_best_split_beats_shared": sum(x > 1.0 for x in gain_rp_over_sp)}), flush=True)


def run_ksteps(args, c3, info):
    """The tile GEMM against K at a fixed M x N (8192 x 28672: 14 tiles of 256 x 256 per CU), so
    that a fit of time (or, under counters, cycles) against K steps separates the cost of a tile's
    start and end from the cost of one K step. Every launch comes after a 512 MiB read flush; the
    K values run in an order shuffled per round (printed, for labelling counter dispatches); C is
    checked bit-identical across rounds."""
    import numpy as np
    import torch

    from concurrent_gemm_dma_amd import workloads as wl

    M, N = 8192, 28672
    Ks = (1024, 2048, 4096, 8192, 16384)
    dev = torch.device("cuda:0")
    A = wl.gen_bf16((M, max(Ks)), ("normal", 0.0, 1.0), wl.seed_for(2, wl.BUF_A))
    dA = torch.from_numpy(A.view(np.int16)).to(dev)
    del A
    B = wl.gen_bf16((max(Ks), N), ("normal", 0.0, 0.02), wl.seed_for(2, wl.BUF_B))
    dB = torch.from_numpy(B.view(np.int16)).to(dev)
    del B
    ops = {K: (dA[:, :K].contiguous(), dB[:K], torch.empty((M, N), dtype=torch.int16, device=dev))
           for K in Ks}
    o = c3.conc_opts(flush_bytes=FLUSH_BYTES)
    times = {K: [] for K in Ks}
    first = {}
    reps = max(3, args.steps)
    for i in range(reps + 1):
        order = list(Ks)
        random.Random(i).shuffle(order)
        print(json.dumps({"mode": "ksteps", "round": i, "order": order}), flush=True)
        for K in order:
            a, b, c = ops[K]
            c.fill_(-1)
            torch.cuda.synchronize()
            t = c3.c3_run_concurrent(c3.gemm_args(a, b, c, M, N, K), None, o)
            if not args.profile:
                if K not in first:
                    first[K] = c.clone()
                elif not torch.equal(first[K], c):
                    raise SystemExit(f"ksteps: C of K={K} differs between rounds")
            if i:
                times[K].append(t["gemm_gpu_ms"])
    for K in Ks:
        ms = statistics.median(times[K])
        print(json.dumps({"mode": "ksteps", "M": M, "N": N, "K": K, "k_steps_per_tile": K // 32,
                          "tiles_per_cu": M * N // (256 * 256) // info["n_cu"],
                          "gemm_ms": round(ms, 4),
                          "tflops": round(2.0 * M * N * K / ms / 1e9, 1)}), flush=True)


def run_mfma_ceiling(args, c3, info):
    """The matrix cores' sustained bf16 rate with nothing but MFMAs in flight (c3_probe_mfma_rate:
    one workgroup of 4 waves per CU, each wave 16 independent 32x32 accumulators), for runs as
    long as the workload-2 and workload-4 GEMMs, each after a 512 MiB read flush, timed with HIP
    events on the probe's stream. The ceiling for any bf16 GEMM on this chip at its power limit."""
    import torch

    n_wg = info["n_cu"]
    s = torch.cuda.Stream()
    out = torch.empty(n_wg * 256, dtype=torch.float64, device="cuda:0")
    reps = max(3, args.steps)
    # random operands (bits toggling as a GEMM's data do) and small-integer ones, for runs about
    # as long as the workload-2 and workload-4 GEMMs
    for random, iters in ((1, 8400), (1, 33600), (0, 8400), (0, 33600)):
        flops = float(n_wg) * 4 * iters * 16 * 32768
        ms = []
        for i in range(reps + 1):
            torch.cuda.synchronize()
            c3.c3_flush_llc(FLUSH_BYTES, s)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            c3.c3_probe_mfma_rate(out, n_wg, iters, random, s)
            e1.record(s)
            torch.cuda.synchronize()
            if i:
                ms.append(e0.elapsed_time(e1))
        m = statistics.median(ms)
        print(json.dumps({"mode": "mfma_ceiling", "operands": "random" if random else "small integers",
                          "workgroups": n_wg, "iterations": iters,
                          "ms": round(m, 4), "tflops": round(flops / m / 1e9, 1),
                          "frac_of_peak": round(flops / m / 1e9 / PEAK_BF16_TFLOPS, 4),
                          "ms_min": round(min(ms), 4), "ms_max": round(max(ms), 4)}), flush=True)


def run_gemm_data(args, c3, info):
    """The tile GEMM of workloads 2 and 4 on three kinds of operands: the workloads' distributions
    (bf16 of N(0, 1) activations and N(0, 0.02) weights), small integers in -2..2 and zeros. The kernel
    runs the same instructions on all three, so its cycles are the same; what changes is how
    many operand bits switch in the matrix cores, and with it the power the chip spends per FLOP
    and so the clock its power limit allows. Every launch comes after the fixed MFMA load and a
    512 MiB read flush (as in the c3 mode); kinds in an order shuffled per round; HIP-event time
    of the GEMM's launch (medians). C is checked bit-identical across rounds (and zero for zero
    operands)."""
    import torch

    from concurrent_gemm_dma_amd import workloads as wl

    precondition = make_preconditioner(c3, info, args)
    o = c3.conc_opts(flush_bytes=FLUSH_BYTES)
    reps = max(3, args.steps)
    for w in (wl.WORKLOADS[2], wl.WORKLOADS[4]):
        M, N, K = w.M, w.N, w.K
        g = torch.Generator(device="cuda").manual_seed(w.wid)
        A = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        B = (torch.randn(K, N, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        ops = {"workload data": (A, B),
               "small integers": (torch.randint(-2, 3, (M, K), device="cuda", generator=g).to(torch.bfloat16),
                                  torch.randint(-2, 3, (K, N), device="cuda", generator=g).to(torch.bfloat16)),
               "zeros": (torch.zeros_like(A), torch.zeros_like(B))}
        C = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
        kinds = list(ops)
        times = {k: [] for k in kinds}
        first = {}
        for i in range(reps + 1):
            order = list(kinds)
            random.Random(i).shuffle(order)
            for k in order:
                a, b = ops[k]
                C.fill_(-1)
                torch.cuda.synchronize()
                precondition()
                t = c3.c3_run_concurrent(c3.gemm_args(a, b, C, M, N, K), None, o)
                if not args.profile:
                    if k not in first:
                        first[k] = C.clone()
                        if k == "zeros" and bool(C.any()):
                            raise SystemExit("gemm_data: C of zero operands is not zero")
                    elif not torch.equal(first[k], C):
                        raise SystemExit(f"gemm_data: C of {k} differs between rounds")
                if i:
                    times[k].append(t["gemm_gpu_ms"])
        flops = 2.0 * M * N * K
        for k in kinds:
            ms = statistics.median(times[k])
            print(json.dumps({"mode": "gemm_data", "workload": w.name, "M": M, "N": N, "K": K,
                              "operands": k, "gemm_ms": round(ms, 4),
                              "tflops": round(flops / ms / 1e9, 1),
                              "frac_of_peak": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}),
                  flush=True)
        del ops, A, B, C, first
        torch.cuda.empty_cache()


def run_gemm_vs_vendor(args, c3, info):
    """The library's GEMM and torch.matmul (hipBLASLt) on the same bf16 operands: alternating
    event-timed single launches (median), then two batches of 20 back-to-back launches each.
    C of the library is checked bit-identical across its launches."""
    import torch

    from concurrent_gemm_dma_amd import workloads as wl

    s = torch.cuda.current_stream()
    shapes = [(w.M, w.N, w.K) for w in (wl.WORKLOADS[2], wl.WORKLOADS[4], wl.WORKLOADS[5], wl.WORKLOADS[3])]
    shapes.insert(3, (8192, 8192, 8192))
    if args.shapes:
        shapes = [tuple(int(x) for x in sh.split("x")) for sh in args.shapes.split(",")]
    for (M, N, K) in shapes:
        g = torch.Generator(device="cuda").manual_seed(M * 31 + N * 7 + K)
        A = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        B = (torch.randn(K, N, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        C = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ours, vendor, first = [], [], None
        for i in range(5 + max(10, args.steps)):
            ev[0].record(s)
            c3.c3_gemm(A, B, C, M, N, K, s)
            ev[1].record(s)
            ev[2].record(s)
            D = A @ B
            ev[3].record(s)
            torch.cuda.synchronize()
            if first is None:
                first = C.clone()
            elif not torch.equal(C, first):
                raise SystemExit("gemm_vs_vendor: C changed between launches")
            if i >= 5:
                ours.append(ev[0].elapsed_time(ev[1]))
                vendor.append(ev[2].elapsed_time(ev[3]))
        b2b = {"ours": [], "vendor": []}
        for name in ("ours", "vendor", "ours", "vendor"):
            torch.cuda.synchronize()
            ev[0].record(s)
            for _ in range(20):
                if name == "ours":
                    c3.c3_gemm(A, B, C, M, N, K, s)
                else:
                    D = A @ B
            ev[1].record(s)
            torch.cuda.synchronize()
            b2b[name].append(ev[0].elapsed_time(ev[1]) / 20)
        f = 2.0 * M * N * K / 1e9
        print(json.dumps({"mode": "gemm_vs_vendor", "shape": f"{M}x{N}x{K}",
                          "ours_ms": round(statistics.median(ours), 4),
                          "vendor_ms": round(statistics.median(vendor), 4),
                          "ours_tflops": round(f / statistics.median(ours), 1),
                          "vendor_tflops": round(f / statistics.median(vendor), 1),
                          "ours_b2b_tflops": [round(f / x, 1) for x in b2b["ours"]],
                          "vendor_b2b_tflops": [round(f / x, 1) for x in b2b["vendor"]],
                          "ours_over_vendor": round(statistics.median(vendor) / statistics.median(ours), 4)}),
              flush=True)
        del A, B, C, D, first


def run_hybrid(args, c3, info):
    """Hybrid mover: concurrent time against the engines' share of the copy (0..1000 per mille in
    steps of 100), the share c3_hybrid_share picks from the untimed first round's isolated times
    (timed in the same rounds as the sweep), and its loss against the best share of the sweep."""
    from concurrent_gemm_dma_amd import workloads as wl

    cases = [(5, g) for g in (128, 256, 512, 768, 1024)] + [(3, 0), (6, 0), (4, 0)]
    reps = max(3, args.steps)
    flush = c3.conc_opts(flush_bytes=FLUSH_BYTES)
    conc_opts = c3.conc_opts(comm_first=True, flush_bytes=FLUSH_BYTES)
    for wid, gmib in cases:
        w = wl.WORKLOADS[wid]
        if gmib:
            w = w.with_gather_total(gmib * MiB)
        s = Setup(c3, w, check=not args.profile)
        shares = list(range(0, 1001, 100))
        iso = {"gemm": [], "sdma": [], "cu": []}
        pure = {"sdma": s.cargs(c3.C3_MOVER_SDMA), "cu": s.cargs(c3.C3_MOVER_CU)}
        hyb = {pm: s.cargs(c3.C3_MOVER_HYBRID, c3.move_opts(sdma_permille=pm)) for pm in shares}
        conc = {pm: [] for pm in shares}
        chosen = None
        for i in range(reps + 1):
            timed = i > 0
            s.poison()
            t = c3.c3_run_concurrent(s.gargs, None, flush)
            s.verify_c("hybrid sweep isolated GEMM")
            iso["gemm"].append(t["t_conc_ns"] * 1e-9)
            for name, (ca, _keep) in pure.items():
                s.poison()
                t = c3.c3_run_concurrent(None, ca, flush)
                s.verify_copy(f"hybrid sweep isolated {name}")
                iso[name].append(t["t_conc_ns"] * 1e-9)
            if chosen is None:
                # the rule's share, from this untimed round's isolated times
                chosen = c3.c3_hybrid_share(iso["gemm"][0], iso["sdma"][0], iso["cu"][0])
                if chosen not in hyb:
                    hyb[chosen] = s.cargs(c3.C3_MOVER_HYBRID, c3.move_opts(sdma_permille=chosen))
                    conc[chosen] = []
            order = sorted(hyb)
            random.Random(3000 + i).shuffle(order)  # no share always runs in the same place
            for pm in order:
                s.poison()
                t = c3.c3_run_concurrent(s.gargs, hyb[pm][0], conc_opts)
                s.verify_copy(f"hybrid {pm}")
                s.verify_c(f"hybrid {pm}")
                if timed:
                    conc[pm].append(t["t_conc_ns"] * 1e-9)
        med = {k: statistics.median(v[1:]) for k, v in iso.items()}
        mean = {pm: statistics.mean(v) for pm, v in conc.items()}
        best = min(mean, key=lambda pm: mean[pm])
        serial = med["gemm"] + min(med["sdma"], med["cu"])
        print(json.dumps({
            "mode": "hybrid", "workload": w.name, "copy": w.copy,
            "copy_mib": round(w.copy_bytes / MiB, 1),
            "t_gemm_ms": round(med["gemm"] * 1e3, 4), "t_sdma_ms": round(med["sdma"] * 1e3, 4),
            "t_cu_ms": round(med["cu"] * 1e3, 4),
            "t_conc_ms": {str(pm): round(mean[pm] * 1e3, 4) for pm in sorted(mean)},
            "chosen_permille": chosen, "t_chosen_ms": round(mean[chosen] * 1e3, 4),
            "chosen_from_timed_medians": c3.c3_hybrid_share(med["gemm"], med["sdma"], med["cu"]),
            "best_permille": best, "t_best_ms": round(mean[best] * 1e3, 4),
            "loss_vs_best": round(mean[chosen] / mean[best] - 1, 4),
            "chosen_vs_sdma_only": round(mean[1000] / mean[chosen], 4),
            "chosen_vs_cu_only": round(mean[0] / mean[chosen], 4),
            "chosen_vs_best_serial": round(serial / mean[chosen], 4)}), flush=True)
        del s


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        log("bench.py: only --gpus 1 is supported (single-GPU build)")
        sys.exit(2)
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        log("bench.py: launched with WORLD_SIZE > 1; this build runs on one GPU only")
        sys.exit(2)

    from concurrent_gemm_dma_amd import _c3 as c3

    c3.c3_init(0)
    info = c3.c3_device_info()
    log("device:", info)
    {"c3": run_c3, "movers": run_movers, "grid": run_grid, "cus": run_cus, "hybrid": run_hybrid,
     "partition": run_partition, "gemm_vs_vendor": run_gemm_vs_vendor,
     "ksteps": run_ksteps, "mfma_ceiling": run_mfma_ceiling,
     "gemm_data": run_gemm_data}[args.mode](args, c3, info)
    c3.c3_finalize()


if __name__ == "__main__":
    main()
