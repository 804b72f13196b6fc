#!/usr/bin/env python3
"""Benchmark of the C3 hot path on one MI355X: a bf16 GEMM concurrent with a collective-shaped
copy, moved by the SDMA engines (headline) and by a CU kernel (baseline).

A step is one concurrent run (c3_run_concurrent) of the whole path over the workload: GEMM and
copy issued (communication first), both completed. Before every step, untimed: the outputs are
poisoned and the Infinity Cache is flushed (inside the library, before its clock starts). After
every step, untimed: the copy destination is compared byte for byte with the oracle's gather and
C bit for bit with the GEMM's isolated result (itself checked against the oracle on sampled
elements). Isolated GEMM and copy times use the same protocol and feed the ideal speedup.

Prints ONE JSON line on stdout. Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", type=int, default=2, help="workload id (1..5)")
    p.add_argument("--gather-mib", type=int, default=0, help="workload 5: total gather MiB")
    p.add_argument("--keep-per-xcc", type=int, default=0,
                   help="GEMM CU mask: CUs kept per XCC (0 = all)")
    p.add_argument("--gemm-first", action="store_true", help="issue the GEMM first")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--profile", action="store_true",
                   help="few steps, no verification or CPU baseline (for rocprofv3 runs)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        log("bench.py: only --gpus 1 is supported (single-GPU build)")
        sys.exit(2)
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        log("bench.py: launched with WORLD_SIZE > 1; this build runs on one GPU only")
        sys.exit(2)

    import numpy as np
    import torch

    import oracle
    from concurrent_gemm_dma_amd import _c3 as c3
    from concurrent_gemm_dma_amd import workloads as wl

    dev = torch.device("cuda:0")
    c3.c3_init(0)
    info = c3.c3_device_info()
    log("device:", info)
    w = wl.WORKLOADS[args.workload]
    if args.gather_mib:
        w = w.with_gather_total(args.gather_mib * MiB)
    M, N, K = w.M, w.N, w.K
    flops = w.gemm_flops
    copy_bytes = w.copy_bytes  # payload S; HBM traffic of the copy is 2S (read + write)

    # ---- inputs (seeded, synthetic), resident in HBM before any timing ----
    t0 = time.time()
    A, B = wl.gen_gemm_operands(w)
    if w.copy == "gather":
        src_np = wl.gen_shards(w)
        want = oracle.gather(src_np)
    else:
        src_np = wl.gen_a2a_source(w)
        want = oracle.all2all_block(src_np, w.units, w.unit_bytes)
    dA = torch.from_numpy(A.view(np.int16)).to(dev)
    dB = torch.from_numpy(B.view(np.int16)).to(dev)
    dC = torch.empty((M, N), dtype=torch.int16, device=dev)
    if w.copy == "gather":
        dsrc = [torch.from_numpy(s).to(dev) for s in src_np]
    else:
        dsrc = torch.from_numpy(src_np).to(dev)
    ddst = torch.empty(want.size, dtype=torch.uint8, device=dev)
    dwant = torch.from_numpy(want).to(dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")

    rows, cols = wl.sample_indices(M, N, 512, seed=w.wid, full_rows=(M // 2,))
    _, ref64, _ = (None, None, None) if args.profile else oracle.gemm_elems(A, B, rows, cols)

    gmask = c3.c3_cu_mask_balanced(args.keep_per_xcc) if args.keep_per_xcc else None
    comm_first = not args.gemm_first

    def cargs(mover):
        if w.copy == "gather":
            return c3.gather_args(ddst, dsrc, w.unit_bytes, mover)
        return c3.all2all_args(ddst, dsrc, w.units, w.unit_bytes, mover)

    gargs = c3.gemm_args(dA, dB, dC, M, N, K)
    poison_i = [0]

    def poison():
        poison_i[0] += 1
        dC.fill_(-1 - (poison_i[0] % 7))
        ddst.fill_((0xA5 + poison_i[0]) & 0xFF)
        torch.cuda.synchronize()

    iso_c = None

    def verify_copy(label):
        if args.profile:
            return
        if not torch.equal(ddst, dwant):
            host = ddst.cpu().numpy()
            raise SystemExit(f"{label}: copy mismatch at byte {oracle.first_diff(want, host)}")

    def verify_c(label):
        nonlocal iso_c
        if iso_c is None:
            iso_c = dC.clone()
            if not args.profile:
                got = iso_c.cpu().numpy().view(np.uint16)[rows, cols]
                rep = oracle.gemm_compare(ref64, got)
                if not oracle.gemm_within_tolerance(rep):
                    raise SystemExit(f"GEMM parity failure vs oracle: {rep}")
                log(f"GEMM sampled parity vs oracle ok ({rep['n']} elems, "
                    f"{rep['n_diff']} differ by one rounding)")
        elif not args.profile and not torch.equal(dC, iso_c):
            raise SystemExit(f"{label}: C differs from the isolated GEMM")

    movers = (("sdma", c3.C3_MOVER_SDMA), ("cu", c3.C3_MOVER_CU))
    copy_args = {name: cargs(mv) for name, mv in movers}
    conc = {}
    for name, mv in movers:
        cmask = None
        if gmask is not None and mv == c3.C3_MOVER_CU:
            cmask = c3.c3_cu_mask_balanced(args.keep_per_xcc, complement=True)
        conc[name] = c3.conc_opts(gemm_mask=gmask, comm_mask=cmask, comm_first=comm_first,
                                  flush_bytes=FLUSH_BYTES)
    iso_g_opts = c3.conc_opts(gemm_mask=gmask, flush_bytes=FLUSH_BYTES)
    iso_c_opts = c3.conc_opts(flush_bytes=FLUSH_BYTES)

    # Every round runs the isolated GEMM, then per mover the isolated copy and the concurrent
    # step, so that clock and thermal drift affect isolated and concurrent times alike.
    t_gemm, g_gpu = [], []
    rec = {name: {"t_copy": [], "c_gpu": [], "t_conc": [], "gk": []} for name, _ in movers}
    torch.cuda.synchronize()
    wall0 = None
    for i in range(args.warmup + args.steps):
        if i == args.warmup:
            torch.cuda.synchronize()
            wall0 = time.time()
        timed = i >= args.warmup
        poison()
        t = c3.c3_run_concurrent(gargs, None, iso_g_opts)
        verify_c(f"isolated GEMM {i}")
        if timed:
            t_gemm.append(t["t_conc_ns"] * 1e-9)
            g_gpu.append(t["gemm_gpu_ms"] * 1e-3)
        for name, mv in movers:
            ca = copy_args[name][0]
            r = rec[name]
            poison()
            t = c3.c3_run_concurrent(None, ca, iso_c_opts)
            verify_copy(f"isolated {name} copy {i}")
            if timed:
                r["t_copy"].append(t["t_conc_ns"] * 1e-9)
                r["c_gpu"].append(t["copy_gpu_ms"] * 1e-3)
            poison()
            t = c3.c3_run_concurrent(gargs, ca, conc[name])
            verify_copy(f"{name} step {i}")
            verify_c(f"{name} step {i}")
            if timed:
                r["t_conc"].append(t["t_conc_ns"] * 1e-9)
                r["gk"].append(t["gemm_gpu_ms"] * 1e-3)
    torch.cuda.synchronize()
    wall = time.time() - wall0
    T_gemm = statistics.median(t_gemm)
    log(f"isolated GEMM: median {T_gemm * 1e3:.3f} ms  ({flops / T_gemm / 1e12:.1f} TFLOP/s host, "
        f"{flops / statistics.median(g_gpu) / 1e12:.1f} TFLOP/s events)")

    results = {}
    for name, _ in movers:
        r = rec[name]
        T_copy = statistics.median(r["t_copy"])
        T_conc = statistics.mean(r["t_conc"])
        c_gpu_med = statistics.median(r["c_gpu"])
        m = c3.c3_derive_metrics(T_gemm, T_copy, T_conc, float(w.gemm_bytes + 2 * copy_bytes),
                                 PEAK_HBM_GBPS * 1e9)
        results[name] = {
            "t_copy_ms": T_copy * 1e3, "t_conc_ms": T_conc * 1e3,
            "t_conc_ms_min": min(r["t_conc"]) * 1e3, "t_conc_ms_max": max(r["t_conc"]) * 1e3,
            "t_conc_ms_std": (statistics.pstdev(r["t_conc"]) * 1e3) if len(r["t_conc"]) > 1 else 0.0,
            "copy_gbps_isolated": 2 * copy_bytes / T_copy / 1e9,
            "copy_gbps_isolated_engine_clock": (2 * copy_bytes / c_gpu_med / 1e9
                                                if c_gpu_med > 0 else None),
            "gemm_tflops_concurrent": flops / T_conc / 1e12,
            "copy_gbps_concurrent": 2 * copy_bytes / T_conc / 1e9,
            "gemm_kernel_ms_concurrent": statistics.mean(r["gk"]) * 1e3,
            **{k: m[k] for k in ("ideal_speedup", "speedup", "uplift_fraction", "ratio_of_ideal",
                                 "gemm_slowdown", "hbm_ceiling", "taxonomy")},
        }
        log(f"{name}: T_copy {T_copy * 1e3:.3f} ms ({results[name]['copy_gbps_isolated']:.0f} GB/s), "
            f"T_conc {T_conc * 1e3:.3f} ms, S {m['speedup']:.4f} / ideal {m['ideal_speedup']:.4f}, "
            f"uplift {m['uplift_fraction'] * 100:.1f}%")

    # ---- roofline of the dominant kernel (the GEMM): HIP events recorded by the library on the
    # GEMM's own stream around every launch of the timed SDMA-concurrent steps ----
    gemm_kernel_s = statistics.mean(rec["sdma"]["gk"])
    achieved_tflops = flops / gemm_kernel_s / 1e12
    roofline = {"bound": "mfma" if M > 64 else "hbm",
                "achieved": None, "peak": None, "unit": None, "frac": None, "traffic": None}
    if M > 64:
        roofline.update(achieved=round(achieved_tflops, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                        frac=round(achieved_tflops / PEAK_BF16_TFLOPS, 4))
    else:
        gbps = w.gemm_bytes / gemm_kernel_s / 1e9
        roofline.update(achieved=round(gbps, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                        frac=round(gbps / PEAK_HBM_GBPS, 4))
    roofline["kernel"] = "gemm_bf16_tile256" if M > 64 else "gemm_bf16_skinny (+splitk_reduce)"
    roofline["kernel_ms"] = round(gemm_kernel_s * 1e3, 4)

    # ---- CPU baseline: the oracle as it stands, on a bounded sample of the same workload ----
    cpu = None
    if not args.no_cpu_baseline and not args.profile:
        nthreads = oracle.threads(0)
        r = 1
        t1 = time.time()
        oracle.gemm_f32acc(A, B, rows=(0, r))
        dt = max(time.time() - t1, 1e-3)
        r = int(max(1, min(M, args.cpu_seconds / dt)))
        t1 = time.time()
        oracle.gemm_f32acc(A, B, rows=(0, r))
        dt = time.time() - t1
        cpu = {"value": round(2.0 * r * N * K / dt / 1e12, 6), "unit": "TFLOP/s",
               "cores": nthreads, "kind": "oracle",
               "sample": f"fp32-accumulate triple-loop GEMM oracle, rows 0..{r - 1} of C "
                         f"({r}x{N}x{K}, {2.0 * r * N * K / 1e9:.1f} GFLOP) in {dt:.1f} s"}
        log("cpu baseline:", cpu)

    head = results["sdma"]
    out = {
        "metric": METRIC,
        "value": round(head["gemm_tflops_concurrent"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["t_conc_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; bf16 N(0,1) activations, N(0,0.02) weights; copy payload as the workload states)",
        "config": {
            "workload": f"{w.name}: bf16 GEMM {M}x{N}x{K} || {w.copy} "
                        f"{w.units}{'x' + str(w.units) if w.copy == 'all2all' else ''} x "
                        f"{w.unit_bytes // MiB} MiB; value = SDMA mover, "
                        f"{'comm-first' if comm_first else 'GEMM-first'}, "
                        f"GEMM CUs {'all' if not gmask else str(args.keep_per_xcc) + '/XCC'}",
            "M": M, "N": N, "K": K, "copy_bytes": copy_bytes,
        },
        "copy_gbps_concurrent": round(head["copy_gbps_concurrent"], 1),
        "pct_of_ideal_uplift": round(head["uplift_fraction"] * 100, 2),
        "pct_of_ideal_ratio": round(head["ratio_of_ideal"] * 100, 2),
        "speedup": round(head["speedup"], 5),
        "ideal_speedup": round(head["ideal_speedup"], 5),
        "gemm_tflops_isolated": round(flops / T_gemm / 1e12, 2),
        "gemm_frac_of_peak_isolated": round(flops / T_gemm / 1e12 / PEAK_BF16_TFLOPS, 4),
        "t_gemm_ms": round(T_gemm * 1e3, 4),
        "movers": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                   for k, v in results.items()},
        "timing": "ms_per_step = mean over the timed steps of the library's host clock from the "
                  "first issue to both operations complete (SDMA cell); isolated and concurrent "
                  "runs interleaved per step, each after a poison + 512 MiB cache flush",
        "wall_s_timed_rounds": round(wall, 3),
        "verified": "every step: copy byte-exact vs oracle, C bit-identical to isolated C; "
                    "isolated C vs oracle on sampled elements",
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    c3.c3_finalize()


if __name__ == "__main__":
    main()
