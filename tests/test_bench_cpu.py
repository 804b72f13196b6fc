"""Host-side checks of bench.py (no GPU work): the one-GPU contract refuses more GPUs before
touching any device, defaults match the documented protocol, the traffic record lookup is
consistent with the committed counter file, and a mover's cell aggregates its timed rounds by
the documented rules."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused(host_only):
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_distributed_launch_is_refused(host_only):
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, BENCH], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 2
    assert "WORLD_SIZE" in r.stderr


def test_defaults(monkeypatch):
    b = load_bench()
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = b.parse()
    assert (a.gpus, a.steps, a.warmup, a.mode, a.workload) == (1, 50, 3, "c3", 4)
    assert b.PEAK_BF16_TFLOPS == 2500.0 and b.PEAK_HBM_GBPS == 8000.0
    # every run of the C3 and grid modes starts after the fixed MFMA load unless asked otherwise
    assert a.no_precondition is False and b.PRECOND_ITERS > 0
    monkeypatch.setattr(sys, "argv", ["bench.py", "--no-precondition"])
    assert b.parse().no_precondition is True
    # 50 timed rounds only in the c3 mode; the sweeps keep 20; an explicit count always wins
    for mode in ("grid", "partition", "gemm_data", "mfma_ceiling"):
        monkeypatch.setattr(sys, "argv", ["bench.py", "--mode", mode])
        assert b.parse().steps == 20, mode
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "7"])
    assert b.parse().steps == 7


def test_traffic_record_lookup_is_consistent():
    """Every record in the traffic file names a kernel and a workload the benchmark knows; while
    its source hash matches, the lookup returns the calibrated bytes, at least the workload's
    algorithmic GEMM bytes."""
    b = load_bench()
    from concurrent_gemm_dma_amd import workloads as wl

    by_name = {w.name: w for w in wl.WORKLOADS.values()}
    rec = json.load(open(os.path.join(ROOT, "profiles", "gemm_traffic.json")))
    assert "gemm_bf16_tile256_dma@" + wl.WORKLOADS[2].name in rec
    for key, r in rec.items():
        kernel, name = key.rsplit("@", 1)
        w = by_name[name]
        t = b.measured_traffic(kernel, w)
        if r["source_sha256"] == b.kernel_source_hash():
            want = int(r["fetch_kib"] * 1024 * r["fetch_scale"] + r["write_kib"] * 1024 * r["write_scale"])
            assert t == want, key
            assert t >= w.gemm_bytes, key
        else:
            assert t is None, key
        assert b.measured_traffic("no_such_kernel", w) is None


def test_gpu_state_never_raises():
    b = load_bench()
    s = b.gpu_state()
    assert s is None or isinstance(s, dict)


def test_mover_cell_aggregates_by_the_documented_rules():
    """bench.mover_cell on synthetic per-round times: the speedup metrics are the oracle's formulas
    applied to the median of each of T_gemm, T_copy and T_conc; the uplift quartiles come from each
    round's own three times; the copy's concurrent rate is its bytes over its median completion
    time; value-like fields use the mean concurrent time."""
    import statistics

    from concurrent_gemm_dma_amd import _c3 as c3
    from oracle import metrics as om

    b = load_bench()
    t_gemm = [10.0e-3, 10.4e-3, 9.8e-3, 10.1e-3, 10.9e-3]
    r = {"t_copy": [0.78e-3, 0.77e-3, 0.80e-3, 0.76e-3, 0.79e-3],
         "t_conc": [10.3e-3, 10.9e-3, 10.2e-3, 10.4e-3, 11.6e-3],
         "c_gpu": [0.75e-3] * 5, "gk": [10.2e-3] * 5,
         "done": [(10.3, 0.80), (10.9, 0.79), (10.2, 0.81), (10.4, 0.78), (11.6, 0.82)]}
    comm_bytes, flops = float(1 << 30), 14.29e12
    res = b.mover_cell(c3, t_gemm, r, comm_bytes=comm_bytes, flops=flops, hbm_total=2e9,
                       best_copy=0.5e-3)
    Tg, Tc, Tx = (statistics.median(x) for x in (t_gemm, r["t_copy"], r["t_conc"]))
    assert res["t_conc_ms"] == pytest.approx(Tx * 1e3)
    assert res["uplift_fraction"] == pytest.approx(om.uplift_fraction(Tg, Tc, Tx), rel=1e-12)
    assert res["speedup"] == pytest.approx(om.realized_speedup(Tg, Tc, Tx), rel=1e-12)
    assert res["ideal_speedup"] == pytest.approx(om.ideal_speedup(Tg, Tc), rel=1e-12)
    assert res["gemm_slowdown"] == pytest.approx(om.gemm_slowdown(Tg, Tx), rel=1e-12)
    per = sorted(om.uplift_fraction(a, c, x) for a, c, x in zip(t_gemm, r["t_copy"], r["t_conc"]))
    assert res["uplift_per_round_p25_median_p75"] == pytest.approx([per[1], per[2], per[3]])
    assert res["uplift_paired_median"] == pytest.approx(per[2])
    assert res["copy_gbps_concurrent"] == pytest.approx(comm_bytes / 0.80e-3 / 1e9)
    assert res["gemm_tflops_concurrent"] == pytest.approx(flops / statistics.mean(r["t_conc"]) / 1e12)
    assert res["speedup_vs_best_serial"] == pytest.approx((Tg + 0.5e-3) / Tx)
    assert res["anomaly_speedup_above_ideal"] is False
    # a concurrent run faster than either alone is flagged
    r2 = dict(r, t_conc=[9.0e-3] * 5)
    assert b.mover_cell(c3, t_gemm, r2, comm_bytes=comm_bytes, flops=flops, hbm_total=2e9,
                        best_copy=0.5e-3)["anomaly_speedup_above_ideal"] is True
