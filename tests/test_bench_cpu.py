"""Host-side checks of bench.py (no GPU work): the one-GPU contract refuses more GPUs before
touching any device, defaults match the documented protocol, and the traffic record lookup is
consistent with the committed counter file."""
import importlib.util
import json
import os
import subprocess
import sys

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
    assert (a.gpus, a.steps, a.warmup, a.mode, a.workload) == (1, 20, 3, "c3", 4)
    assert b.PEAK_BF16_TFLOPS == 2500.0 and b.PEAK_HBM_GBPS == 8000.0


def test_traffic_record_lookup_is_consistent():
    b = load_bench()
    from concurrent_gemm_dma_amd import workloads as wl

    w = wl.WORKLOADS[2]
    rec = json.load(open(os.path.join(ROOT, "profiles", "gemm_traffic.json")))
    key = f"gemm_bf16_tile256_dma@{w.name}"
    t = b.measured_traffic("gemm_bf16_tile256_dma", w)
    if rec[key]["source_sha256"] == b.kernel_source_hash():
        r = rec[key]
        want = int(r["fetch_kib"] * 1024 * r["fetch_scale"] + r["write_kib"] * 1024 * r["write_scale"])
        assert t == want
        # the GEMM moves at least its algorithmic bytes
        assert t >= w.gemm_bytes
    else:
        assert t is None
    assert b.measured_traffic("no_such_kernel", w) is None


def test_gpu_state_never_raises():
    b = load_bench()
    s = b.gpu_state()
    assert s is None or isinstance(s, dict)
