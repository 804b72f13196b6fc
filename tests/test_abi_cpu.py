"""Host-only checks of the C-ABI library: it loads, exports every symbol include/c3.h declares,
shares torch's single HIP/ROCr runtime, rejects calls before c3_init, and its host-side metric
arithmetic agrees with the oracle's independent formulas. No GPU work is issued here."""
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "c3.h")


@pytest.fixture(scope="module")
def c3():
    from concurrent_gemm_dma_amd import _c3

    if not os.path.exists(_c3.LIB_PATH):
        from concurrent_gemm_dma_amd.build import build

        build()
    _c3.load()
    return _c3


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:c3_status|const char\*)\s+(c3_\w+)\s*\(", text, re.M)))


def test_header_and_binding_agree(c3):
    assert declared_functions() == sorted(c3.EXPORTS)


def test_exports_every_declared_symbol(c3):
    L = c3.load()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_one_hip_and_one_rocr_runtime(c3):
    maps = open("/proc/self/maps").read()
    hip = set(re.findall(r"(\S*/libamdhip64\.so\S*)", maps))
    hsa = set(re.findall(r"(\S*/libhsa-runtime64\.so\S*)", maps))
    assert len(hip) == 1 and len(hsa) == 1, (hip, hsa)


def test_calls_before_init_are_rejected(c3):
    # require_init fails before any HIP call is made
    assert c3.call("c3_gemm", None, None, None, 1, 8, 8, None) == c3.C3_E_NOT_INIT
    assert "c3_init" in c3.c3_last_error()
    assert c3.call("c3_gemm_noalloc", None, None, None, 1, 8, 8, None) == c3.C3_E_NOT_INIT
    assert "c3_init" in c3.c3_last_error()
    info = c3.c3_info()
    assert c3.call("c3_device_info", info) == c3.C3_E_NOT_INIT


def test_struct_layouts_match_c_compiler(c3, tmp_path, host_only):
    """Every binding struct's size and field offsets equal what a C compiler makes of c3.h."""
    import ctypes
    import subprocess

    structs = [c3.c3_info, c3.c3_move_opts, c3.c3_gemm_args, c3.c3_copy_args, c3.c3_conc_opts,
               c3.c3_timing, c3.c3_metrics, c3.c3_slowdown_curve]
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "c3.h"', "int main(void) {"]
    want = []
    for st in structs:
        name = st.__name__
        lines.append(f'printf("%zu\\n", sizeof({name}));')
        want.append(ctypes.sizeof(st))
        for fname, _ in st._fields_:
            lines.append(f'printf("%zu\\n", offsetof({name}, {fname}));')
            want.append(getattr(st, fname).offset)
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), "-o", str(exe), str(src)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert got == want


def test_struct_sizes_match_header_layout(c3):
    import ctypes

    assert ctypes.sizeof(c3.c3_move_opts) == 40
    assert ctypes.sizeof(c3.c3_gemm_args) == 48
    assert ctypes.sizeof(c3.c3_copy_args) == 56 + 40 + 24
    assert ctypes.sizeof(c3.c3_conc_opts) == 32 + 32 + 8 + 8
    assert ctypes.sizeof(c3.c3_timing) == 8 * 8 + 16 + 16 + 2 * 4 * c3.C3_MAX_MASK_WORDS
    assert ctypes.sizeof(c3.c3_metrics) == 6 * 8 + 8
    assert ctypes.sizeof(c3.c3_info) == 12 * 4 + 8 + 64


def test_metrics_agree_with_oracle(c3):
    from oracle import metrics as om

    rng = np.random.Generator(np.random.PCG64(21))
    for _ in range(200):
        tg, tc = rng.uniform(0.1, 10.0, size=2)
        tconc = rng.uniform(max(tg, tc) * 0.9, (tg + tc) * 1.1)
        nbytes = rng.uniform(0, 1e12)
        bw = 8e12
        got = c3.c3_derive_metrics(tg, tc, tconc, nbytes, bw)
        want = om.all_metrics(tg, tc, tconc, bytes_total=nbytes, bw_bytes_per_s=bw)
        for k in ("ideal_speedup", "speedup", "uplift_fraction", "ratio_of_ideal", "gemm_slowdown",
                  "hbm_ceiling"):
            assert got[k] == pytest.approx(want[k], rel=1e-12), k
        assert got["taxonomy"] == want["taxonomy"]
    assert math.isnan(c3.c3_derive_metrics(1.0, 0.0, 1.0)["uplift_fraction"])
    with pytest.raises(c3.C3Error):
        c3.c3_derive_metrics(0.0, 0.0, 1.0)


def test_partition_heuristic_matches_oracle(c3):
    """libc3's host-side heuristic against the oracle's: same choice and bit-identical
    predictions on random tables; same rejections."""
    import random

    from oracle import partition as P

    rng = random.Random(12)
    opts = (1, 2, 4, 8, 16)
    for trial in range(300):
        g = {32 - c: rng.uniform(1.0, 3.0) for c in opts}
        cm = {c: rng.uniform(0.5, 20.0) for c in opts}
        if trial % 7 == 0:  # force ties
            cm = {c: 1.0 for c in opts}
            g = {32 - c: 1.0 for c in opts}
        tg, tc = rng.uniform(0, 5), rng.uniform(0, 5)
        want = P.predict_partition(g, cm, tg, tc, 32, opts)
        got = c3.c3_predict_partition(g, cm, tg, tc, 32, opts)
        assert got[0] == want[0] and got[1] == want[1], (trial, got, want)
    for f, b in ((2.0 * 8192 ** 3, 6.0 * 8192 ** 2), (0.0, 2.0 ** 31), (1e9, 1e9)):
        assert c3.c3_roofline_time(f, b, 2.5e15, 8e12) == P.roofline_time(f, b, 2.5e15, 8e12)
    with pytest.raises(c3.C3Error):
        c3.c3_predict_partition({31: 1.0}, {1: 1.0}, 1.0, 1.0, 32, (2,))
    with pytest.raises(c3.C3Error):
        c3.c3_predict_partition({31: 1.0}, {1: 1.0}, 1.0, 1.0, 32, (32,))
    with pytest.raises(c3.C3Error):
        c3.c3_roofline_time(1.0, 1.0, 1.0, 1.0, 0.0)


def test_hybrid_share_closed_forms(c3):
    """The hybrid mover's engine share balances f * t_sdma against t_gemm + (1 - f) * t_cu:
    closed-form cases, the clamp, and brute force over every permille on random times."""
    import random

    assert c3.c3_hybrid_share(0.0, 2.0, 2.0) == 500        # no GEMM, equal movers: half each
    assert c3.c3_hybrid_share(0.0, 3.0, 1.0) == 250        # engines 3x slower: a quarter
    assert c3.c3_hybrid_share(1.0, 3.0, 1.0) == 500        # (1 + 1) / (3 + 1)
    assert c3.c3_hybrid_share(10.0, 1.0, 0.25) == 1000     # GEMM outlasts the whole DMA copy
    assert c3.c3_hybrid_share(1.0, 1.0, 0.25) == 1000      # GEMM as long as the DMA copy: f = 1
    assert c3.c3_hybrid_share(0.75, 1.0, 0.25) == 800      # (0.75 + 0.25) / (1 + 0.25)

    def model(pm, tg, ts, tc):
        f = pm / 1000.0
        return max(f * ts, tg + (1.0 - f) * tc)

    rng = random.Random(5)
    for _ in range(500):
        tg, ts, tc = rng.uniform(0, 3), rng.uniform(0.01, 3), rng.uniform(0.01, 3)
        got = c3.c3_hybrid_share(tg, ts, tc)
        assert 0 <= got <= 1000
        best = min(model(pm, tg, ts, tc) for pm in range(1001))
        # rounding f to thousandths costs at most 0.5/1000 of the slower mover's time
        assert model(got, tg, ts, tc) <= best + 0.5e-3 * max(ts, tc) + 1e-12, (tg, ts, tc, got)
    for bad in ((-1.0, 1.0, 1.0), (1.0, 0.0, 1.0), (1.0, 1.0, 0.0), (float("nan"), 1.0, 1.0),
                (1.0, float("inf"), 1.0)):
        with pytest.raises(c3.C3Error):
            c3.c3_hybrid_share(*bad)


def test_readme_c_example_compiles(tmp_path):
    """The C usage example in README.md compiles against include/c3.h as C11."""
    import re
    import shutil
    import subprocess

    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    readme = open(os.path.join(os.path.dirname(HEADER), "..", "README.md")).read()
    blocks = re.findall(r"```c\n(.*?)```", readme, re.S)
    assert blocks, "README.md has no C example"
    src = tmp_path / "example.c"
    src.write_text(blocks[0])
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-fsyntax-only", "-I",
                        os.path.dirname(HEADER), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr

