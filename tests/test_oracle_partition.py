"""Pins of the oracle's CU-partitioning heuristic (roofline estimate, GEMM class, lookup-table
prediction, scoring) against hand-worked values and limiting cases."""
import math

import pytest

from oracle import partition as P

PEAK_F = 2.5e15
PEAK_W = 8.0e12


def test_roofline_time_hand_values():
    # compute-bound: 2 * 8192^3 flops = 1.0995e12; at 70% of 2.5 PF -> 0.62832 ms
    f = 2.0 * 8192 ** 3
    b = 2.0 * 3 * 8192 * 8192
    assert math.isclose(P.roofline_time(f, b, PEAK_F, PEAK_W), f / (0.7 * PEAK_F), rel_tol=1e-15)
    assert math.isclose(P.roofline_time(f, b, PEAK_F, PEAK_W), 6.2832e-4, rel_tol=1e-4)
    # memory-bound: a 1 GiB copy moves 2 GiB; at 70% of 8 TB/s -> 383.5 us
    assert math.isclose(P.roofline_time(0.0, 2.0 * 2 ** 30, PEAK_F, PEAK_W), 3.8347e-4, rel_tol=1e-4)
    # efficiency 1 is the plain roofline
    assert P.roofline_time(4.0, 1.0, 2.0, 1.0, efficiency=1.0) == 2.0
    with pytest.raises(ValueError):
        P.roofline_time(1.0, 1.0, PEAK_F, PEAK_W, efficiency=0.0)


def test_gemm_class():
    def fb(M, N, K):
        return 2.0 * M * N * K, 2.0 * (M * K + K * N + M * N)

    assert P.gemm_class(*fb(8192, 28672, 8192), PEAK_F, PEAK_W) == "compute"
    assert P.gemm_class(*fb(16, 28672, 8192), PEAK_F, PEAK_W) == "memory"
    # machine balance 2.5e15 / 8e12 = 312.5 flop/byte: a square bf16 GEMM reaches it at
    # n / 3 = 312.5, i.e. n = 937.5
    assert P.gemm_class(*fb(936, 936, 936), PEAK_F, PEAK_W) == "memory"
    assert P.gemm_class(*fb(940, 940, 940), PEAK_F, PEAK_W) == "compute"


# GEMM slows as 32 / k on k of 32 CUs; the collective needs 4 CUs per XCC to saturate.
LINEAR_G = {k: 32.0 / k for k in (16, 24, 28, 30, 31)}
SAT_C = {1: 4.0, 2: 2.0, 4: 1.0, 8: 1.0, 16: 1.0}
OPTS = (1, 2, 4, 8, 16)


def test_predict_hand_worked():
    # T_G = 3, T_C = 1:  c=1: max(3*32/31, 4) = 4;  c=2: max(3*32/30, 2) = 3.2;
    # c=4: max(3*32/28, 1) = 3.4286;  c=8: max(3*32/24, 1) = 4;  c=16: max(6, 1) = 6
    c, preds = P.predict_partition(LINEAR_G, SAT_C, 3.0, 1.0, 32, OPTS)
    assert c == 2
    want = [4.0, 3.2, 96.0 / 28.0, 4.0, 6.0]
    assert all(math.isclose(p, w, rel_tol=1e-15) for p, w in zip(preds, want))
    # a longer collective moves the choice to more CUs: T_C = 4 -> c=4 gives max(3.43, 4) = 4,
    # c=8 gives max(4, 4) = 4 (tie -> smaller c), c=2 gives 8
    c, preds = P.predict_partition(LINEAR_G, SAT_C, 3.0, 4.0, 32, OPTS)
    assert c == 4 and preds[2] == 4.0 and preds[3] == 4.0


def test_predict_limits():
    flat = {k: 1.0 for k in (16, 24, 28, 30, 31)}
    # a GEMM that does not care about CUs: give the collective the most
    assert P.predict_partition(flat, SAT_C, 1.0, 1.0, 32, OPTS)[0] == 4  # first c reaching 1.0
    steep_c = {1: 16.0, 2: 8.0, 4: 4.0, 8: 2.0, 16: 1.0}
    assert P.predict_partition(flat, steep_c, 1.0, 1.0, 32, OPTS)[0] == 16
    # a collective that does not care: take the fewest CUs from the GEMM
    flat_c = {c: 1.0 for c in OPTS}
    assert P.predict_partition(LINEAR_G, flat_c, 1.0, 1.0, 32, OPTS)[0] == 1
    # zero-length collective: every split costs the GEMM's slowdown only -> c = 1
    assert P.predict_partition(LINEAR_G, SAT_C, 1.0, 0.0, 32, OPTS)[0] == 1


def test_predict_errors():
    with pytest.raises(ValueError):
        P.predict_partition(LINEAR_G, SAT_C, 1.0, 1.0, 32, (3,))  # 3 and 29 not in the tables
    with pytest.raises(ValueError):
        P.predict_partition(LINEAR_G, SAT_C, 1.0, 1.0, 32, (32,))
    with pytest.raises(ValueError):
        P.predict_partition(LINEAR_G, SAT_C, 1.0, 1.0, 32, ())


def test_score():
    measured = {1: 5.0, 2: 4.0, 4: 4.04, 8: 4.0, 16: 6.0}
    assert P.score(2, measured) == (True, 0.0)       # best (tie with 8 goes to the smaller c)
    hit, loss = P.score(4, measured)
    assert not hit and math.isclose(loss, 0.01)
    hit, loss = P.score(8, measured)
    assert not hit and loss == 0.0
    with pytest.raises(ValueError):
        P.score(3, measured)
