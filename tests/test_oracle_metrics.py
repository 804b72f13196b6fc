"""Pins for the oracle's derived C3 metrics: closed forms, and consistency of the chosen reading
of "% of ideal speedup" with the figures the paper prints (tests/golden/pages_figures.json)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import metrics as m

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def test_ideal_closed_forms():
    assert m.ideal_speedup(3.0, 3.0) == 2.0
    assert m.ideal_speedup(5.0, 0.0) == 1.0
    assert m.ideal_speedup(1.0, 3.0) == pytest.approx(4.0 / 3.0)
    rng = np.random.Generator(np.random.PCG64(5))
    for tg, tc in rng.uniform(1e-6, 1.0, size=(1000, 2)):
        s = m.ideal_speedup(tg, tc)
        assert 1.0 <= s <= 2.0
        assert (s == 2.0) == (tg == tc)
    with pytest.raises(ValueError):
        m.ideal_speedup(0.0, 0.0)


def test_realized_and_uplift():
    tg, tc = 4.0, 2.0
    # perfect overlap: concurrent time = max -> speedup = ideal, uplift fraction 1
    assert m.realized_speedup(tg, tc, 4.0) == pytest.approx(1.5)
    assert m.uplift_fraction(tg, tc, 4.0) == pytest.approx(1.0)
    assert m.ratio_of_ideal(tg, tc, 4.0) == pytest.approx(1.0)
    # no overlap: concurrent time = serial -> speedup 1, uplift 0
    assert m.uplift_fraction(tg, tc, 6.0) == pytest.approx(0.0)
    assert m.ratio_of_ideal(tg, tc, 6.0) == pytest.approx(1.0 / 1.5)
    # halfway
    assert m.uplift_fraction(tg, tc, 6.0 / 1.25) == pytest.approx(0.5)
    assert math.isnan(m.uplift_fraction(1.0, 0.0, 1.0))


def test_taxonomy_and_ceiling():
    assert m.taxonomy(1.0, 1.1) == "GC-equal"
    assert m.taxonomy(1.0, 1.15) == "GC-equal"
    assert m.taxonomy(1.0, 1.2) == "C-long"
    assert m.taxonomy(2.0, 1.0) == "G-long"
    # with ample bandwidth the ceiling equals the ideal; with scarce bandwidth it is lower
    assert m.hbm_ceiling(2.0, 1.0, 1.0, 1e9) == pytest.approx(m.ideal_speedup(2.0, 1.0))
    assert m.hbm_ceiling(2.0, 1.0, 6.0, 2.0) == pytest.approx(1.0)
    assert m.gemm_slowdown(2.0, 2.2) == pytest.approx(0.1)


def test_reading_of_percent_of_ideal_matches_pages():
    """The ideal speedup is at most 2. Read as a plain ratio S / S_ideal, the paper's c3_base
    21% would force S <= 0.42, a slowdown, but the abstract says C3 gives uplifts; read as the
    fraction of the ideal uplift, every printed percentage in (0, 1) means 1 < S < S_ideal.
    The largest printed speedup (1.67x) must not exceed the largest ideal (2)."""
    g = json.load(open(GOLDEN))
    for entry in g["percent_of_ideal"].values():
        p = entry["value"]
        # uplift reading: S = 1 + p (S_ideal - 1) lies in (1, S_ideal) for any S_ideal in (1, 2]
        for s_ideal in (1.01, 1.5, 2.0):
            s = 1.0 + p * (s_ideal - 1.0)
            assert 1.0 < s < s_ideal
            t_g = 1.0
            t_c = s_ideal - 1.0          # so that ideal = (1 + t_c) / 1 = s_ideal
            t_conc = (t_g + t_c) / s
            assert m.uplift_fraction(t_g, t_c, t_conc) == pytest.approx(p)
    assert g["percent_of_ideal"]["c3_base"]["value"] * 2.0 < 1.0  # plain ratio -> slowdown
    assert g["max_speedup_over_serial"]["value"] <= 2.0
    a2a = g["all_to_all_speedup"]
    assert 1.0 < a2a["c3_base"] < a2a["conccl"] <= 2.0


def test_all_metrics_keys():
    d = m.all_metrics(2.0, 1.0, 2.5, bytes_total=8e12, bw_bytes_per_s=8e12)
    assert set(d) >= {"ideal_speedup", "speedup", "uplift_fraction", "ratio_of_ideal",
                      "taxonomy", "gemm_slowdown", "hbm_ceiling"}
    assert d["taxonomy"] == "G-long"
