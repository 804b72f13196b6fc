"""Derived C3 metrics, oracle side (test infrastructure only; pure Python, no library code).

Source: "Optimizing ML Concurrent Computation and Communication with GPU DMA Engines"
(arXiv 2412.14335).
  * Ideal speedup (abstract; Section IV-B3, Fig. 7): serial time (computation plus
    communication) over the larger of the two, every time taken from an isolated run.
  * "% of ideal speedup" (abstract; Pith review, circularity check): the abstract's figures
    (21%, 42%, 72%) only make sense as the fraction of the ideal *uplift* that is realized,
    (S - 1) / (S_ideal - 1): a plain ratio S / S_ideal of 21% would mean running far slower
    than serial, which contradicts the abstract's statement that C3 gives uplifts. Both forms
    are computed; the uplift fraction is the headline reading.
  * Taxonomy (Section III, Fig. 4): G-long, C-long or GC-equal. The thresholds reach us
    garbled ("115% and 15%"); the reading taken is GC-equal when the longer isolated time is
    at most 1.15x the shorter, else G-long (GEMM longer) or C-long (communication longer).
  * HBM-aware ceiling: the paper attributes the residual gap to shared HBM bandwidth
    (Section VI-F); with both operations moving bytes through HBM, the concurrent time cannot
    drop below total bytes / bandwidth, so S <= (T_g + T_c) / max(T_g, T_c, bytes / BW).
"""
from __future__ import annotations

import math


def ideal_speedup(t_gemm: float, t_copy: float) -> float:
    """(T_gemm + T_copy) / max(T_gemm, T_copy) from isolated runs; in [1, 2]."""
    if t_gemm < 0 or t_copy < 0 or max(t_gemm, t_copy) <= 0:
        raise ValueError("times must be non-negative with a positive maximum")
    return (t_gemm + t_copy) / max(t_gemm, t_copy)


def realized_speedup(t_gemm: float, t_copy: float, t_conc: float) -> float:
    """Serial time (T_gemm + T_copy) over the measured concurrent time."""
    if t_conc <= 0:
        raise ValueError("t_conc must be positive")
    return (t_gemm + t_copy) / t_conc


def uplift_fraction(t_gemm: float, t_copy: float, t_conc: float) -> float:
    """(S - 1) / (S_ideal - 1); NaN when the ideal uplift is zero (one time is zero)."""
    s_ideal = ideal_speedup(t_gemm, t_copy)
    s = realized_speedup(t_gemm, t_copy, t_conc)
    if s_ideal == 1.0:
        return float("nan")
    return (s - 1.0) / (s_ideal - 1.0)


def ratio_of_ideal(t_gemm: float, t_copy: float, t_conc: float) -> float:
    """The plain ratio S / S_ideal (secondary reading)."""
    return realized_speedup(t_gemm, t_copy, t_conc) / ideal_speedup(t_gemm, t_copy)


def taxonomy(t_gemm: float, t_copy: float, threshold: float = 1.15) -> str:
    """'GC-equal' if max/min <= threshold, else 'G-long' or 'C-long'."""
    lo, hi = min(t_gemm, t_copy), max(t_gemm, t_copy)
    if lo > 0 and hi / lo <= threshold:
        return "GC-equal"
    return "G-long" if t_gemm > t_copy else "C-long"


def hbm_ceiling(t_gemm: float, t_copy: float, bytes_total: float, bw_bytes_per_s: float) -> float:
    """Upper bound on S when both operations share one HBM of bandwidth bw."""
    floor_t = max(t_gemm, t_copy, bytes_total / bw_bytes_per_s)
    return (t_gemm + t_copy) / floor_t


def gemm_slowdown(t_gemm: float, t_conc: float) -> float:
    """T_conc / T_gemm - 1: how much longer the GEMM-bound concurrent run takes than the GEMM alone."""
    return t_conc / t_gemm - 1.0


def all_metrics(t_gemm: float, t_copy: float, t_conc: float, bytes_total: float = 0.0,
                bw_bytes_per_s: float = 8.0e12) -> dict:
    out = {
        "ideal_speedup": ideal_speedup(t_gemm, t_copy),
        "speedup": realized_speedup(t_gemm, t_copy, t_conc),
        "uplift_fraction": uplift_fraction(t_gemm, t_copy, t_conc),
        "ratio_of_ideal": ratio_of_ideal(t_gemm, t_copy, t_conc),
        "taxonomy": taxonomy(t_gemm, t_copy),
        "gemm_slowdown": gemm_slowdown(t_gemm, t_conc) if t_gemm > 0 else math.nan,
    }
    if bytes_total > 0:
        out["hbm_ceiling"] = hbm_ceiling(t_gemm, t_copy, bytes_total, bw_bytes_per_s)
    return out
