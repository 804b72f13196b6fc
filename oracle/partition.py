"""CU-partitioning heuristic, oracle side -- TEST INFRASTRUCTURE ONLY (pure Python, no library
code; only the test suite and the benchmark's cpu_baseline leg may import it).

Source: "Optimizing ML Concurrent Computation and Communication with GPU DMA Engines"
(arXiv 2412.14335) as the Pith review of it reports:
  * resource partitioning (c3_rp, Section V-B): the GEMM and a CU-based collective run on
    disjoint sets of CUs; the paper's figure is the best of a sweep over power-of-two CU
    allocations (review, free parameters; referee minor comment 3);
  * the heuristic (Section V-C): a one-time lookup table of kernel slowdowns plus a roofline
    model with a 0.70 efficiency factor picks the allocation (review, "If this is right";
    free parameters); it matched the sweep's best in 24 of 30 scenarios, losing at most 1.5%
    ("Significance").

Reading taken (the pages name the ingredients, not the formula):
  1. A slowdown curve S(k) = T(kernel on k CUs per XCC) / T(kernel on all CUs), measured once
     per kernel class (a compute-bound GEMM, a memory-bound GEMM, each collective kind) and
     looked up, not interpolated: a split the table does not hold is an error.
  2. Isolated times come from a roofline at 70% efficiency:
     T = max(flops / (0.70 * peak_flops), bytes / (0.70 * peak_bandwidth)); a GEMM's class is
     the roofline term that dominates.
  3. For a split that gives the collective c CUs per XCC and the GEMM the other N - c, the two
     kernels run side by side on disjoint CUs, so the predicted concurrent time is
     max(T_G * S_G(N - c), T_C * S_C(c)).
  4. The split with the smallest prediction is chosen; a tie goes to the smaller c (fewer CUs
     taken from the GEMM).
  5. Scoring against the exhaustive sweep: a hit when the chosen split is the measured best;
     loss = T_conc(chosen) / T_conc(best) - 1.
"""
from __future__ import annotations

from typing import Mapping, Sequence

EFFICIENCY = 0.70


def roofline_time(flops: float, nbytes: float, peak_flops: float, peak_bw: float,
                  efficiency: float = EFFICIENCY) -> float:
    """max(flops / (eff * peak_flops), bytes / (eff * peak_bw)), in seconds for SI inputs."""
    if flops < 0 or nbytes < 0 or peak_flops <= 0 or peak_bw <= 0 or not 0 < efficiency <= 1:
        raise ValueError("roofline_time: need flops, bytes >= 0, peaks > 0, 0 < efficiency <= 1")
    return max(flops / (efficiency * peak_flops), nbytes / (efficiency * peak_bw))


def gemm_class(flops: float, nbytes: float, peak_flops: float, peak_bw: float) -> str:
    """'compute' when the compute term of the roofline is at least the memory term."""
    return "compute" if flops / peak_flops >= nbytes / peak_bw else "memory"


def lookup(curve: Mapping[int, float], k: int) -> float:
    """Slowdown at k CUs per XCC from a table {k: T(k) / T(all)}."""
    if k not in curve:
        raise ValueError(f"slowdown table has no entry for {k} CUs per XCC")
    return float(curve[k])


def predict_partition(gemm_curve: Mapping[int, float], comm_curve: Mapping[int, float],
                      t_gemm: float, t_comm: float, cus_per_xcc: int,
                      options: Sequence[int]) -> tuple[int, list[float]]:
    """(chosen c, predicted concurrent time of every option in order)."""
    if t_gemm < 0 or t_comm < 0:
        raise ValueError("times must be non-negative")
    if not options:
        raise ValueError("no split to choose from")
    preds = []
    for c in options:
        if not 0 < c < cus_per_xcc:
            raise ValueError(f"split {c} leaves no CU to one side")
        preds.append(max(t_gemm * lookup(gemm_curve, cus_per_xcc - c), t_comm * lookup(comm_curve, c)))
    best = None
    for c, p in zip(options, preds):
        if best is None or p < best[1] or (p == best[1] and c < best[0]):
            best = (c, p)
    return best[0], preds


def score(chosen: int, measured: Mapping[int, float]) -> tuple[bool, float]:
    """(hit, loss) of a chosen split against measured concurrent times {c: T_conc}."""
    if chosen not in measured:
        raise ValueError("the chosen split was not measured")
    best_t = min(measured.values())
    best_c = min(c for c, t in measured.items() if t == best_t)
    return chosen == best_c, measured[chosen] / best_t - 1.0
