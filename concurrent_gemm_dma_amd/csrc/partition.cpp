// partition.cpp -- the CU-partitioning heuristic: a one-time lookup table of kernel slowdowns
// against the CUs they get, plus a roofline estimate of isolated times at 70% efficiency, picks
// the CU split between a GEMM and a CU-based collective ("Optimizing ML Concurrent Computation
// and Communication with GPU DMA Engines", Section V-B resource partitioning, Section V-C
// heuristic, as the Pith review reports them). The two kernels run on disjoint CUs, so a split
// is predicted to take as long as the slower of the two under it. Also the share of a copy
// the hybrid mover gives the SDMA engines. Host arithmetic only.
#include <cmath>

#include "c3_internal.h"

namespace {

// Slowdown at k CUs per XCC, or a negative value when the curve has no entry for k.
double lookup(const c3_slowdown_curve& c, int k) {
    for (int i = 0; i < c.n; ++i)
        if (c.cus_per_xcc[i] == k) return c.slowdown[i];
    return -1.0;
}

c3_status check_curve(const c3_slowdown_curve* c, const char* what) {
    if (!c) return c3::fail(C3_E_INVALID, "%s curve is NULL", what);
    if (c->n < 1 || c->n > C3_MAX_CURVE)
        return c3::fail(C3_E_INVALID, "%s curve: n must be in [1, %d]", what, C3_MAX_CURVE);
    for (int i = 0; i < c->n; ++i) {
        if (!(c->slowdown[i] > 0) || !std::isfinite(c->slowdown[i]))
            return c3::fail(C3_E_INVALID, "%s curve: slowdown %d must be finite and > 0", what, i);
        for (int j = 0; j < i; ++j)
            if (c->cus_per_xcc[j] == c->cus_per_xcc[i])
                return c3::fail(C3_E_INVALID, "%s curve: %d CUs listed twice", what, c->cus_per_xcc[i]);
    }
    return C3_OK;
}

}  // namespace

extern "C" {

c3_status c3_roofline_time(double flops, double bytes, double peak_flops, double peak_bw,
                           double efficiency, double* t_out) {
    if (!t_out) return c3::fail(C3_E_INVALID, "c3_roofline_time: t_out is NULL");
    if (!(flops >= 0) || !(bytes >= 0) || !(peak_flops > 0) || !(peak_bw > 0) ||
        !(efficiency > 0 && efficiency <= 1))
        return c3::fail(C3_E_INVALID,
                        "c3_roofline_time: need flops, bytes >= 0, peaks > 0, 0 < efficiency <= 1");
    *t_out = std::fmax(flops / (efficiency * peak_flops), bytes / (efficiency * peak_bw));
    return C3_OK;
}

c3_status c3_predict_partition(const c3_slowdown_curve* gemm, const c3_slowdown_curve* comm,
                               double t_gemm, double t_comm, int cus_per_xcc,
                               const int32_t* options, int n_options, int32_t* chosen_out,
                               double* predicted_out) {
    C3_TRY(check_curve(gemm, "GEMM"));
    C3_TRY(check_curve(comm, "communication"));
    if (!chosen_out) return c3::fail(C3_E_INVALID, "c3_predict_partition: chosen_out is NULL");
    if (!options || n_options < 1) return c3::fail(C3_E_INVALID, "c3_predict_partition: no options");
    if (!(t_gemm >= 0) || !(t_comm >= 0))
        return c3::fail(C3_E_INVALID, "c3_predict_partition: times must be >= 0");
    int best_c = 0;
    double best_t = 0.0;
    for (int i = 0; i < n_options; ++i) {
        const int c = options[i];
        if (c <= 0 || c >= cus_per_xcc)
            return c3::fail(C3_E_INVALID, "split %d leaves no CU to one side", c);
        const double sg = lookup(*gemm, cus_per_xcc - c), sc = lookup(*comm, c);
        if (sg < 0 || sc < 0)
            return c3::fail(C3_E_INVALID, "slowdown table lacks %d (GEMM) or %d (communication) CUs",
                            cus_per_xcc - c, c);
        const double p = std::fmax(t_gemm * sg, t_comm * sc);
        if (predicted_out) predicted_out[i] = p;
        if (i == 0 || p < best_t || (p == best_t && c < best_c)) {
            best_c = c;
            best_t = p;
        }
    }
    *chosen_out = best_c;
    return C3_OK;
}

c3_status c3_hybrid_share(double t_gemm, double t_sdma, double t_cu, int32_t* permille_out) {
    if (!permille_out) return c3::fail(C3_E_INVALID, "c3_hybrid_share: permille_out is NULL");
    if (!(t_gemm >= 0) || !(t_sdma > 0) || !(t_cu > 0) || !std::isfinite(t_gemm) ||
        !std::isfinite(t_sdma) || !std::isfinite(t_cu))
        return c3::fail(C3_E_INVALID, "c3_hybrid_share: need finite t_gemm >= 0, t_sdma > 0, t_cu > 0");
    // engines' part f * t_sdma against the GEMM plus the CUs' part, t_gemm + (1 - f) * t_cu
    const double f = std::fmin(1.0, (t_gemm + t_cu) / (t_sdma + t_cu));
    *permille_out = (int32_t)std::lround(1000.0 * f);
    return C3_OK;
}

}  // extern "C"
