/*
 * oracle.c -- plain CPU oracle for the C3 hot path. TEST INFRASTRUCTURE ONLY (see oracle.h).
 *
 * Every routine is the literal definition of one result, written as plainly as possible:
 * no blocking, no reordering of any element's arithmetic, no vector intrinsics. OpenMP only
 * splits independent output elements (or independent memcpy calls) between threads.
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no fast-math), see oracle/build.py.
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------ */
/* bf16 format                                                                                  */
/* ------------------------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t bits_from_f32(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

uint32_t orc_f32_bits_from_bf16(uint16_t h) { return (uint32_t)h << 16; }

static float f32_from_bf16(uint16_t h) { return f32_from_bits(orc_f32_bits_from_bf16(h)); }

/*
 * Round an fp32 to bf16, nearest with ties to even, by integer arithmetic on the bit pattern:
 * adding 0x7FFF plus the lowest kept bit, then truncating the low 16 bits, rounds the 16
 * dropped bits up exactly when they exceed one half, or equal one half with an odd kept part.
 * A carry out of the mantissa steps the exponent (and the largest finite values round to Inf),
 * as IEEE rounding requires. NaNs are kept NaN (quiet bit forced so truncation cannot make Inf).
 */
uint16_t orc_bf16_from_f32_bits(uint32_t u) {
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u) {
        return (uint16_t)((u >> 16) | 0x0040u);
    }
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/*
 * Round an fp64 to bf16 with a single rounding: bf16 keeps 8 significant bits, so a finite
 * nonzero x with |x| in [2^(e-1), 2^e) is rounded to a multiple of 2^(e-8); below the smallest
 * normal (2^-126) the spacing stays 2^-133 (bf16 subnormals). nearbyint() in the default
 * rounding mode rounds half to even; the power-of-two scalings are exact. The rounded value
 * has at most 8 significant bits, so it converts to fp32 exactly, except a result of 2^128,
 * which converts to Inf (overflow under round-to-nearest).
 */
uint16_t orc_bf16_from_f64(double x) {
    if (isnan(x)) {
        return (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u);
    }
    if (isinf(x) || x == 0.0) {
        return (uint16_t)(bits_from_f32((float)x) >> 16);
    }
    int e = 0;
    (void)frexp(x, &e);
    int q = e - 8;
    if (q < -133) q = -133;
    double r = ldexp(nearbyint(ldexp(x, -q)), q);
    return (uint16_t)(bits_from_f32((float)r) >> 16);
}

void orc_bf16_from_f32_bits_array(const uint32_t* in, uint16_t* out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f32_bits(in[i]);
}

void orc_bf16_from_f64_array(const double* in, uint16_t* out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f64(in[i]);
}

int orc_threads(int nthreads) { return nthreads > 0 ? nthreads : omp_get_max_threads(); }

/* ------------------------------------------------------------------------------------------ */
/* GEMM                                                                                         */
/* ------------------------------------------------------------------------------------------ */

/* One element with fp32 accumulation, k ascending from a +0.0f start. */
static float dot_f32(const uint16_t* A, const uint16_t* B, int64_t N, int64_t K, int64_t i,
                     int64_t j) {
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float a = f32_from_bf16(A[i * K + k]);
        float b = f32_from_bf16(B[k * N + j]);
        acc = acc + a * b;
    }
    return acc;
}

/* One element with fp64 accumulation, k ascending; every bf16 x bf16 product is exact in fp64. */
static double dot_f64(const uint16_t* A, const uint16_t* B, int64_t N, int64_t K, int64_t i,
                      int64_t j) {
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double a = (double)f32_from_bf16(A[i * K + k]);
        double b = (double)f32_from_bf16(B[k * N + j]);
        s = s + a * b;
    }
    return s;
}

void orc_gemm_f32acc_rows(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                          int64_t row_begin, int64_t row_end, uint16_t* C_out, float* acc_out,
                          int nthreads) {
    (void)M;
    const int64_t rows = row_end - row_begin;
    const int64_t total = rows * N;
#pragma omp parallel for schedule(static) num_threads(orc_threads(nthreads))
    for (int64_t t = 0; t < total; ++t) {
        const int64_t i = row_begin + t / N;
        const int64_t j = t % N;
        const float acc = dot_f32(A, B, N, K, i, j);
        C_out[t] = orc_bf16_from_f32_bits(bits_from_f32(acc));
        if (acc_out) acc_out[t] = acc;
    }
}

void orc_gemm_f64acc_rows(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                          int64_t row_begin, int64_t row_end, uint16_t* C_out, double* sum_out,
                          int nthreads) {
    (void)M;
    const int64_t rows = row_end - row_begin;
    const int64_t total = rows * N;
#pragma omp parallel for schedule(static) num_threads(orc_threads(nthreads))
    for (int64_t t = 0; t < total; ++t) {
        const int64_t i = row_begin + t / N;
        const int64_t j = t % N;
        const double s = dot_f64(A, B, N, K, i, j);
        if (C_out) C_out[t] = orc_bf16_from_f64(s);
        if (sum_out) sum_out[t] = s;
    }
}

int orc_gemm_elems(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                   const int64_t* rows, const int64_t* cols, int64_t n, uint16_t* c32,
                   uint16_t* c64, double* s64, int nthreads) {
    for (int64_t t = 0; t < n; ++t) {
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -1;
    }
#pragma omp parallel for schedule(dynamic, 16) num_threads(orc_threads(nthreads))
    for (int64_t t = 0; t < n; ++t) {
        if (c32) c32[t] = orc_bf16_from_f32_bits(bits_from_f32(dot_f32(A, B, N, K, rows[t], cols[t])));
        if (c64 || s64) {
            const double s = dot_f64(A, B, N, K, rows[t], cols[t]);
            if (c64) c64[t] = orc_bf16_from_f64(s);
            if (s64) s64[t] = s;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Collective-shaped copies                                                                     */
/* ------------------------------------------------------------------------------------------ */

void orc_gather(void* dst, const void* const* shards, int n_shards, size_t shard_bytes) {
    for (int i = 0; i < n_shards; ++i) {
        memcpy((unsigned char*)dst + (size_t)i * shard_bytes, shards[i], shard_bytes);
    }
}

void orc_all2all_block(void* dst, const void* src, int grid, size_t block_bytes) {
    for (int i = 0; i < grid; ++i) {
        for (int j = 0; j < grid; ++j) {
            const size_t from = ((size_t)i * (size_t)grid + (size_t)j) * block_bytes;
            const size_t to = ((size_t)j * (size_t)grid + (size_t)i) * block_bytes;
            memcpy((unsigned char*)dst + to, (const unsigned char*)src + from, block_bytes);
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* All-reduce local share: reduce-scatter (arithmetic) then all-gather (copy)                   */
/* ------------------------------------------------------------------------------------------ */

/*
 * Reduce-scatter local share: element e of this rank's chunk is the sum of the `world` ranks'
 * contributions in[0][e], ..., in[world-1][e]. Reading taken (the pages give no precision or
 * order): fp32 accumulation, starting from rank 0's value and adding ranks 1, 2, ... in order,
 * one rounding to bf16 at the end.
 */
void orc_reduce_sum_bf16(const uint16_t* const* in, int world, size_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < (int64_t)n; ++e) {
        float acc = f32_from_bf16(in[0][e]);
        for (int r = 1; r < world; ++r) {
            acc = acc + f32_from_bf16(in[r][e]);
        }
        out[e] = orc_bf16_from_f32_bits(bits_from_f32(acc));
    }
}

/*
 * All-reduce local share = reduce-scatter, then all-gather of the reduced chunks: `reduced`
 * receives this rank's reduced chunk; dst slot i (chunk_elems bf16 each) receives `reduced` for
 * i == rank and the other ranks' reduced chunks peers[i] otherwise.
 */
void orc_allreduce_local(const uint16_t* const* contribs, const uint16_t* const* peers, int world,
                         int rank, size_t chunk_elems, uint16_t* reduced, uint16_t* dst) {
    orc_reduce_sum_bf16(contribs, world, chunk_elems, reduced);
    for (int i = 0; i < world; ++i) {
        const uint16_t* from = (i == rank) ? reduced : peers[i];
        memcpy(dst + (size_t)i * chunk_elems, from, chunk_elems * sizeof(uint16_t));
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Checkers                                                                                     */
/* ------------------------------------------------------------------------------------------ */

int64_t orc_first_diff(const void* a, const void* b, size_t n) {
    const unsigned char* pa = (const unsigned char*)a;
    const unsigned char* pb = (const unsigned char*)b;
    for (size_t i = 0; i < n; ++i) {
        if (pa[i] != pb[i]) return (int64_t)i;
    }
    return -1;
}

void orc_gemm_compare(const uint16_t* ref, const uint16_t* got, int64_t n, double tol,
                      orc_gemm_report* rep) {
    int64_t n_diff = 0, n_viol = 0, first = -1, nonfinite = 0;
    double max_scaled = 0.0, num = 0.0, den = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        const double r = (double)f32_from_bf16(ref[t]);
        const double g = (double)f32_from_bf16(got[t]);
        if (ref[t] != got[t]) ++n_diff;
        if (!isfinite(g)) ++nonfinite;
        const double d = fabs(g - r);
        const double scale = fabs(r) > 1.0 ? fabs(r) : 1.0;
        const double scaled = d / scale;
        const int bad = !(scaled <= tol); /* NaN compares false -> counted as a violation */
        if (bad) {
            ++n_viol;
            if (first < 0) first = t;
        }
        if (scaled > max_scaled || isnan(scaled)) max_scaled = scaled;
        num += (g - r) * (g - r);
        den += r * r;
    }
    rep->n = n;
    rep->n_diff = n_diff;
    rep->n_violations = n_viol;
    rep->first_violation = first;
    rep->max_scaled_err = max_scaled;
    rep->frob_rel = den > 0.0 ? sqrt(num) / sqrt(den) : (num > 0.0 ? INFINITY : 0.0);
    rep->n_nonfinite = nonfinite;
}
