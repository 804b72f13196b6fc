/*
 * oracle.h -- plain CPU oracle for the C3 hot path (concurrent bf16 GEMM + collective-shaped copy).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke entry point and the benchmark's
 * cpu_baseline leg may load or call this code. The product library (libc3) shares no code,
 * header, helper or constant with it, and neither side includes or links the other.
 *
 * Source of what is computed: "Optimizing ML Concurrent Computation and Communication with GPU
 * DMA Engines" (Agrawal, Aga, Pati, Islam; arXiv 2412.14335).
 *   - Concurrency (C3) changes when work runs, never what it computes (abstract; Fig. 1): the
 *     concurrent results are exactly the serial results, so each oracle routine is the plain
 *     definition of one result.
 *   - GEMM: the paper runs GEMM kernels from LLaMA training (Section IV, Fig. 5a) but names no
 *     precision. Reading taken here: bf16 operands, row-major A[M][K], B[K][N], C[M][N],
 *     C = A.B with no scaling, bias or accumulation into C, bf16 result rounded to nearest even.
 *   - All-gather / all-to-all: the ConCCL proof-of-concepts split the collective into individual
 *     transfers (Pith review of arXiv 2412.14335, skeptic critique "load-bearing attack";
 *     Section VI-B). On one GPU the data movement is the local share: gather 8 shards into one
 *     buffer, or transpose an 8x8 grid of blocks. Bytes are moved verbatim.
 *   - Correctness check: every output buffer must be compared against a CPU reference after
 *     each concurrent run (Pith review, skeptic critique "concrete test").
 *
 * Parity pins live in the test suite (brute force in fp64, closed-form error bounds, identity /
 * zero / integer-exact invariants, per-byte loops, an independent bf16 rounding formulation).
 */
#ifndef C3_ORACLE_H
#define C3_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- bf16 format (1 sign, 8 exponent, 7 stored mantissa bits; the top half of an IEEE fp32) ---- */

/* fp32 bit pattern -> bf16 bit pattern, round to nearest, ties to even. NaN -> quiet NaN. */
uint16_t orc_bf16_from_f32_bits(uint32_t f32_bits);
/* fp64 value -> bf16 bit pattern with ONE rounding (nearest, ties to even), no detour via fp32. */
uint16_t orc_bf16_from_f64(double x);
/* bf16 bit pattern -> fp32 bit pattern (exact). */
uint32_t orc_f32_bits_from_bf16(uint16_t h);
/* Array forms of the two conversions above. */
void orc_bf16_from_f32_bits_array(const uint32_t* in, uint16_t* out, size_t n);
void orc_bf16_from_f64_array(const double* in, uint16_t* out, size_t n);

/* ---- GEMM, C = A.B (bf16 in, bf16 out) ---- */

/*
 * fp32-accumulate triple loop: for each (i, j), acc = +0.0f, then for k = 0, 1, ..., K-1:
 * acc = acc + fp32(A[i][k]) * fp32(B[k][j]) in fp32, then C[i][j] = bf16_rne(acc).
 * Rows [row_begin, row_end) of C are written to C_out (row-major, (row_end-row_begin) x N).
 * acc_out, if not NULL, receives the unrounded fp32 sums in the same layout.
 * nthreads <= 0 uses every available core; threads only split independent output elements.
 */
void orc_gemm_f32acc_rows(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                          int64_t row_begin, int64_t row_end, uint16_t* C_out, float* acc_out,
                          int nthreads);

/*
 * fp64-accumulate reference: for each (i, j), s = sum_k fp64(A[i][k]) * fp64(B[k][j]) with k
 * ascending (each product is exact in fp64), then C[i][j] = bf16_rne(s) with one rounding.
 * Same row-range convention as above. sum_out, if not NULL, receives the fp64 sums.
 */
void orc_gemm_f64acc_rows(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                          int64_t row_begin, int64_t row_end, uint16_t* C_out, double* sum_out,
                          int nthreads);

/*
 * Selected elements (rows[t], cols[t]) for t < n, both accumulation kinds at once:
 * c32[t] = bf16 of the fp32-accumulate sum, c64[t] = bf16 of the fp64 sum (either may be NULL),
 * s64[t] = the fp64 sum (may be NULL). Returns -1 if an index is out of range, else 0.
 */
int orc_gemm_elems(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                   const int64_t* rows, const int64_t* cols, int64_t n, uint16_t* c32,
                   uint16_t* c64, double* s64, int nthreads);

/* ---- Collective-shaped copies (local share on one GPU) ---- */

/* All-gather local share: dst[i*shard_bytes + b] = shards[i][b], i < n_shards, b < shard_bytes. */
void orc_gather(void* dst, const void* const* shards, int n_shards, size_t shard_bytes);

/*
 * All-to-all local share as a block transpose of a grid x grid array of blocks:
 * source block (i, j) at byte offset (i*grid + j)*block_bytes is copied verbatim to
 * destination offset (j*grid + i)*block_bytes.
 */
void orc_all2all_block(void* dst, const void* src, int grid, size_t block_bytes);

/* ---- All-reduce local share (reduce-scatter + all-gather) ---- */

/*
 * DMA engines do no arithmetic, so an all-reduce is split into a reduce-scatter (the sum, on the
 * compute units) and an all-gather of the reduced chunks (a copy, which the engines can do)
 * (L3 Synthesis page on 2412.14335, section 3 "attack surface", Attack 1; Pith review, "Reading
 * between the lines"). On one GPU only the local share exists.
 *
 * Reduce-scatter local share: out[e] = bf16_rne(fp32 sum of in[r][e]), the sum started from
 * rank 0's value with ranks 1..world-1 added in order (reading taken: the pages fix neither
 * precision nor order). world >= 1; n elements per rank.
 */
void orc_reduce_sum_bf16(const uint16_t* const* in, int world, size_t n, uint16_t* out);

/*
 * All-reduce local share: reduced = orc_reduce_sum_bf16(contribs); then dst slot i (chunk_elems
 * elements) = reduced if i == rank, else peers[i] (the other ranks' reduced chunks; peers[rank]
 * is not read).
 */
void orc_allreduce_local(const uint16_t* const* contribs, const uint16_t* const* peers, int world,
                         int rank, size_t chunk_elems, uint16_t* reduced, uint16_t* dst);

/* ---- Checkers ---- */

/* Offset of the first differing byte, or -1 if the two ranges are equal. */
int64_t orc_first_diff(const void* a, const void* b, size_t n);

typedef struct {
    int64_t n;               /* elements compared */
    int64_t n_diff;          /* elements whose bf16 bit patterns differ */
    int64_t n_violations;    /* elements with |got - ref| > tol * max(1, |ref|) (NaN counts) */
    int64_t first_violation; /* index of the first violation, -1 if none */
    double max_scaled_err;   /* max over elements of |got - ref| / max(1, |ref|) */
    double frob_rel;         /* ||got - ref||_F / ||ref||_F (0 if both are zero) */
    int64_t n_nonfinite;     /* elements of got that are Inf or NaN */
} orc_gemm_report;

/* Elementwise and Frobenius comparison of two bf16 arrays (values decoded exactly to fp64). */
void orc_gemm_compare(const uint16_t* ref, const uint16_t* got, int64_t n, double tol,
                      orc_gemm_report* rep);

/* Number of threads the oracle's parallel loops use for a given request (for reporting). */
int orc_threads(int nthreads);

#ifdef __cplusplus
}
#endif

#endif /* C3_ORACLE_H */
