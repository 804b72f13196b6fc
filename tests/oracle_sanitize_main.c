/* Drives every function of the C oracle on small and edge-case inputs. It is built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by test_oracle_sanitizers.py. A memory error or
 * undefined behaviour aborts the run with a report. The checks below only confirm that the calls
 * did something sensible; parity itself is pinned by the other oracle tests. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static int fails = 0;
#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++fails;                                               \
        }                                                          \
    } while (0)

static uint16_t* bf16_array(size_t n, unsigned seed) {
    uint16_t* a = malloc((n ? n : 1) * sizeof(uint16_t));
    srand(seed);
    for (size_t i = 0; i < n; ++i) {
        const float v = (float)(rand() % 9 - 4) * 0.25f;
        uint32_t b;
        memcpy(&b, &v, 4);
        a[i] = orc_bf16_from_f32_bits(b);
    }
    return a;
}

int main(void) {
    /* conversions, including the special values */
    const uint32_t specials[] = {0x00000000u, 0x80000000u, 0x7F800000u, 0xFF800000u, 0x7FC00000u,
                                 0x7F800001u, 0x00000001u, 0x807FFFFFu, 0x3F808000u, 0x3F818000u,
                                 0x7F7FFFFFu};
    uint16_t out16[16];
    orc_bf16_from_f32_bits_array(specials, out16, sizeof specials / sizeof specials[0]);
    CHECK(out16[2] == 0x7F80 && out16[3] == 0xFF80);
    const double d[] = {0.0, -0.0, 1.0 / 3.0, 1e300, -1e-300, NAN, INFINITY};
    orc_bf16_from_f64_array(d, out16, 7);
    CHECK(out16[4] == 0x8000 && (out16[5] & 0x7FFF) > 0x7F80);
    CHECK(orc_f32_bits_from_bf16(0x3F80) == 0x3F800000u);
    orc_bf16_from_f32_bits_array(specials, out16, 0);

    /* GEMM: ragged shape, row sub-ranges, both accumulations, selected elements */
    const int64_t M = 7, N = 9, K = 13;
    uint16_t *A = bf16_array(M * K, 1), *B = bf16_array(K * N, 2);
    uint16_t *C32 = malloc(M * N * 2), *C64 = malloc(M * N * 2);
    float* acc = malloc(M * N * sizeof(float));
    double* sum = malloc(M * N * sizeof(double));
    orc_gemm_f32acc_rows(A, B, M, N, K, 0, M, C32, acc, 0);
    orc_gemm_f64acc_rows(A, B, M, N, K, 0, M, C64, sum, 2);
    /* quarter-integer entries: every partial sum is exact, so both agree bit for bit */
    CHECK(memcmp(C32, C64, M * N * 2) == 0);
    orc_gemm_f32acc_rows(A, B, M, N, K, 3, 5, C32, NULL, 1);
    CHECK(memcmp(C32, C64 + 3 * N, 2 * N * 2) == 0);
    orc_gemm_f32acc_rows(A, B, M, N, K, 4, 4, C32, NULL, 1); /* empty range */
    const int64_t rows[] = {0, 6, 3}, cols[] = {0, 8, 4}, bad[] = {7, 0, 0};
    uint16_t c32[3], c64[3];
    double s64[3];
    CHECK(orc_gemm_elems(A, B, M, N, K, rows, cols, 3, c32, c64, s64, 0) == 0);
    CHECK(c32[1] == C64[6 * N + 8] && c64[2] == C64[3 * N + 4]);
    CHECK(orc_gemm_elems(A, B, M, N, K, bad, cols, 3, c32, NULL, NULL, 1) == -1);
    CHECK(orc_gemm_elems(A, B, M, N, K, rows, cols, 0, NULL, NULL, NULL, 1) == 0);

    /* copies: ragged sizes, empty and single-shard cases */
    uint8_t src[3 * 3 * 5], dst[3 * 3 * 5];
    for (int i = 0; i < (int)sizeof src; ++i) src[i] = (uint8_t)(i * 7 + 1);
    const void* shards[3] = {src, src + 15, src + 30};
    orc_gather(dst, shards, 3, 15);
    CHECK(memcmp(dst, src, 45) == 0);
    orc_gather(dst, shards, 0, 15);
    orc_gather(dst, shards, 3, 0);
    orc_all2all_block(dst, src, 3, 5);
    CHECK(memcmp(dst + (1 * 3 + 2) * 5, src + (2 * 3 + 1) * 5, 5) == 0);
    orc_all2all_block(dst, src, 1, 45);
    CHECK(memcmp(dst, src, 45) == 0);
    CHECK(orc_first_diff(dst, src, 45) == -1 && orc_first_diff(dst, src, 0) == -1);
    dst[44] ^= 1;
    CHECK(orc_first_diff(dst, src, 45) == 44);

    /* reduce-scatter and all-reduce: one rank, many ranks, NULL peer at this rank */
    enum { W = 64, E = 11 };
    uint16_t* contrib[W];
    for (int r = 0; r < W; ++r) contrib[r] = bf16_array(E, 100 + r);
    uint16_t red[E], red1[E], gathered[W * E];
    orc_reduce_sum_bf16((const uint16_t* const*)contrib, 1, E, red1);
    CHECK(memcmp(red1, contrib[0], E * 2) == 0);
    orc_reduce_sum_bf16((const uint16_t* const*)contrib, W, E, red);
    orc_reduce_sum_bf16((const uint16_t* const*)contrib, W, 0, red);
    const uint16_t* peers[W];
    for (int r = 0; r < W; ++r) peers[r] = r == 5 ? NULL : contrib[(r + 1) % W];
    orc_allreduce_local((const uint16_t* const*)contrib, peers, W, 5, E, red, gathered);
    CHECK(memcmp(gathered + 5 * E, red, E * 2) == 0 && memcmp(gathered, contrib[1], E * 2) == 0);

    /* checker, including non-finite values and an empty comparison */
    orc_gemm_report rep;
    orc_gemm_compare(C64, C64, M * N, 1e-2, &rep);
    CHECK(rep.n == M * N && rep.n_diff == 0 && rep.n_violations == 0);
    uint16_t got[4] = {0x3F80, 0x7FC0, 0x7F80, 0x0000}, ref[4] = {0x3F80, 0x3F80, 0x3F80, 0x0000};
    orc_gemm_compare(ref, got, 4, 1e-2, &rep);
    CHECK(rep.n_nonfinite == 2 && rep.n_violations == 2 && rep.first_violation == 1);
    orc_gemm_compare(ref, got, 0, 1e-2, &rep);
    CHECK(orc_threads(0) >= 1 && orc_threads(3) == 3);

    for (int r = 0; r < W; ++r) free(contrib[r]);
    free(A);
    free(B);
    free(C32);
    free(C64);
    free(acc);
    free(sum);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    puts("oracle sanitizer run: ok");
    return 0;
}
