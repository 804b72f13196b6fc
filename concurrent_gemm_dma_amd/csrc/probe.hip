// probe.hip -- the matrix cores' sustained bf16 rate on this device with nothing but MFMAs in
// flight: no loads, no LDS, no stores until the end. It bounds what any bf16 GEMM kernel can
// reach here, because under sustained MFMA load the chip runs at the clock its power limit
// allows, not at the nominal 2.4 GHz the vendor peak assumes.
//
// One workgroup per CU, 4 waves (one per SIMD, as the 256x256 tile kernel runs). Each wave keeps
// 16 independent 32x32 fp32 accumulators (256 accumulation registers, as the tile kernel) and
// issues `iters` rounds of 16 v_mfma_f32_32x32x16_bf16 on two operand sets used alternately, so
// that the multipliers' inputs change from one MFMA to the next as they do in a GEMM. The power an
// MFMA draws depends on how many operand bits toggle, so there are two kinds of operands:
//   random = 0: small integers (-2..2) from a fixed formula: few mantissa bits toggle, but every
//               product and partial sum is an exact integer, so the result has a closed form the
//               host checks (total of all accumulators of a wave = iters * 8 * (S0 + S1), S_s =
//               sum over k of (sum over rows of X_s[.][k]) * (sum over columns of Y_s[k][.]));
//   random = 1: bf16 values with random sign, exponent in [-2, 1] and mantissa bits from a hash,
//               as the bits of a GEMM's data toggle; the same closed form then holds up to fp32
//               rounding.
#include "c3_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Operand values: X_s[i][k] and Y_s[k][j] for i, j in [0, 32), k in [0, 16), s in {0, 1}.
__device__ __forceinline__ float probe_bits(uint32_t seed) {
    const uint32_t h = seed * 2654435761u;
    const uint32_t bits = ((h >> 31) << 15) | ((125u + ((h >> 20) & 3u)) << 7) | (h & 0x7Fu);
    return __uint_as_float(bits << 16);
}
__device__ __forceinline__ float probe_x(int random, int s, int i, int k) {
    return random ? probe_bits((uint32_t)(i * 16 + k + s * 512 + 1))
                  : (float)(((i * 31 + k * 17 + s * 7 + 3) % 5) - 2);
}
__device__ __forceinline__ float probe_y(int random, int s, int k, int j) {
    return random ? probe_bits((uint32_t)(k * 32 + j + s * 512 + 1025))
                  : (float)(((k * 13 + j * 29 + s * 11 + 1) % 5) - 2);
}

__global__ __launch_bounds__(256, 1) void mfma_rate_probe(double* __restrict__ out, int iters,
                                                         int random) {
    const int lane = threadIdx.x & 63;
    // lane l holds row (or column) l % 32 and k in [8 * (l / 32), 8 * (l / 32) + 8)
    bf16x8_t x[2], y[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = 8 * (lane >> 5) + e;
            x[s][e] = static_cast<__bf16>(probe_x(random, s, lane & 31, k));
            y[s][e] = static_cast<__bf16>(probe_y(random, s, k, lane & 31));
        }
    f32x16_t acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = f32x16_t{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[j & 1], y[j & 1], acc[j], 0, 0, 0);
    }
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += (double)acc[j][r];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

}  // namespace

namespace c3 {

c3_status mfma_probe_enqueue(int n_workgroups, int iters, int random, double* out_dev,
                             hipStream_t stream) {
    hipLaunchKernelGGL(mfma_rate_probe, dim3(n_workgroups), dim3(256), 0, stream, out_dev, iters,
                       random);
    C3_HIP_TRY(hipGetLastError());
    return C3_OK;
}

}  // namespace c3
