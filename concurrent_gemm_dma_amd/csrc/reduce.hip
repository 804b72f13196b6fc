// reduce.hip -- the arithmetic half of an all-reduce on the compute units: the reduce-scatter's
// local share sums `world` bf16 contributions to this rank's chunk element by element. DMA
// engines cannot add, so an all-reduce is a reduce-scatter on CUs followed by an all-gather that
// the engines can move (L3 Synthesis page on 2412.14335, section 3, Attack 1; Pith review of
// "Optimizing ML Concurrent Computation and Communication with GPU DMA Engines", Reading
// between the lines).
//
// Arithmetic (fixed so results are reproducible bit for bit): fp32 accumulation starting from
// rank 0's value, ranks added in order, one round-to-nearest-even to bf16 at the end.
//
// Vector path: when every pointer is 16-byte aligned, each lane owns 8 consecutive elements
// (16 bytes per rank), issues the loads of up to 8 ranks before adding them, and a wavefront
// reads 1 KiB contiguous per rank per access. HBM-bound: (world + 1) * chunk bytes per call.
// Misaligned pointers and the last (n mod 8) elements take a per-element path.
#include "c3_internal.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBatch = 8;  // ranks whose loads are in flight together

struct InTable {
    uint64_t p[c3::kMaxWorld];
};

__device__ __forceinline__ float lo_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__device__ __forceinline__ void accumulate(float (&acc)[8], const u32x4_t v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc[2 * q] += lo_f32(v[q]);
        acc[2 * q + 1] += hi_f32(v[q]);
    }
}

// Round two fp32 to bf16 (nearest even, hardware conversion) and pack them, first in the low half.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t p = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, p);
}

// One piece per lane and streaming (non-temporal) loads and stores measured fastest on MI355X:
// 8 ranks x 32 MiB in 51.8 us = 5.83 TB/s of (world + 1) * chunk bytes; 2 or 4 pieces per lane
// were 4% and 35% slower (fewer, longer workgroups), ordinary loads and stores 11% slower.
constexpr int kPieces = 1;  // 16-byte pieces per lane

__device__ __forceinline__ u32x4_t load16(const u32x4_t* p) { return __builtin_nontemporal_load(p); }

// Workgroup b owns pieces [b * kPieces * kThreads, (b + 1) * kPieces * kThreads); lane t takes
// pieces t, t + kThreads, ... of that range (each access coalesced across the wavefront).
__global__ __launch_bounds__(kThreads) void reduce_sum_vec(const InTable t, int world,
                                                          u32x4_t* out, uint64_t n16) {
    const uint64_t first = (uint64_t)blockIdx.x * (kPieces * kThreads) + threadIdx.x;
    float acc[kPieces][8];
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
        const uint64_t i = first + (uint64_t)q * kThreads;
        if (i < n16) {
            const u32x4_t v = load16(reinterpret_cast<const u32x4_t*>(t.p[0]) + i);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                acc[q][2 * h] = lo_f32(v[h]);
                acc[q][2 * h + 1] = hi_f32(v[h]);
            }
        }
    }
    for (int r0 = 1; r0 < world; r0 += kBatch) {
        u32x4_t v[kBatch][kPieces];
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
#pragma unroll
            for (int q = 0; q < kPieces; ++q) {
                const uint64_t i = first + (uint64_t)q * kThreads;
                if (r0 + j < world && i < n16)
                    v[j][q] = load16(reinterpret_cast<const u32x4_t*>(t.p[r0 + j]) + i);
            }
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
#pragma unroll
            for (int q = 0; q < kPieces; ++q)
                if (r0 + j < world && first + (uint64_t)q * kThreads < n16) accumulate(acc[q], v[j][q]);
    }
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
        const uint64_t i = first + (uint64_t)q * kThreads;
        if (i < n16) {
            u32x4_t o;
#pragma unroll
            for (int h = 0; h < 4; ++h) o[h] = pack2(acc[q][2 * h], acc[q][2 * h + 1]);
            __builtin_nontemporal_store(o, out + i);
        }
    }
}

// Per-element path: elements [first, first + n) of every rank, grid-stride.
__global__ __launch_bounds__(kThreads) void reduce_sum_elem(const InTable t, int world,
                                                           uint16_t* out, uint64_t first,
                                                           uint64_t n) {
    for (uint64_t k = (uint64_t)blockIdx.x * kThreads + threadIdx.x; k < n;
         k += (uint64_t)gridDim.x * kThreads) {
        const uint64_t e = first + k;
        float acc = lo_f32(reinterpret_cast<const uint16_t*>(t.p[0])[e]);
        for (int r = 1; r < world; ++r) acc += lo_f32(reinterpret_cast<const uint16_t*>(t.p[r])[e]);
        out[e] = (uint16_t)(pack2(acc, 0.f) & 0xFFFFu);
    }
}

}  // namespace

namespace c3 {

c3_status reduce_enqueue(const ReduceArgs& a, hipStream_t stream) {
    if (a.elems == 0) return C3_OK;
    if (a.world < 1 || a.world > kMaxWorld) return fail(C3_E_INVALID, "reduce: bad world %d", a.world);
    InTable t{};
    uintptr_t align = (uintptr_t)a.out;
    for (int r = 0; r < a.world; ++r) {
        t.p[r] = (uint64_t)(uintptr_t)a.in[r];
        align |= (uintptr_t)a.in[r];
    }
    const uint64_t n16 = (align & 15) == 0 ? a.elems / 8 : 0;
    if (n16) {
        const uint64_t per_block = (uint64_t)kPieces * kThreads;
        const uint64_t blocks = (n16 + per_block - 1) / per_block;
        if (blocks > 0x7FFFFFFFull) return fail(C3_E_INVALID, "reduce: chunk too large for one launch");
        hipLaunchKernelGGL(reduce_sum_vec, dim3((unsigned)blocks), dim3(kThreads), 0, stream, t,
                           a.world, static_cast<u32x4_t*>(a.out), n16);
        C3_HIP_TRY(hipGetLastError());
    }
    const uint64_t done = n16 * 8;
    if (done < a.elems) {
        const uint64_t rest = a.elems - done;
        const unsigned blocks = (unsigned)std::min<uint64_t>(4096, (rest + kThreads - 1) / kThreads);
        hipLaunchKernelGGL(reduce_sum_elem, dim3(blocks), dim3(kThreads), 0, stream, t, a.world,
                           static_cast<uint16_t*>(a.out), done, rest);
        C3_HIP_TRY(hipGetLastError());
    }
    return C3_OK;
}

}  // namespace c3
