// gemm.hip -- bf16 GEMM C[M][N] = A[M][K] . B[K][N] for gfx950 (CDNA4), fp32 accumulation,
// round-to-nearest-even bf16 result. Row-major operands, no alpha/beta.
//
// The paper's computation is the GEMM of LLaMA-class training layers ("Optimizing ML Concurrent
// Computation and Communication with GPU DMA Engines", Section IV, Fig. 5a). Two kernels:
//
// * tile256_dma: 256x256 output tile per workgroup, 4 waves (2x2), each wave 128x128 built from
//   4x4 v_mfma_f32_32x32x16_bf16. Operands go global -> LDS directly (LDS-direct buffer loads),
//   K step 32: A in slabs of 64 k (full 128-byte lines), three in LDS, B in four 32-k stages.
//   The MFMA is fed transposed (B^T as the row operand, A^T as the
//   column operand), so each lane's accumulators are 4 consecutive columns of one C row; the
//   epilogue regroups them through LDS into 16-byte runs along C's rows. B stays K x N in LDS and is read with the LDS transpose load
//   (ds_read_b64_tr_b16), which hands each lane 4 consecutive k of one column. With fewer tiles
//   than CUs, K can also be split over a second grid dimension (fp32 partials, summed in split
//   order by splitk_reduce). Shapes with M > 64 use this kernel unless the 128 kernel wins.
// * tile128_dma: the same at 128x128 (4 waves of 64x64), two workgroups per CU, for mid-size
//   shapes where a 256x256 grid leaves most CUs idle and K is too short for a split to pay.
// * skinny: all M (<= 64) rows x 256 columns per workgroup, K split across workgroups
//   (deterministic: fp32 partials per split, summed in split order by a second kernel),
//   v_mfma_f32_16x16x32_bf16. For M <= 64, where the GEMM streams B once and is bound by HBM
//   bandwidth.
//
// Global loads and C stores use raw buffer instructions whose resource covers only the valid
// part of the operand: anything past it reads as zero / is dropped, and ragged M, N, K edges are
// masked explicitly by pointing the lane at an out-of-range offset.
#include "c3_internal.h"

#include <algorithm>
#include <cstdlib>
#include <map>
#include <type_traits>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define C3_LDS __attribute__((address_space(3)))

// Raw buffer resource word 3 for gfx9-family parts (32-bit data format, no swizzle, no stride).
constexpr int kRsrcWord3 = 0x00020000;
// Any offset >= the resource's record count reads zero / drops the store.
constexpr uint32_t kOOB = 0x80000000u;
constexpr uint64_t kMaxRecords = 0x7FFFFFF0ull;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    uint64_t n = bytes <= 0 ? 0ull : (uint64_t)bytes;
    if (n > kMaxRecords) n = kMaxRecords;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// The same with the non-temporal cache policy (the instruction's nt bit, cache-policy operand 2
// on gfx950), for data read exactly once: measured on a 448 MiB stream of 512-byte row pieces,
// 6.75 TB/s against 6.17 TB/s with the default policy.
__device__ __forceinline__ u32x4_t load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}

__device__ __forceinline__ void store8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2_t v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

__device__ __forceinline__ void lds_store16(char* lds, uint32_t off, u32x4_t v) {
    *reinterpret_cast<C3_LDS u32x4_t*>((C3_LDS char*)lds + off) = v;
}

__device__ __forceinline__ bf16x8_t lds_load16(const char* lds, uint32_t off) {
    return *reinterpret_cast<const C3_LDS bf16x8_t*>((const C3_LDS char*)lds + off);
}

// Two LDS transpose loads (4 k each) form one 8-k MFMA row operand.
__device__ __forceinline__ bf16x8_t lds_load_tr8(const char* lds, uint32_t off_lo,
                                                 uint32_t off_hi) {
    i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<C3_LDS i16x4_t*>((C3_LDS char*)lds + off_lo));
    i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<C3_LDS i16x4_t*>((C3_LDS char*)lds + off_hi));
    i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
}

// Round 4 fp32 to bf16 (nearest even; v_cvt_pk_bf16_f32) and pack.
__device__ __forceinline__ u32x2_t pack_bf16x4(float a, float b, float c, float d) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t p0 = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    bf16x2_t p1 = {static_cast<__bf16>(c), static_cast<__bf16>(d)};
    u32x2_t r;
    r.x = __builtin_bit_cast(uint32_t, p0);
    r.y = __builtin_bit_cast(uint32_t, p1);
    return r;
}

// LDS swizzles (16-byte chunk index XOR), chosen so the MFMA operand reads below touch distinct
// banks both when the LDS serves 16 lanes x 8 B (32 banks) and 32 lanes x 8 B (64 banks) per
// cycle.
// A tiles: rows of 64 k (128 B = 8 chunks); chunk ^= (row & 7) ^ bit 3 of row.
__device__ __forceinline__ int swz_a(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// B tiles: rows of 256 n (512 B = 32 chunks); chunk ^= f(row & 3), f = {0, 6, 10, 12}.
__device__ __forceinline__ int swz_b(int krow) {
    const int r = krow & 3;
    return (r << 2) ^ (((r ^ (r >> 1)) & 1) << 1);
}

// Workgroup -> output tile. The dispatcher deals workgroups to the XCDs in turn: workgroup b runs
// on XCD (b + s) mod 8, where the start s moves on from one dispatch to the next (measured, on
// plain and CU-masked queues alike), so the workgroups of one residue b mod 8 share an XCD.
// Renumber so that each residue gets a contiguous range of logical tiles, then walk tiles in
// groups of GROUP_M tile rows so that the tiles resident at one time on an XCD share A rows and B
// columns in its L2.
template <int GROUP_M>
__device__ __forceinline__ void map_tile(int bid, int nblocks, int tiles_m, int tiles_n, int& tm,
                                         int& tn) {
    int logical = bid;
    if (nblocks >= 8) {
        const int q = nblocks >> 3, rem = nblocks & 7;
        const int x = bid & 7, local = bid >> 3;
        logical = x * q + (x < rem ? x : rem) + local;
    }
    const int per_group = GROUP_M * tiles_n;
    const int group = logical / per_group;
    const int first_m = group * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int in_group = logical - group * per_group;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

// ------------------------------------------------------------------------------------------------
// 256 x 256 tile kernel, LDS-direct loads
// ------------------------------------------------------------------------------------------------
// 4 waves (2x2), each 128x128 = 4x4 v_mfma_f32_32x32x16_bf16. Operands go global -> LDS directly
// (buffer_load_dwordx4 ... lds: each wave-instruction fills 1 KiB of LDS, lane t's 16 bytes at
// byte 16*t), so no registers stage them. K step 32. A is loaded in slabs of 64 k (each row's
// 128 bytes whole, so every L1 -> L2 request is a full line: a third fewer requests than 64-byte
// half rows, and less power under the chip's power limit), three slabs in LDS (96 KiB), each
// serving two steps; B in four stages of 32 k (64 KiB). Each step issues B of step k+3 and one
// half (128 rows) of the slab four to five steps ahead. Per step: read the second half of this
// step's fragments, run the first half's MFMAs, wait for step k+1 and barrier, issue the A half,
// read the first half of step k+1's fragments, run the second half's MFMAs.
namespace td {
constexpr int BM = 256, BN = 256, BK = 32, NT = 256, NSTAGE = 4;  // NSTAGE: B stages
constexpr int B_STAGE = BK * BN * 2;  // 16 KiB: 32 rows of 512 B
constexpr int GROUP_M = 4;            // tile rows walked together on one XCD (map_tile)
constexpr int LOADS_PER_STAGE = 8;    // per wave and step: 4 A (half slab) + 4 B wave-instructions
}  // namespace td

// A rows of 64 B (4 chunks): chunk ^= 2*(r2^r3) + (r1^r2) (r_i = bit i of the row). Distinct
// within every 8 consecutive rows of one parity and within every 4 rows 4 apart, so 8 or 16
// lanes reading 16 B from consecutive rows hit distinct banks.
__device__ __forceinline__ int swz_a32(int row) {
    const int b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b3 = (row >> 3) & 1;
    return ((b2 ^ b3) << 1) | (b1 ^ b2);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define C3_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// Raw buffer resource as four dwords (gfx9 layout: base, base_hi | stride << 16, records, word 3).
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc_words(const void* base, int64_t bytes) {
    uint64_t n = bytes <= 0 ? 0ull : (uint64_t)bytes;
    if (n > kMaxRecords) n = kMaxRecords;
    const uint64_t a = (uint64_t)(uintptr_t)base;
    i32x4_t w;
    w.x = (int)(uint32_t)a;
    w.y = (int)((uint32_t)(a >> 32) & 0xFFFFu);
    w.z = (int)(uint32_t)n;
    w.w = kRsrcWord3;
    return w;
}

// One LDS-direct 16-byte load per lane: lane t's 16 bytes from `voff` land at LDS byte address
// lds_addr + 16*t (lds_addr wave-uniform). Issued through inline asm so that the compiler's wait
// insertion, which cannot tell these writes from the transpose reads of other LDS stages and
// would wait for every outstanding load before each read, leaves them alone; the kernel waits
// on the vector-memory counter itself (C3_WAIT_VMCNT) before it reads a stage. M0 carries the
// LDS address; nothing else in these kernels uses M0.
__device__ __forceinline__ void lds_dma16_at(i32x4_t r, uint32_t lds_addr, uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(lds_addr), "v"(voff), "s"(r)
        : "memory", "m0");
}

template <uint32_t OFF>
__device__ __forceinline__ void lds_dma16_so(i32x4_t r, uint32_t lds_base, uint32_t voff,
                                             uint32_t soff) {
    asm volatile(
        "s_add_u32 m0, %0, %4\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(lds_base), "v"(voff), "s"(r), "s"(soff), "n"(OFF)
        : "memory", "m0", "scc");
}

__device__ __forceinline__ void lds_dma16(i32x4_t r, char* lds, uint32_t voff) {
    lds_dma16_at(r, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(C3_LDS char*)lds), voff);
}

// SPLIT = false: the whole K, bf16 C. SPLIT = true: K split y = blockIdx.y, fp32 partials to
// ws[y][M][N] for splitk_reduce (a template parameter so that the two epilogues never share the
// register budget of one kernel).
template <bool SPLIT>
__global__ __launch_bounds__(256, 1) void gemm_bf16_tile256_dma(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    float* __restrict__ ws, int M, int N, int K, int k_per_split, int tiles_m, int tiles_n) {
    using namespace td;
    // A in slabs of 64 k ([256 rows][128 B], three buffers); B in 32-k stages (four buffers)
    constexpr int A_SLAB = BM * 64 * 2;                     // 32 KiB
    constexpr int B_REGION = 3 * A_SLAB;                    // 96 KiB
    __shared__ __attribute__((aligned(1024))) char smem[B_REGION + NSTAGE * B_STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int tm, tn;
    map_tile<GROUP_M>(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    // K split y = blockIdx.y covers k in [kbeg, kbeg + Ke); A keeps its row stride K.
    const int kbeg = SPLIT ? blockIdx.y * k_per_split : 0;
    const int Ke = SPLIT ? min(K, kbeg + k_per_split) - kbeg : K;
    if (SPLIT) {
        A += kbeg;
        B += (size_t)kbeg * N;
    }

    // ---- global -> LDS addressing. Wave w fills, per A half slab, blocks 4w+i (8 rows each)
    // and, per B stage, blocks 4w+j (2 k rows each); lane t lands at byte 16*t of the 1 KiB
    // block.
    const i32x4_t rA =
        make_rsrc_words(A + (size_t)m0 * K, (int64_t)(M - m0) * K * 2 - (int64_t)kbeg * 2);
    // half h of slab j: wave w, instruction i covers rows 128h + 32w + 8i + lane/8, 128 B each;
    // lane t lands at chunk position t%8 and loads global chunk (t%8) ^ swz_a(row)
    int a_c[4];
    uint32_t a_g[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 32 * wave + 8 * i + (lane >> 3);
        a_c[i] = (lane & 7) ^ swz_a(row);
        a_g[i] = (uint32_t)row * (uint32_t)K * 2u + (uint32_t)a_c[i] * 16u;
    }
    const uint32_t a_hstep = 128u * (uint32_t)K * 2u;
    uint32_t b_g[4];
    bool b_ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int krow = 2 * (wave * 4 + j) + (lane >> 5);
        const int nc = (lane & 31) ^ swz_b(krow);
        b_g[j] = (uint32_t)krow * (uint32_t)N * 2u + (uint32_t)nc * 16u;
        b_ok[j] = (n0 + nc * 8) < N;
    }
    auto issue_B = [&](int k0, int st) {
        const i32x4_t rB =
            make_rsrc_words(B + (size_t)k0 * N + n0, ((int64_t)(Ke - k0) * N - n0) * 2);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            lds_dma16(rB, smem + B_REGION + st * B_STAGE + (wave * 4 + j) * 1024, b_ok[j] ? b_g[j] : kOOB);
    };
    auto issue_A_half = [&](int slab, int h) {
        const int k0 = 64 * slab;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = (k0 + a_c[i] * 8) < Ke;
            lds_dma16(rA, smem + (slab % 3) * A_SLAB + (16 * h + 4 * wave + i) * 1024,
                      ok ? a_g[i] + (uint32_t)h * a_hstep + (uint32_t)k0 * 2u : kOOB);
        }
    };

    // ---- LDS -> MFMA operand addressing ----
    const int ar = lane & 31;
    uint32_t a_rd[2];  // even step; an odd step reads chunk + 4, i.e. byte offset ^ 64
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
        a_rd[kk] = (uint32_t)(wm * 128 + ar) * 128u +
                   (uint32_t)((((kk * 2) + (lane >> 5)) ^ swz_a(ar)) << 4);
    const int G = lane >> 4, p = lane & 15;
    const int b_sw = swz_b(p >> 2);
    uint32_t b_rd[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        const int nc = wn * 16 + ni * 4 + 2 * (G & 1) + ((p >> 1) & 1);
        b_rd[ni] = (uint32_t)(8 * (G >> 1) + (p >> 2)) * 512u + (uint32_t)((nc ^ b_sw) << 4) +
                   (uint32_t)((p & 1) * 8);
    }

    f32x16_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x16_t{};

    const int nk = (Ke + BK - 1) / BK;
    // Prologue, in the order the steady state issues (step kt issues B of step kt+3, then half
    // 1 - kt%2 of slab (kt+5)/2): slab 0, B0, slab 1 first half, B1, slab 1 second half, B2,
    // slab 2 first half. Loads past the end read zeros into buffers nothing reads.
    issue_A_half(0, 0);
    issue_A_half(0, 1);
    issue_B(0, 0);
    issue_A_half(1, 0);
    issue_B(BK, 1);
    issue_A_half(1, 1);
    issue_B(2 * BK, 2);
    issue_A_half(2, 0);
    C3_WAIT_VMCNT(5 * 4);  // slab 0 and B0 landed
    __syncthreads();

    // With one wave per SIMD the MFMA pipe idles whenever the wave issues anything else between
    // two MFMAs, so every other instruction is slotted one-for-one behind an MFMA (scheduling
    // fences after each slot keep this order): while an MFMA occupies the pipe for its 32
    // cycles the wave issues the next LDS read or LDS-direct load, and the next MFMA is ready
    // the moment the pipe frees.
    bf16x8_t cf[2][4];
    i16x4_t rlo[2][4], rhi[2][4];
    // kt: the step whose fragments are read (A slab kt/2, parity kt%2; B stage kt%4)
    auto read_item = [&](int kt, int kk, int set, int j) {
        const char* As = smem + ((kt >> 1) % 3) * A_SLAB;
        const char* Bs = smem + B_REGION + (kt & (NSTAGE - 1)) * B_STAGE;
        if (j < 4) {
            cf[set][j] = lds_load16(As, (a_rd[kk] ^ ((uint32_t)(kt & 1) << 6)) + j * 4096u);
        } else {
            const int ni = (j - 4) >> 1;
            const uint32_t off = b_rd[ni] + kk * 8192u + ((j - 4) & 1) * 2048u;
            const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                reinterpret_cast<C3_LDS i16x4_t*>((C3_LDS char*)Bs + off));
            if ((j - 4) & 1) rhi[set][ni] = v;
            else rlo[set][ni] = v;
        }
    };
    // The 16 MFMAs of a k-slice walk the 4x4 blocks row by row, odd rows backwards, so that from
    // one MFMA to the next only one operand changes (the row operand at a row's end stays).
    auto mfma_item = [&](int set, int i) {
        const int mi = i >> 2, ni = (mi & 1) ? 3 - (i & 3) : (i & 3);
        const i16x8_t rv = __builtin_shufflevector(rlo[set][ni], rhi[set][ni], 0, 1, 2, 3, 4, 5, 6, 7);
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, rv),
                                                              cf[set][mi], acc[mi][ni], 0, 0, 0);
    };
    // Wave-uniform LDS byte addresses of this wave's LDS-direct destinations in stage 0.
    const uint32_t lds_base = (uint32_t)(uintptr_t)(C3_LDS char*)smem;
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane((uint32_t)wave);
    const uint32_t b_dst0 = lds_base + (uint32_t)B_REGION + wave_u * 4096u;

    // One K step, with compile-time flags (each loop body stays straight-line: branches around
    // the MFMA sequence cost the accumulators their registers):
    //   BA - first half issues the B half of step kt+3 into buffer (kt+3)%4 (split refill; that
    //        buffer's last reader, step kt-1, finished before the previous step's barrier),
    //   RA - second half issues half 1 - kt%2 of slab (kt+5)/2 (rows 128h..128h+127),
    //   NX - second half reads step kt+1's first fragments.
    auto step = [&](int kt, auto ba_c, auto ra_c, auto nx_c) {
        constexpr bool BA = decltype(ba_c)::value;
        constexpr bool RA = decltype(ra_c)::value;
        constexpr bool NX = decltype(nx_c)::value;
        const int s3 = (kt + NSTAGE - 1) & (NSTAGE - 1);
        const int k3 = (kt + NSTAGE - 1) * BK;
        i32x4_t rB3{};
        if (BA) rB3 = make_rsrc_words(B + (size_t)k3 * N + n0, ((int64_t)(Ke - k3) * N - n0) * 2);
        const uint32_t b_dst3 = b_dst0 + (uint32_t)s3 * B_STAGE;
        // first half: MFMAs of k-slice 0 (set 0) with the reads of k-slice 1 (set 1)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mfma_item(0, i);
            if (i < 12) read_item(kt, 1, 1, i);
            if (BA && i >= 4 && i < 8)
                lds_dma16_at(rB3, b_dst3 + (i - 4) * 1024u, b_ok[i - 4] ? b_g[i - 4] : kOOB);
            __builtin_amdgcn_sched_barrier(0);
        }
        // step kt+1 landed for this wave (steps kt+2, kt+3 may still be in flight); this
        // wave's reads of step kt are done; then every wave is past both points
        if (RA || kt + 3 < nk) C3_WAIT_VMCNT(2 * LOADS_PER_STAGE);
        else if (kt + 2 < nk) C3_WAIT_VMCNT(1 * LOADS_PER_STAGE);
        else C3_WAIT_VMCNT(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // second half: MFMAs of k-slice 1 (set 1) with the reads of step kt+1's k-slice 0
        // (set 0) and the refill of this step's buffer for step kt+4
        // refill: half 1 - kt%2 of slab (kt+5)/2 (its buffer's slab, (kt+5)/2 - 3, was last
        // read by steps kt-1 and kt, both finished at the barrier above)
        const int slab = (kt + 5) >> 1, h = 1 - (kt & 1);
        const int ka = 64 * slab;
        const uint32_t a_dst = lds_base + (uint32_t)((slab % 3) * A_SLAB) +
                               (uint32_t)((16 * h + 4 * (int)wave_u) * 1024);
        const uint32_t a_off = (uint32_t)h * a_hstep + (uint32_t)ka * 2u;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mfma_item(1, i);
            if (NX && i < 12) read_item(kt + 1, 0, 0, i);
            if (RA && i < 4)
                lds_dma16_at(rA, a_dst + i * 1024u,
                             (ka + a_c[i] * 8) < Ke ? a_g[i] + a_off : kOOB);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Fast steps (while every load they issue lies wholly inside K): twelve steps per iteration (the
    // period of the four B stages and the three A slabs of two steps), so every LDS address is a
    // constant; B's resource keeps the maximum record count and only its base moves; A's loads
    // keep their lane offsets (one set per half of the rows, so that rows past M stay out of
    // range in the lane offset itself) and take the slab's k offset in the scalar offset (fa0:
    // the group's k offset, advanced by six slabs per group).
    // With one wave per SIMD a wave issues at most one instruction every four cycles, so a
    // 32-cycle MFMA covers seven others; the few scalar updates left sit in slots that issue
    // nothing else, which keeps every slot at five non-MFMA instructions or fewer.
    uint32_t fb_lo = 0, fb_hi = 0, fa0 = 0;
    const uint64_t fb_step = (uint64_t)BK * (uint64_t)N * 2u;
    const uint32_t fbs_lo = (uint32_t)fb_step, fbs_hi = (uint32_t)(fb_step >> 32);
    const uint32_t wave_lds = lds_base + wave_u * 4096u;
    uint32_t b_vo[4], a_vo1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        b_vo[j] = b_ok[j] ? b_g[j] : kOOB;
        a_vo1[j] = a_g[j] + a_hstep;
    }
    auto step_fast = [&](auto r_c) {
        constexpr int R = decltype(r_c)::value;            // kt mod 12
        constexpr int S3 = (R + NSTAGE - 1) & (NSTAGE - 1);
        constexpr uint32_t B_DST3 = (uint32_t)(B_REGION + S3 * B_STAGE);
        constexpr int SLAB = (R + 5) >> 1, H = 1 - (R & 1);
        constexpr uint32_t A_DST = (uint32_t)((SLAB % 3) * A_SLAB + 16 * H * 1024);
        constexpr uint32_t A_K = (uint32_t)(128 * SLAB);     // slab's k offset within the group, bytes
        i32x4_t rBf;
        rBf.x = (int)fb_lo;
        rBf.y = (int)fb_hi;
        rBf.z = (int)kMaxRecords;
        rBf.w = kRsrcWord3;
        uint32_t a_so = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mfma_item(0, i);
            if (i < 12) read_item(R, 1, 1, i);
            if (i == 4) lds_dma16_so<B_DST3 + 0u>(rBf, wave_lds, b_vo[0], 0u);
            if (i == 5) lds_dma16_so<B_DST3 + 1024u>(rBf, wave_lds, b_vo[1], 0u);
            if (i == 6) lds_dma16_so<B_DST3 + 2048u>(rBf, wave_lds, b_vo[2], 0u);
            if (i == 7) lds_dma16_so<B_DST3 + 3072u>(rBf, wave_lds, b_vo[3], 0u);
            if (i == 12)
                asm volatile("s_add_u32 %0, %1, %2" : "=s"(a_so) : "s"(fa0), "n"(A_K) : "scc");
            if (i == 13)
                asm volatile("s_add_u32 %0, %0, %2\n\ts_addc_u32 %1, %1, %3"
                             : "+s"(fb_lo), "+s"(fb_hi)
                             : "s"(fbs_lo), "s"(fbs_hi)
                             : "scc");
            if (R == 11 && i == 14)
                asm volatile("s_add_u32 %0, %0, %1" : "+s"(fa0) : "n"(128 * 6) : "scc");
            __builtin_amdgcn_sched_barrier(0);
        }
        C3_WAIT_VMCNT(2 * LOADS_PER_STAGE);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mfma_item(1, i);
            if (i < 12) read_item(R + 1, 0, 0, i);
            if (i == 0) lds_dma16_so<A_DST + 0u>(rA, wave_lds, H ? a_vo1[0] : a_g[0], a_so);
            if (i == 1) lds_dma16_so<A_DST + 1024u>(rA, wave_lds, H ? a_vo1[1] : a_g[1], a_so);
            if (i == 2) lds_dma16_so<A_DST + 2048u>(rA, wave_lds, H ? a_vo1[2] : a_g[2], a_so);
            if (i == 3) lds_dma16_so<A_DST + 3072u>(rA, wave_lds, H ? a_vo1[3] : a_g[3], a_so);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    using T = std::true_type;
    using F = std::false_type;

#pragma unroll
    for (int j = 0; j < 12; ++j) read_item(0, 0, 0, j);
    int kt = 0;
    const int nkf = Ke / BK;
    {
        const uint64_t b0 = (uint64_t)(uintptr_t)(B + (size_t)(NSTAGE - 1) * BK * N + n0);
        fb_lo = (uint32_t)b0;
        fb_hi = (uint32_t)(b0 >> 32);
        fa0 = 0u;
    }
    for (; kt + 18 <= nkf; kt += 12) {
        step_fast(std::integral_constant<int, 0>{});
        step_fast(std::integral_constant<int, 1>{});
        step_fast(std::integral_constant<int, 2>{});
        step_fast(std::integral_constant<int, 3>{});
        step_fast(std::integral_constant<int, 4>{});
        step_fast(std::integral_constant<int, 5>{});
        step_fast(std::integral_constant<int, 6>{});
        step_fast(std::integral_constant<int, 7>{});
        step_fast(std::integral_constant<int, 8>{});
        step_fast(std::integral_constant<int, 9>{});
        step_fast(std::integral_constant<int, 10>{});
        step_fast(std::integral_constant<int, 11>{});
    }
    // Past the last whole group (kt % 12 == 0 here), fast steps go on, in the group's phase, for
    // as long as the loads a step issues lie wholly inside K: B of step kt+3 and the slab
    // (kt+5)/2. The test only turns false as kt grows and kt moves only when a step runs, so
    // once one test fails every later one fails too.
    auto fast_ok = [&](int k) { return k + NSTAGE <= nkf && 64 * ((k + 5) >> 1) + 64 <= Ke; };
    if (fast_ok(kt)) { step_fast(std::integral_constant<int, 0>{}); ++kt; }
    if (fast_ok(kt)) { step_fast(std::integral_constant<int, 1>{}); ++kt; }
    if (fast_ok(kt)) { step_fast(std::integral_constant<int, 2>{}); ++kt; }
    if (fast_ok(kt)) { step_fast(std::integral_constant<int, 3>{}); ++kt; }
    if (fast_ok(kt)) { step_fast(std::integral_constant<int, 4>{}); ++kt; }
    if (fast_ok(kt)) { step_fast(std::integral_constant<int, 5>{}); ++kt; }
    if (fast_ok(kt)) { step_fast(std::integral_constant<int, 6>{}); ++kt; }
    if (fast_ok(kt)) { step_fast(std::integral_constant<int, 7>{}); ++kt; }
    if (fast_ok(kt)) { step_fast(std::integral_constant<int, 8>{}); ++kt; }
    if (fast_ok(kt)) { step_fast(std::integral_constant<int, 9>{}); ++kt; }
    if (fast_ok(kt)) { step_fast(std::integral_constant<int, 10>{}); ++kt; }
    if (fast_ok(kt)) { step_fast(std::integral_constant<int, 11>{}); ++kt; }
    for (; kt + NSTAGE < nk; ++kt) step(kt, T{}, T{}, T{});
    if (kt + NSTAGE - 1 < nk) {
        step(kt, T{}, F{}, T{});
        ++kt;
    }
    for (; kt + 1 < nk; ++kt) step(kt, F{}, F{}, T{});
    if (kt < nk) step(kt, F{}, F{}, F{});

    // ---- epilogue: lane holds C[m][n..n+3], m = mi*32 + lane%32, n = ni*32 + 8g + 4*(lane/32);
    // one K split writes bf16 C, several write fp32 partials ws[y][m][n] for splitk_reduce
    if (!SPLIT) {
        // Stored straight from the accumulator layout, each store instruction would write 16
        // bytes into each of 32 rows, and the 64 such stores per wave hold the CU's vector memory
        // path for about 15 000 cycles per tile. So each wave stages its 128 x 128 bf16 sub-tile in
        // LDS (free once every wave has read its last fragments; 32 KiB per wave, rows of 256 B)
        // and stores it back as 16 bytes per lane along the rows: four 256-byte row pieces per
        // instruction, 32 instructions per wave. Layout: 16-byte chunk ^= (row >> 1) & 15, and
        // the two 8-byte halves of a chunk swapped in odd rows. The LDS serves 512 bytes per
        // cycle (128 banks of 4 bytes) when it can: a wave's 8-byte writes (32 rows, two halves
        // each) then fill 64 distinct 8-byte slots of two rows' 512 bytes, and its 16-byte reads
        // (four rows of 16 chunks) cover each pair of rows once; with 256 bytes (64 banks) per
        // cycle the 32 lanes of one half-row write and the 16 lanes of one row read still touch
        // every bank once. Reads of odd rows swap the halves back.
        // N is a multiple of 8, so a 16-byte chunk lies wholly inside or wholly outside N.
        __syncthreads();
        C3_LDS char* stg = (C3_LDS char*)smem + wave * (BM / 2) * (BN / 2) * 2;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int r = mi * 32 + (lane & 31);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int chunk = ni * 4 + g;
                    const uint32_t off = (uint32_t)r * 256u +
                                         (uint32_t)((chunk ^ ((r >> 1) & 15)) << 4) +
                                         8u * (uint32_t)((lane >> 5) ^ (r & 1));
                    const f32x16_t& a = acc[mi][ni];
                    *reinterpret_cast<C3_LDS u32x2_t*>(stg + off) =
                        pack_bf16x4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
                }
        }
        const __amdgpu_buffer_rsrc_t rC =
            make_rsrc(C + (size_t)m0 * N + n0, ((int64_t)(M - m0) * N - n0) * 2);
        const int chunk = lane & 15;
        const int nl = wn * 128 + chunk * 8;
        const bool nvalid = (n0 + nl) < N;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int r = i * 4 + (lane >> 4);
            u32x4_t v = *reinterpret_cast<const C3_LDS u32x4_t*>(
                stg + (uint32_t)r * 256u + (uint32_t)((chunk ^ ((r >> 1) & 15)) << 4));
            if (r & 1) v = __builtin_shufflevector(v, v, 2, 3, 0, 1);
            const int ml = wm * 128 + r;
            const bool ok = nvalid && (m0 + ml) < M;
            store16(rC, ok ? ((uint32_t)ml * (uint32_t)N + (uint32_t)nl) * 2u : kOOB, v);
        }
    } else {
        float* wsb = ws + ((size_t)blockIdx.y * M + m0) * N + n0;
        const __amdgpu_buffer_rsrc_t rW = make_rsrc(wsb, ((int64_t)(M - m0) * N - n0) * 4);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int ml = wm * 128 + mi * 32 + (lane & 31);
            const bool mvalid = (m0 + ml) < M;
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int nl = wn * 128 + ni * 32 + 8 * g + 4 * (lane >> 5);
                    const bool ok = mvalid && (n0 + nl) < N;
                    const uint32_t off =
                        ok ? ((uint32_t)ml * (uint32_t)N + (uint32_t)nl) * 4u : kOOB;
                    const f32x16_t& a = acc[mi][ni];
                    const f32x4_t v = {a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
                    store16(rW, off, __builtin_bit_cast(u32x4_t, v));
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// 128 x 128 tile kernel, LDS-direct loads, two workgroups per CU
// ------------------------------------------------------------------------------------------------
// For shapes with fewer 256x256 tiles than CUs. 4 waves (2x2), each 64x64 = 2x2
// v_mfma_f32_32x32x16_bf16 (64 accumulators per lane), K step 32, four LDS stages of 16 KiB
// (A [128][32], B [32][128]); two workgroups share a CU, so one's LDS reads and barriers hide
// behind the other's MFMAs instead of a hand-interleaved schedule.
namespace tq {
constexpr int BM = 128, BN = 128, BK = 32, NT = 256, NSTAGE = 4;
constexpr int A_STAGE = BM * BK * 2;  // 8 KiB: 128 rows of 64 B
constexpr int B_STAGE = BK * BN * 2;  // 8 KiB: 32 rows of 256 B
constexpr int STAGE = A_STAGE + B_STAGE;
constexpr int GROUP_M = 4;
}  // namespace tq

__global__ __launch_bounds__(256, 2) void gemm_bf16_tile128_dma(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    int M, int N, int K, int tiles_m, int tiles_n) {
    using namespace tq;
    __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int tm, tn;
    map_tile<GROUP_M>(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // ---- global -> LDS: wave w fills A blocks 2w, 2w+1 (16 rows of 64 B each) and B blocks
    // 2w, 2w+1 (4 k rows of 256 B each); lane t lands at byte 16*t of the 1 KiB block.
    const i32x4_t rA = make_rsrc_words(A + (size_t)m0 * K, (int64_t)(M - m0) * K * 2);
    const int a_row0 = 16 * (wave * 2) + (lane >> 2);           // + 16*j
    const int a_kc = (lane & 3) ^ swz_a32(a_row0);               // same for j = 0, 1
    const uint32_t a_g0 = (uint32_t)a_row0 * (uint32_t)K * 2u + (uint32_t)a_kc * 16u;
    const uint32_t a_gstep = 16u * (uint32_t)K * 2u;
    uint32_t b_g[2];
    bool b_ok[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int krow = 4 * (wave * 2 + j) + (lane >> 4);
        const int nc = (lane & 15) ^ swz_b(krow);
        b_g[j] = (uint32_t)krow * (uint32_t)N * 2u + (uint32_t)nc * 16u;
        b_ok[j] = (n0 + nc * 8) < N;
    }
    auto issue_stage = [&](int k0, int s) {
        char* As = smem + s * STAGE;
        char* Bs = As + A_STAGE;
        const bool a_ok = (k0 + a_kc * 8) < K;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            lds_dma16(rA, As + (wave * 2 + j) * 1024,
                      a_ok ? a_g0 + (uint32_t)j * a_gstep + (uint32_t)k0 * 2u : kOOB);
        const i32x4_t rB =
            make_rsrc_words(B + (size_t)k0 * N + n0, ((int64_t)(K - k0) * N - n0) * 2);
#pragma unroll
        for (int j = 0; j < 2; ++j) lds_dma16(rB, Bs + (wave * 2 + j) * 1024, b_ok[j] ? b_g[j] : kOOB);
    };

    // ---- LDS -> MFMA operands (as in the 256 kernel, with 64-row / 64-column wave tiles) ----
    const int ar = lane & 31;
    uint32_t a_rd[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
        a_rd[kk] = (uint32_t)(wm * 64 + ar) * 64u +
                   (uint32_t)((((kk * 2) + (lane >> 5)) ^ swz_a32(ar)) << 4);
    const int G = lane >> 4, p = lane & 15;
    const int b_sw = swz_b(p >> 2);
    uint32_t b_rd[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int nc = wn * 8 + ni * 4 + 2 * (G & 1) + ((p >> 1) & 1);
        b_rd[ni] = (uint32_t)(8 * (G >> 1) + (p >> 2)) * 256u + (uint32_t)((nc ^ b_sw) << 4) +
                   (uint32_t)((p & 1) * 8);
    }

    f32x16_t acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16_t{};

    const int nk = (K + BK - 1) / BK;
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
        if (s < nk) issue_stage(s * BK, s);
    // stage 0 landed: at most the loads of stages 1 and 2 (4 per stage per wave) outstanding
    if (nk >= 3) C3_WAIT_VMCNT(8);
    else if (nk == 2) C3_WAIT_VMCNT(4);
    else C3_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();

    auto compute = [&](const char* As) {
        const char* Bs = As + A_STAGE;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8_t colop[2], rowop[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) colop[mi] = lds_load16(As, a_rd[kk] + mi * 2048u);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                rowop[ni] = lds_load_tr8(Bs, b_rd[ni] + kk * 4096u, b_rd[ni] + kk * 4096u + 1024u);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rowop[ni], colop[mi],
                                                                          acc[mi][ni], 0, 0, 0);
        }
    };

    // Fast steps (as in the 256 kernel): while the refill of step kt+3 lies wholly inside K,
    // four steps per iteration, one per stage, so that stage addresses are constants; A's lane
    // offsets stay fixed and the k offset rides in the scalar offset; B's resource keeps the
    // maximum record count and only its base moves. Per step that leaves four loads, the twelve
    // LDS reads, eight MFMAs and two scalar updates, instead of the general step's per-step
    // resource, address and branch work.
    int kt = 0;
    const int nkf = K / BK;
    if (kt + 7 <= nkf) {
        const uint32_t lds_base = (uint32_t)(uintptr_t)(C3_LDS char*)smem;
        const uint32_t wave_lds = lds_base + __builtin_amdgcn_readfirstlane((uint32_t)wave) * 2048u;
        uint32_t a_vo[2], b_vo[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            a_vo[j] = a_g0 + (uint32_t)j * a_gstep;
            b_vo[j] = b_ok[j] ? b_g[j] : kOOB;
        }
        const uint64_t b0 = (uint64_t)(uintptr_t)(B + (size_t)(NSTAGE - 1) * BK * N + n0);
        uint32_t fb_lo = (uint32_t)b0, fb_hi = (uint32_t)(b0 >> 32);
        uint32_t fa_so = (uint32_t)(NSTAGE - 1) * BK * 2u;
        const uint64_t fb_step = (uint64_t)BK * (uint64_t)N * 2u;
        const uint32_t fbs_lo = (uint32_t)fb_step, fbs_hi = (uint32_t)(fb_step >> 32);
        auto step_fast = [&](auto s_c) {
            constexpr int S = decltype(s_c)::value;
            constexpr uint32_t DST = (uint32_t)(((S + NSTAGE - 1) & (NSTAGE - 1)) * STAGE);
            i32x4_t rBf;
            rBf.x = (int)fb_lo;
            rBf.y = (int)fb_hi;
            rBf.z = (int)kMaxRecords;
            rBf.w = kRsrcWord3;
            lds_dma16_so<DST + 0u>(rA, wave_lds, a_vo[0], fa_so);
            lds_dma16_so<DST + 1024u>(rA, wave_lds, a_vo[1], fa_so);
            lds_dma16_so<DST + A_STAGE + 0u>(rBf, wave_lds, b_vo[0], 0u);
            lds_dma16_so<DST + A_STAGE + 1024u>(rBf, wave_lds, b_vo[1], 0u);
            asm volatile("s_add_u32 %0, %0, %1" : "+s"(fa_so) : "n"(BK * 2) : "scc");
            asm volatile("s_add_u32 %0, %0, %2\n\ts_addc_u32 %1, %1, %3"
                         : "+s"(fb_lo), "+s"(fb_hi)
                         : "s"(fbs_lo), "s"(fbs_hi)
                         : "scc");
            compute(smem + S * STAGE);
            C3_WAIT_VMCNT(8);                    // step kt+1 landed (kt+2, kt+3 in flight)
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
        };
        for (; kt + 7 <= nkf; kt += 4) {
            step_fast(std::integral_constant<int, 0>{});
            step_fast(std::integral_constant<int, 1>{});
            step_fast(std::integral_constant<int, 2>{});
            step_fast(std::integral_constant<int, 3>{});
        }
    }

    for (; kt < nk; ++kt) {
        // refill the buffer step kt-1 used (every wave finished it before the last barrier)
        if (kt + NSTAGE - 1 < nk) issue_stage((kt + NSTAGE - 1) * BK, (kt + NSTAGE - 1) & (NSTAGE - 1));
        compute(smem + (kt & (NSTAGE - 1)) * STAGE);
        // step kt+1 landed for this wave (stages kt+2, kt+3 may be in flight); this wave's
        // reads of step kt are done; then every wave is past both points
        const int g = min(max(nk - kt - 2, 0), NSTAGE - 2);
        if (g >= 2) C3_WAIT_VMCNT(8);
        else if (g == 1) C3_WAIT_VMCNT(4);
        else C3_WAIT_VMCNT(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
    }

    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(C + (size_t)m0 * N + n0, ((int64_t)(M - m0) * N - n0) * 2);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const int ml = wm * 64 + mi * 32 + (lane & 31);
        const bool mvalid = (m0 + ml) < M;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nl = wn * 64 + ni * 32 + 8 * g + 4 * (lane >> 5);
                const bool ok = mvalid && (n0 + nl) < N;
                const uint32_t off = ok ? ((uint32_t)ml * (uint32_t)N + (uint32_t)nl) * 2u : kOOB;
                const f32x16_t& a = acc[mi][ni];
                store8(rC, off, pack_bf16x4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]));
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Skinny (small M) split-K kernel
// ------------------------------------------------------------------------------------------------
namespace sk {
constexpr int BM = 16, BN = 256, BK = 64, NT = 256;  // BM: one MFMA tile row block
constexpr int B_STAGE = BK * BN * 2;                 // 32 KiB
constexpr int B_LD = BK * BN / 8 / NT;               // 8
}  // namespace sk

// grid: x = N tiles of 256, y = K splits, z = M blocks of 16*MT rows. Each workgroup covers k in
// [y*k_per_split, min(K, (y+1)*k_per_split)) for all 16*MT of its rows, so B is streamed from
// memory once whatever M is (<= 64). With splits == 1 it writes bf16 C; otherwise fp32 partials
// to ws[y][m][n] (m < Mpad = 16*MT*gridDim.z).
template <int MT>
__global__ __launch_bounds__(256, 2) void gemm_bf16_skinny(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    float* __restrict__ ws, int M, int N, int K, int k_per_split) {
    using namespace sk;
    constexpr int ROWS = BM * MT;
    constexpr int A_STAGE = ROWS * BK * 2;  // MT * 2 KiB
    constexpr int STAGE = A_STAGE + B_STAGE;
    constexpr int A_CHUNKS = ROWS * BK / 8;  // 16-byte chunks per stage
    constexpr int A_LD = (A_CHUNKS + NT - 1) / NT;
    __shared__ __attribute__((aligned(128))) char smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.z * ROWS;
    const int kbeg = blockIdx.y * k_per_split;
    const int kend = min(K, kbeg + k_per_split);

    // A: chunk c = tid + NT*i (c < A_CHUNKS): row c/8, k chunk c%8.
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(A + (size_t)m0 * K, (int64_t)(M - m0) * K * 2);
    uint32_t a_g0[A_LD], a_s0[A_LD];
    int a_kc[A_LD];
    bool a_loader[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int c = tid + NT * i;
        const int row = (c >> 3) % ROWS;
        a_loader[i] = c < A_CHUNKS;
        a_kc[i] = c & 7;
        a_g0[i] = (uint32_t)row * (uint32_t)K * 2u + (uint32_t)a_kc[i] * 16u;
        a_s0[i] = (uint32_t)row * 128u + (uint32_t)((a_kc[i] ^ swz_a(row)) << 4);
    }
    // B: same 64 x 256 stage layout as the tile kernel.
    const int b_row = tid >> 5, b_nc = tid & 31;
    const bool b_nvalid = (n0 + b_nc * 8) < N;
    const uint32_t b_g0 = (uint32_t)b_row * (uint32_t)N * 2u + (uint32_t)b_nc * 16u;
    const uint32_t b_gstep = 8u * (uint32_t)N * 2u;
    const uint32_t b_s0 = (uint32_t)b_row * 512u + (uint32_t)((b_nc ^ swz_b(b_row)) << 4);

    // Column operand (A^T, 16 x 32 per MFMA): lane reads row 16*mt + lane%16, k chunk
    // kk*4 + lane/16.
    const int ar = lane & 15;
    uint32_t a_rd[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
        a_rd[kk] = (uint32_t)ar * 128u + (uint32_t)((((kk * 4) + (lane >> 4)) ^ swz_a(ar)) << 4);
    // Row operand (B^T, 16 n x 32 k): lane group G supplies k rows 8G + p/4 (+4h, +32kk),
    // n = 64*wave + 16*ni + 4*(p%4).
    const int G = lane >> 4, p = lane & 15;
    const int b_sw = swz_b(p >> 2);
    uint32_t b_rd[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        const int nc = wave * 8 + ni * 2 + ((p >> 1) & 1);
        b_rd[ni] = (uint32_t)(8 * G + (p >> 2)) * 512u + (uint32_t)((nc ^ b_sw) << 4) +
                   (uint32_t)((p & 1) * 8);
    }

    f32x4_t acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mt][ni] = f32x4_t{};

    // Register staging sets: with two, the loads would run two K steps ahead of the MFMAs. One
    // is used: two measured no faster (85-160 us either way for the skinny workloads), so bytes
    // in flight are not what limits this stream once the grid holds about two workgroups per CU;
    // B, read once, is loaded with the non-temporal policy (8-10% faster on 16..64 x 28672 x
    // 8192). A form with LDS-direct loads and three 32-k stages in flight was bit-identical and
    // up to 30% faster when only a few workgroups share the chip, but 2-11% slower with the
    // workgroups this split count gives, so it is not used.
    constexpr int PF = 1;
    u32x4_t ra[PF][A_LD], rb[PF][B_LD];
    auto load_stage = [&](int k0, int set) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const bool ok = a_loader[i] && (k0 + a_kc[i] * 8) < kend;
            ra[set][i] = load16(rA, ok ? a_g0[i] + (uint32_t)k0 * 2u : kOOB);
        }
        const __amdgpu_buffer_rsrc_t rB =
            make_rsrc(B + (size_t)k0 * N + n0, ((int64_t)(kend - k0) * N - n0) * 2);
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            rb[set][i] = load16_stream(rB, b_nvalid ? b_g0 + (uint32_t)i * b_gstep : kOOB);
    };
    auto store_stage = [&](int s, int set) {
        char* As = smem + s * STAGE;
        char* Bs = As + A_STAGE;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            if (a_loader[i]) lds_store16(As, a_s0[i], ra[set][i]);
#pragma unroll
        for (int i = 0; i < B_LD; ++i) lds_store16(Bs, b_s0 + (uint32_t)i * 4096u, rb[set][i]);
    };
    auto compute_stage = [&](int s) {
        const char* As = smem + s * STAGE;
        const char* Bs = As + A_STAGE;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8_t colop[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) colop[mt] = lds_load16(As, a_rd[kk] + mt * 2048u);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const bf16x8_t rowop = lds_load_tr8(Bs, b_rd[ni] + kk * 16384u,
                                                    b_rd[ni] + kk * 16384u + 2048u);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rowop, colop[mt],
                                                                          acc[mt][ni], 0, 0, 0);
            }
        }
    };

    const int nk = (kend - kbeg + BK - 1) / BK;
    // K step kt computes LDS stage kt%2. Register set indices must be compile-time constants
    // (a runtime index would put the staging registers in scratch memory), so the loop body
    // is written for an even and an odd step.
    auto body = [&](int kt, auto odd_c) {
        constexpr int ODD = decltype(odd_c)::value;
        // stage kt+PF into the register set that stage kt held (already stored to LDS)
        if (kt + PF < nk) load_stage(kbeg + (kt + PF) * BK, PF == 2 ? ODD : 0);
        compute_stage(ODD);
        if (kt + 1 < nk) store_stage(ODD ^ 1, PF == 2 ? (ODD ^ 1) : 0);
        __syncthreads();
    };
    if (nk > 0) {
        load_stage(kbeg, 0);
        store_stage(0, 0);
        if (PF == 2 && nk > 1) load_stage(kbeg + BK, PF - 1);
        __syncthreads();
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            body(kt, std::integral_constant<int, 0>{});
            body(kt + 1, std::integral_constant<int, 1>{});
        }
        if (kt < nk) body(kt, std::integral_constant<int, 0>{});
    }

    // lane holds D[n][m] for m = 16*mt + lane%16, n = 64*wave + 16*ni + 4*(lane/16) + v
    if (gridDim.y == 1) {
        const __amdgpu_buffer_rsrc_t rC =
            make_rsrc(C + (size_t)m0 * N + n0, ((int64_t)(M - m0) * N - n0) * 2);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int ml = mt * BM + (lane & 15);
            const bool mvalid = (m0 + ml) < M;
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const int nl = wave * 64 + ni * 16 + 4 * (lane >> 4);
                const bool ok = mvalid && (n0 + nl) < N;
                const uint32_t off = ok ? ((uint32_t)ml * (uint32_t)N + (uint32_t)nl) * 2u : kOOB;
                store8(rC, off, pack_bf16x4(acc[mt][ni][0], acc[mt][ni][1], acc[mt][ni][2],
                                            acc[mt][ni][3]));
            }
        }
    } else {
        const int mpad = gridDim.z * ROWS;
        float* wsb = ws + ((size_t)blockIdx.y * mpad + m0) * N + n0;
        const __amdgpu_buffer_rsrc_t rW = make_rsrc(wsb, ((int64_t)(mpad - m0) * N - n0) * 4);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int ml = mt * BM + (lane & 15);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const int nl = wave * 64 + ni * 16 + 4 * (lane >> 4);
                const bool ok = (n0 + nl) < N;
                const uint32_t off = ok ? ((uint32_t)ml * (uint32_t)N + (uint32_t)nl) * 4u : kOOB;
                store16(rW, off, __builtin_bit_cast(u32x4_t, acc[mt][ni]));
            }
        }
    }
}

// C[m][n..n+3] = bf16(sum over splits s = 0, 1, ... of ws[s][m][n..n+3]), in that order.
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ ws,
                                                    uint16_t* __restrict__ C, int M, int N,
                                                    int mpad, int splits) {
    const int nq = N >> 2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)M * nq) return;
    const int m = (int)(idx / nq);
    const int n = (int)(idx - (int64_t)m * nq) * 4;
    f32x4_t s = *reinterpret_cast<const f32x4_t*>(ws + (size_t)m * N + n);
    for (int k = 1; k < splits; ++k)
        s += *reinterpret_cast<const f32x4_t*>(ws + ((size_t)k * mpad + m) * N + n);
    *reinterpret_cast<u32x2_t*>(C + (size_t)m * N + n) = pack_bf16x4(s[0], s[1], s[2], s[3]);
}

constexpr int64_t kMaxDim = 1 << 21;

// Split-K partials of c3_gemm_noalloc: one fixed array per device, loaded with the code object
// and held until the process ends, instead of a workspace allocated per stream. In host code the
// name is only a stand-in: kernels get the device address bound by gemm_scratch_bind.
constexpr size_t kScratchBytes = C3_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];
constexpr int kMaxDevices = 64;
float* g_scratch_dev[kMaxDevices] = {};

struct Workspace {
    float* ptr = nullptr;
    size_t bytes = 0;
};
std::map<hipStream_t, Workspace>& workspaces() {
    static std::map<hipStream_t, Workspace> w;
    return w;
}

int env_int(const char* name, int dflt) {
    const char* v = std::getenv(name);
    return (v && *v) ? std::atoi(v) : dflt;
}

// K splits for the tile kernel from a cost model, in microseconds, measured on MI355X: a 32-deep
// K step of a 256x256 tile takes about 0.77 us on one CU; with splits, the fp32 partials are
// written and read back at about 3.5 TB/s and the reduction launch adds about 4 us. Time of s
// splits = waves * steps per split * 0.77 (+ partial traffic + 4 if s > 1); the smallest wins,
// ties to fewer splits. With at least as many tiles as CUs this is always 1.
int choose_splits(int64_t M, int64_t N, int64_t K, int tiles, int n_cu, int max_splits,
                  double* t_out) {
    constexpr double kStepUs = 0.77, kPartialBytesPerUs = 3.5e6, kReduceLaunchUs = 4.0;
    int best = 1;
    double best_t = 0.0;
    for (int s = 1; s <= max_splits; ++s) {
        int64_t kps = (K + s - 1) / s;
        kps = (kps + td::BK - 1) / td::BK * td::BK;
        const int64_t splits = (K + kps - 1) / kps;
        if (splits != s) continue;  // the same split as a smaller s
        const int64_t waves = ((int64_t)tiles * s + n_cu - 1) / n_cu;
        double t = (double)waves * (double)(kps / td::BK) * kStepUs;
        if (s > 1) t += kReduceLaunchUs + (double)s * (double)M * (double)N * 8.0 / kPartialBytesPerUs;
        if (s == 1 || t < best_t) {
            best = s;
            best_t = t;
        }
    }
    if (t_out) *t_out = best_t;
    return best;
}

// Time of the 128x128 tile kernel in the same units (measured on MI355X for 64-512 tiles of
// 128x128): a 32-deep K step takes about 0.5 us with one workgroup on a CU and about 0.62 us
// for each of two sharing one.
double tile128_time(int64_t M, int64_t N, int64_t K, int n_cu) {
    constexpr double kStepAloneUs = 0.5, kStepSharedUs = 0.62;
    const int64_t tiles = ((M + tq::BM - 1) / tq::BM) * ((N + tq::BN - 1) / tq::BN);
    const double steps = (double)((K + tq::BK - 1) / tq::BK);
    if (tiles <= n_cu) return steps * kStepAloneUs;
    const int64_t waves = (tiles + 2 * n_cu - 1) / (2 * n_cu);
    return (double)waves * steps * kStepSharedUs;
}

}  // namespace

namespace c3 {

c3_status gemm_validate(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K) {
    if (!A || !B || !C) return fail(C3_E_INVALID, "c3_gemm: null operand pointer");
    if (M < 1 || N < 1 || K < 1 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return fail(C3_E_INVALID, "c3_gemm: M, N, K must be in [1, %lld] (got %lld, %lld, %lld)",
                    (long long)kMaxDim, (long long)M, (long long)N, (long long)K);
    if (K % 8 || N % 8)
        return fail(C3_E_INVALID, "c3_gemm: K and N must be multiples of 8 (got K=%lld N=%lld)",
                    (long long)K, (long long)N);
    if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 15)
        return fail(C3_E_INVALID, "c3_gemm: A, B, C must be 16-byte aligned");
    const size_t a_bytes = (size_t)M * K * 2, b_bytes = (size_t)K * N * 2, c_bytes = (size_t)M * N * 2;
    C3_TRY(check_device_ptr(A, a_bytes, "A"));
    C3_TRY(check_device_ptr(B, b_bytes, "B"));
    C3_TRY(check_device_ptr(C, c_bytes, "C"));
    if (ranges_overlap(A, a_bytes, C, c_bytes) || ranges_overlap(B, b_bytes, C, c_bytes))
        return fail(C3_E_OVERLAP, "c3_gemm: C overlaps A or B");
    return C3_OK;
}

// The split-K fp32 workspace of `stream`: grown on demand (hipFree waits for work still using
// the old one), kept until c3_finalize.
static c3_status ensure_workspace(hipStream_t stream, size_t need, GemmPlan* p) {
    Workspace& w = workspaces()[stream];
    if (w.bytes < need) {
        if (w.ptr) C3_HIP_TRY(hipFree(w.ptr));
        w.ptr = nullptr;
        w.bytes = 0;
        C3_HIP_TRY(hipMalloc(&w.ptr, need));
        w.bytes = need;
    }
    p->workspace = w.ptr;
    p->workspace_bytes = need;
    return C3_OK;
}

// Device address of `device`'s scratch array (called at c3_init with that device current).
c3_status gemm_scratch_bind(int device) {
    if (device < 0 || device >= kMaxDevices)
        return fail(C3_E_UNSUPPORTED, "device %d: the no-allocation scratch covers devices 0..%d",
                    device, kMaxDevices - 1);
    void* p = nullptr;
    C3_HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(C3_E_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_dev[device] = static_cast<float*>(p);
    return C3_OK;
}

// The split-K partials of a plan: the stream's workspace (allocated on first need), or with
// `noalloc` the device's fixed scratch array, refused when the partials do not fit in it.
static c3_status partials(hipStream_t stream, size_t need, bool noalloc, GemmPlan* p) {
    if (!noalloc) return ensure_workspace(stream, need, p);
    if (need > kScratchBytes)
        return fail(C3_E_INVALID,
                    "c3_gemm_noalloc: this shape splits K into %d parts whose fp32 partials need "
                    "%zu bytes, above the %zu-byte scratch (use c3_gemm)",
                    p->splits, need, kScratchBytes);
    const int dev = ctx().device;
    float* w = (dev >= 0 && dev < kMaxDevices) ? g_scratch_dev[dev] : nullptr;
    if (!w) return fail(C3_E_NOT_INIT, "c3_gemm_noalloc: no scratch bound for device %d", dev);
    p->workspace = w;
    p->workspace_bytes = need;
    return C3_OK;
}

c3_status gemm_plan(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                    hipStream_t stream, GemmPlan* plan, bool noalloc) {
    C3_TRY(gemm_validate(A, B, C, M, N, K));
    GemmPlan p;
    p.A = A;
    p.B = B;
    p.C = C;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    if (M <= 64) {
        p.kind = 1;
        p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);  // 16-row MFMA tiles per workgroup (one M block)
        const int tiles = (int)((N + sk::BN - 1) / sk::BN);
        const int n_cu = ctx().info.n_cu > 0 ? ctx().info.n_cu : 256;
        // As many K splits as keep every workgroup resident at once (two per CU): a partial
        // second wave of workgroups would idle most of the chip while it runs.
        int splits = env_int("C3_SKINNY_SPLITS", 0);
        if (splits <= 0) splits = std::max(1, (2 * n_cu) / tiles);
        const int max_splits = std::max(1, (int)(K / (4 * sk::BK)));
        splits = std::max(1, std::min(splits, max_splits));
        int kps = (int)((K + splits - 1) / splits);
        kps = (kps + sk::BK - 1) / sk::BK * sk::BK;
        splits = (int)((K + kps - 1) / kps);
        p.splits = splits;
        p.k_per_split = kps;
        if (splits > 1) {
            const size_t mpad = (size_t)sk::BM * p.mt;
            const size_t need = (size_t)splits * mpad * (size_t)N * sizeof(float);
            C3_TRY(partials(stream, need, noalloc, &p));
        }
    } else {
        p.kind = 0;
        // Fewer output tiles than CUs: K may be split too, so that more of the chip works
        // (each split keeps at least 4 K steps so that the LDS pipeline fills); fp32 partials
        // are summed in split order by splitk_reduce. The count follows the device's CU count,
        // never a stream's CU mask, so C is the same under any mask.
        const int tiles = ((p.M + td::BM - 1) / td::BM) * ((p.N + td::BN - 1) / td::BN);
        const int n_cu = ctx().info.n_cu > 0 ? ctx().info.n_cu : 256;
        const int max_splits = std::max(1, std::min(256, (int)(K / (4 * td::BK))));
        int splits = env_int("C3_GEMM_SPLITS", 0);
        double t256 = 0.0;
        const int auto_splits = choose_splits(M, N, K, tiles, n_cu, max_splits, &t256);
        if (splits <= 0) splits = auto_splits;
        splits = std::max(1, std::min(splits, max_splits));
        // With fewer 256x256 tiles than CUs the 128x128 kernel may be faster (more workgroups,
        // no partial sums); the same model decides. C3_GEMM_TILE=128 / 256 forces the choice.
        const int tile = env_int("C3_GEMM_TILE", 0);
        if (tile == 128 ||
            (tile != 256 && tiles < n_cu && env_int("C3_GEMM_SPLITS", 0) <= 0 &&
             tile128_time(M, N, K, n_cu) < t256)) {
            p.kind = 2;
            *plan = p;
            return C3_OK;
        }
        int kps = (int)((K + splits - 1) / splits);
        kps = (kps + td::BK - 1) / td::BK * td::BK;
        splits = (int)((K + kps - 1) / kps);
        p.splits = splits;
        p.k_per_split = splits > 1 ? kps : (int)K;
        if (splits > 1) {
            const size_t need = (size_t)splits * (size_t)M * (size_t)N * sizeof(float);
            C3_TRY(partials(stream, need, noalloc, &p));
        }
    }
    *plan = p;
    return C3_OK;
}

c3_status gemm_enqueue(const GemmPlan& p, hipStream_t stream) {
    const auto* A = static_cast<const uint16_t*>(p.A);
    const auto* B = static_cast<const uint16_t*>(p.B);
    auto* C = static_cast<uint16_t*>(p.C);
    if (p.kind == 2) {
        const int tiles_m = (p.M + tq::BM - 1) / tq::BM;
        const int tiles_n = (p.N + tq::BN - 1) / tq::BN;
        hipLaunchKernelGGL(gemm_bf16_tile128_dma, dim3(tiles_m * tiles_n), dim3(tq::NT), 0, stream,
                           A, B, C, p.M, p.N, p.K, tiles_m, tiles_n);
        C3_HIP_TRY(hipGetLastError());
        return C3_OK;
    }
    if (p.kind == 0) {
        const int tiles_m = (p.M + td::BM - 1) / td::BM;
        const int tiles_n = (p.N + td::BN - 1) / td::BN;
        if (p.splits > 1 && !p.workspace) return fail(C3_E_INVALID, "split-K plan without workspace");
        if (p.splits > 1)
            hipLaunchKernelGGL(gemm_bf16_tile256_dma<true>, dim3(tiles_m * tiles_n, p.splits),
                               dim3(td::NT), 0, stream, A, B, C, p.workspace, p.M, p.N, p.K,
                               p.k_per_split, tiles_m, tiles_n);
        else
            hipLaunchKernelGGL(gemm_bf16_tile256_dma<false>, dim3(tiles_m * tiles_n), dim3(td::NT),
                               0, stream, A, B, C, nullptr, p.M, p.N, p.K, p.K, tiles_m, tiles_n);
        C3_HIP_TRY(hipGetLastError());
        if (p.splits > 1) {
            const int64_t quads = (int64_t)p.M * (p.N / 4);
            hipLaunchKernelGGL(splitk_reduce, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0,
                               stream, p.workspace, C, p.M, p.N, p.M, p.splits);
        }
        C3_HIP_TRY(hipGetLastError());
        return C3_OK;
    }
    const int tiles_n = (p.N + sk::BN - 1) / sk::BN;
    if (p.splits > 1 && !p.workspace) return fail(C3_E_INVALID, "split-K plan without workspace");
    const dim3 grid(tiles_n, p.splits, 1);  // M <= 64: one block of 16*mt rows
    if (p.mt == 1)
        hipLaunchKernelGGL(gemm_bf16_skinny<1>, grid, dim3(sk::NT), 0, stream, A, B, C, p.workspace,
                           p.M, p.N, p.K, p.k_per_split);
    else if (p.mt == 2)
        hipLaunchKernelGGL(gemm_bf16_skinny<2>, grid, dim3(sk::NT), 0, stream, A, B, C, p.workspace,
                           p.M, p.N, p.K, p.k_per_split);
    else
        hipLaunchKernelGGL(gemm_bf16_skinny<4>, grid, dim3(sk::NT), 0, stream, A, B, C, p.workspace,
                           p.M, p.N, p.K, p.k_per_split);
    C3_HIP_TRY(hipGetLastError());
    if (p.splits > 1) {
        const int64_t quads = (int64_t)p.M * (p.N / 4);
        const int blocks = (int)((quads + 255) / 256);
        hipLaunchKernelGGL(splitk_reduce, dim3(blocks), dim3(256), 0, stream, p.workspace, C, p.M,
                           p.N, sk::BM * p.mt, p.splits);
        C3_HIP_TRY(hipGetLastError());
    }
    return C3_OK;
}

void gemm_release_workspaces() {
    for (auto& kv : workspaces())
        if (kv.second.ptr) (void)hipFree(kv.second.ptr);
    workspaces().clear();
}

}  // namespace c3
