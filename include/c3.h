/*
 * c3.h -- C ABI of libc3: concurrent computation and communication (C3) on one MI355X (gfx950).
 *
 * What the library does, after "Optimizing ML Concurrent Computation and Communication with GPU
 * DMA Engines" (Agrawal, Aga, Pati, Islam; arXiv 2412.14335):
 *   - a dense GEMM runs concurrently with a collective-shaped data movement (abstract, Fig. 1);
 *   - the collective is an all-gather (FSDP) or an all-to-all (MoE) (Section III, Fig. 4); on
 *     one GPU only its local share exists: gather 8 shards into one buffer, or transpose an
 *     8x8 grid of blocks;
 *   - the data movement is done either by a copy kernel on the compute units (the baseline the
 *     paper calls c3_base) or by the SDMA engines, with the collective split into individual
 *     transfers, each put on an engine through hsa_amd_memory_async_copy_on_engine (ConCCL,
 *     Section VI-B; Pith review of arXiv 2412.14335, skeptic critique "load-bearing attack");
 *   - two C3 controls: issue the communication first (schedule prioritization: the kernel with
 *     fewer workgroups first) and split the compute units between the two (resource
 *     partitioning, Section V-B, Fig. 8; removing CUs from memory-bound GEMMs, Section VI-F).
 *
 * Conventions for every entry point:
 *   - extern "C"; no C++ exception crosses the boundary; nothing here aborts or prints.
 *   - Every function returns a c3_status. On anything but C3_OK, c3_last_error() gives a
 *     human-readable reason (thread-local; valid until the next call on the same thread).
 *   - Device pointers are HIP device memory of the device passed to c3_init (hipMalloc or a
 *     torch CUDA tensor's data pointer). The caller owns every buffer it passes; the library
 *     never frees them. Host pointers are only accepted where a parameter says "host".
 *   - A `stream` parameter is a hipStream_t passed as void*; NULL means the null stream.
 *   - Sizes are in bytes unless named M, N, K (elements).
 *   - Calls are serialized by one internal mutex. Kernel faults surface asynchronously at the
 *     next synchronizing call, as in HIP.
 */
#ifndef C3_H
#define C3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define C3_ABI_VERSION 5
#define C3_MAX_MASK_WORDS 8 /* CU masks cover up to 256 CUs, bit i = CU i as the driver numbers it */
#define C3_MAX_SEGMENTS 4096
#define C3_MAX_WORLD 64 /* ranks of a reduce-scatter / all-reduce local share */

typedef enum {
    C3_OK = 0,
    C3_E_INVALID = 1,     /* bad argument: null pointer, zero or inconsistent size, alignment */
    C3_E_HIP = 2,         /* a HIP runtime call failed */
    C3_E_HSA = 3,         /* a ROCr (HSA) call failed, or an SDMA copy reported an error */
    C3_E_NO_SDMA = 4,     /* no SDMA engine is available for device-local copies */
    C3_E_TIMEOUT = 5,     /* a completion wait exceeded its limit */
    C3_E_OVERLAP = 6,     /* source and destination (or GEMM input and output) ranges overlap */
    C3_E_UNSUPPORTED = 7, /* a valid request this build does not perform (e.g. priority != 0) */
    C3_E_NOT_INIT = 8     /* c3_init has not succeeded yet */
} c3_status;

/* C3_MOVER_HYBRID splits every segment of the copy: its first sdma_permille thousandths (rounded
 * down to a multiple of 256 bytes) go to the SDMA engines, the rest to the CU copy kernel, and
 * the two parts run at the same time. Not one of the paper's movers: on MI355X the engines move
 * a device-local copy several times slower than the CUs do, so when the copy is long beside the
 * GEMM a pure DMA offload makes the run copy-bound; moving part of it on the CUs shortens it. */
typedef enum { C3_MOVER_CU = 0, C3_MOVER_SDMA = 1, C3_MOVER_HYBRID = 2 } c3_mover;
typedef enum { C3_COPY_GATHER = 0, C3_COPY_ALL2ALL = 1, C3_COPY_ALLREDUCE = 2 } c3_copy_kind;

/* Test hooks for the SDMA mover, all forced from the host (no GPU fault is ever provoked):
 * DROP  - chunk `fault_chunk` is not issued and its completion is faked: the destination keeps
 *         its old bytes, so the caller's byte-exact check must fail;
 * STUCK - chunk `fault_chunk` is not issued and never completes: the wait ends in C3_E_TIMEOUT
 *         (every real chunk is still waited for first);
 * ERROR - chunk `fault_chunk` is not issued and its signal is set negative, the way ROCr reports
 *         a failed copy: the call returns C3_E_HSA after every real chunk completed. */
typedef enum {
    C3_FAULT_NONE = 0,
    C3_FAULT_DROP_CHUNK = 1,
    C3_FAULT_STUCK_CHUNK = 2,
    C3_FAULT_ERROR_CHUNK = 3
} c3_fault;

typedef enum { C3_TAX_GC_EQUAL = 0, C3_TAX_G_LONG = 1, C3_TAX_C_LONG = 2 } c3_taxonomy;

typedef struct {
    int32_t hip_device;
    int32_t n_cu;                /* compute units (hipDeviceProp_t.multiProcessorCount) */
    int32_t n_xcc;               /* accelerator complex dies (HSA_AMD_AGENT_INFO_NUM_XCC) */
    int32_t n_sdma;              /* SDMA engines (HSA_AMD_AGENT_INFO_NUM_SDMA_ENG) */
    int32_t n_sdma_xgmi;         /* xGMI SDMA engines (HSA_AMD_AGENT_INFO_NUM_SDMA_XGMI_ENG) */
    uint32_t sdma_engine_mask;   /* engines (one-hot HSA_AMD_SDMA_ENGINE_i bits) that completed a
                                    byte-exact device-local probe copy at c3_init */
    uint32_t sdma_status_mask;   /* hsa_amd_memory_copy_engine_status(gpu, gpu), as reported */
    uint32_t sdma_preferred_mask;/* ROCr's preferred engines for device-local copies (0 = none) */
    int32_t max_clock_mhz;       /* peak engine clock */
    int32_t lds_bytes_per_cu;    /* LDS per CU */
    int32_t l2_bytes;            /* L2 size reported by HIP */
    int32_t reserved;
    uint64_t hbm_bytes;          /* device memory */
    char arch[64];               /* gcnArchName, e.g. "gfx950:sramecc+:xnack-" */
} c3_info;

/* Options for one data movement. Zero-initialised means defaults. */
typedef struct {
    uint64_t chunk_bytes;  /* SDMA: split every segment into chunks of at most this many bytes
                              (0 = one transfer per shard or block, the paper's direct scheme,
                              each cut into equal 256-byte-multiple pieces of at least 128 KiB
                              until there are at least as many transfers as engines, and into
                              pieces of at most 16 MiB) */
    uint32_t engine_mask;  /* SDMA: use only these engines (one-hot HSA_AMD_SDMA_ENGINE_i bits;
                              0 = every engine available for device-local copies). Chunk c goes
                              to the (c mod n)-th engine of the mask. */
    int32_t nontemporal;   /* CU: 1 = streaming (non-temporal) loads and stores */
    int32_t cu_blocks;     /* CU: workgroups to launch (0 = one per 8 KiB of payload) */
    int32_t timeout_ms;    /* SDMA: wait limit per call (0 = 20000 ms) */
    int32_t fault_mode;    /* c3_fault test hook (0 = off) */
    int32_t fault_chunk;   /* chunk index the fault hook applies to */
    int32_t sdma_permille; /* HYBRID: share of every segment moved by the engines, in thousandths
                              (0..1000; 0 = all on the CUs, 1000 = all on the engines; see
                              c3_hybrid_share); ignored by the other movers */
} c3_move_opts;

/* One GEMM, C[M][N] = A[M][K] . B[K][N], bf16 row-major, fp32 accumulation, bf16 result. */
typedef struct {
    const void* A;
    const void* B;
    void* C;
    int64_t M, N, K;
} c3_gemm_args;

/* One collective's local share (see c3_gather, c3_all2all_block and c3_allreduce_local for the
 * layouts). For C3_COPY_ALLREDUCE, `mover` moves the all-gather half; the reduce-scatter half
 * always runs on the compute units. */
typedef struct {
    int32_t kind;               /* c3_copy_kind */
    int32_t mover;              /* c3_mover */
    void* dst;
    const void* const* shards;  /* gather: host array of n_shards device pointers;
                                   all-reduce: the n_shards (= world) ranks' contributions */
    int32_t n_shards;
    int32_t grid;               /* all-to-all: grid x grid blocks */
    uint64_t shard_bytes;       /* gather: bytes per shard; all-reduce: bytes per chunk */
    const void* src;            /* all-to-all: source holding grid*grid blocks */
    uint64_t block_bytes;       /* all-to-all: bytes per block */
    c3_move_opts opts;
    const void* const* peers;   /* all-reduce: host array of world device pointers, the other
                                   ranks' reduced chunks (entry `rank` is not read) */
    void* reduced;              /* all-reduce: this rank's reduced chunk (shard_bytes) */
    int32_t rank;               /* all-reduce: slot of `reduced` in dst */
    int32_t reserved;
} c3_copy_args;

/* Controls of one concurrent run. Zero-initialised means: all CUs for both, GEMM issued first,
 * no flush. */
typedef struct {
    uint32_t gemm_cu_mask[C3_MAX_MASK_WORDS]; /* all zero = every CU */
    uint32_t comm_cu_mask[C3_MAX_MASK_WORDS]; /* all zero = every CU (CU-mover copies and any
                                                 reduce-scatter) */
    int32_t comm_first;   /* 1 = start the communication before the GEMM (SDMA: each engine's
                             first transfer is issued before the GEMM launch, the engine's
                             other transfers right after it, queued behind the first) */
    int32_t use_priority; /* must be 0: every stream stays at default priority; the
                             prioritization control is the issue order (comm_first) */
    uint64_t flush_bytes; /* > 0: before the timed region, read this many bytes of a library
                             scratch buffer through the caches, evicting the last-level
                             (Infinity) cache; dirty lines are written back then, not in the
                             timed run (at least 32 KiB, else no flush) */
} c3_conc_opts;

/* Timings of one run. Host times use a monotonic clock and start just before the first issue. */
typedef struct {
    int64_t t_conc_ns;       /* first issue -> both operations observed complete */
    int64_t t_gemm_done_ns;  /* first issue -> GEMM completion observed (0 if no GEMM) */
    int64_t t_copy_done_ns;  /* first issue -> copy completion observed (0 if no copy) */
    int64_t t_issue_ns;      /* time spent issuing both operations */
    double gemm_gpu_ms;      /* HIP events around the GEMM launch(es) */
    double copy_gpu_ms;      /* CU mover: HIP events; SDMA: last end - first start of the
                                engines' own copy timestamps (all-reduce: plus the
                                reduce-scatter's kernel time); HYBRID: the larger of the two */
    int64_t sdma_first_start_ns; /* SDMA timestamps relative to the earliest chunk start */
    int64_t sdma_last_end_ns;
    int32_t n_chunks;        /* transfers issued (SDMA) or segments copied (CU); HYBRID: both */
    uint32_t engines_used;   /* SDMA engines that received a chunk */
    int32_t applied_priority;/* always 0 (default priority) */
    int32_t comm_issued_first;
    int64_t t_reduce_done_ns;/* all-reduce: first issue -> reduce-scatter completion observed */
    double reduce_gpu_ms;    /* all-reduce: HIP events around the reduce-scatter kernel(s) */
    /* CU masks the run actually applied, after normalisation (an all-zero request becomes every
     * CU of the device; bits past the device's last CU are dropped). gemm_applied_mask is the
     * GEMM stream's mask (all zero when no GEMM ran); comm_applied_mask is the communication
     * stream's (all zero when no kernel of the copy ran on the CUs, e.g. a pure SDMA copy). */
    uint32_t gemm_applied_mask[C3_MAX_MASK_WORDS];
    uint32_t comm_applied_mask[C3_MAX_MASK_WORDS];
} c3_timing;

#define C3_MAX_CURVE 16

/* One row of the one-time lookup table of kernel slowdowns (Section V-C): a kernel's time on
 * cus_per_xcc[i] CUs of every XCC relative to its time on all CUs. */
typedef struct {
    int32_t n;                          /* entries used, 1..C3_MAX_CURVE */
    int32_t reserved;
    int32_t cus_per_xcc[C3_MAX_CURVE];  /* distinct, each in [1, CUs per XCC] */
    double slowdown[C3_MAX_CURVE];      /* T(cus_per_xcc[i]) / T(all CUs), > 0 */
} c3_slowdown_curve;

/* Derived metrics of one concurrent run (abstract; Section IV-B3, Fig. 7). */
typedef struct {
    double ideal_speedup;   /* (T_gemm + T_copy) / max(T_gemm, T_copy) */
    double speedup;         /* (T_gemm + T_copy) / T_conc */
    double uplift_fraction; /* (speedup - 1) / (ideal_speedup - 1): "% of ideal speedup" */
    double ratio_of_ideal;  /* speedup / ideal_speedup (the literal ratio, secondary) */
    double gemm_slowdown;   /* T_conc / T_gemm - 1 */
    double hbm_ceiling;     /* (T_gemm + T_copy) / max(T_gemm, T_copy, bytes / bandwidth) */
    int32_t taxonomy;       /* c3_taxonomy: GC-equal when max/min <= 1.15 (Section III) */
    int32_t reserved;
} c3_metrics;

/* ---------------------------------------------------------------------------------------------
 * Set-up
 * ------------------------------------------------------------------------------------------- */

/* Bind the library to HIP device `hip_device` and its ROCr agent; discover CUs, XCCs and the
 * SDMA engines usable for device-local copies: every candidate engine (those the copy-engine
 * status reports, else one per SDMA engine the agent counts; the environment variable
 * C3_SDMA_ENGINE_MASK overrides the candidates) copies 256 KiB device-to-device once, and only
 * engines whose copy completes byte-exact within 2 s are used. Idempotent for the same device;
 * a different device returns C3_E_UNSUPPORTED. Finding no SDMA engine is not an error here
 * (c3_info.sdma_engine_mask = 0; SDMA copies then return C3_E_NO_SDMA). */
c3_status c3_init(int hip_device);

/* Release library-owned streams, events, signals and scratch memory. Safe to call twice. */
c3_status c3_finalize(void);

/* Text of the last non-OK status on this thread (never NULL). */
const char* c3_last_error(void);

/* Fill *out (host) with what c3_init discovered. */
c3_status c3_device_info(c3_info* out);

/* ---------------------------------------------------------------------------------------------
 * Streams and CU masks (resource partitioning, Section V-B)
 * ------------------------------------------------------------------------------------------- */

/* Create a stream restricted to the CUs in `cu_mask` (host array of n_words 32-bit words, bit i
 * = CU i). n_words = 0 or a NULL mask means every CU. The stream is always created with an
 * explicit mask so it gets a hardware queue of its own. `priority` must be 0
 * (C3_E_UNSUPPORTED otherwise). The library owns the stream until c3_stream_destroy or
 * c3_finalize. */
c3_status c3_stream_create(const uint32_t* cu_mask, int n_words, int priority, void** out);
c3_status c3_stream_destroy(void* stream);

/* Build a CU mask (host array of C3_MAX_MASK_WORDS words) that keeps `keep_per_xcc` CUs on
 * every XCC (0 < keep_per_xcc <= CUs per XCC), or its complement when complement = 1. The
 * driver spreads mask bit i onto XCC (i mod n_xcc), so the first keep_per_xcc * n_xcc bits are
 * kept. */
c3_status c3_cu_mask_balanced(int keep_per_xcc, int complement, uint32_t* mask_out);

/* Record where `n_blocks` one-wave workgroups ran: out_dev (device, 2*n_blocks uint32) gets the
 * raw HW_ID and XCC_ID registers of each workgroup. Synchronous. Used to verify CU masks. */
c3_status c3_probe_placement(void* stream, int n_blocks, uint32_t* out_dev);

/* Measurement probe: the matrix cores' sustained bf16 rate on this device with nothing but MFMAs
 * in flight, the ceiling for any bf16 GEMM here (under sustained MFMA load the chip runs at the
 * clock its power limit allows, and the power an MFMA draws depends on how many operand bits
 * toggle). n_workgroups workgroups of 4 waves; each wave keeps 16 independent 32x32 fp32
 * accumulators and issues `iterations` rounds of 16 v_mfma_f32_32x32x16_bf16, i.e.
 * n_workgroups * 4 * iterations * 16 * 32768 FLOP, on two operand sets used alternately:
 * random = 0: small integers (-2..2), every sum exact; random = 1: random signs, exponents and
 * mantissas, as a GEMM's data. out_dev (device, n_workgroups * 256 doubles) gets each lane's sum
 * of its accumulators; a wave's 64 sums total iterations * 8 * (S0 + S1) (exactly for random = 0,
 * up to fp32 rounding for random = 1; the operand formulas are in probe.hip). Stream-ordered and
 * asynchronous (time it with events on `stream`). 1 <= n_workgroups <= 65536,
 * 1 <= iterations <= 262144 (the largest count whose integer sums stay exact in fp32),
 * random in {0, 1}, else C3_E_INVALID. */
c3_status c3_probe_mfma_rate(void* stream, int n_workgroups, int iterations, int random,
                             double* out_dev);

/* ---------------------------------------------------------------------------------------------
 * The two operations (isolated)
 * ------------------------------------------------------------------------------------------- */

/* GEMM C = A.B: A[M][K], B[K][N], C[M][N], bf16 row-major, device memory, 16-byte aligned,
 * K % 8 == 0 and N % 8 == 0 (rows are read in 16-byte pieces), 1 <= M, N, K <= 2^21.
 * fp32 accumulation; C is overwritten with the sum rounded to nearest-even bf16 (no alpha,
 * beta, bias). Deterministic: no atomics, fixed reduction order, same bits on every run and
 * under any CU mask. Stream-ordered and asynchronous. A/B must not overlap C (C3_E_OVERLAP).
 * M <= 64, and shapes with fewer 256x256 output tiles than CUs where a cost model says it pays,
 * split K over workgroups: fp32 partials in a workspace the library allocates per stream on first
 * need (kept until c3_finalize), summed in split order. The split count depends only on the
 * shape and the device, so the bits do not change between calls.
 * GEMM kernels of LLaMA-70B/405B training are the paper's computation (Section IV, Fig. 5a). */
c3_status c3_gemm(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                  void* stream);

/* c3_gemm for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. Same arguments, kernels, plan and bits as
 * c3_gemm, but a shape whose plan splits K keeps its fp32 partials in a fixed device array of
 * C3_NOALLOC_SCRATCH_BYTES loaded with the library (one per device, held until the process
 * ends) instead of a workspace the library allocates. Nothing is allocated or freed, on the
 * device or through any allocating library routine; the array needs no clearing (every partial
 * the reduction reads is written first by the same call).
 * Errors: as c3_gemm; C3_E_INVALID, before anything is launched, when the shape's K split needs
 * more than C3_NOALLOC_SCRATCH_BYTES of partials (c3_last_error gives the size; c3_gemm runs
 * it). Shapes that do not split K (every shape with at least as many 256x256 output tiles as
 * CUs) use no scratch and have no limit.
 * Every call on one device shares that device's array: two calls that may overlap in time on
 * that device (different streams, or another host thread's call) race and give wrong results;
 * order them on one stream or synchronize between them. */
#define C3_NOALLOC_SCRATCH_BYTES (16u << 20)
c3_status c3_gemm_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                          void* stream);

/* All-gather local share: dst[i*shard_bytes + b] = shards[i][b] for i < n_shards,
 * b < shard_bytes. `shards` is a host array of n_shards device pointers; dst is device memory of
 * n_shards*shard_bytes bytes. Any alignment and size (shard_bytes = 0 is a no-op).
 * CU mover: stream-ordered and asynchronous. SDMA mover: synchronizes `stream` first (the copy
 * has no stream), issues one transfer per shard (or per chunk_bytes piece) round-robin over the
 * engines, and returns when every transfer completed. HYBRID mover: synchronizes `stream`,
 * issues the engines' share, enqueues the CU kernel for the rest on `stream` and returns when
 * the engines' transfers completed (the CU part is stream-ordered). opt->sdma_permille outside
 * 0..1000 is C3_E_INVALID. Sources must not overlap dst.
 * (Section VI-B; Pith review skeptic critique "load-bearing attack".) */
c3_status c3_gather(void* dst, const void* const* shards, int n_shards, size_t shard_bytes,
                    c3_mover mover, const c3_move_opts* opt, void* stream);

/* All-to-all local share as a block transpose: src holds grid*grid blocks of block_bytes, block
 * (i, j) at byte offset (i*grid + j)*block_bytes; it is copied verbatim to dst offset
 * (j*grid + i)*block_bytes. Out of place; src and dst must not overlap. Movers and completion as
 * for c3_gather (one transfer per block by default). (Section VI-B; Pith review forward
 * implications on all-to-all.) */
c3_status c3_all2all_block(void* dst, const void* src, int grid, size_t block_bytes,
                           c3_mover mover, const c3_move_opts* opt, void* stream);

/* Reduce-scatter local share on the compute units: out[e] = sum over r < world of
 * contribs[r][e], bf16 elements, e < chunk_bytes / 2. The sum is accumulated in fp32 starting
 * from rank 0's value with ranks added in order, then rounded once to nearest-even bf16 (a NaN
 * stays a NaN; its payload is not specified). `contribs` is a host array of world device
 * pointers; 1 <= world <= C3_MAX_WORLD; chunk_bytes must be even (0 is a no-op); any 2-byte
 * alignment (16-byte aligned pointers take the vector path). `out` must not overlap any
 * contribution (C3_E_OVERLAP). Stream-ordered and asynchronous. `opt` is unused (may be NULL).
 * DMA engines do no arithmetic, so this half of an all-reduce stays on the CUs (L3 Synthesis
 * page on 2412.14335, section 3, Attack 1; Pith review, Reading between the lines). */
c3_status c3_reduce_scatter(void* out, const void* const* contribs, int world, size_t chunk_bytes,
                            const c3_move_opts* opt, void* stream);

/* All-reduce local share = reduce-scatter, then all-gather of the reduced chunks:
 * reduced = c3_reduce_scatter(contribs); then dst slot i (chunk_bytes each, world slots) receives
 * `reduced` for i == rank and peers[i] otherwise. `peers` is a host array of world device
 * pointers (peers[rank] is not read); on one GPU they stand in for the chunks the other ranks
 * reduced. The all-gather starts only after the reduce-scatter completed and is moved by
 * `ag_mover`: CU - both halves stream-ordered and asynchronous on `stream`; SDMA - the
 * reduce-scatter runs on `stream`, the call waits for it, issues the transfers and returns when
 * they completed; HYBRID - as SDMA for the engines' share, the CU share enqueued on `stream`. dst and reduced must not overlap each other or any contribution or peer.
 * (Same passages as c3_reduce_scatter; the all-gather is c3_gather's.) */
c3_status c3_allreduce_local(void* dst, void* reduced, const void* const* contribs,
                             const void* const* peers, int world, int rank, size_t chunk_bytes,
                             c3_mover ag_mover, const c3_move_opts* opt, void* stream);

/* Read `bytes` of a library-owned scratch buffer on `stream`, which evicts the Infinity Cache
 * and leaves it holding clean lines (writes one word per workgroup into the scratch's first
 * 8 KiB). Allocates the scratch on first use or growth; below 32 KiB nothing is done. */
c3_status c3_flush_llc(size_t bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Concurrent run (C3)
 * ------------------------------------------------------------------------------------------- */

/* Run one GEMM and one copy concurrently and return when both completed (abstract, Fig. 1).
 * g or c may be NULL: then only the other one runs, under the same protocol (an isolated run,
 * as the ideal speedup requires, Section IV-B3). `o` may be NULL (defaults). `t` (host) may be
 * NULL.
 * Protocol: wait for the device to be idle; optionally flush; start the clock; issue the
 * communication then the GEMM if o->comm_first, else the GEMM then the communication (the GEMM
 * on a stream masked to o->gemm_cu_mask, a CU-mover copy on a second stream masked to
 * o->comm_cu_mask, an SDMA copy on the engines); poll both for completion; stop the clock.
 * An all-reduce (c->kind = C3_COPY_ALLREDUCE) runs its reduce-scatter on the o->comm_cu_mask
 * stream whatever the mover; with the SDMA mover the host issues the all-gather transfers as
 * soon as it observes the reduce-scatter complete (t_reduce_done_ns).
 * HYBRID mover: the engines' share is issued first (for an all-reduce, once the reduce-scatter
 * is observed complete), the CU share runs on the o->comm_cu_mask stream, and the copy is
 * complete when both are.
 * Library streams are created once per distinct mask and reused. Errors of either operation are
 * reported after both have finished. */
c3_status c3_run_concurrent(const c3_gemm_args* g, const c3_copy_args* c, const c3_conc_opts* o,
                            c3_timing* t);

/* Derived metrics from isolated times t_gemm, t_copy and concurrent time t_conc (any one unit),
 * plus total bytes both operations move and the memory bandwidth (bytes per that unit) for the
 * HBM-aware ceiling (bytes_total = 0 skips it: hbm_ceiling = ideal). Host arithmetic only.
 * (Abstract; Section III; Section IV-B3.) */
c3_status c3_derive_metrics(double t_gemm, double t_copy, double t_conc, double bytes_total,
                            double bandwidth, c3_metrics* out);

/* ---------------------------------------------------------------------------------------------
 * CU-partitioning heuristic (host arithmetic only; no device work)
 * ------------------------------------------------------------------------------------------- */

/* Roofline time estimate: *t_out = max(flops / (efficiency * peak_flops),
 * bytes / (efficiency * peak_bw)). The paper's heuristic uses efficiency 0.70 (Section V-C).
 * Needs flops, bytes >= 0, peaks > 0, 0 < efficiency <= 1. */
c3_status c3_roofline_time(double flops, double bytes, double peak_flops, double peak_bw,
                           double efficiency, double* t_out);

/* Choose how many CUs per XCC to give a CU-based collective running beside a GEMM (resource
 * partitioning, Section V-B; heuristic, Section V-C). For each candidate options[i] = c
 * (0 < c < cus_per_xcc) the predicted concurrent time is
 *     max(t_gemm * S_G(cus_per_xcc - c), t_comm * S_C(c)),
 * S looked up (not interpolated) in the two curves; a value the curve lacks is C3_E_INVALID.
 * *chosen_out = the option with the smallest prediction (ties: the smaller c);
 * predicted_out (host array of n_options, may be NULL) receives every prediction in order.
 * t_gemm, t_comm >= 0 (measured isolated times or c3_roofline_time estimates). */
c3_status c3_predict_partition(const c3_slowdown_curve* gemm, const c3_slowdown_curve* comm,
                               double t_gemm, double t_comm, int cus_per_xcc,
                               const int32_t* options, int n_options, int32_t* chosen_out,
                               double* predicted_out);

/* Share of a copy for the SDMA engines under C3_MOVER_HYBRID (host arithmetic only), from the
 * isolated times of the GEMM (t_gemm; 0 = no GEMM), of the whole copy on the engines (t_sdma)
 * and of the whole copy on the CUs (t_cu). Model: the engines' share runs beside the GEMM at its
 * isolated rate, while a CU copy beside a GEMM on the same CUs adds about its own isolated time
 * to the GEMM's (what MI355X measures for compute-bound GEMMs). The run then takes
 *     max(f * t_sdma, t_gemm + (1 - f) * t_cu),
 * smallest at f = (t_gemm + t_cu) / (t_sdma + t_cu), clamped to [0, 1].
 * *permille_out = f in thousandths, rounded to nearest. Needs t_gemm >= 0, t_sdma > 0, t_cu > 0
 * (finite), else C3_E_INVALID. Not from the paper: its DMA engines keep pace with CU
 * collectives at large sizes, MI355X's do not. */
c3_status c3_hybrid_share(double t_gemm, double t_sdma, double t_cu, int32_t* permille_out);

#ifdef __cplusplus
}
#endif

#endif /* C3_H */
