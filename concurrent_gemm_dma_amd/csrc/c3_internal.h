// Internal declarations of libc3 (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "c3.h"

namespace c3 {

// ---- errors -------------------------------------------------------------------------------
c3_status fail(c3_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

#define C3_HIP_TRY(call)                                                                      \
    do {                                                                                      \
        hipError_t e_ = (call);                                                               \
        if (e_ != hipSuccess)                                                                 \
            return ::c3::fail(C3_E_HIP, "%s failed: %s (%s:%d)", #call, hipGetErrorString(e_), \
                              __FILE__, __LINE__);                                            \
    } while (0)

#define C3_HSA_TRY(call)                                                                      \
    do {                                                                                      \
        hsa_status_t s_ = (call);                                                             \
        if (s_ != HSA_STATUS_SUCCESS) {                                                       \
            const char* m_ = nullptr;                                                         \
            hsa_status_string(s_, &m_);                                                       \
            return ::c3::fail(C3_E_HSA, "%s failed: %s (%s:%d)", #call, m_ ? m_ : "?",        \
                              __FILE__, __LINE__);                                            \
        }                                                                                     \
    } while (0)

#define C3_TRY(expr)                      \
    do {                                  \
        c3_status st_ = (expr);           \
        if (st_ != C3_OK) return st_;     \
    } while (0)

// ---- library state --------------------------------------------------------------------------
struct Context {
    bool inited = false;
    int device = -1;
    hsa_agent_t agent{};
    c3_info info{};
    std::vector<uint32_t> sdma_engines;  // one-hot engine ids usable for device-local copies
    void* flush_buf = nullptr;
    size_t flush_bytes = 0;
};
Context& ctx();
std::recursive_mutex& api_mutex();
c3_status require_init();

// ---- argument checks --------------------------------------------------------------------------
c3_status check_device_ptr(const void* p, size_t bytes, const char* what);
bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb);

// ---- GEMM (gemm.hip) ----------------------------------------------------------------------------
struct GemmPlan {
    const void* A = nullptr;
    const void* B = nullptr;
    void* C = nullptr;
    int M = 0, N = 0, K = 0;
    int kind = 0;          // 0 = 256x256 tile kernel, 1 = skinny split-K kernel, 2 = 128x128 tile
    int mt = 1;            // skinny: 16-row MFMA tiles per workgroup (1, 2 or 4)
    int splits = 1;        // skinny: K splits (1 = write bf16 directly)
    int k_per_split = 0;
    float* workspace = nullptr;  // skinny, splits > 1: fp32 partials [splits][Mpad][N]
    size_t workspace_bytes = 0;
};
c3_status gemm_validate(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K);
// Choose the kernel and (for split-K) make sure a workspace exists for `stream`. May allocate,
// unless `noalloc`: then split-K partials go to the device's fixed scratch array, and a plan
// whose partials do not fit there is refused (C3_E_INVALID).
c3_status gemm_plan(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                    hipStream_t stream, GemmPlan* plan, bool noalloc = false);
// Bind the fixed scratch array of `device` (must be the current device). Called by c3_init.
c3_status gemm_scratch_bind(int device);
// Launch only (no allocation, no synchronization).
c3_status gemm_enqueue(const GemmPlan& plan, hipStream_t stream);
void gemm_release_workspaces();

// ---- copies (copy.hip) ----------------------------------------------------------------------------
struct Segment {
    const void* src;
    void* dst;
    uint64_t bytes;
};
c3_status copy_cu_enqueue(const std::vector<Segment>& segs, const c3_move_opts& o,
                          hipStream_t stream);
c3_status flush_enqueue(void* buf, size_t bytes, hipStream_t stream);
c3_status probe_enqueue(int n_blocks, uint32_t* out_dev, hipStream_t stream);

// ---- MFMA rate probe (probe.hip) ---------------------------------------------------------------
c3_status mfma_probe_enqueue(int n_workgroups, int iters, int random, double* out_dev,
                             hipStream_t stream);

// ---- reduce-scatter (reduce.hip) ------------------------------------------------------------------
constexpr int kMaxWorld = C3_MAX_WORLD;
struct ReduceArgs {
    const void* in[kMaxWorld] = {};
    int world = 0;
    void* out = nullptr;
    uint64_t elems = 0;  // bf16 elements per rank
};
// Launch only: out[e] = bf16(fp32 sum of in[0..world-1][e] in rank order).
c3_status reduce_enqueue(const ReduceArgs& a, hipStream_t stream);

// A collective's local share as launched: optional reduce-scatter, then copy segments.
struct CommPlan {
    bool has_reduce = false;
    ReduceArgs reduce;
    std::vector<Segment> segs;
};
// Validate a c3_copy_args and turn it into a plan (no launch, no allocation on the device).
c3_status comm_plan(const c3_copy_args& a, CommPlan* plan);

// The copy segments each mover takes. CU: all on the CUs; SDMA: all on the engines; HYBRID: the
// first sdma_permille thousandths of every segment (rounded down to 256 bytes) on the engines,
// the rest on the CUs, empty parts dropped. use_dma / use_cu say whether each side has work.
struct MoverSplit {
    std::vector<Segment> dma, cu;
    bool use_dma = false, use_cu = false;
};
c3_status split_movers(int mover, const c3_move_opts& o, const std::vector<Segment>& segs,
                       MoverSplit* out);

// ---- SDMA (sdma.cpp) ----------------------------------------------------------------------------
c3_status sdma_discover();
void sdma_release();

struct SdmaOp {
    std::vector<Segment> chunks;        // the transfers, in issue order
    std::vector<uint32_t> engines;      // engine ids; chunk i goes to engines[i mod n]
    size_t next = 0;                    // first chunk not yet taken up (issued or faked)
    std::vector<hsa_signal_t> signals;  // one per chunk taken up
    std::vector<uint32_t> engine_of;    // engine id per chunk taken up
    std::vector<int> issued;            // 1 if the chunk was handed to ROCr
    uint32_t engines_used = 0;
    int fault_mode = 0;
    int fault_chunk = -1;
    int64_t deadline_ns = 0;
};
// Split segments into chunks and issue them on the engines (host returns right after issue).
// With first_round_only, only the first chunk of each engine is issued; sdma_issue_rest issues
// the others. An engine runs its transfers in issue order, so the rest only queue behind the
// first round. On an error nothing is left in flight and the op counts as never issued.
c3_status sdma_issue(const std::vector<Segment>& segs, const c3_move_opts& o, SdmaOp* op,
                     bool first_round_only = false);
// Issue the chunks sdma_issue held back. On an error the op still needs sdma_finish, which
// waits for everything issued.
c3_status sdma_issue_rest(SdmaOp* op);
// Nonblocking: true once every chunk's signal has left the "pending" state.
bool sdma_done(const SdmaOp& op);
// Wait for all chunks (bounded by the op's deadline), collect errors and timestamps, and return
// the signals to the pool. Always waits for every chunk that was really issued.
c3_status sdma_finish(SdmaOp* op, c3_timing* t);

// ---- streams and timing (concurrent.cpp) ---------------------------------------------------------
c3_status stream_for_mask(const uint32_t* mask, hipStream_t* out);
void release_streams();
int64_t now_ns();

}  // namespace c3
