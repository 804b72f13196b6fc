// abi.cpp -- the extern "C" entry points declared in include/c3.h. Each one takes the library
// mutex, validates its arguments before any launch, and converts C++ exceptions into a status.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <exception>
#include <limits>

#include "c3_internal.h"

namespace c3 {
const char* last_error_text();
c3_status init_device(int hip_device);
void finalize_device();
c3_status stream_for_role(int role, const uint32_t* mask, hipStream_t* out);
c3_status user_stream_create(const uint32_t* mask, int n_words, hipStream_t* out);
c3_status user_stream_destroy(hipStream_t s);
c3_status ensure_flush_buffer(size_t bytes);
c3_status run_concurrent(const c3_gemm_args* g, const c3_copy_args* c, const c3_conc_opts* o,
                         c3_timing* t);

// Validate a reduce-scatter local share: world contributions of chunk_bytes (bf16) into out.
c3_status reduce_args(void* out, const void* const* contribs, int world, size_t chunk_bytes,
                      ReduceArgs* r) {
    if (world < 1 || world > kMaxWorld)
        return fail(C3_E_INVALID, "reduce-scatter: world must be in [1, %d]", kMaxWorld);
    if (chunk_bytes % 2) return fail(C3_E_INVALID, "reduce-scatter: chunk_bytes must be even (bf16)");
    if (!contribs) return fail(C3_E_INVALID, "reduce-scatter: contributions array is NULL");
    if (!out) return fail(C3_E_INVALID, "reduce-scatter: output is NULL");
    r->world = world;
    r->out = out;
    r->elems = chunk_bytes / 2;
    if (chunk_bytes == 0) return C3_OK;
    C3_TRY(check_device_ptr(out, chunk_bytes, "reduce-scatter output"));
    for (int i = 0; i < world; ++i) {
        C3_TRY(check_device_ptr(contribs[i], chunk_bytes, "reduce-scatter contribution"));
        if (ranges_overlap(contribs[i], chunk_bytes, out, chunk_bytes))
            return fail(C3_E_OVERLAP, "reduce-scatter: contribution %d overlaps the output", i);
        r->in[i] = contribs[i];
    }
    return C3_OK;
}

c3_status comm_plan(const c3_copy_args& a, CommPlan* plan) {
    plan->has_reduce = false;
    plan->segs.clear();
    std::vector<Segment>* segs = &plan->segs;
    if (!a.dst) return fail(C3_E_INVALID, "copy: dst is NULL");
    if (a.kind == C3_COPY_GATHER) {
        if (a.n_shards < 0 || a.n_shards > C3_MAX_SEGMENTS)
            return fail(C3_E_INVALID, "gather: n_shards must be in [0, %d]", C3_MAX_SEGMENTS);
        if (a.n_shards > 0 && !a.shards) return fail(C3_E_INVALID, "gather: shards array is NULL");
        if (a.shard_bytes && (uint64_t)a.n_shards > std::numeric_limits<uint64_t>::max() / a.shard_bytes)
            return fail(C3_E_INVALID, "gather: size overflow");
        const size_t total = (size_t)a.n_shards * a.shard_bytes;
        if (total == 0) return C3_OK;
        C3_TRY(check_device_ptr(a.dst, total, "gather dst"));
        for (int i = 0; i < a.n_shards; ++i) {
            C3_TRY(check_device_ptr(a.shards[i], a.shard_bytes, "gather shard"));
            if (ranges_overlap(a.shards[i], a.shard_bytes, a.dst, total))
                return fail(C3_E_OVERLAP, "gather: shard %d overlaps dst", i);
            segs->push_back({a.shards[i], static_cast<char*>(a.dst) + (size_t)i * a.shard_bytes,
                             a.shard_bytes});
        }
        return C3_OK;
    }
    if (a.kind == C3_COPY_ALL2ALL) {
        if (a.grid < 1 || (int64_t)a.grid * a.grid > C3_MAX_SEGMENTS)
            return fail(C3_E_INVALID, "all2all: grid must be in [1, 64]");
        if (!a.src) return fail(C3_E_INVALID, "all2all: src is NULL");
        const uint64_t nb = (uint64_t)a.grid * (uint64_t)a.grid;
        if (a.block_bytes && nb > std::numeric_limits<uint64_t>::max() / a.block_bytes)
            return fail(C3_E_INVALID, "all2all: size overflow");
        const size_t total = (size_t)(nb * a.block_bytes);
        if (total == 0) return C3_OK;
        C3_TRY(check_device_ptr(a.src, total, "all2all src"));
        C3_TRY(check_device_ptr(a.dst, total, "all2all dst"));
        if (ranges_overlap(a.src, total, a.dst, total))
            return fail(C3_E_OVERLAP, "all2all: src overlaps dst");
        for (int i = 0; i < a.grid; ++i)
            for (int j = 0; j < a.grid; ++j) {
                const size_t from = ((size_t)i * a.grid + j) * a.block_bytes;
                const size_t to = ((size_t)j * a.grid + i) * a.block_bytes;
                segs->push_back({static_cast<const char*>(a.src) + from,
                                 static_cast<char*>(a.dst) + to, a.block_bytes});
            }
        return C3_OK;
    }
    if (a.kind == C3_COPY_ALLREDUCE) {
        const int world = a.n_shards;
        const size_t chunk = a.shard_bytes;
        C3_TRY(reduce_args(a.reduced, a.shards, world, chunk, &plan->reduce));
        if (a.rank < 0 || a.rank >= world)
            return fail(C3_E_INVALID, "all-reduce: rank must be in [0, world)");
        if (world > 1 && !a.peers) return fail(C3_E_INVALID, "all-reduce: peers array is NULL");
        if (chunk == 0) return C3_OK;
        if (chunk > (std::numeric_limits<size_t>::max() >> 7))  // world <= 64 = 2^6
            return fail(C3_E_INVALID, "all-reduce: size overflow");
        const size_t total = (size_t)world * chunk;
        C3_TRY(check_device_ptr(a.dst, total, "all-reduce dst"));
        if (ranges_overlap(a.reduced, chunk, a.dst, total))
            return fail(C3_E_OVERLAP, "all-reduce: reduced chunk overlaps dst");
        for (int i = 0; i < world; ++i)
            if (ranges_overlap(a.shards[i], chunk, a.dst, total))
                return fail(C3_E_OVERLAP, "all-reduce: contribution %d overlaps dst", i);
        for (int i = 0; i < world; ++i) {
            const void* src = a.reduced;
            if (i != a.rank) {
                C3_TRY(check_device_ptr(a.peers[i], chunk, "all-reduce peer chunk"));
                if (ranges_overlap(a.peers[i], chunk, a.dst, total))
                    return fail(C3_E_OVERLAP, "all-reduce: peer chunk %d overlaps dst", i);
                if (ranges_overlap(a.peers[i], chunk, a.reduced, chunk))
                    return fail(C3_E_OVERLAP, "all-reduce: peer chunk %d overlaps the reduced chunk", i);
                src = a.peers[i];
            }
            segs->push_back({src, static_cast<char*>(a.dst) + (size_t)i * chunk, chunk});
        }
        plan->has_reduce = true;
        return C3_OK;
    }
    return fail(C3_E_INVALID, "copy: unknown kind %d", a.kind);
}

c3_status split_movers(int mover, const c3_move_opts& o, const std::vector<Segment>& segs,
                       MoverSplit* out) {
    *out = MoverSplit{};
    if (mover == C3_MOVER_CU) {
        out->cu = segs;
        out->use_cu = true;
        return C3_OK;
    }
    if (mover == C3_MOVER_SDMA) {
        out->dma = segs;
        out->use_dma = true;
        return C3_OK;
    }
    if (mover != C3_MOVER_HYBRID) return fail(C3_E_INVALID, "unknown mover %d", mover);
    if (o.sdma_permille < 0 || o.sdma_permille > 1000)
        return fail(C3_E_INVALID, "hybrid mover: sdma_permille must be in [0, 1000], got %d",
                    o.sdma_permille);
    for (const Segment& s : segs) {
        if (s.bytes == 0) continue;
        // bytes < 2^64 / 1000 for any buffer that fits a device; 256-byte multiples keep the
        // CU part's alignment that of the segment
        uint64_t head = s.bytes;
        if (o.sdma_permille < 1000)
            head = (s.bytes / 1000 * (uint64_t)o.sdma_permille +
                    s.bytes % 1000 * (uint64_t)o.sdma_permille / 1000) & ~uint64_t(255);
        if (head) out->dma.push_back({s.src, s.dst, head});
        if (head < s.bytes)
            out->cu.push_back({static_cast<const char*>(s.src) + head, static_cast<char*>(s.dst) + head,
                               s.bytes - head});
    }
    out->use_dma = !out->dma.empty();
    out->use_cu = !out->cu.empty();
    return C3_OK;
}

// Isolated collective on `stream`: the reduce-scatter (if any) and a CU-mover copy are
// enqueued; with the SDMA mover the stream is drained first, then the transfers are issued and
// waited for; the hybrid mover drains the stream, issues the engines' share, enqueues the CUs'
// share and waits for the engines.
c3_status copy_isolated(const c3_copy_args& a, hipStream_t stream) {
    CommPlan plan;
    C3_TRY(comm_plan(a, &plan));
    MoverSplit ms;
    C3_TRY(split_movers(a.mover, a.opts, plan.segs, &ms));
    if (plan.has_reduce) C3_TRY(reduce_enqueue(plan.reduce, stream));
    if (plan.segs.empty()) return C3_OK;
    if (!ms.use_dma) return copy_cu_enqueue(ms.cu, a.opts, stream);
    C3_HIP_TRY(hipStreamSynchronize(stream));
    SdmaOp op;
    C3_TRY(sdma_issue(ms.dma, a.opts, &op));
    c3_status st = C3_OK;
    if (ms.use_cu) st = copy_cu_enqueue(ms.cu, a.opts, stream);
    c3_timing t{};
    const c3_status st_dma = sdma_finish(&op, &t);
    return st != C3_OK ? st : st_dma;
}

}  // namespace c3

using namespace c3;

#define C3_ENTRY(body)                                                      \
    try {                                                                   \
        std::lock_guard<std::recursive_mutex> lock_(api_mutex());           \
        body                                                                \
    } catch (const std::exception& e) {                                     \
        return fail(C3_E_INVALID, "internal exception: %s", e.what());      \
    } catch (...) {                                                         \
        return fail(C3_E_INVALID, "internal exception");                    \
    }

extern "C" {

c3_status c3_init(int hip_device) { C3_ENTRY(return init_device(hip_device);) }

c3_status c3_finalize(void) {
    C3_ENTRY(finalize_device(); return C3_OK;)
}

const char* c3_last_error(void) { return last_error_text(); }

c3_status c3_device_info(c3_info* out) {
    C3_ENTRY({
        C3_TRY(require_init());
        if (!out) return fail(C3_E_INVALID, "c3_device_info: out is NULL");
        *out = ctx().info;
        return C3_OK;
    })
}

c3_status c3_stream_create(const uint32_t* cu_mask, int n_words, int priority, void** out) {
    C3_ENTRY({
        C3_TRY(require_init());
        if (!out) return fail(C3_E_INVALID, "c3_stream_create: out is NULL");
        if (priority != 0)
            return fail(C3_E_UNSUPPORTED,
                        "c3_stream_create: only default-priority streams are created "
                        "(prioritize by issue order)");
        if (n_words > 0 && !cu_mask) return fail(C3_E_INVALID, "c3_stream_create: mask is NULL");
        hipStream_t s = nullptr;
        C3_TRY(user_stream_create(cu_mask, n_words, &s));
        *out = s;
        return C3_OK;
    })
}

c3_status c3_stream_destroy(void* stream) {
    C3_ENTRY({
        C3_TRY(require_init());
        return user_stream_destroy(static_cast<hipStream_t>(stream));
    })
}

c3_status c3_cu_mask_balanced(int keep_per_xcc, int complement, uint32_t* mask_out) {
    C3_ENTRY({
        C3_TRY(require_init());
        if (!mask_out) return fail(C3_E_INVALID, "mask_out is NULL");
        const c3_info& d = ctx().info;
        const int per = d.n_cu / d.n_xcc;
        if (keep_per_xcc < 1 || keep_per_xcc > per)
            return fail(C3_E_INVALID, "keep_per_xcc must be in [1, %d]", per);
        if (complement && keep_per_xcc == per)
            return fail(C3_E_INVALID, "complement of a full mask is empty");
        std::memset(mask_out, 0, sizeof(uint32_t) * C3_MAX_MASK_WORDS);
        const int kept = keep_per_xcc * d.n_xcc;
        for (int b = 0; b < d.n_cu && b < 32 * C3_MAX_MASK_WORDS; ++b) {
            const bool in = b < kept;
            if (in != (complement != 0)) mask_out[b / 32] |= 1u << (b % 32);
        }
        return C3_OK;
    })
}

c3_status c3_probe_placement(void* stream, int n_blocks, uint32_t* out_dev) {
    C3_ENTRY({
        C3_TRY(require_init());
        if (n_blocks < 1 || n_blocks > 65536)
            return fail(C3_E_INVALID, "n_blocks must be in [1, 65536]");
        C3_TRY(check_device_ptr(out_dev, (size_t)n_blocks * 8, "probe out"));
        hipStream_t s = static_cast<hipStream_t>(stream);
        C3_TRY(probe_enqueue(n_blocks, out_dev, s));
        C3_HIP_TRY(hipStreamSynchronize(s));
        return C3_OK;
    })
}

c3_status c3_probe_mfma_rate(void* stream, int n_workgroups, int iterations, int random,
                             double* out_dev) {
    C3_ENTRY({
        C3_TRY(require_init());
        if (n_workgroups < 1 || n_workgroups > 65536)
            return fail(C3_E_INVALID, "n_workgroups must be in [1, 65536]");
        if (iterations < 1 || iterations > 262144)
            return fail(C3_E_INVALID, "iterations must be in [1, 262144]");
        C3_TRY(check_device_ptr(out_dev, (size_t)n_workgroups * 256 * sizeof(double), "probe out"));
        if (random != 0 && random != 1) return fail(C3_E_INVALID, "random must be 0 or 1");
        return mfma_probe_enqueue(n_workgroups, iterations, random, out_dev,
                                  static_cast<hipStream_t>(stream));
    })
}

c3_status c3_gemm(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                  void* stream) {
    C3_ENTRY({
        C3_TRY(require_init());
        hipStream_t s = static_cast<hipStream_t>(stream);
        GemmPlan plan;
        C3_TRY(gemm_plan(A, B, C, M, N, K, s, &plan));
        return gemm_enqueue(plan, s);
    })
}

c3_status c3_gemm_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                          void* stream) {
    C3_ENTRY({
        C3_TRY(require_init());
        hipStream_t s = static_cast<hipStream_t>(stream);
        GemmPlan plan;
        C3_TRY(gemm_plan(A, B, C, M, N, K, s, &plan, /*noalloc=*/true));
        return gemm_enqueue(plan, s);
    })
}

c3_status c3_gather(void* dst, const void* const* shards, int n_shards, size_t shard_bytes,
                    c3_mover mover, const c3_move_opts* opt, void* stream) {
    C3_ENTRY({
        C3_TRY(require_init());
        c3_copy_args a{};
        a.kind = C3_COPY_GATHER;
        a.mover = mover;
        a.dst = dst;
        a.shards = shards;
        a.n_shards = n_shards;
        a.shard_bytes = shard_bytes;
        if (opt) a.opts = *opt;
        return copy_isolated(a, static_cast<hipStream_t>(stream));
    })
}

c3_status c3_all2all_block(void* dst, const void* src, int grid, size_t block_bytes,
                           c3_mover mover, const c3_move_opts* opt, void* stream) {
    C3_ENTRY({
        C3_TRY(require_init());
        c3_copy_args a{};
        a.kind = C3_COPY_ALL2ALL;
        a.mover = mover;
        a.dst = dst;
        a.src = src;
        a.grid = grid;
        a.block_bytes = block_bytes;
        if (opt) a.opts = *opt;
        return copy_isolated(a, static_cast<hipStream_t>(stream));
    })
}

c3_status c3_reduce_scatter(void* out, const void* const* contribs, int world, size_t chunk_bytes,
                            const c3_move_opts* opt, void* stream) {
    (void)opt;
    C3_ENTRY({
        C3_TRY(require_init());
        ReduceArgs r;
        C3_TRY(reduce_args(out, contribs, world, chunk_bytes, &r));
        return reduce_enqueue(r, static_cast<hipStream_t>(stream));
    })
}

c3_status c3_allreduce_local(void* dst, void* reduced, const void* const* contribs,
                             const void* const* peers, int world, int rank, size_t chunk_bytes,
                             c3_mover ag_mover, const c3_move_opts* opt, void* stream) {
    C3_ENTRY({
        C3_TRY(require_init());
        c3_copy_args a{};
        a.kind = C3_COPY_ALLREDUCE;
        a.mover = ag_mover;
        a.dst = dst;
        a.shards = contribs;
        a.n_shards = world;
        a.shard_bytes = chunk_bytes;
        a.peers = peers;
        a.reduced = reduced;
        a.rank = rank;
        if (opt) a.opts = *opt;
        return copy_isolated(a, static_cast<hipStream_t>(stream));
    })
}

c3_status c3_flush_llc(size_t bytes, void* stream) {
    C3_ENTRY({
        C3_TRY(require_init());
        if (bytes == 0) return C3_OK;
        C3_TRY(ensure_flush_buffer(bytes));
        return flush_enqueue(ctx().flush_buf, bytes, static_cast<hipStream_t>(stream));
    })
}

c3_status c3_run_concurrent(const c3_gemm_args* g, const c3_copy_args* c, const c3_conc_opts* o,
                            c3_timing* t) {
    C3_ENTRY({
        C3_TRY(require_init());
        return run_concurrent(g, c, o, t);
    })
}

c3_status c3_derive_metrics(double t_gemm, double t_copy, double t_conc, double bytes_total,
                            double bandwidth, c3_metrics* out) {
    if (!out) return fail(C3_E_INVALID, "c3_derive_metrics: out is NULL");
    if (!(t_gemm >= 0) || !(t_copy >= 0) || !(t_conc > 0) || !(std::max(t_gemm, t_copy) > 0))
        return fail(C3_E_INVALID, "c3_derive_metrics: need t_gemm, t_copy >= 0, max > 0, t_conc > 0");
    const double serial = t_gemm + t_copy;
    const double longest = std::max(t_gemm, t_copy);
    const double shortest = std::min(t_gemm, t_copy);
    c3_metrics m{};
    m.ideal_speedup = serial / longest;
    m.speedup = serial / t_conc;
    m.uplift_fraction = m.ideal_speedup == 1.0 ? std::nan("")
                                               : (m.speedup - 1.0) / (m.ideal_speedup - 1.0);
    m.ratio_of_ideal = m.speedup / m.ideal_speedup;
    m.gemm_slowdown = t_gemm > 0 ? t_conc / t_gemm - 1.0 : std::nan("");
    double floor_t = longest;
    if (bytes_total > 0 && bandwidth > 0) floor_t = std::max(floor_t, bytes_total / bandwidth);
    m.hbm_ceiling = serial / floor_t;
    if (shortest > 0 && longest / shortest <= 1.15) m.taxonomy = C3_TAX_GC_EQUAL;
    else m.taxonomy = t_gemm > t_copy ? C3_TAX_G_LONG : C3_TAX_C_LONG;
    *out = m;
    return C3_OK;
}

}  // extern "C"
