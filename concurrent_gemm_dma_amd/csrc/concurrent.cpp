// concurrent.cpp -- the C3 controller: CU-masked streams, issue order, completion and timing of
// one GEMM running concurrently with one collective-shaped copy ("Optimizing ML Concurrent
// Computation and Communication with GPU DMA Engines": abstract and Fig. 1 for the concurrent
// run; Section IV-B3 for isolated times; Section V-B and Fig. 8 for schedule prioritization and
// CU partitioning; Section VI-F for removing CUs from the GEMM when the copy runs on DMA).
//
// * Partitioning: the GEMM runs on a stream created with hipExtStreamCreateWithCUMask; a
//   CU-mover copy runs on a second masked stream (typically the complement). Every library
//   stream carries an explicit mask (all CUs when unrestricted) so that each gets a hardware
//   queue of its own and the two operations can really overlap.
// * Prioritization: the communication is issued before the GEMM (comm_first); with the SDMA
//   engines, each engine's first transfer goes before the GEMM launch and its others right after
//   it, queued behind the first. Streams keep the default priority.
// * Completion: the host polls the GEMM's end event and the copy's end event (CU mover) or
//   completion signals (SDMA mover) and timestamps each completion on a monotonic clock.
// * All-reduce (reduce-scatter + all-gather; L3 Synthesis page on 2412.14335, section 3,
//   Attack 1): the reduce-scatter kernel runs on the communication stream whatever the mover;
//   a CU-mover all-gather follows it on that stream, an SDMA all-gather is issued by the
//   polling loop as soon as the reduce-scatter's end event has completed.
// * Hybrid mover: the engines' share of every segment and the CUs' share run at the same time,
//   the latter on the communication stream; the copy is complete when both are.
#include <algorithm>
#include <array>
#include <chrono>
#include <cmath>
#include <map>
#include <set>

#include "c3_internal.h"

namespace c3 {

int64_t now_ns() {
    return std::chrono::duration_cast<std::chrono::nanoseconds>(
               std::chrono::steady_clock::now().time_since_epoch())
        .count();
}

namespace {

using MaskKey = std::pair<int, std::array<uint32_t, C3_MAX_MASK_WORDS>>;

std::map<MaskKey, hipStream_t>& stream_cache() {
    static std::map<MaskKey, hipStream_t> m;
    return m;
}

std::set<hipStream_t>& user_streams() {
    static std::set<hipStream_t> s;
    return s;
}

struct Events {
    hipEvent_t g0 = nullptr, g1 = nullptr, c0 = nullptr, c1 = nullptr, r1 = nullptr;
};
Events& events() {
    static Events e;
    return e;
}

int mask_words() { return std::max(1, (ctx().info.n_cu + 31) / 32); }

// Normalise a mask: all-zero means every CU; bits beyond the device's CUs are dropped.
std::array<uint32_t, C3_MAX_MASK_WORDS> normalise(const uint32_t* mask, int n_words) {
    std::array<uint32_t, C3_MAX_MASK_WORDS> m{};
    bool any = false;
    for (int i = 0; i < n_words && i < C3_MAX_MASK_WORDS; ++i) {
        m[i] = mask ? mask[i] : 0u;
        any |= m[i] != 0;
    }
    const int n_cu = ctx().info.n_cu;
    for (int b = 0; b < 32 * C3_MAX_MASK_WORDS; ++b) {
        const bool in_device = b < n_cu;
        uint32_t& w = m[b / 32];
        const uint32_t bit = 1u << (b % 32);
        if (!any) w = in_device ? (w | bit) : (w & ~bit);
        else if (!in_device) w &= ~bit;
    }
    return m;
}

c3_status create_masked(const std::array<uint32_t, C3_MAX_MASK_WORDS>& m, hipStream_t* out) {
    bool any = false;
    for (uint32_t w : m) any |= w != 0;
    if (!any) return fail(C3_E_INVALID, "CU mask selects no CU of this device");
    C3_HIP_TRY(hipExtStreamCreateWithCUMask(out, (uint32_t)mask_words(), m.data()));
    return C3_OK;
}

c3_status ensure_events() {
    Events& e = events();
    if (!e.g0) {
        C3_HIP_TRY(hipEventCreate(&e.g0));
        C3_HIP_TRY(hipEventCreate(&e.g1));
        C3_HIP_TRY(hipEventCreate(&e.c0));
        C3_HIP_TRY(hipEventCreate(&e.c1));
        C3_HIP_TRY(hipEventCreate(&e.r1));
    }
    return C3_OK;
}

}  // namespace

// role 0 = GEMM, 1 = communication: the two roles never share a stream, even with equal masks.
c3_status stream_for_role(int role, const uint32_t* mask, hipStream_t* out) {
    const auto m = normalise(mask, C3_MAX_MASK_WORDS);
    const MaskKey key{role, m};
    auto& cache = stream_cache();
    auto it = cache.find(key);
    if (it != cache.end()) {
        *out = it->second;
        return C3_OK;
    }
    hipStream_t s = nullptr;
    C3_TRY(create_masked(m, &s));
    cache[key] = s;
    *out = s;
    return C3_OK;
}

c3_status stream_for_mask(const uint32_t* mask, hipStream_t* out) { return stream_for_role(0, mask, out); }

c3_status user_stream_create(const uint32_t* mask, int n_words, hipStream_t* out) {
    if (n_words < 0 || n_words > C3_MAX_MASK_WORDS)
        return fail(C3_E_INVALID, "n_words must be in [0, %d]", C3_MAX_MASK_WORDS);
    const auto m = normalise(n_words ? mask : nullptr, n_words);
    hipStream_t s = nullptr;
    C3_TRY(create_masked(m, &s));
    user_streams().insert(s);
    *out = s;
    return C3_OK;
}

c3_status user_stream_destroy(hipStream_t s) {
    auto& us = user_streams();
    if (!us.count(s)) return fail(C3_E_INVALID, "stream %p was not created by c3_stream_create", (void*)s);
    us.erase(s);
    C3_HIP_TRY(hipStreamDestroy(s));
    return C3_OK;
}

void release_streams() {
    for (auto& kv : stream_cache()) (void)hipStreamDestroy(kv.second);
    stream_cache().clear();
    for (hipStream_t s : user_streams()) (void)hipStreamDestroy(s);
    user_streams().clear();
    Events& e = events();
    for (hipEvent_t* ev : {&e.g0, &e.g1, &e.c0, &e.c1, &e.r1})
        if (*ev) {
            (void)hipEventDestroy(*ev);
            *ev = nullptr;
        }
}

c3_status ensure_flush_buffer(size_t bytes) {
    Context& c = ctx();
    if (c.flush_bytes >= bytes) return C3_OK;
    if (c.flush_buf) C3_HIP_TRY(hipFree(c.flush_buf));
    c.flush_buf = nullptr;
    c.flush_bytes = 0;
    C3_HIP_TRY(hipMalloc(&c.flush_buf, bytes));
    c.flush_bytes = bytes;
    return C3_OK;
}

c3_status run_concurrent(const c3_gemm_args* g, const c3_copy_args* c, const c3_conc_opts* o_in,
                         c3_timing* t_out) {
    c3_conc_opts o{};
    if (o_in) o = *o_in;
    if (o.use_priority)
        return fail(C3_E_UNSUPPORTED,
                    "stream priorities are not used: every stream stays at default priority; "
                    "prioritize with comm_first (issue order)");
    if (!g && !c) return fail(C3_E_INVALID, "c3_run_concurrent: neither a GEMM nor a copy given");

    // ---- validation and planning (may allocate; all before the clock starts) ----
    GemmPlan plan;
    hipStream_t gs = nullptr, cs = nullptr;
    if (g) {
        C3_TRY(stream_for_role(0, o.gemm_cu_mask, &gs));
        C3_TRY(gemm_plan(g->A, g->B, g->C, g->M, g->N, g->K, gs, &plan));
    }
    CommPlan cp;
    const std::vector<Segment>& segs = cp.segs;
    MoverSplit split;
    c3_move_opts mo{};
    if (c) {
        C3_TRY(comm_plan(*c, &cp));
        mo = c->opts;
        C3_TRY(split_movers(c->mover, mo, cp.segs, &split));
    }
    // the communication stream carries the reduce-scatter and the CUs' share of the copy
    const bool need_cs = c && (split.use_cu || cp.has_reduce);
    if (need_cs) C3_TRY(stream_for_role(1, o.comm_cu_mask, &cs));
    if (c && g) {
        const size_t a_b = (size_t)g->M * g->K * 2, b_b = (size_t)g->K * g->N * 2,
                     c_b = (size_t)g->M * g->N * 2;
        auto clash = [&](const void* src, const void* dst, size_t n) {
            return ranges_overlap(dst, n, g->A, a_b) || ranges_overlap(dst, n, g->B, b_b) ||
                   ranges_overlap(dst, n, g->C, c_b) || ranges_overlap(src, n, g->C, c_b);
        };
        for (const Segment& s : segs)
            if (clash(s.src, s.dst, s.bytes))
                return fail(C3_E_OVERLAP, "copy buffers overlap the GEMM's operands");
        if (cp.has_reduce) {
            const size_t n = cp.reduce.elems * 2;
            for (int r = 0; r < cp.reduce.world; ++r)
                if (clash(cp.reduce.in[r], cp.reduce.out, n))
                    return fail(C3_E_OVERLAP, "reduce-scatter buffers overlap the GEMM's operands");
        }
    }
    C3_TRY(ensure_events());
    Events& ev = events();

    // ---- idle device, optional last-level-cache flush ----
    C3_HIP_TRY(hipDeviceSynchronize());
    if (o.flush_bytes) {
        C3_TRY(ensure_flush_buffer((size_t)o.flush_bytes));
        C3_TRY(flush_enqueue(ctx().flush_buf, (size_t)o.flush_bytes, gs ? gs : cs));
        C3_HIP_TRY(hipDeviceSynchronize());
    }

    // ---- issue ----
    SdmaOp op;
    c3_status gemm_st = C3_OK, copy_st = C3_OK;
    bool gemm_issued = false;
    bool stream_issued = false;  // c0 .. c1 recorded on the communication stream
    bool reduce_issued = false;
    bool sdma_issued = false;
    // the engines' share of an all-reduce waits for the reduce-scatter (host-observed)
    bool sdma_pending = false;
    auto issue_gemm = [&]() {
        if (hipEventRecord(ev.g0, gs) != hipSuccess) {
            gemm_st = fail(C3_E_HIP, "hipEventRecord failed");
            return;
        }
        gemm_st = gemm_enqueue(plan, gs);
        if (gemm_st == C3_OK && hipEventRecord(ev.g1, gs) != hipSuccess)
            gemm_st = fail(C3_E_HIP, "hipEventRecord failed");
        gemm_issued = gemm_st == C3_OK;
    };
    auto issue_copy = [&]() {
        // with nothing to wait for, the engines go first: their host-side issue is the slower.
        // Communication first, beside a GEMM: every engine gets its first transfer before the
        // GEMM is launched and the rest right after it (handing 64 transfers to the engines
        // takes the host about 60 us, which the GEMM launch would otherwise wait behind).
        if (split.use_dma && !cp.has_reduce) {
            copy_st = sdma_issue(split.dma, mo, &op, /*first_round_only=*/o.comm_first && g);
            if (copy_st != C3_OK) return;
            sdma_issued = true;
        }
        if (need_cs) {
            if (hipEventRecord(ev.c0, cs) != hipSuccess) {
                copy_st = fail(C3_E_HIP, "hipEventRecord failed");
                return;
            }
            if (cp.has_reduce) {
                copy_st = reduce_enqueue(cp.reduce, cs);
                if (copy_st == C3_OK && hipEventRecord(ev.r1, cs) != hipSuccess)
                    copy_st = fail(C3_E_HIP, "hipEventRecord failed");
                if (copy_st != C3_OK) return;
                reduce_issued = true;
            }
            if (split.use_cu) {
                copy_st = copy_cu_enqueue(split.cu, mo, cs);
                if (copy_st != C3_OK) return;
            }
            if (hipEventRecord(ev.c1, cs) != hipSuccess) {
                copy_st = fail(C3_E_HIP, "hipEventRecord failed");
                return;
            }
            stream_issued = true;
        }
        if (split.use_dma && cp.has_reduce) sdma_pending = true;  // issued from the polling loop
    };

    const int64_t t0 = now_ns();
    if (c && o.comm_first) issue_copy();
    if (g) issue_gemm();
    if (sdma_issued && copy_st == C3_OK && op.next < op.chunks.size()) copy_st = sdma_issue_rest(&op);
    if (c && !o.comm_first) issue_copy();
    const int64_t t_issue = now_ns() - t0;

    // ---- poll for completion: the copy is complete when the communication stream's end event
    // and every engine transfer are ----
    bool gdone = !gemm_issued;
    bool cu_done = !stream_issued, dma_done = !(sdma_issued || sdma_pending);
    bool reduce_seen = !reduce_issued;
    if (copy_st != C3_OK) {
        // a launch failed part way: nothing more is issued; what was is drained below
        cu_done = dma_done = reduce_seen = true;
        sdma_pending = false;
    }
    bool cdone = cu_done && dma_done;
    int64_t tg = 0, tc = 0, tr = 0;
    while (!(gdone && cdone)) {
        if (!gdone) {
            const hipError_t e = hipEventQuery(ev.g1);
            if (e == hipSuccess) {
                gdone = true;
                tg = now_ns() - t0;
            } else if (e != hipErrorNotReady) {
                gemm_st = fail(C3_E_HIP, "GEMM completion query failed: %s", hipGetErrorString(e));
                gdone = true;
            }
        }
        if (!reduce_seen) {
            const hipError_t e = hipEventQuery(ev.r1);
            if (e == hipSuccess) {
                reduce_seen = true;
                tr = now_ns() - t0;
                if (sdma_pending) {
                    // all-gather on the engines: issued once the reduced chunk exists
                    sdma_pending = false;
                    copy_st = sdma_issue(split.dma, mo, &op);
                    if (copy_st == C3_OK) sdma_issued = true;
                    else dma_done = true;
                }
            } else if (e != hipErrorNotReady) {
                copy_st = fail(C3_E_HIP, "reduce-scatter completion query failed: %s",
                               hipGetErrorString(e));
                reduce_seen = true;
                if (sdma_pending) {
                    sdma_pending = false;
                    dma_done = true;
                }
            }
        }
        if (!cu_done) {
            const hipError_t e = hipEventQuery(ev.c1);
            if (e == hipSuccess) {
                cu_done = true;
            } else if (e != hipErrorNotReady) {
                copy_st = fail(C3_E_HIP, "copy completion query failed: %s", hipGetErrorString(e));
                cu_done = true;
            }
        }
        if (!dma_done && !sdma_pending) {
            if (sdma_done(op)) dma_done = true;
            else if (now_ns() > op.deadline_ns) dma_done = true;  // sdma_finish reports the timeout
        }
        if (!cdone && cu_done && dma_done) {
            cdone = true;
            tc = now_ns() - t0;
        }
    }
    const int64_t t1 = now_ns();

    c3_timing t{};
    if (sdma_issued) {
        const c3_status st = sdma_finish(&op, &t);
        if (st != C3_OK) copy_st = st;
    }
    // Make sure nothing is still running before returning (errors included).
    if (gemm_issued) (void)hipEventSynchronize(ev.g1);
    if (cs) (void)hipStreamSynchronize(cs);
    if (reduce_issued) {
        if (!tr) tr = now_ns() - t0;  // first observed here (the copy finished before a poll saw it)
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, ev.c0, ev.r1) == hipSuccess) t.reduce_gpu_ms = ms;
        t.t_reduce_done_ns = tr;
    }

    t.t_conc_ns = t1 - t0;
    t.t_gemm_done_ns = tg;
    t.t_copy_done_ns = tc;
    t.t_issue_ns = t_issue;
    t.applied_priority = 0;
    t.comm_issued_first = (c && o.comm_first) ? 1 : 0;
    if (g) {
        const auto m = normalise(o.gemm_cu_mask, C3_MAX_MASK_WORDS);
        std::copy(m.begin(), m.end(), t.gemm_applied_mask);
    }
    if (need_cs) {
        const auto m = normalise(o.comm_cu_mask, C3_MAX_MASK_WORDS);
        std::copy(m.begin(), m.end(), t.comm_applied_mask);
    }
    if (gemm_issued) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, ev.g0, ev.g1) == hipSuccess) t.gemm_gpu_ms = ms;
    }
    if (stream_issued) {
        // the stream's span covers the reduce-scatter and the CUs' share; the engines' span
        // (from their own timestamps) covers only their transfers, so an all-reduce adds the
        // reduce-scatter's kernel time to it
        float ms = 0.f;
        const double stream_ms = hipEventElapsedTime(&ms, ev.c0, ev.c1) == hipSuccess ? ms : 0.0;
        if (sdma_issued) {
            const double dma_ms = t.copy_gpu_ms + (cp.has_reduce ? t.reduce_gpu_ms : 0.0);
            t.copy_gpu_ms = std::max(stream_ms, dma_ms);
            if (split.use_cu) t.n_chunks += (int32_t)split.cu.size();
        } else {
            t.copy_gpu_ms = stream_ms;
            t.n_chunks = (int32_t)split.cu.size();
        }
    }
    if (t_out) *t_out = t;
    if (gemm_st != C3_OK) return gemm_st;
    if (copy_st != C3_OK) return copy_st;
    C3_HIP_TRY(hipGetLastError());
    return C3_OK;
}

}  // namespace c3
