// sdma.cpp -- the SDMA mover: a collective's local share moved by the GPU's system DMA engines,
// which use no compute units and bypass the L1/L2 caches ("Optimizing ML Concurrent Computation
// and Communication with GPU DMA Engines", Sections II-A and VI-A). As in the paper's ConCCL
// proof-of-concepts (Section VI-B), the collective is split into individual transfers and each
// transfer is put on an engine from the CPU with hsa_amd_memory_async_copy_on_engine.
//
// Design on gfx950:
// * Engines: for a copy from a GPU to itself the copy-engine status call may report no engine,
//   so the candidates are one engine id per SDMA engine the agent counts, and each candidate is
//   kept only if a probe copy on it completes byte-exact at initialisation. Chunk c goes to
//   engine list[c mod n] (round robin). By default every shard or block is one transfer, cut
//   into equal 256-byte-aligned pieces (of at least 128 KiB) until there are at least as many
//   transfers as engines: one engine moves only ~100 GB/s, so the 8 shards of an all-gather as
//   8 transfers would leave half of 16 engines idle. Pieces are also kept to at most 16 MiB.
//   The hybrid mover hands this path the engines' share of every segment.
// * force_copy_on_sdma = true on every call: for a same-device copy ROCr would otherwise use a
//   blit kernel, i.e. compute units, which would defeat the purpose.
// * One completion signal per chunk (initial value 1, decremented to 0 by the engine, negative
//   on error), drawn from a pool, so that per-chunk engine timestamps
//   (hsa_amd_profiling_get_async_copy_time) can be read back as evidence of overlap.
// * The host issues and returns; completion is polled (sdma_done) or waited for (sdma_finish)
//   with a deadline. A chunk that was really issued is always waited for before its signal is
//   reused or an error is returned, so no engine can still be writing after a call returns,
//   unless the engine itself hangs (then the signal is leaked, never reused).
#include <algorithm>
#include <chrono>
#include <cstdlib>
#include <cstring>

#include "c3_internal.h"

namespace c3 {
namespace {

std::vector<hsa_signal_t>& signal_pool() {
    static std::vector<hsa_signal_t> pool;
    return pool;
}

c3_status get_signal(hsa_signal_t* out) {
    auto& pool = signal_pool();
    if (!pool.empty()) {
        *out = pool.back();
        pool.pop_back();
        return C3_OK;
    }
    C3_HSA_TRY(hsa_signal_create(1, 0, nullptr, out));
    return C3_OK;
}

void put_signal(hsa_signal_t s) { signal_pool().push_back(s); }

uint64_t system_tick_hz() {
    static uint64_t hz = 0;
    if (!hz) {
        uint64_t f = 0;
        if (hsa_system_get_info(HSA_SYSTEM_INFO_TIMESTAMP_FREQUENCY, &f) == HSA_STATUS_SUCCESS && f)
            hz = f;
        else
            hz = 1000000000ull;
    }
    return hz;
}

bool profiling_on = false;

}  // namespace

c3_status sdma_discover() {
    Context& c = ctx();
    uint32_t n = 0;
    if (hsa_agent_get_info(c.agent, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_NUM_SDMA_ENG, &n) ==
        HSA_STATUS_SUCCESS)
        c.info.n_sdma = (int32_t)n;
    n = 0;
    if (hsa_agent_get_info(c.agent, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_NUM_SDMA_XGMI_ENG, &n) ==
        HSA_STATUS_SUCCESS)
        c.info.n_sdma_xgmi = (int32_t)n;
    uint32_t status_mask = 0;
    if (hsa_amd_memory_copy_engine_status(c.agent, c.agent, &status_mask) != HSA_STATUS_SUCCESS)
        status_mask = 0;
    c.info.sdma_status_mask = status_mask;
    uint32_t pref = 0;
    if (hsa_amd_memory_get_preferred_copy_engine(c.agent, c.agent, &pref) != HSA_STATUS_SUCCESS)
        pref = 0;
    c.info.sdma_preferred_mask = pref;
    profiling_on = hsa_amd_profiling_async_copy_enable(true) == HSA_STATUS_SUCCESS;

    // Candidates: what the status call reports for a device-local copy, else one engine id per
    // SDMA engine the agent counts (ids are one-hot bits), unless the environment overrides.
    uint32_t cand = status_mask;
    if (!cand) {
        const int total = std::min(16, c.info.n_sdma + c.info.n_sdma_xgmi);
        for (int b = 0; b < total; ++b) cand |= 1u << b;
    }
    if (const char* env = std::getenv("C3_SDMA_ENGINE_MASK"))
        if (*env) cand = (uint32_t)std::strtoul(env, nullptr, 0);
    c.sdma_engines.clear();
    c.info.sdma_engine_mask = 0;
    if (!cand) return C3_OK;

    // Probe each candidate with one byte-checked device-to-device copy.
    constexpr size_t kProbe = 256 * 1024;
    void* src = nullptr;
    void* dst = nullptr;
    C3_HIP_TRY(hipMalloc(&src, kProbe));
    c3_status st = C3_OK;
    std::vector<uint8_t> want(kProbe), got(kProbe);
    for (size_t i = 0; i < kProbe; ++i) want[i] = (uint8_t)((i * 131u + 7u) ^ (i >> 9));
    if (hipMalloc(&dst, kProbe) != hipSuccess ||
        hipMemcpy(src, want.data(), kProbe, hipMemcpyHostToDevice) != hipSuccess) {
        st = fail(C3_E_HIP, "SDMA probe: buffer set-up failed");
    }
    hsa_signal_t sig{};
    if (st == C3_OK && hsa_signal_create(1, 0, nullptr, &sig) != HSA_STATUS_SUCCESS)
        st = fail(C3_E_HSA, "SDMA probe: hsa_signal_create failed");
    for (int b = 0; st == C3_OK && b < 16; ++b) {
        const uint32_t engine = 1u << b;
        if (!(cand & engine)) continue;
        if (hipMemset(dst, 0, kProbe) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
            st = fail(C3_E_HIP, "SDMA probe: clearing the destination failed");
            break;
        }
        hsa_signal_store_screlease(sig, 1);
        if (hsa_amd_memory_async_copy_on_engine(dst, c.agent, src, c.agent, kProbe, 0, nullptr, sig,
                                                (hsa_amd_sdma_engine_id_t)engine,
                                                true) != HSA_STATUS_SUCCESS)
            continue;
        const int64_t deadline = now_ns() + 2000000000ll;
        hsa_signal_value_t v = hsa_signal_load_scacquire(sig);
        while (v >= 1 && now_ns() < deadline)
            v = hsa_signal_wait_scacquire(sig, HSA_SIGNAL_CONDITION_LT, 1,
                                          system_tick_hz() / 100, HSA_WAIT_STATE_ACTIVE);
        if (v >= 1) {
            // The engine never finished: it may still write dst and decrement the signal, so
            // neither is released (both are leaked on purpose) and initialisation fails.
            return fail(C3_E_TIMEOUT, "SDMA probe: engine 0x%x did not complete", engine);
        }
        if (v != 0) continue;
        if (hipMemcpy(got.data(), dst, kProbe, hipMemcpyDeviceToHost) != hipSuccess) {
            st = fail(C3_E_HIP, "SDMA probe: read-back failed");
            break;
        }
        if (std::memcmp(got.data(), want.data(), kProbe) == 0) {
            c.sdma_engines.push_back(engine);
            c.info.sdma_engine_mask |= engine;
        }
    }
    if (sig.handle) hsa_signal_destroy(sig);
    if (dst) (void)hipFree(dst);
    (void)hipFree(src);
    return st;
}

void sdma_release() {
    for (hsa_signal_t s : signal_pool()) hsa_signal_destroy(s);
    signal_pool().clear();
    if (profiling_on) hsa_amd_profiling_async_copy_enable(false);
    profiling_on = false;
}

namespace {

// Hand chunks op->next .. end-1 to ROCr, chunk i on engine engines[i mod n]. On an error the
// chunk that failed is marked complete and not issued; what was issued before it stays in the
// op for sdma_finish to drain.
c3_status issue_chunks(SdmaOp* op, size_t end) {
    Context& c = ctx();
    for (size_t& i = op->next; i < end; ++i) {
        hsa_signal_t sig;
        C3_TRY(get_signal(&sig));
        const uint32_t engine = op->engines[i % op->engines.size()];
        const Segment& ch = op->chunks[i];
        op->signals.push_back(sig);
        op->engine_of.push_back(engine);
        const bool faulted = op->fault_mode != C3_FAULT_NONE && (int)i == op->fault_chunk;
        if (faulted) {
            const hsa_signal_value_t v = op->fault_mode == C3_FAULT_DROP_CHUNK  ? 0
                                         : op->fault_mode == C3_FAULT_ERROR_CHUNK ? -1
                                                                                  : 1;
            hsa_signal_store_screlease(sig, v);
            op->issued.push_back(0);
            continue;
        }
        hsa_signal_store_screlease(sig, 1);
        const hsa_status_t hs = hsa_amd_memory_async_copy_on_engine(
            ch.dst, c.agent, ch.src, c.agent, ch.bytes, 0, nullptr, sig,
            (hsa_amd_sdma_engine_id_t)engine, true);
        if (hs != HSA_STATUS_SUCCESS) {
            // nothing was queued for this chunk: mark it complete
            hsa_signal_store_screlease(sig, 0);
            op->issued.push_back(0);
            const char* m = nullptr;
            hsa_status_string(hs, &m);
            const size_t failed = i++;
            return fail(C3_E_HSA, "hsa_amd_memory_async_copy_on_engine(chunk %zu, engine 0x%x, %llu B): %s",
                        failed, engine, (unsigned long long)ch.bytes, m ? m : "?");
        }
        op->issued.push_back(1);
        op->engines_used |= engine;
    }
    return C3_OK;
}

}  // namespace

c3_status sdma_issue(const std::vector<Segment>& segs, const c3_move_opts& o, SdmaOp* op,
                     bool first_round_only) {
    Context& c = ctx();
    std::vector<uint32_t> engines;
    for (uint32_t e : c.sdma_engines)
        if (o.engine_mask == 0 || (o.engine_mask & e)) engines.push_back(e);
    if (engines.empty())
        return fail(C3_E_NO_SDMA,
                    "no SDMA engine for device-local copies (available mask 0x%x, requested 0x%x)",
                    c.info.sdma_engine_mask, o.engine_mask);

    // Default split: one transfer per segment (shard or block), each cut into just enough
    // pieces that there are at least as many transfers as engines (one engine moves only
    // ~100 GB/s, so a gather of 8 shards would otherwise leave half of 16 engines idle).
    // Pieces stay at least 128 KiB: below that the host-side cost of one more transfer
    // outweighs the engine time it saves (1 MiB gather: 22 us as 8 transfers, 25 us as 16).
    constexpr uint64_t kMinPiece = 128 * 1024;
    // ...and at most 16 MiB: on some boxes a single transfer of 32 MiB or more ran at two thirds
    // of an engine's usual rate (1 GiB gather: 2.16 ms as 16 x 64 MiB, 1.48 ms as 64 x 16 MiB),
    // while 16 MiB pieces cost at most 2.4% where large ones are at full rate.
    constexpr uint64_t kMaxPiece = 16ull << 20;
    size_t nonempty = 0;
    for (const Segment& s : segs) nonempty += s.bytes != 0;
    const uint64_t pieces =
        nonempty ? std::max<uint64_t>(1, (engines.size() + nonempty - 1) / nonempty) : 1;
    const int timeout_ms = o.timeout_ms > 0 ? o.timeout_ms : 20000;

    *op = SdmaOp{};
    for (const Segment& s : segs) {
        if (s.bytes == 0) continue;
        uint64_t step = o.chunk_bytes;
        if (!step) {
            const uint64_t p = std::max<uint64_t>({1, std::min<uint64_t>(pieces, s.bytes / kMinPiece),
                                                    (s.bytes + kMaxPiece - 1) / kMaxPiece});
            step = (s.bytes + p - 1) / p;
            step = (step + 255) & ~uint64_t(255);  // 256-byte multiples keep pieces aligned
        }
        for (uint64_t off = 0; off < s.bytes; off += step)
            op->chunks.push_back({static_cast<const char*>(s.src) + off,
                                  static_cast<char*>(s.dst) + off, std::min(step, s.bytes - off)});
    }
    op->engines = std::move(engines);
    op->fault_mode = o.fault_mode;
    op->fault_chunk = o.fault_chunk;
    op->deadline_ns = now_ns() + (int64_t)timeout_ms * 1000000ll;
    op->signals.reserve(op->chunks.size());
    const size_t n = op->chunks.size();
    const c3_status st = issue_chunks(op, first_round_only ? std::min(n, op->engines.size()) : n);
    if (st != C3_OK) {
        // drain what was issued; the caller treats the op as never issued
        c3_timing ignore{};
        (void)sdma_finish(op, &ignore);
    }
    return st;
}

c3_status sdma_issue_rest(SdmaOp* op) { return issue_chunks(op, op->chunks.size()); }

bool sdma_done(const SdmaOp& op) {
    for (hsa_signal_t s : op.signals)
        if (hsa_signal_load_scacquire(s) >= 1) return false;
    return true;
}

c3_status sdma_finish(SdmaOp* op, c3_timing* t) {
    const size_t n = op->signals.size();
    bool hung = false;           // a really issued chunk did not finish in time
    bool stuck = false;          // a hook-held chunk never finished (expected for STUCK)
    int errored = -1;
    // really issued chunks first, so none is in flight when we give up on a held one
    for (int pass = 0; pass < 2; ++pass) {
        for (size_t i = 0; i < n; ++i) {
            if ((pass == 0) != (op->issued[i] == 1)) continue;
            hsa_signal_t s = op->signals[i];
            hsa_signal_value_t v = hsa_signal_load_scacquire(s);
            while (v >= 1) {
                const int64_t left = op->deadline_ns - now_ns();
                if (left <= 0) break;
                const uint64_t hint_ns = (uint64_t)std::min<int64_t>(left, 2000000);
                const uint64_t hint_ticks = hint_ns * system_tick_hz() / 1000000000ull;
                v = hsa_signal_wait_scacquire(s, HSA_SIGNAL_CONDITION_LT, 1, hint_ticks,
                                              HSA_WAIT_STATE_ACTIVE);
            }
            if (v >= 1) {
                if (op->issued[i]) hung = true;
                else stuck = true;
            } else if (v < 0 && errored < 0) {
                errored = (int)i;
            }
        }
    }

    // engine timestamps of the real chunks
    if (t) {
        t->n_chunks = (int32_t)n;
        t->engines_used = op->engines_used;
        if (profiling_on && !hung) {
            uint64_t first = UINT64_MAX, last = 0;
            for (size_t i = 0; i < n; ++i) {
                if (!op->issued[i]) continue;
                hsa_amd_profiling_async_copy_time_t ct{};
                if (hsa_amd_profiling_get_async_copy_time(op->signals[i], &ct) == HSA_STATUS_SUCCESS &&
                    ct.end >= ct.start && ct.start) {
                    first = std::min(first, ct.start);
                    last = std::max(last, ct.end);
                }
            }
            if (last > 0 && first != UINT64_MAX) {
                const double ns = (double)(last - first) * 1e9 / (double)system_tick_hz();
                t->copy_gpu_ms = ns * 1e-6;
                t->sdma_first_start_ns = 0;
                t->sdma_last_end_ns = (int64_t)ns;
            }
        }
    }

    // return signals: never recycle one an engine may still decrement
    for (size_t i = 0; i < n; ++i) {
        const hsa_signal_value_t v = hsa_signal_load_scacquire(op->signals[i]);
        if (v < 1 || !op->issued[i]) put_signal(op->signals[i]);
    }
    op->signals.clear();

    if (hung) return fail(C3_E_TIMEOUT, "SDMA copy did not complete before the deadline");
    if (errored >= 0)
        return fail(C3_E_HSA, "SDMA copy of chunk %d reported an error (negative completion signal)",
                    errored);
    if (stuck) return fail(C3_E_TIMEOUT, "SDMA chunk held by the test hook never completed");
    return C3_OK;
}

}  // namespace c3
