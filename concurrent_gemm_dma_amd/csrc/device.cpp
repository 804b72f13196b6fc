// device.cpp -- library state, errors, device binding (HIP device <-> ROCr agent) and argument
// checks shared by the entry points.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "c3_internal.h"

namespace c3 {

namespace {
thread_local std::string g_last_error = "no error";
}

c3_status fail(c3_status st, const char* fmt, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

void clear_error() { g_last_error = "no error"; }

const char* last_error_text() { return g_last_error.c_str(); }

Context& ctx() {
    static Context c;
    return c;
}

std::recursive_mutex& api_mutex() {
    static std::recursive_mutex m;
    return m;
}

c3_status require_init() {
    if (!ctx().inited) return fail(C3_E_NOT_INIT, "c3_init has not been called (or failed)");
    return C3_OK;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!na || !nb) return false;
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

// The range [p, p + bytes) must lie inside one device allocation owned by our agent. This keeps
// every kernel and engine inside memory the caller really owns: a short buffer is rejected here
// instead of being overrun on the GPU.
c3_status check_device_ptr(const void* p, size_t bytes, const char* what) {
    if (!p) return fail(C3_E_INVALID, "%s is NULL", what);
    if (bytes == 0) return C3_OK;
    hsa_amd_pointer_info_t info;
    std::memset(&info, 0, sizeof info);
    info.size = sizeof info;
    const hsa_status_t s = hsa_amd_pointer_info(p, &info, nullptr, nullptr, nullptr);
    if (s != HSA_STATUS_SUCCESS) return fail(C3_E_HSA, "hsa_amd_pointer_info(%s) failed", what);
    if (info.type == HSA_EXT_POINTER_TYPE_UNKNOWN)
        return fail(C3_E_INVALID, "%s (%p) is not device memory known to the runtime", what, p);
    if (info.type == HSA_EXT_POINTER_TYPE_LOCKED)
        return fail(C3_E_INVALID, "%s (%p) is pinned host memory, not device memory", what, p);
    if (info.agentOwner.handle != ctx().agent.handle)
        return fail(C3_E_INVALID, "%s (%p) belongs to another device", what, p);
    const uintptr_t base = (uintptr_t)info.agentBaseAddress;
    const uintptr_t q = (uintptr_t)p;
    if (q < base || q + bytes > base + info.sizeInBytes || q + bytes < q)
        return fail(C3_E_INVALID,
                    "%s: %zu bytes at %p run past its allocation (%zu bytes at %p)", what, bytes, p,
                    (size_t)info.sizeInBytes, info.agentBaseAddress);
    return C3_OK;
}

c3_status init_device(int hip_device) {
    Context& c = ctx();
    if (c.inited) {
        if (c.device == hip_device) return C3_OK;
        return fail(C3_E_UNSUPPORTED, "already bound to device %d (asked for %d)", c.device,
                    hip_device);
    }
    int n = 0;
    C3_HIP_TRY(hipGetDeviceCount(&n));
    if (hip_device < 0 || hip_device >= n)
        return fail(C3_E_INVALID, "device %d out of range (%d devices)", hip_device, n);
    C3_HIP_TRY(hipSetDevice(hip_device));
    hipDeviceProp_t prop;
    C3_HIP_TRY(hipGetDeviceProperties(&prop, hip_device));

    // HIP has initialised ROCr already; this only takes a reference.
    C3_HSA_TRY(hsa_init());

    // The agent that owns a fresh allocation of this device is its ROCr agent.
    void* probe = nullptr;
    C3_HIP_TRY(hipMalloc(&probe, 4096));
    hsa_amd_pointer_info_t info;
    std::memset(&info, 0, sizeof info);
    info.size = sizeof info;
    const hsa_status_t ps = hsa_amd_pointer_info(probe, &info, nullptr, nullptr, nullptr);
    (void)hipFree(probe);
    if (ps != HSA_STATUS_SUCCESS || info.type == HSA_EXT_POINTER_TYPE_UNKNOWN)
        return fail(C3_E_HSA,
                    "could not map HIP device %d to a ROCr agent (is a second HIP/ROCr runtime "
                    "loaded in this process?)", hip_device);
    c.agent = info.agentOwner;

    c3_info& d = c.info;
    std::memset(&d, 0, sizeof d);
    d.hip_device = hip_device;
    d.n_cu = prop.multiProcessorCount;
    d.max_clock_mhz = prop.clockRate / 1000;
    d.lds_bytes_per_cu = (int32_t)prop.maxSharedMemoryPerMultiProcessor;
    d.l2_bytes = prop.l2CacheSize;
    d.hbm_bytes = prop.totalGlobalMem;
    std::snprintf(d.arch, sizeof d.arch, "%s", prop.gcnArchName);
    uint32_t v = 0;
    if (hsa_agent_get_info(c.agent, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_NUM_XCC, &v) ==
        HSA_STATUS_SUCCESS)
        d.n_xcc = (int32_t)v;
    if (d.n_xcc <= 0) d.n_xcc = 1;
    c.device = hip_device;
    C3_TRY(gemm_scratch_bind(hip_device));
    C3_TRY(sdma_discover());
    c.inited = true;
    return C3_OK;
}

void finalize_device() {
    Context& c = ctx();
    if (!c.inited) return;
    (void)hipDeviceSynchronize();
    release_streams();
    gemm_release_workspaces();
    if (c.flush_buf) (void)hipFree(c.flush_buf);
    c.flush_buf = nullptr;
    c.flush_bytes = 0;
    sdma_release();
    hsa_shut_down();
    c.inited = false;
    c.device = -1;
    c.sdma_engines.clear();
}

}  // namespace c3
