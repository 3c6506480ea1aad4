// C-ABI entry points that enqueue work: argument checks, then kernel launches.
// Every check happens before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "da2_internal.hpp"

namespace da2 {
hipError_t launch_prep(const Geo& g, const Layout& L, const void* q, const void* k, const void* v, void* ws,
                       hipStream_t stream);
hipError_t launch_draft(const Geo& g, const Layout& L, void* ws, hipStream_t stream);
hipError_t launch_set_labels(const Geo& g, const Layout& L, void* ws, const int8_t* labels, hipStream_t stream);
hipError_t launch_attention(const Geo& g, const Layout& L, const void* ws, void* out, int out_fp32,
                            hipStream_t stream);
}  // namespace da2

namespace {

da2_status check_ws(const da2_plan_t* plan, const void* ws, size_t bytes) {
    if (!ws) return DA2_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return DA2_ERR_WORKSPACE;
    if (bytes < plan->ws.total) return DA2_ERR_WORKSPACE;
    return DA2_OK;
}

// The HIP error behind the last DA2_ERR_HIP of this thread.
thread_local hipError_t g_last_hip = hipSuccess;

da2_status hip_fail(hipError_t e) {
    g_last_hip = e;
    return DA2_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// 16-byte vector loads/stores of rows need 8-element alignment of the strides.
bool strides_vectorizable(const da2::Geo& g) {
    return g.stride_n % 8 == 0 && g.stride_h % 8 == 0 && g.stride_b % 8 == 0;
}
bool out_strides_vectorizable(const da2::Geo& g) {
    return g.ostride_n % 8 == 0 && g.ostride_h % 8 == 0 && g.ostride_b % 8 == 0;
}

}  // namespace

extern "C" da2_status da2_prepare(const da2_plan_t* plan, const void* q, const void* k, const void* v,
                                  void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (!plan || !q || !k || !v) return DA2_ERR_INVALID_ARG;
    da2_status st = check_ws(plan, workspace, workspace_bytes);
    if (st != DA2_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !strides_vectorizable(plan->geo)) return DA2_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (hipError_t e = da2::launch_prep(plan->geo, plan->ws, q, k, v, workspace, s); e != hipSuccess)
        return hip_fail(e);
    if (hipError_t e = da2::launch_draft(plan->geo, plan->ws, workspace, s); e != hipSuccess) return hip_fail(e);
    return DA2_OK;
}

extern "C" da2_status da2_attention(const da2_plan_t* plan, const void* workspace, size_t workspace_bytes, void* out,
                                    void* hip_stream) {
    if (!plan || !out) return DA2_ERR_INVALID_ARG;
    da2_status st = check_ws(plan, workspace, workspace_bytes);
    if (st != DA2_OK) return st;
    if (!aligned16(out) || !out_strides_vectorizable(plan->geo)) return DA2_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const int out_fp32 = plan->cfg.out_dtype == DA2_OUT_FP32;
    if (hipError_t e = da2::launch_attention(plan->geo, plan->ws, workspace, out, out_fp32, s); e != hipSuccess)
        return hip_fail(e);
    return DA2_OK;
}

extern "C" da2_status da2_set_labels(const da2_plan_t* plan, void* workspace, size_t workspace_bytes,
                                     const int8_t* labels_dev, void* hip_stream) {
    if (!plan || !labels_dev) return DA2_ERR_INVALID_ARG;
    da2_status st = check_ws(plan, workspace, workspace_bytes);
    if (st != DA2_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (hipError_t e = da2::launch_set_labels(plan->geo, plan->ws, workspace, labels_dev, s); e != hipSuccess)
        return hip_fail(e);
    return DA2_OK;
}

extern "C" int da2_last_hip_error(const char** name) {
    if (name) *name = hipGetErrorName(g_last_hip);
    return static_cast<int>(g_last_hip);
}

// ---- the entry point that allocates nothing ----
// Its workspace is this file-scope device array (one copy per GPU, held
// until the process ends). In host code the name `scratch` is only a
// stand-in for the symbol, never a device address: host code uses the
// address hipGetSymbolAddress returns for the device, looked up once per
// device with that device current and kept in g_scratch.
namespace {

static __device__ __align__(256) __attribute__((used)) uint8_t scratch[DA2_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, null until looked up

// The device address of `scratch` on the device that runs `stream`.
da2_status scratch_address(hipStream_t stream, void** out) {
    int cur = -1;
    if (hipError_t e = hipGetDevice(&cur); e != hipSuccess) return hip_fail(e);
    int dev = cur;
    if (stream) {
        hipDevice_t d = 0;
        if (hipError_t e = hipStreamGetDevice(stream, &d); e != hipSuccess) return hip_fail(e);
        dev = static_cast<int>(d);
    }
    if (dev < 0 || dev >= kMaxDevices) return DA2_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        if (dev != cur)
            if (hipError_t e = hipSetDevice(dev); e != hipSuccess) return hip_fail(e);
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess && r != hipSuccess) return hip_fail(r);
        }
        if (e != hipSuccess) return hip_fail(e);
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return DA2_OK;
}

}  // namespace

extern "C" da2_status da2_forward_scratch(const da2_plan_t* plan, const void* q, const void* k, const void* v,
                                          void* out, void* hip_stream) {
    if (!plan || !q || !k || !v || !out) return DA2_ERR_INVALID_ARG;
    if (plan->ws.total > DA2_SCRATCH_BYTES) return DA2_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !strides_vectorizable(plan->geo) ||
        !out_strides_vectorizable(plan->geo))
        return DA2_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    void* ws = nullptr;
    if (da2_status st = scratch_address(s, &ws); st != DA2_OK) return st;
    // every byte of the workspace that a later kernel reads is written by an
    // earlier one in this call, so the array needs no clearing between calls
    if (hipError_t e = da2::launch_prep(plan->geo, plan->ws, q, k, v, ws, s); e != hipSuccess) return hip_fail(e);
    if (hipError_t e = da2::launch_draft(plan->geo, plan->ws, ws, s); e != hipSuccess) return hip_fail(e);
    const int out_fp32 = plan->cfg.out_dtype == DA2_OUT_FP32;
    if (hipError_t e = da2::launch_attention(plan->geo, plan->ws, ws, out, out_fp32, s); e != hipSuccess)
        return hip_fail(e);
    return DA2_OK;
}
