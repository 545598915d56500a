// moe_route_ffn_combine_noalloc: the one-call layer (router, gate/up + SwiGLU,
// down projection, weighted combine) with its workspace in a fixed device array
// of this library, for callers that cannot allocate device memory.
//
// `scratch` below is a file-scope __device__ array: every GPU the library runs
// on holds its own copy until the process ends.  In host code its name is only a
// host-side stand-in; the device address is taken once per device with
// hipGetSymbolAddress (on the first call with that device current) and passed
// to the kernels like any workspace pointer.
#include <mutex>

#include "common.h"
#include "ffn.h"

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;  // 16 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

// Device address of this device's scratch array (looked up once per device).
int scratch_ptr(void **out) {
    int dev = 0;
    MOE_TRY_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return moe::fail(MOE_E_STATE, "noalloc: device %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return moe::fail_hip(e, "hipGetSymbolAddress(scratch)");
        if (!p) return moe::fail(MOE_E_STATE, "noalloc: no scratch address on device %d", dev);
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace

extern "C" size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int moe_route_ffn_combine_noalloc(const uint16_t *x, int T, int H, int I, const float *w_router,
                                             const float *bias, int E, int k, const void *const *expert_table,
                                             const void *shared_slab, int32_t *topk_idx, float *topk_w, uint16_t *out,
                                             const void *prefetch, size_t prefetch_bytes, void *stream) {
    const char *who = "route_ffn_combine_noalloc";
    if (T < 0) return moe::fail(MOE_E_ARG, "%s: T=%d < 0", who, T);
    if (!prefetch && prefetch_bytes) return moe::fail(MOE_E_ARG, "%s: %zu prefetch bytes at NULL", who, prefetch_bytes);
    if (T == 0) return MOE_OK;
    if (H <= 0 || I <= 0 || E <= 0 || k <= 0)
        return moe::fail(MOE_E_SHAPE, "%s: H=%d I=%d E=%d k=%d", who, H, I, E, k);
    const size_t need = moe_route_ffn_combine_workspace_bytes(T, H, I, E, k, shared_slab != nullptr);
    if (need > kScratchBytes)
        return moe::fail(MOE_E_NOMEM, "%s: T=%d H=%d I=%d E=%d k=%d needs %zu bytes of workspace, more than the %zu of "
                         "the library's fixed scratch (use moe_route_ffn_combine with a workspace)",
                         who, T, H, I, E, k, need, kScratchBytes);
    void *ws = nullptr;
    const int rc = scratch_ptr(&ws);
    if (rc != MOE_OK) return rc;
    // the workspace contents don't matter to the kernels: nothing to clear
    return moe::route_ffn_combine_impl(x, T, H, I, w_router, bias, E, k, expert_table, shared_slab, topk_idx, topk_w,
                                       out, ws, kScratchBytes, prefetch, prefetch_bytes, false, stream);
}
