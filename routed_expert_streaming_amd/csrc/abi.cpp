// Status codes, thread-local error state and format helpers of the C ABI.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>

#include "moe.h"
#include "dequant.h"

namespace {
thread_local int g_last_hip = 0;
thread_local char g_last_msg[512] = "";
}  // namespace

namespace moe {

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_msg, sizeof g_last_msg, fmt, ap);
    va_end(ap);
    return status;
}

int fail_hip(hipError_t err, const char *what) {
    g_last_hip = (int)err;
    snprintf(g_last_msg, sizeof g_last_msg, "%s failed: %s (%d)", what, hipGetErrorString(err), (int)err);
    return MOE_E_HIP;
}

}  // namespace moe

extern "C" const char *moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_E_ARG: return "invalid argument";
        case MOE_E_SHAPE: return "unsupported shape";
        case MOE_E_NOT_PINNED: return "host memory is not pinned";
        case MOE_E_NOMEM: return "workspace or pool too small";
        case MOE_E_CAPACITY: return "more experts requested than cache slots";
        case MOE_E_HIP: return "HIP runtime error";
        case MOE_E_STATE: return "invalid state";
        default: return "unknown status";
    }
}

extern "C" int moe_last_hip_error(void) { return g_last_hip; }

extern "C" const char *moe_last_error_message(void) { return g_last_msg; }

extern "C" int moe_version(void) { return 100; }

extern "C" size_t moe_expert_bytes_mx(int hidden, int inter) {
    if (hidden <= 0 || inter <= 0 || hidden % 32 || inter % 32) return 0;
    return (size_t)2 * inter * moe::mx_row_bytes(hidden) + (size_t)hidden * moe::mx_row_bytes(inter);
}

extern "C" size_t moe_expert_bytes_sb(int hidden, int inter) {
    if (hidden <= 0 || inter <= 0 || hidden % 256 || inter % 256) return 0;
    return (size_t)2 * inter * moe::sb_row_bytes(hidden) + (size_t)hidden * moe::sb_row_bytes(inter);
}

extern "C" size_t moe_expert_bytes(int hidden, int inter) {
    if (hidden <= 0 || inter <= 0 || hidden % 32 || inter % 32) return 0;
    // 2*inter gate/up rows of `hidden` columns and `hidden` down rows of `inter`
    // columns; a row holds K/2 code bytes and K/32 4-byte records, padded to 16
    // bytes (1.875 * hidden * inter when both are multiples of 128)
    return (size_t)2 * inter * moe::slab_row_bytes(hidden) + (size_t)hidden * moe::slab_row_bytes(inter);
}
