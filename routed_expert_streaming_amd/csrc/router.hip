// Router: fp64-accumulated logits rounded once to fp32, then a wavefront top-k
// (ties to the lower expert index) and the softmax over the selected k.
//
// Follows the LayerStoRm README ("TL;DR": the router tells which experts each
// token activates) and the glm-flash-lite page ("How it works": 8 experts per
// layer per token).  Each bf16 x fp32 product is exact in fp64 and the sum is
// rounded once, so the selected indices do not depend on summation order
// (up to fp64 rounding of the sum itself).
//
// Two logit kernels:
//  * small T (decode, T <= 32): one wavefront per expert streams that expert's
//    router row once for every token; the last workgroup to finish (atomic
//    ticket) runs the top-k for all tokens, so decode needs one launch;
//  * large T (prefill): 64x64 register-tiled fp64 product through LDS, then a
//    top-k kernel with one wavefront per token.
#include "common.h"

namespace {

constexpr int kTopkMaxK = 64;
constexpr int kMaxE = 1024;

// Order-preserving key: larger logit first, then lower index.  Key 0 never
// occurs for finite logits, so it marks taken/empty entries.
__device__ __forceinline__ unsigned long long topk_key(float l, int e) {
    if (l == 0.0f) l = 0.0f;  // -0 and +0 compare equal: same key
    uint32_t u = __float_as_uint(l);
    uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ float key_logit(unsigned long long key) {
    uint32_t ord = (uint32_t)(key >> 32);
    uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
    return __uint_as_float(u);
}

__device__ __forceinline__ int key_index(unsigned long long key) {
    return (int)(0xFFFFFFFFu - (uint32_t)key);
}

// One wavefront: top-k of one token's E logits, then the renormalised softmax.
__device__ void wave_topk(const float *lg, int E, int k, int32_t *idx_out, float *w_out) {
    const int lane = threadIdx.x & 63;
    constexpr int kPer = kMaxE / 64;
    unsigned long long keys[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        int e = lane + 64 * j;
        keys[j] = (e < E) ? topk_key(lg[e], e) : 0ull;
    }
    float my_logit = 0.0f;
    int my_index = 0;
    for (int i = 0; i < k; ++i) {
        unsigned long long best = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) best = keys[j] > best ? keys[j] : best;
        best = wave_max_u64(best);
        int e = key_index(best);
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (lane + 64 * j == e) keys[j] = 0ull;  // owner drops the winner
        if (lane == i) {
            my_logit = key_logit(best);
            my_index = e;
        }
    }
    // softmax over the k selected, max is slot 0
    float top = __shfl(my_logit, 0, 64);
    float ex = (lane < k) ? expf(my_logit - top) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
    if (lane < k) {
        idx_out[lane] = my_index;
        w_out[lane] = ex / sum;
    }
}

// ---------------------------------------------------------------- small T
template <int TMAX>
__global__ __launch_bounds__(256) void router_small_kernel(const uint16_t *__restrict__ x, int T, int H,
                                                           const float *__restrict__ wr,
                                                           const float *__restrict__ bias, int E, int k,
                                                           float *__restrict__ logits, unsigned *ticket,
                                                           int32_t *__restrict__ idx, float *__restrict__ w) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + wave;
    if (e < E) {
        double acc[TMAX];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) acc[t] = 0.0;
        const float *row = wr + (size_t)e * H;
        for (int h = lane * 4; h < H; h += 256) {
            float4 wv = *reinterpret_cast<const float4 *>(row + h);
#pragma unroll
            for (int t = 0; t < TMAX; ++t) {
                if (t < T) {
                    uint2 xv = *reinterpret_cast<const uint2 *>(x + (size_t)t * H + h);
                    double a = acc[t];
                    a += (double)bf16_bits_to_f32(xv.x & 0xFFFFu) * (double)wv.x;
                    a += (double)bf16_bits_to_f32(xv.x >> 16) * (double)wv.y;
                    a += (double)bf16_bits_to_f32(xv.y & 0xFFFFu) * (double)wv.z;
                    a += (double)bf16_bits_to_f32(xv.y >> 16) * (double)wv.w;
                    acc[t] = a;
                }
            }
        }
        const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t < T) {
                double s = wave_sum_f64(acc[t]);
                if (lane == 0) logits[(size_t)t * E + e] = (float)(s + b);
            }
        }
    }
    // Last workgroup to finish runs the top-k for every token.
    __shared__ unsigned s_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (atomicAdd(ticket, 1u) == gridDim.x - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int t = wave; t < T; t += 4) wave_topk(logits + (size_t)t * E, E, k, idx + (size_t)t * k, w + (size_t)t * k);
    if (threadIdx.x == 0) *ticket = 0u;  // ready for the next call
}

// ---------------------------------------------------------------- large T
constexpr int kTT = 64, kTE = 64, kTK = 16;

__global__ __launch_bounds__(256) void router_tiled_kernel(const uint16_t *__restrict__ x, int T, int H,
                                                           const float *__restrict__ wr,
                                                           const float *__restrict__ bias, int E,
                                                           float *__restrict__ logits) {
    __shared__ double xs[kTK][kTT];
    __shared__ double ws[kTK][kTE];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int t0 = blockIdx.x * kTT, e0 = blockIdx.y * kTE;
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    for (int k0 = 0; k0 < H; k0 += kTK) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int id = tid + 256 * r;
            int row = id >> 4, kk = id & 15;
            int t = t0 + row, e = e0 + row;
            xs[kk][row] = (t < T) ? (double)bf16_bits_to_f32(x[(size_t)t * H + k0 + kk]) : 0.0;
            ws[kk][row] = (e < E) ? (double)wr[(size_t)e * H + k0 + kk] : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kTK; ++kk) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int t = t0 + ty * 4 + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int e = e0 + tx * 4 + j;
            if (e < E) logits[(size_t)t * E + e] = (float)(acc[i][j] + (bias ? (double)bias[e] : 0.0));
        }
    }
}

__global__ __launch_bounds__(256) void router_topk_kernel(const float *__restrict__ logits, int T, int E, int k,
                                                          int32_t *__restrict__ idx, float *__restrict__ w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    wave_topk(logits + (size_t)t * E, E, k, idx + (size_t)t * k, w + (size_t)t * k);
}

constexpr size_t kTicketBytes = 256;

}  // namespace

extern "C" size_t moe_router_workspace_bytes(int T, int E) {
    if (T < 0 || E <= 0) return 0;
    return kTicketBytes + moe::align_up((size_t)T * (size_t)E * sizeof(float), 256);
}

extern "C" int moe_router_topk(const uint16_t *x, int T, int H, const float *w_router, const float *bias, int E,
                               int k, int32_t *topk_idx, float *topk_w, void *workspace, size_t workspace_bytes,
                               void *stream) {
    if (T < 0) return moe::fail(MOE_E_ARG, "router: T=%d < 0", T);
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !topk_idx || !topk_w || !workspace) return moe::fail(MOE_E_ARG, "router: NULL pointer");
    if (H <= 0 || H % 32 != 0) return moe::fail(MOE_E_SHAPE, "router: H=%d must be a positive multiple of 32", H);
    if (E <= 0 || E > kMaxE) return moe::fail(MOE_E_SHAPE, "router: E=%d outside 1..%d", E, kMaxE);
    if (k < 1 || k > E || k > kTopkMaxK) return moe::fail(MOE_E_SHAPE, "router: k=%d outside 1..min(E,64)", k);
    if (workspace_bytes < moe_router_workspace_bytes(T, E))
        return moe::fail(MOE_E_NOMEM, "router: workspace %zu < %zu bytes", workspace_bytes,
                         moe_router_workspace_bytes(T, E));
    hipStream_t s = (hipStream_t)stream;
    unsigned *ticket = (unsigned *)workspace;
    float *logits = (float *)((char *)workspace + kTicketBytes);
    const dim3 block(256);
    const dim3 grid_small((E + 3) / 4);
    if (T <= 32) {
        if (T == 1)
            hipLaunchKernelGGL(router_small_kernel<1>, grid_small, block, 0, s, x, T, H, w_router, bias, E, k, logits,
                               ticket, topk_idx, topk_w);
        else if (T <= 4)
            hipLaunchKernelGGL(router_small_kernel<4>, grid_small, block, 0, s, x, T, H, w_router, bias, E, k, logits,
                               ticket, topk_idx, topk_w);
        else if (T <= 8)
            hipLaunchKernelGGL(router_small_kernel<8>, grid_small, block, 0, s, x, T, H, w_router, bias, E, k, logits,
                               ticket, topk_idx, topk_w);
        else
            hipLaunchKernelGGL(router_small_kernel<32>, grid_small, block, 0, s, x, T, H, w_router, bias, E, k,
                               logits, ticket, topk_idx, topk_w);
        MOE_LAUNCH_CHECK("router_small_kernel");
        return MOE_OK;
    }
    dim3 grid((T + kTT - 1) / kTT, (E + kTE - 1) / kTE);
    hipLaunchKernelGGL(router_tiled_kernel, grid, block, 0, s, x, T, H, w_router, bias, E, logits);
    MOE_LAUNCH_CHECK("router_tiled_kernel");
    hipLaunchKernelGGL(router_topk_kernel, dim3((T + 3) / 4), block, 0, s, logits, T, E, k, topk_idx, topk_w);
    MOE_LAUNCH_CHECK("router_topk_kernel");
    return MOE_OK;
}
