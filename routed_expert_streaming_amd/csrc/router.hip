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
//  * small T (decode, T <= 32): one wavefront per (expert, H slice) streams
//    that piece of the router row once for every token, then one wavefront per
//    token sums the slices in order and runs the top-k;
//  * large T (prefill): 64x64 register-tiled fp64 product through LDS, then a
//    top-k kernel with one wavefront per token.
#include "common.h"
#include "router.h"
#include "topk.h"

namespace {

using moe::kTopkMaxK;
constexpr int kMaxE = moe::kTopkMaxE;
constexpr int kPer = moe::kTopkPer;

// One wavefront: top-k of the codes in registers, softmax, write slot i from lane i.
template <int PER>
__device__ __forceinline__ void wave_topk_write(uint32_t (&ord)[PER], int k, int32_t *idx_out, float *w_out) {
    float slot_logit;
    int slot_index;
    moe::topk_select(ord, k, slot_logit, slot_index);
    const float w = moe::topk_softmax(slot_logit, k);
    const int lane = threadIdx.x & 63;
    if (lane < k) {
        idx_out[lane] = slot_index;
        w_out[lane] = w;
    }
}

// ---------------------------------------------------------------- small T
// Kernel 1: one wavefront per (expert, 1024-column slice of H): 16 router
// weights per lane loaded at once, fp64 products, a fixed butterfly, and the
// slice's partial sum written per token.  Kernel 2: one wavefront per token adds
// the partials of each logit in slice order plus the bias, rounds once to fp32
// and runs the top-k.  (A single kernel with a last-workgroup ticket would need
// an agent-scope fence per workgroup, which costs more than the second launch.)
using moe::kSlice;
using moe::kMaxSlices;
constexpr int kSmallT = 32;

template <int TMAX>
__global__ __launch_bounds__(256) void router_partial_kernel(const uint16_t *__restrict__ x, int T, int H,
                                                             const float *__restrict__ wr, int E,
                                                             double *__restrict__ partial) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nslices = (H + kSlice - 1) / kSlice;
    const int item = blockIdx.x * 4 + wave;  // (expert, slice)
    const int e = item / nslices, sl = item - e * nslices;
    if (e >= E) return;
    const int h0 = sl * kSlice;
    const float *row = wr + (size_t)e * H;
    float4 wv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int h = h0 + lane * 4 + 256 * j;
        wv[j] = (h < H) ? *reinterpret_cast<const float4 *>(row + h) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t < T) {
            double a = 0.0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int h = h0 + lane * 4 + 256 * j;
                if (h < H) {
                    const uint2 xv = *reinterpret_cast<const uint2 *>(x + (size_t)t * H + h);
                    a += (double)bf16_bits_to_f32(xv.x & 0xFFFFu) * (double)wv[j].x;
                    a += (double)bf16_bits_to_f32(xv.x >> 16) * (double)wv[j].y;
                    a += (double)bf16_bits_to_f32(xv.y & 0xFFFFu) * (double)wv[j].z;
                    a += (double)bf16_bits_to_f32(xv.y >> 16) * (double)wv[j].w;
                }
            }
            a = wave_sum_f64(a);
            if (lane == 0) partial[((size_t)t * E + e) * kMaxSlices + sl] = a;
        }
    }
}

template <int PER>
__global__ __launch_bounds__(256) void router_finalize_kernel(const double *__restrict__ partial, int T, int H,
                                                              const float *__restrict__ bias, int E, int k,
                                                              float *__restrict__ logits, int32_t *__restrict__ idx,
                                                              float *__restrict__ w) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int nslices = (H + kSlice - 1) / kSlice;
    uint32_t ord[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = lane + 64 * j;
        ord[j] = 0u;
        if (e < E) {
            const float l = moe::router_logit(partial + (size_t)t * E * kMaxSlices, nslices, bias, e);
            logits[(size_t)t * E + e] = l;  // kept for inspection; the top-k reads registers
            ord[j] = moe::topk_ord(l);
        }
    }
    wave_topk_write(ord, k, idx + (size_t)t * k, w + (size_t)t * k);
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
    const int lane = threadIdx.x & 63;
    uint32_t ord[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int e = lane + 64 * j;
        ord[j] = (e < E) ? moe::topk_ord(logits[(size_t)t * E + e]) : 0u;
    }
    wave_topk_write(ord, k, idx + (size_t)t * k, w + (size_t)t * k);
}

constexpr size_t kHeaderBytes = 256;  // reserved header before the logits

}  // namespace

namespace moe {

float *router_logits(void *workspace) { return (float *)((char *)workspace + kHeaderBytes); }

double *router_partials_buf(void *workspace, int T, int E) {
    return (double *)((char *)workspace + kHeaderBytes + align_up((size_t)T * (size_t)E * sizeof(float), 256));
}

int router_partials(const uint16_t *x, int T, int H, const float *w_router, int E, double *partial, hipStream_t s) {
    const int nslices = (H + kSlice - 1) / kSlice;
    const dim3 grid((E * nslices + 3) / 4), block(256);
    if (T == 1)
        hipLaunchKernelGGL(router_partial_kernel<1>, grid, block, 0, s, x, T, H, w_router, E, partial);
    else if (T <= 4)
        hipLaunchKernelGGL(router_partial_kernel<4>, grid, block, 0, s, x, T, H, w_router, E, partial);
    else if (T <= 8)
        hipLaunchKernelGGL(router_partial_kernel<8>, grid, block, 0, s, x, T, H, w_router, E, partial);
    else
        hipLaunchKernelGGL(router_partial_kernel<32>, grid, block, 0, s, x, T, H, w_router, E, partial);
    MOE_LAUNCH_CHECK("router_partial_kernel");
    return MOE_OK;
}

}  // namespace moe

extern "C" size_t moe_router_workspace_bytes(int T, int E) {
    if (T < 0 || E <= 0) return 0;
    const size_t logits = moe::align_up((size_t)T * (size_t)E * sizeof(float), 256);
    const size_t partial = T <= kSmallT ? (size_t)T * (size_t)E * kMaxSlices * sizeof(double) : 0;
    return kHeaderBytes + logits + partial;
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
    if (H > kSlice * kMaxSlices) return moe::fail(MOE_E_SHAPE, "router: H=%d above %d", H, kSlice * kMaxSlices);
    hipStream_t s = (hipStream_t)stream;
    float *logits = moe::router_logits(workspace);
    double *partial = moe::router_partials_buf(workspace, T, E);
    const dim3 block(256);
    if (T <= kSmallT) {
        int rc = moe::router_partials(x, T, H, w_router, E, partial, s);
        if (rc != MOE_OK) return rc;
        const dim3 grid_f((T + 3) / 4);
        if (E <= 64)
            hipLaunchKernelGGL(router_finalize_kernel<1>, grid_f, block, 0, s, partial, T, H, bias, E, k, logits,
                               topk_idx, topk_w);
        else if (E <= 128)
            hipLaunchKernelGGL(router_finalize_kernel<2>, grid_f, block, 0, s, partial, T, H, bias, E, k, logits,
                               topk_idx, topk_w);
        else if (E <= 256)
            hipLaunchKernelGGL(router_finalize_kernel<4>, grid_f, block, 0, s, partial, T, H, bias, E, k, logits,
                               topk_idx, topk_w);
        else
            hipLaunchKernelGGL(router_finalize_kernel<kPer>, grid_f, block, 0, s, partial, T, H, bias, E, k, logits,
                               topk_idx, topk_w);
        MOE_LAUNCH_CHECK("router_finalize_kernel");
        return MOE_OK;
    }
    dim3 grid((T + kTT - 1) / kTT, (E + kTE - 1) / kTE);
    hipLaunchKernelGGL(router_tiled_kernel, grid, block, 0, s, x, T, H, w_router, bias, E, logits);
    MOE_LAUNCH_CHECK("router_tiled_kernel");
    hipLaunchKernelGGL(router_topk_kernel, dim3((T + 3) / 4), block, 0, s, logits, T, E, k, topk_idx, topk_w);
    MOE_LAUNCH_CHECK("router_topk_kernel");
    return MOE_OK;
}
