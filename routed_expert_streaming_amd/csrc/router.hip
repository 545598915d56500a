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
//  * large T (prefill): the product on the fp64 matrix cores (32 x 32 tiles),
//    then a top-k kernel with one wavefront per token.
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

// Both kernels take grid.y = layers: layer y reads x + y*T*H, the router rows
// + y*E*H and the bias + y*E, and writes its partials and logits in its own
// workspace slice (ws_stride bytes apart) and its top-k at + y*T*k.
template <int TMAX>
__global__ __launch_bounds__(256) void router_partial_kernel(const uint16_t *__restrict__ x, int T, int H,
                                                             const float *__restrict__ wr, int E,
                                                             double *__restrict__ partial, size_t ws_stride) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    x += (size_t)blockIdx.y * T * H;
    wr += (size_t)blockIdx.y * E * H;
    partial = (double *)((char *)partial + blockIdx.y * ws_stride);
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
                                                              float *__restrict__ w, size_t ws_stride) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    partial = (const double *)((const char *)partial + blockIdx.y * ws_stride);
    logits = (float *)((char *)logits + blockIdx.y * ws_stride);
    if (bias) bias += (size_t)blockIdx.y * E;
    idx += (size_t)blockIdx.y * T * k;
    w += (size_t)blockIdx.y * T * k;
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
// Prefill router on the fp64 matrix cores: logits[t][e] = sum_h x[t][h] Wr[e][h]
// + bias[e] with every product exact in fp64 (v_mfma_f64_16x16x4_f64), summed in
// fp64 and rounded once to fp32.  A workgroup owns 32 tokens x 32 experts; each
// wave one 16 x 16 tile.  K streams in chunks of 64 columns through two LDS
// buffers (x and Wr converted to fp64 on the way in, exact); the next chunk's
// loads are in flight in registers while the current one is multiplied.
// Lane layout of v_mfma_f64_16x16x4_f64 (checked on gfx950): lane l holds
// A[l%16][l/16], B[l/16][l%16], and C[4*j + l/16][l%16] for j < 4.
typedef double f64x4_t __attribute__((ext_vector_type(4)));
constexpr int kRT = 32, kRE = 32, kRK = 64, kRStride = kRK + 1;  // fp64 LDS rows padded by one

__global__ __launch_bounds__(256) void router_mfma_kernel(const uint16_t *__restrict__ x, int T, int H,
                                                          const float *__restrict__ wr,
                                                          const float *__restrict__ bias, int E,
                                                          float *__restrict__ logits) {
    __shared__ double xs[2][kRT * kRStride];
    __shared__ double ws[2][kRE * kRStride];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int t0 = blockIdx.x * kRT, e0 = blockIdx.y * kRE;
    const int nchunks = (H + kRK - 1) / kRK;
    // one chunk per thread: 8 bf16 of x (row tid/8, cols 8*(tid%8)..) and 8 fp32 of Wr
    const int lrow = tid >> 3, lcol = (tid & 7) * 8;
    uint4 xv, wv0, wv1;
    auto load = [&](int c) {
        const int k = c * kRK + lcol, t = t0 + lrow, e = e0 + lrow;
        xv = (t < T && k < H) ? *reinterpret_cast<const uint4 *>(x + (size_t)t * H + k) : make_uint4(0u, 0u, 0u, 0u);
        if (e < E && k < H) {
            wv0 = *reinterpret_cast<const uint4 *>(wr + (size_t)e * H + k);
            wv1 = *reinterpret_cast<const uint4 *>(wr + (size_t)e * H + k + 4);
        } else {
            wv0 = wv1 = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store = [&](int b) {
        double *xr = &xs[b][lrow * kRStride + lcol];
        double *wq = &ws[b][lrow * kRStride + lcol];
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            xr[2 * j] = (double)bf16_bits_to_f32(xw[j] & 0xFFFFu);
            xr[2 * j + 1] = (double)bf16_bits_to_f32(xw[j] >> 16);
        }
        const uint32_t ww[8] = {wv0.x, wv0.y, wv0.z, wv0.w, wv1.x, wv1.y, wv1.z, wv1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) wq[j] = (double)__uint_as_float(ww[j]);
    };
    f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
    load(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
        const int b = c & 1;
        if (c + 1 < nchunks) load(c + 1);
        const double *xa = &xs[b][(wm * 16 + (lane & 15)) * kRStride + (lane >> 4)];
        const double *wb = &ws[b][(wn * 16 + (lane & 15)) * kRStride + (lane >> 4)];
#pragma unroll
        for (int kk = 0; kk < kRK / 4; ++kk) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xa[4 * kk], wb[4 * kk], acc, 0, 0, 0);
        if (c + 1 < nchunks) store(b ^ 1);
        __syncthreads();
    }
    const int e = e0 + wn * 16 + (lane & 15);
    if (e < E) {
        const double bb = bias ? (double)bias[e] : 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = t0 + wm * 16 + 4 * j + (lane >> 4);
            if (t < T) logits[(size_t)t * E + e] = (float)(acc[j] + bb);
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

int router_partials(const uint16_t *x, int T, int H, const float *w_router, int E, double *partial, hipStream_t s,
                    int layers, size_t ws_stride) {
    const int nslices = (H + kSlice - 1) / kSlice;
    const dim3 grid((E * nslices + 3) / 4, layers), block(256);
    if (T == 1)
        hipLaunchKernelGGL(router_partial_kernel<1>, grid, block, 0, s, x, T, H, w_router, E, partial, ws_stride);
    else if (T <= 4)
        hipLaunchKernelGGL(router_partial_kernel<4>, grid, block, 0, s, x, T, H, w_router, E, partial, ws_stride);
    else if (T <= 8)
        hipLaunchKernelGGL(router_partial_kernel<8>, grid, block, 0, s, x, T, H, w_router, E, partial, ws_stride);
    else
        hipLaunchKernelGGL(router_partial_kernel<32>, grid, block, 0, s, x, T, H, w_router, E, partial, ws_stride);
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

extern "C" size_t moe_router_layers_workspace_bytes(int n_layers, int T, int E);

namespace {

// Bytes between the workspace slices of consecutive layers.
size_t layer_stride(int T, int E) { return moe::align_up(moe_router_workspace_bytes(T, E), 256); }

// Shared body of the single-layer and layer-batched entry points: `layers`
// independent routers, layer l using workspace slice l (ws_stride bytes apart).
int router_run(const uint16_t *x, int layers, int T, int H, const float *w_router, const float *bias, int E, int k,
               int32_t *topk_idx, float *topk_w, void *workspace, size_t workspace_bytes, void *stream,
               const char *who) {
    if (T < 0 || layers < 0) return moe::fail(MOE_E_ARG, "%s: T=%d, layers=%d must be >= 0", who, T, layers);
    if (T == 0 || layers == 0) return MOE_OK;
    if (!x || !w_router || !topk_idx || !topk_w || !workspace) return moe::fail(MOE_E_ARG, "%s: NULL pointer", who);
    if (H <= 0 || H % 32 != 0) return moe::fail(MOE_E_SHAPE, "%s: H=%d must be a positive multiple of 32", who, H);
    if (E <= 0 || E > kMaxE) return moe::fail(MOE_E_SHAPE, "%s: E=%d outside 1..%d", who, E, kMaxE);
    if (k < 1 || k > E || k > kTopkMaxK) return moe::fail(MOE_E_SHAPE, "%s: k=%d outside 1..min(E,64)", who, k);
    if (layers > 65535) return moe::fail(MOE_E_SHAPE, "%s: layers=%d above 65535", who, layers);
    const size_t per = layer_stride(T, E), need = moe_router_layers_workspace_bytes(layers, T, E);
    if (workspace_bytes < need) return moe::fail(MOE_E_NOMEM, "%s: workspace %zu < %zu bytes", who, workspace_bytes, need);
    if (H > kSlice * kMaxSlices) return moe::fail(MOE_E_SHAPE, "%s: H=%d above %d", who, H, kSlice * kMaxSlices);
    hipStream_t s = (hipStream_t)stream;
    const dim3 block(256);
    if (T <= kSmallT) {
        float *logits = moe::router_logits(workspace);
        double *partial = moe::router_partials_buf(workspace, T, E);
        int rc = moe::router_partials(x, T, H, w_router, E, partial, s, layers, per);
        if (rc != MOE_OK) return rc;
        const dim3 grid_f((T + 3) / 4, layers);
        if (E <= 64)
            hipLaunchKernelGGL(router_finalize_kernel<1>, grid_f, block, 0, s, partial, T, H, bias, E, k, logits,
                               topk_idx, topk_w, per);
        else if (E <= 128)
            hipLaunchKernelGGL(router_finalize_kernel<2>, grid_f, block, 0, s, partial, T, H, bias, E, k, logits,
                               topk_idx, topk_w, per);
        else if (E <= 256)
            hipLaunchKernelGGL(router_finalize_kernel<4>, grid_f, block, 0, s, partial, T, H, bias, E, k, logits,
                               topk_idx, topk_w, per);
        else
            hipLaunchKernelGGL(router_finalize_kernel<kPer>, grid_f, block, 0, s, partial, T, H, bias, E, k, logits,
                               topk_idx, topk_w, per);
        MOE_LAUNCH_CHECK("router_finalize_kernel");
        return MOE_OK;
    }
    for (int l = 0; l < layers; ++l) {
        const size_t xo = (size_t)l * T * H, wo = (size_t)l * E * H, io = (size_t)l * T * k;
        float *logits = moe::router_logits((char *)workspace + (size_t)l * per);
        dim3 grid((T + kRT - 1) / kRT, (E + kRE - 1) / kRE);
        hipLaunchKernelGGL(router_mfma_kernel, grid, block, 0, s, x + xo, T, H, w_router + wo,
                           bias ? bias + (size_t)l * E : nullptr, E, logits);
        MOE_LAUNCH_CHECK("router_mfma_kernel");
        hipLaunchKernelGGL(router_topk_kernel, dim3((T + 3) / 4), block, 0, s, logits, T, E, k, topk_idx + io,
                           topk_w + io);
        MOE_LAUNCH_CHECK("router_topk_kernel");
    }
    return MOE_OK;
}

}  // namespace

extern "C" int moe_router_topk(const uint16_t *x, int T, int H, const float *w_router, const float *bias, int E,
                               int k, int32_t *topk_idx, float *topk_w, void *workspace, size_t workspace_bytes,
                               void *stream) {
    return router_run(x, 1, T, H, w_router, bias, E, k, topk_idx, topk_w, workspace, workspace_bytes, stream,
                      "router");
}

extern "C" size_t moe_router_layers_workspace_bytes(int n_layers, int T, int E) {
    if (n_layers <= 0 || moe_router_workspace_bytes(T, E) == 0) return 0;
    return (size_t)(n_layers - 1) * layer_stride(T, E) + moe_router_workspace_bytes(T, E);
}

extern "C" int moe_router_topk_layers(const uint16_t *x, int n_layers, int T, int H, const float *w_router,
                                      const float *bias, int E, int k, int32_t *topk_idx, float *topk_w,
                                      void *workspace, size_t workspace_bytes, void *stream) {
    return router_run(x, n_layers, T, H, w_router, bias, E, k, topk_idx, topk_w, workspace, workspace_bytes, stream,
                      "router_layers");
}
