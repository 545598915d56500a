// Router pieces shared between the router entry point and the fused
// router + expert-FFN path: the per-slice fp64 partial logits and the rule that
// turns them into one fp32 logit.
#pragma once
#include "common.h"

namespace moe {

constexpr int kSlice = 1024;    // H columns per partial sum
constexpr int kMaxSlices = 16;  // H <= 16384

// Logit of expert e from its slice partials (token-major layout
// [T][E][kMaxSlices], already offset to the token): the partials are added in
// slice order, then the bias, in fp64, and the sum is rounded once to fp32.
__device__ __forceinline__ float router_logit(const double *partial_t, int nslices, const float *bias, int e) {
    const double *p = partial_t + (size_t)e * kMaxSlices;
    double s = 0.0;
    for (int i = 0; i < nslices; ++i) s += p[i];
    return (float)(s + (bias ? (double)bias[e] : 0.0));
}

// The same rule for nslices <= 4 with the partials already loaded.
__device__ __forceinline__ float router_logit4(const double (&q)[4], int nslices, float bias) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (i < nslices) s += q[i];
    return (float)(s + (double)bias);
}

// Workspace layout of the router: 256-byte header, fp32 logits [T][E], then the
// fp64 partials [T][E][kMaxSlices] (small T only).
float *router_logits(void *workspace);
double *router_partials_buf(void *workspace, int T, int E);

// Launch the partial-logit kernel for T <= 32 tokens; with layers > 1, layer l
// reads x + l*T*H and w_router + l*E*H and writes partial + l*ws_stride bytes.
int router_partials(const uint16_t *x, int T, int H, const float *w_router, int E, double *partial, hipStream_t s,
                    int layers = 1, size_t ws_stride = 0);

}  // namespace moe
