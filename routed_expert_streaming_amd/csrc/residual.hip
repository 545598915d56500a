// Residual stream between chained MoE layers: the step that connects layer l's
// output to layer l+1's input when the layers run as a chain (so that a layer's
// routing is only known once the layer before it has finished, the setting in
// which the next layer's experts are predicted and prefetched: LayerStoRm
// README, "Status and limitations", predictive expert prefetching; "References",
// gating lookahead behind the expert prefetch predictor).  The pages describe no
// block around the MoE layers; this is the plainest pre-norm residual block with
// the attention half left out and no learned norm weight:
//   resid[t,:] += out[t,:]                                (fp32)
//   x_next[t,:] = bf16( resid[t,:] / sqrt(mean_h resid[t,h]^2 + eps) )
// One workgroup per token row; the sum of squares is taken in a fixed order
// (per thread in index order, a butterfly per wave, then the waves in order), so
// results are reproducible run to run.  HBM-bound: it reads and writes the
// residual row once and writes the bf16 row.
#include "common.h"

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void residual_norm_kernel(const uint16_t *__restrict__ add,
                                                                  float *__restrict__ resid, int H, float eps,
                                                                  uint16_t *__restrict__ x_next) {
    const size_t row = (size_t)blockIdx.x * H;
    float *r = resid + row;
    uint16_t *xo = x_next + row;
    const int tid = threadIdx.x;
    float ss = 0.0f;
    for (int i = tid; i < H; i += kThreads) {
        float v = r[i];
        if (add) {
            v += bf16_bits_to_f32(add[row + i]);
            r[i] = v;
        }
        ss = fmaf(v, v, ss);
    }
    ss = group_sum<64>(ss);
    __shared__ float part[kThreads / 64];
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    float tot = part[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) tot += part[w];
    const float inv = 1.0f / sqrtf(tot / (float)H + eps);
    for (int i = tid; i < H; i += kThreads) xo[i] = (uint16_t)f32_to_bf16_bits(r[i] * inv);
}

}  // namespace

extern "C" int moe_residual_norm(const uint16_t *add, float *resid, int T, int H, float eps, uint16_t *x_next,
                                 void *stream) {
    if (T < 0 || H <= 0) return moe::fail(MOE_E_ARG, "residual_norm: T=%d, H=%d", T, H);
    if (!(eps >= 0.0f) || eps > 1.0f) return moe::fail(MOE_E_ARG, "residual_norm: eps=%g outside [0, 1]", (double)eps);
    if (T == 0) return MOE_OK;
    if (!resid || !x_next) return moe::fail(MOE_E_ARG, "residual_norm: NULL pointer");
    hipLaunchKernelGGL(residual_norm_kernel, dim3(T), dim3(kThreads), 0, (hipStream_t)stream, add, resid, H, eps,
                       x_next);
    MOE_LAUNCH_CHECK("residual_norm_kernel");
    return MOE_OK;
}
