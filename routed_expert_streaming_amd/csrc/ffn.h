// Internal interface between the expert-FFN entry point and its kernel families.
#pragma once
#include "common.h"

namespace moe {

struct FfnArgs {
    const uint16_t *x;          // [T, H] bf16 activations
    int T, H, I, E, k;
    const int32_t *topk_idx;    // [T, k]
    const void *const *table;   // [E] slab pointers of this layer
    const void *shared;         // shared expert slab or nullptr
    const uint8_t *mask;        // [E] or nullptr
    int grouped;                // 0: one group per (token, slot) pair; 1: one group per expert
    int n_routed_groups;        // T*k (pairs) or E (grouped)
    const int32_t *count;       // [E]     (grouped)
    const int32_t *offset;      // [E + 1] (grouped)
    const int32_t *pair_of_row; // [T*k]   (grouped)
    uint16_t *h;                // [T*k + T*shared, I] bf16 SwiGLU output
    float *y;                   // [T*k + T*shared, H] fp32 expert outputs
    const uint8_t **pair_slab;  // [T*k + T*shared] or nullptr: slab of each pair (nullptr = masked),
                                // written by the one-token gate/up kernel, read by the down kernel
    int fmt;                    // expert weight format: 0 = fp16 scale/min blocks, 1 = MXFP4, 2 = super-blocks
    int min_m, max_m;           // grouped kernels skip groups with fewer / more tokens than these
    int compact;                // MFMA kernel: workgroups take the active groups in rank order (see the kernel)
    const uint8_t *prefetch;    // or nullptr: bytes the one-token down kernel reads into the device caches
    size_t prefetch_bytes;      // for the caller's next call (read and discarded, 1 KB per wave)
    const int32_t *act_scale;   // scaled MXFP4 MFMA kernels: E8M0 scale of each activation row (x or h),
                                // whose elements are then FP8 digit pairs (moe_quant_act_mx), not bf16
};

// Router finish fused into the one-token gate/up kernel: the per-slice fp64
// partial logits of the token and where to publish the routing.
struct RouteArgs {
    const double *partial;  // [E][kMaxSlices] partial logits of the token
    const float *bias;      // [E] or nullptr
    int E, nslices;
    float *logits;          // [E] fp32 logits (written by one wave of the kernel)
    int32_t *idx_out;       // [k] selected experts
    float *w_out;           // [k] their renormalised weights
};

// Gate/up + SwiGLU (x -> h) and down projection (h -> y) with the dequant-GEMV
// kernels.  max_m: largest number of tokens any group can have.
int ffn_gemv_gate_up(const FfnArgs &a, int max_m, hipStream_t s);
int ffn_gemv_down(const FfnArgs &a, int max_m, hipStream_t s);

// Decode kernels (pair grouping, few tokens): true if this shape is covered.
bool decode_supported(const FfnArgs &a);
int decode_gate_up(const FfnArgs &a, hipStream_t s);
// out == nullptr: write y; otherwise apply the weighted combine into out [T, H].
int decode_down(const FfnArgs &a, const float *topk_w, uint16_t *out, hipStream_t s);
// One token with the router finished inside gate/up (a.topk_idx unused; the
// down kernel must then read ra.idx_out / ra.w_out).
bool decode1_routed_supported(const FfnArgs &a, int E);
// True if decode_gate_up runs the one-token kernel, which fills a.pair_slab.
bool decode1_publishes_slabs(const FfnArgs &a);
int decode1_routed_gate_up(const FfnArgs &a, const RouteArgs &ra, hipStream_t s);

// MFMA grouped GEMM (prefill): needs the expert grouping and H, I multiples of 128.
bool mfma_supported(const FfnArgs &a);
int mfma_gate_up(const FfnArgs &a, hipStream_t s);
int mfma_down(const FfnArgs &a, hipStream_t s);
// MXFP4 on the block-scaled FP4 matrix cores: a.x (gate/up) or a.h (down) hold
// FP8 digit pairs from quant_act with their row scales in a.act_scale.
int mfma_gate_up_scaled(const FfnArgs &a, hipStream_t s);
int mfma_down_scaled(const FfnArgs &a, hipStream_t s);
// bf16 rows -> FP8 digit pairs (hi, lo) in the scaled kernels' A-operand order
// plus one E8M0 scale per row (in place allowed: out may equal x).
int quant_act(const uint16_t *x, int rows, int K, uint8_t *out, int32_t *scale, hipStream_t s);

// (token, slot) pairs the one-token down kernel combines (routed slots + shared).
constexpr int kDown1MaxPairs = 16;

// Tokens from which the automatic choice uses the MFMA kernels.
constexpr int kMfmaMinTokens = 128;
// Tokens of a group that one grouped-GEMV pass stages (LDS for the activations);
// larger groups go to the MFMA kernels when their shapes allow.
constexpr int kGemvOnePass = 4;

// moe_route_ffn_combine; fork = false runs the split path's two parts in order
// on `stream` (no helper stream, no events: nothing is allocated).
int route_ffn_combine_impl(const uint16_t *x, int T, int H, int I, const float *w_router, const float *bias, int E,
                           int k, const void *const *expert_table, const void *shared_slab, int32_t *topk_idx,
                           float *topk_w, uint16_t *out, void *workspace, size_t workspace_bytes,
                           const void *prefetch, size_t prefetch_bytes, bool fork, void *stream);

// Counting sort of pairs by expert (see moe_permute).
int permute_launch(const int32_t *topk_idx, int T, int k, int E, int32_t *count, int32_t *offset,
                   int32_t *pair_of_row, hipStream_t s);

}  // namespace moe
