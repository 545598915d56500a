// Wavefront top-k over router logits and the softmax over the selected k,
// shared by the router kernels and the fused router + gate/up kernel so both
// select and weight experts identically.
//
// Selection order: larger fp32 logit first, ties to the lower expert index
// (-0 and +0 are equal).  Each logit is mapped to an order-preserving 32-bit
// code; the wave maximum of the codes is found with DPP row shifts and
// broadcasts, and the lowest index holding it with a ballot, so a selection
// round costs a few dozen instructions and no LDS traffic.
#pragma once
#include "common.h"

namespace moe {

constexpr int kTopkMaxK = 64;
constexpr int kTopkMaxE = 1024;
constexpr int kTopkPer = kTopkMaxE / 64;  // logits per lane at most

// order-preserving code of a logit; 0 never occurs for finite logits and marks
// empty or taken entries
__device__ __forceinline__ uint32_t topk_ord(float l) {
    if (l == 0.0f) l = 0.0f;  // -0 -> +0
    const uint32_t u = __float_as_uint(l);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float topk_logit(uint32_t ord) {
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// Wave-wide max of an unsigned value, returned in every lane (inclusive scans
// inside 16-lane rows, then row broadcasts; lane 63 ends with the total).
__device__ __forceinline__ uint32_t topk_wave_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k over codes held in registers (lane l holds experts l, l+64, ...; code 0
// = absent).  Afterwards lane i < k holds slot i: its logit and expert index;
// slots are in selection order.  All lanes must be active.
template <int PER>
__device__ __forceinline__ void topk_select(uint32_t (&ord)[PER], int k, float &slot_logit, int &slot_index) {
    const int lane = threadIdx.x & 63;
    slot_logit = 0.0f;
    slot_index = 0;
    for (int i = 0; i < k; ++i) {
        uint32_t best = 0;
        int best_j = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (ord[j] > best) {  // strict: the lower index wins a tie inside the lane
                best = ord[j];
                best_j = j;
            }
        const uint32_t top = topk_wave_max(best);
        // lowest index holding the maximum: lanes whose best sits in register j
        // hold indices 64j + lane, so the first j with a match, then its lowest lane
        uint32_t e = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const uint64_t m = __ballot(best == top && best_j == j);
            if (m) {
                e = 64u * j + (uint32_t)(__ffsll((long long)m) - 1);
                break;
            }
        }
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if ((uint32_t)(lane + 64 * j) == e) ord[j] = 0u;  // the owner drops the winner
        if (lane == i) {
            slot_logit = topk_logit(top);
            slot_index = (int)e;
        }
    }
}

// Renormalised softmax over the k selected logits (slot 0 holds the maximum);
// lane i < k returns the weight of slot i.
__device__ __forceinline__ float topk_softmax(float slot_logit, int k) {
    const int lane = threadIdx.x & 63;
    const float top = __shfl(slot_logit, 0, 64);
    const float ex = (lane < k) ? expf(slot_logit - top) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
    return ex / sum;
}

}  // namespace moe
