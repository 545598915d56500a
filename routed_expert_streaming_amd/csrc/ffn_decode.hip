// Expert FFN kernels for decode (a few tokens, one kernel group per (token, slot)
// pair): the same fused 4-bit block dequant + dot2 arithmetic as the general
// GEMV kernels, organised for streaming bandwidth when every weight byte is read
// exactly once and the whole launch moves only tens of megabytes.
//
//  * Activations of all tokens are staged into LDS once per workgroup, so a
//    workgroup can then stream any number of weight rows.
//  * Each group of LPR lanes walks a contiguous run of "units" (one weight row
//    of one expert) and keeps D units of loads in flight in a register ring:
//    the loads of unit u+D are issued before unit u is computed.
//  * gate/up: units are (pair, row) over the concatenated pairs; h = silu(g)*u.
//  * down: units are (row, pair), pairs innermost, so one lane group owns all
//    pairs of an output row and can apply the weighted combine itself, in the
//    same order as the stand-alone combine kernel (slot 0..k-1, then shared).
//    No workgroup ever needs another workgroup's result.
#include <algorithm>

#include "common.h"
#include "dequant.h"
#include "ffn.h"

namespace {

// Build-time tuning knobs (defaults are the tuned values).
#ifndef MOE_DECODE_WG_PER_CU
#define MOE_DECODE_WG_PER_CU 2  // target workgroups per compute unit
#endif
#ifndef MOE_DECODE_D_GU
#define MOE_DECODE_D_GU 5  // gate/up units in flight per lane group (H = 4096)
#endif
#ifndef MOE_DECODE_D_DN
#define MOE_DECODE_D_DN 8  // down units in flight per lane group (I = 1536)
#endif

constexpr int kMaxTok = 4;      // tokens per launch on this path
constexpr int kMaxGroups = 64;  // T*k + 1



// Stage n activation rows (K columns, bf16) into LDS in dot2 pair order plus
// the fp32 block sums (same layout as the general kernels).
__device__ __forceinline__ void stage_all(const uint16_t *__restrict__ act, int K, int n, uint4 *X, float *S) {
    const int nblk = K >> 5;
    for (int id = threadIdx.x; id < n * nblk; id += blockDim.x) {
        const int m = id / nblk, b = id - m * nblk;
        const uint4 *src = reinterpret_cast<const uint4 *>(act + (size_t)m * K + 32 * b);
        uint4 d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = src[j];  // the whole block in one round trip
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint4 p;
            p.x = (d[j].x & 0xFFFFu) | (d[j].z << 16);
            p.y = (d[j].x >> 16) | (d[j].z & 0xFFFF0000u);
            p.z = (d[j].y & 0xFFFFu) | (d[j].w << 16);
            p.w = (d[j].y >> 16) | (d[j].w & 0xFFFF0000u);
            X[(m * 4 + j) * nblk + b] = p;
            const uint32_t v[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s += bf16_bits_to_f32(v[q] & 0xFFFFu);
                s += bf16_bits_to_f32(v[q] >> 16);
            }
        }
        S[m * nblk + b] = s;
    }
}

__device__ __forceinline__ void load_group_slabs(const moe::FfnArgs &a, const uint8_t **gslab, int G) {
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
        const uint8_t *p = nullptr;
        if (g < a.n_routed_groups) {
            const int e = a.topk_idx[g];
            if (!a.mask || a.mask[e]) p = (const uint8_t *)a.table[e];
        } else {
            p = (const uint8_t *)a.shared;
        }
        gslab[g] = p;
    }
}

// ---------------------------------------------------------------- gate/up
template <int LPR, int BPL, int D>
__global__ __launch_bounds__(256) void decode_gate_up_kernel(moe::FfnArgs a, int units_per_sg) {
    constexpr int RPW = 64 / LPR;
    const int H = a.H, I = a.I, T = a.T, nblk = H >> 5;
    const int G = a.n_routed_groups + (a.shared ? 1 : 0);
    const long long Q = (long long)G * I;
    extern __shared__ uint4 lds[];
    uint4 *X = lds;
    float *S = reinterpret_cast<float *>(lds + (size_t)T * 4 * nblk);
    __shared__ const uint8_t *gslab[kMaxGroups];
    load_group_slabs(a, gslab, G);
    __syncthreads();

    const uint32_t magic = moe_magic_vgpr();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPR, c = lane % LPR;
    const long long sg = ((long long)blockIdx.x * 4 + wave) * RPW + sub;
    const long long q0 = sg * units_per_sg;
    const int n = (int)max(0LL, min(q0 + units_per_sg, Q) - q0);  // units of this lane group
    const size_t m13 = (size_t)I * H * 5 / 8;
    const size_t cbytes = (size_t)I * H / 2;

    uint4 c0[D][BPL], c1[D][BPL];
    uint32_t p0[D][BPL], p1[D][BPL];
    // issue cursor (unit index, group, row) walks ahead of the compute cursor
    int ui = 0, gi = (int)(q0 / I), ri = (int)(q0 - (long long)gi * I);
    auto issue = [&](int j) {
        if (ui < n) {
            const uint8_t *slab = gslab[gi];
            if (slab) {
#pragma unroll
                for (int b = 0; b < BPL; ++b) {
                    const int blk = c + b * LPR;
                    c0[j][b] = load_stream_u4(slab + (size_t)ri * (H / 2) + 16 * blk);
                    p0[j][b] = load_stream_u32(slab + cbytes + ((size_t)ri * nblk + blk) * 4);
                    c1[j][b] = load_stream_u4(slab + m13 + (size_t)ri * (H / 2) + 16 * blk);
                    p1[j][b] = load_stream_u32(slab + m13 + cbytes + ((size_t)ri * nblk + blk) * 4);
                }
            }
        }
        ++ui;
        if (++ri == I) {
            ri = 0;
            ++gi;
        }
    };
#pragma unroll
    for (int j = 0; j < D; ++j) issue(j);
    stage_all(a.x, H, T, X, S);
    __syncthreads();

    int g = (int)(q0 / I), r = (int)(q0 - (long long)g * I);  // compute cursor
    for (int base = 0; base < n; base += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            if (base + j >= n) break;
            if (gslab[g]) {
                const bool routed = g < a.n_routed_groups;
                const int t_begin = routed ? g / a.k : 0, t_end = routed ? t_begin + 1 : T;
                for (int t = t_begin; t < t_end; ++t) {
                    float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
                    for (int b = 0; b < BPL; ++b) {
                        const int blk = c + b * LPR;
                        const uint4 *xb = X + (size_t)(t * 4) * nblk + blk;
                        const float Sb = S[t * nblk + blk];
                        v0 += moe_block_value(p0[j][b], moe_block_dot(c0[j][b], xb, nblk, magic), Sb);
                        v1 += moe_block_value(p1[j][b], moe_block_dot(c1[j][b], xb, nblk, magic), Sb);
                    }
                    v0 = moe_group_sum<LPR>(v0);
                    v1 = moe_group_sum<LPR>(v1);
                    if (moe_group_sum_owner<LPR>(c)) {
                        const int row = routed ? g : T * a.k + t;
                        a.h[(size_t)row * I + r] = (uint16_t)f32_to_bf16_bits(v0 / (1.0f + expf(-v0)) * v1);
                    }
                }
            }
            issue(j);  // slot j is free again: request the unit D ahead
            if (++r == I) {
                r = 0;
                ++g;
            }
        }
    }
}

// ---------------------------------------------------------------- down (+ combine)
template <int LPR, int BPL, int D, bool COMBINE>
__global__ __launch_bounds__(256) void decode_down_kernel(moe::FfnArgs a, const float *__restrict__ topk_w,
                                                          uint16_t *__restrict__ out, int rows_per_sg) {
    constexpr int RPW = 64 / LPR;
    const int H = a.H, I = a.I, T = a.T, k = a.k, nblk = I >> 5;
    const int G = a.n_routed_groups + (a.shared ? 1 : 0);
    const int P = T * k + (a.shared ? T : 0);
    extern __shared__ uint4 lds[];
    uint4 *X = lds;
    float *S = reinterpret_cast<float *>(lds + (size_t)P * 4 * nblk);
    __shared__ const uint8_t *gslab[kMaxGroups];
    __shared__ float wts[kMaxGroups];
    load_group_slabs(a, gslab, G);
    if (COMBINE)
        for (int i = threadIdx.x; i < T * k; i += blockDim.x) wts[i] = topk_w[i];
    __syncthreads();

    const uint32_t magic = moe_magic_vgpr();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPR, c = lane % LPR;
    const long long sg = ((long long)blockIdx.x * 4 + wave) * RPW + sub;
    const int r_first = (int)min<long long>(sg * rows_per_sg, H);
    const int r_last = (int)min<long long>((long long)r_first + rows_per_sg, H);
    const int n_units = (r_last - r_first) * G;  // (row, pair) units, pairs innermost
    const size_t m2 = 2 * ((size_t)I * H * 5 / 8);
    const size_t cbytes = (size_t)H * I / 2;

    uint4 cw[D][BPL];
    uint32_t pw[D][BPL];
    int ui = 0, ri = r_first, gi = 0;
    auto issue = [&](int j) {
        if (ui < n_units) {
            const uint8_t *slab = gslab[gi];
            if (slab) {
#pragma unroll
                for (int b = 0; b < BPL; ++b) {
                    const int blk = c + b * LPR;
                    cw[j][b] = load_stream_u4(slab + m2 + (size_t)ri * (I / 2) + 16 * blk);
                    pw[j][b] = load_stream_u32(slab + m2 + cbytes + ((size_t)ri * nblk + blk) * 4);
                }
            }
        }
        ++ui;
        if (++gi == G) {
            gi = 0;
            ++ri;
        }
    };
#pragma unroll
    for (int j = 0; j < D; ++j) issue(j);
    stage_all(a.h, I, P, X, S);
    __syncthreads();

    float acc[kMaxTok];
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) acc[t] = 0.0f;
    int rr = r_first, g = 0;
    for (int base = 0; base < n_units; base += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            if (base + j >= n_units) break;
            if (gslab[g]) {
                const bool routed = g < a.n_routed_groups;
                const int t_begin = routed ? g / k : 0, t_end = routed ? t_begin + 1 : T;
                for (int t = t_begin; t < t_end; ++t) {
                    const int hrow = routed ? g : T * k + t;
                    float v = 0.0f;
#pragma unroll
                    for (int b = 0; b < BPL; ++b) {
                        const int blk = c + b * LPR;
                        v += moe_block_value(pw[j][b],
                                             moe_block_dot(cw[j][b], X + (size_t)(hrow * 4) * nblk + blk, nblk, magic),
                                             S[hrow * nblk + blk]);
                    }
                    v = moe_group_sum<LPR>(v);
                    if (moe_group_sum_owner<LPR>(c)) {
                        if (COMBINE) {
#pragma unroll
                            for (int tt = 0; tt < kMaxTok; ++tt)
                                if (tt == t) acc[tt] = routed ? fmaf(wts[g], v, acc[tt]) : acc[tt] + v;
                        } else {
                            a.y[(size_t)hrow * H + rr] = v;
                        }
                    }
                }
            }
            issue(j);
            if (COMBINE && g == G - 1 && moe_group_sum_owner<LPR>(c)) {
#pragma unroll
                for (int tt = 0; tt < kMaxTok; ++tt) {
                    if (tt < T) out[(size_t)tt * H + rr] = (uint16_t)f32_to_bf16_bits(acc[tt]);
                    acc[tt] = 0.0f;
                }
            }
            if (++g == G) {
                g = 0;
                ++rr;
            }
        }
    }
}

int g_num_cus = 0;

int num_cus() {
    if (g_num_cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        g_num_cus = n;
    }
    return g_num_cus;
}

template <typename K>
int raise_lds(K kernel, size_t lds) {
    if (lds <= 64 * 1024) return MOE_OK;
    hipError_t e = hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return moe::fail_hip(e, "hipFuncSetAttribute(decode kernel)");
    return MOE_OK;
}

template <int LPR, int BPL, int D>
int launch_gate_up(const moe::FfnArgs &a, hipStream_t s) {
    constexpr int RPW = 64 / LPR;
    const int G = a.n_routed_groups + (a.shared ? 1 : 0);
    const long long Q = (long long)G * a.I;
    const long long target_sg = (long long)MOE_DECODE_WG_PER_CU * num_cus() * 4 * RPW;
    const int ups = (int)std::max<long long>(1, (Q + target_sg - 1) / target_sg);
    const long long nsg = (Q + ups - 1) / ups;
    const int grid = (int)((nsg + 4 * RPW - 1) / (4 * RPW));
    const size_t lds = (size_t)a.T * (a.H >> 5) * (4 * 16 + 4);
    int rc = raise_lds(decode_gate_up_kernel<LPR, BPL, D>, lds);
    if (rc != MOE_OK) return rc;
    hipLaunchKernelGGL((decode_gate_up_kernel<LPR, BPL, D>), dim3(grid), dim3(256), lds, s, a, ups);
    MOE_LAUNCH_CHECK("decode_gate_up_kernel");
    return MOE_OK;
}

template <int LPR, int BPL, int D>
int launch_down(const moe::FfnArgs &a, const float *topk_w, uint16_t *out, hipStream_t s) {
    constexpr int RPW = 64 / LPR;
    const long long target_sg = (long long)MOE_DECODE_WG_PER_CU * num_cus() * 4 * RPW;
    const int rps = (int)std::max<long long>(1, (a.H + target_sg - 1) / target_sg);
    const long long nsg = (a.H + rps - 1) / rps;
    const int grid = (int)((nsg + 4 * RPW - 1) / (4 * RPW));
    const int P = a.T * a.k + (a.shared ? a.T : 0);
    const size_t lds = (size_t)P * (a.I >> 5) * (4 * 16 + 4);
    if (out) {
        int rc = raise_lds(decode_down_kernel<LPR, BPL, D, true>, lds);
        if (rc != MOE_OK) return rc;
        hipLaunchKernelGGL((decode_down_kernel<LPR, BPL, D, true>), dim3(grid), dim3(256), lds, s, a, topk_w, out,
                           rps);
    } else {
        int rc = raise_lds(decode_down_kernel<LPR, BPL, D, false>, lds);
        if (rc != MOE_OK) return rc;
        hipLaunchKernelGGL((decode_down_kernel<LPR, BPL, D, false>), dim3(grid), dim3(256), lds, s, a, topk_w,
                           out, rps);
    }
    MOE_LAUNCH_CHECK("decode_down_kernel");
    return MOE_OK;
}

}  // namespace

namespace moe {

bool decode_supported(const FfnArgs &a) {
    if (a.grouped || a.T > kMaxTok) return false;
    const int G = a.n_routed_groups + (a.shared ? 1 : 0);
    const int P = a.T * a.k + (a.shared ? a.T : 0);
    if (G > kMaxGroups || P > 16) return false;
    const int nh = a.H >> 5, ni = a.I >> 5;
    const bool gu = nh == 128 || nh == 192 || nh == 8 || nh == 64;
    const bool dn = ni == 48 || ni == 64 || ni == 4 || ni == 128;
    return gu && dn;
}

int decode_gate_up(const FfnArgs &a, hipStream_t s) {
    switch (a.H >> 5) {
        case 128: return launch_gate_up<64, 2, MOE_DECODE_D_GU>(a, s);
        case 192: return launch_gate_up<64, 3, 3>(a, s);
        case 64: return launch_gate_up<64, 1, 6>(a, s);
        case 8: return launch_gate_up<8, 1, 4>(a, s);
        default: return fail(MOE_E_SHAPE, "decode gate/up: H=%d not supported", a.H);
    }
}

int decode_down(const FfnArgs &a, const float *topk_w, uint16_t *out, hipStream_t s) {
    switch (a.I >> 5) {
        case 48: return launch_down<16, 3, MOE_DECODE_D_DN>(a, topk_w, out, s);
        case 64: return launch_down<64, 1, 8>(a, topk_w, out, s);
        case 128: return launch_down<64, 2, 6>(a, topk_w, out, s);
        case 4: return launch_down<4, 1, 8>(a, topk_w, out, s);
        default: return fail(MOE_E_SHAPE, "decode down: I=%d not supported", a.I);
    }
}

}  // namespace moe
