// Expert FFN for few tokens per expert (decode): fused 4-bit block dequant +
// GEMV, gate/up with SwiGLU in one kernel and the down projection in another.
//
// Method (LayerStoRm README "TL;DR": each token runs only the few experts the
// router picked; the expert weights are 4-bit block-quantised, README
// "Install": UD-Q4_K_XL weights): for each expert and each of its tokens
//   g = W1 x, u = W3 x, h = bf16(silu(g) * u), y = W2 h,
// W = scale * q + min per 32-column block.
//
// Kernel design (gfx950, wave64):
//  * Each lane owns whole 32-column blocks: one 16-byte code load (32 nibbles)
//    plus one 4-byte (scale, min) record per block, so a row is read with
//    fully used, coalesced 16 B/lane loads.  LPR lanes share a row (LPR = 64
//    for K = 4096/6144/2048, 16 for K = 1536), BPL blocks per lane.
//  * The activation row(s) of the expert's tokens are staged once per
//    workgroup in LDS, already permuted into the bf16 pairs the nibble
//    extraction produces, so the inner loop is: mask+or a nibble pair into a
//    bf16 pair (128 + q) and one v_dot2_f32_bf16 per two weights.  The block
//    result is scale*acc + (min - 128*scale) * sum(x_block), which equals
//    sum((scale*q + min) * x) exactly in real arithmetic.
//  * Partial sums of the LPR lanes of a row meet in a fixed butterfly, so the
//    output is reproducible run to run.
//  * The other weight formats use the same structure with their own block
//    terms, the ones the one-token kernels use: MXFP4 blocks through the scaled
//    FP4-to-bf16 convert (activations staged in column order, scale 2^(v-127)
//    applied to the block's fp32 sum), super-block headers turned into each
//    block's scale and min and then the format-0 identity.
#include <type_traits>

#include "common.h"
#include "dequant.h"
#include "ffn.h"

namespace {

constexpr int kMT = 4;  // tokens staged per pass
static_assert(kMT >= moe::kGemvOnePass, "a one-pass group must fit one staging pass");


struct Group {
    const uint8_t *slab;
    int M;
    int routed;  // group id within routed groups, or -1 for the shared expert
};

__device__ __forceinline__ Group resolve_group(const moe::FfnArgs &a, int g) {
    Group out{nullptr, 0, -1};
    if (g < a.n_routed_groups) {
        int e;
        int M;
        if (a.grouped) {
            e = g;
            M = a.count[e];
        } else {
            e = a.topk_idx[g];
            M = 1;
        }
        if (M == 0 || M < a.min_m || M > a.max_m || (a.mask && a.mask[e] == 0)) return out;
        out.slab = (const uint8_t *)a.table[e];
        out.M = M;
        out.routed = g;
    } else if (a.shared && a.T >= a.min_m && a.T <= a.max_m) {
        out.slab = (const uint8_t *)a.shared;
        out.M = a.T;
    }
    return out;
}

// Output row (in h / y) of the m-th token of a group.
__device__ __forceinline__ int group_row(const moe::FfnArgs &a, const Group &gr, int m) {
    if (gr.routed < 0) return a.T * a.k + m;
    if (a.grouped) return a.pair_of_row[a.offset[gr.routed] + m];
    return gr.routed;
}

// Stage mcount activation rows (bf16, K columns) into LDS:
//   X[(m*4 + j)*nblk + b] = the 8 values of word j of block b, as bf16 pairs
//                           (v0,v4), (v1,v5), (v2,v6), (v3,v7) -- for MXFP4
//                           (NATURAL) in column order (v0,v1) .. (v6,v7)
//   S[m*nblk + b]         = fp32 sum of the block's 32 values (in index order)
template <bool NATURAL>
__device__ __forceinline__ void stage_rows(const uint16_t *__restrict__ act, int K, const int *src_rows, int mcount,
                                           uint4 *X, float *S) {
    const int nblk = K >> 5;
    for (int id = threadIdx.x; id < mcount * nblk; id += blockDim.x) {
        const int m = id / nblk, b = id - m * nblk;
        const uint4 *src = reinterpret_cast<const uint4 *>(act + (size_t)src_rows[m] * K + 32 * b);
        uint4 d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = src[j];  // the whole block in one round trip
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint4 p = d[j];
            if constexpr (!NATURAL) {
                p.x = (d[j].x & 0xFFFFu) | (d[j].z << 16);
                p.y = (d[j].x >> 16) | (d[j].z & 0xFFFF0000u);
                p.z = (d[j].y & 0xFFFFu) | (d[j].w << 16);
                p.w = (d[j].y >> 16) | (d[j].w & 0xFFFF0000u);
            }
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

// One workgroup owns one group (expert) and `iters` row steps of ROWS_PER_STEP
// rows (RPW rows per wave per step): it stages the group's activation rows in
// LDS once per pass of up to mt_cap tokens and walks its steps with the weights
// of the next D steps in flight in registers (a ring of D slots, the loop
// unrolled by D so every slot is a fixed set of registers).  The weights of a
// row are dotted with every staged token before the slot is refilled.
// FMT: weight format -- 0: (fp16 scale, fp16 min) record per block; 1: MXFP4,
// one E8M0 scale byte per block; 2: super-blocks, one 16-byte header per 8
// blocks (each lane reads the header of each of its blocks).
#ifndef MOE_GEMV_WAVES_PER_EU
#define MOE_GEMV_WAVES_PER_EU 2
#endif
template <int BPL, bool GATEUP, int FMT>
struct GemvSlot {
    using Param = std::conditional_t<FMT == 2, uint4, uint32_t>;
    uint4 c0[BPL], c1[GATEUP ? BPL : 1];
    Param p0[BPL], p1[GATEUP ? BPL : 1];
};

// the block parameters of block blk of a row (codes at row, parameters at row + K/2)
template <int FMT>
__device__ __forceinline__ std::conditional_t<FMT == 2, uint4, uint32_t> load_param(const uint8_t *row, int K, int blk) {
    if constexpr (FMT == 2)
        return load_stream_u4(row + K / 2 + 16 * (blk >> 3));
    else if constexpr (FMT == 1)
        return load_stream_u8(row + K / 2 + blk);
    else
        return load_stream_u32(row + K / 2 + 4 * blk);
}

// sum over block blk of W * x for one staged token (xb: the block's first word, S: its sum)
template <int FMT>
__device__ __forceinline__ float block_term(const uint4 c, std::conditional_t<FMT == 2, uint4, uint32_t> p,
                                            const uint4 *xb, int stride, float S, int blk, uint32_t magic) {
    if constexpr (FMT == 1)
        return moe_mx_block_value(p, moe_mx_block_dot(c, xb, stride));
    else if constexpr (FMT == 2)
        return moe_sb_block_value(p, blk & 7, moe_block_dot(c, xb, stride, magic), S);
    else
        return moe_block_value(p, moe_block_dot(c, xb, stride, magic), S);
}

template <int LPR, int BPL, int D, bool GATEUP, int FMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MOE_GEMV_WAVES_PER_EU)))
void ffn_gemv_kernel(moe::FfnArgs a, int tiles, int mt_cap, int iters) {
    constexpr int RPW = 64 / LPR;              // rows per wave per step
    constexpr int ROWS_PER_STEP = 4 * RPW;     // rows per workgroup per step
    const int K = GATEUP ? a.H : a.I;
    const int R = GATEUP ? a.I : a.H;
    const int nblk = K >> 5;
    const int g = blockIdx.x / tiles, tile = blockIdx.x - g * tiles;
    const Group gr = resolve_group(a, g);
    if (gr.M == 0) return;
    const int row0 = tile * iters * ROWS_PER_STEP;
    if (row0 >= R) return;
    const int nsteps = min(iters, (R - row0 + ROWS_PER_STEP - 1) / ROWS_PER_STEP);

    // matrix rows: W1 and W3 (gate/up) or W2 (down); codes, then records at + K/2
    const moe::MatRows m0 = GATEUP ? moe::slab_w1<FMT>(gr.slab, a.H, a.I) : moe::slab_w2<FMT>(gr.slab, a.H, a.I);
    const moe::MatRows m1 = moe::slab_w3<FMT>(gr.slab, a.H, a.I);

    extern __shared__ uint4 lds[];
    uint4 *X = lds;
    float *S = reinterpret_cast<float *>(lds + (size_t)mt_cap * 4 * nblk);
    __shared__ int src_rows[kMT];
    __shared__ int out_rows[kMT];

    const uint32_t magic = moe_magic_vgpr();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPR, c = lane % LPR;
    const int rbase = row0 + wave * RPW + sub;  // this lane group's row in step 0

    // rows past R re-read row R-1 (valid memory) and are not stored
    auto load = [&](GemvSlot<BPL, GATEUP, FMT> &sl, int step) {
        const int r = min(rbase + step * ROWS_PER_STEP, R - 1);
        const uint8_t *row0 = m0.row0 + (size_t)r * m0.stride, *row1 = m1.row0 + (size_t)r * m1.stride;
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
            const int blk = min(c + b * LPR, nblk - 1);
            sl.c0[b] = load_stream_u4(row0 + 16 * blk);
            sl.p0[b] = load_param<FMT>(row0, K, blk);
            if constexpr (GATEUP) {
                sl.c1[b] = load_stream_u4(row1 + 16 * blk);
                sl.p1[b] = load_param<FMT>(row1, K, blk);
            }
        }
    };
    auto compute = [&](const GemvSlot<BPL, GATEUP, FMT> &sl, int step, int mcount) {
        const int r = rbase + step * ROWS_PER_STEP;
        for (int m = 0; m < mcount; ++m) {
            float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
            for (int b = 0; b < BPL; ++b) {
                const int blk = c + b * LPR;
                if (blk < nblk) {
                    const uint4 *xb = X + (size_t)(m * 4) * nblk + blk;
                    const float Sb = S[m * nblk + blk];
                    v0 += block_term<FMT>(sl.c0[b], sl.p0[b], xb, nblk, Sb, blk, magic);
                    if constexpr (GATEUP) v1 += block_term<FMT>(sl.c1[b], sl.p1[b], xb, nblk, Sb, blk, magic);
                }
            }
            v0 = moe_group_sum<LPR>(v0);
            if constexpr (GATEUP) v1 = moe_group_sum<LPR>(v1);
            if (moe_group_sum_owner<LPR>(c) && r < R) {
                if constexpr (GATEUP) {
                    const float hval = v0 / (1.0f + expf(-v0)) * v1;
                    a.h[(size_t)out_rows[m] * a.I + r] = (uint16_t)f32_to_bf16_bits(hval);
                } else {
                    a.y[(size_t)out_rows[m] * a.H + r] = v0;
                }
            }
        }
    };

    GemvSlot<BPL, GATEUP, FMT> slot[D];
    for (int pass = 0; pass < gr.M; pass += mt_cap) {
        const int mcount = min(mt_cap, gr.M - pass);
        // the first D steps' weights are requested before the activations are staged
#pragma unroll
        for (int d = 0; d < D; ++d) load(slot[d], d);
        if (threadIdx.x < mcount) {
            const int row = group_row(a, gr, pass + threadIdx.x);
            out_rows[threadIdx.x] = row;
            src_rows[threadIdx.x] = GATEUP ? (gr.routed < 0 ? pass + (int)threadIdx.x : row / a.k) : row;
        }
        __syncthreads();
        stage_rows<FMT == 1>(GATEUP ? a.x : a.h, K, src_rows, mcount, X, S);
        __syncthreads();
        for (int i0 = 0; i0 < nsteps; i0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int i = i0 + d;
                if (i < nsteps) {
                    compute(slot[d], i, mcount);
                    if (i + D < nsteps) load(slot[d], i + D);
                }
            }
        }
        __syncthreads();  // the next pass restages X and the row tables
    }
}

// rows of one row step in flight per wave: D steps of (GATEUP ? 2 : 1) * BPL
// 16-byte blocks per lane, about MOE_GEMV_BLOCKS_IN_FLIGHT blocks
#ifndef MOE_GEMV_BLOCKS_IN_FLIGHT
#define MOE_GEMV_BLOCKS_IN_FLIGHT 6
#endif
template <int BPL, bool GATEUP>
constexpr int steps_in_flight() {
    constexpr int per = (GATEUP ? 2 : 1) * BPL;
    return per >= MOE_GEMV_BLOCKS_IN_FLIGHT ? 1 : (MOE_GEMV_BLOCKS_IN_FLIGHT + per - 1) / per;
}
#ifndef MOE_GEMV_ITERS
#define MOE_GEMV_ITERS 8
#endif

template <int LPR, int BPL, bool GATEUP, int FMT>
int launch_one(const moe::FfnArgs &a, int R, int K, int n_groups, int max_m, hipStream_t s) {
    constexpr int D = steps_in_flight<BPL, GATEUP>();
    constexpr int ROWS_PER_STEP = 4 * (64 / LPR);
    const int iters = MOE_GEMV_ITERS;
    const int tiles = (R + ROWS_PER_STEP * iters - 1) / (ROWS_PER_STEP * iters);
    const int nblk = K / 32;
    const int mt_cap = max_m < kMT ? max_m : kMT;
    const size_t lds_bytes = (size_t)mt_cap * nblk * (4 * 16 + 4);
    if (lds_bytes > 64 * 1024) {
        static bool raised = false;
        if (!raised) {
            hipError_t e = hipFuncSetAttribute((const void *)ffn_gemv_kernel<LPR, BPL, D, GATEUP, FMT>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
            if (e != hipSuccess) return moe::fail_hip(e, "hipFuncSetAttribute(ffn_gemv_kernel)");
            raised = true;
        }
    }
    hipLaunchKernelGGL((ffn_gemv_kernel<LPR, BPL, D, GATEUP, FMT>), dim3((unsigned)n_groups * tiles), dim3(256), lds_bytes,
                       s, a, tiles, mt_cap, iters);
    MOE_LAUNCH_CHECK("ffn_gemv_kernel");
    return MOE_OK;
}

template <bool GATEUP, int FMT>
int launch_phase(const moe::FfnArgs &a, int n_groups, int max_m, hipStream_t s) {
    const int K = GATEUP ? a.H : a.I;
    const int R = GATEUP ? a.I : a.H;
    const int nblk = K / 32;
#define MOE_TRY_SHAPE(L, B) \
    if (nblk == (L) * (B)) return launch_one<L, B, GATEUP, FMT>(a, R, K, n_groups, max_m, s);
    MOE_TRY_SHAPE(64, 1) MOE_TRY_SHAPE(64, 2) MOE_TRY_SHAPE(64, 3) MOE_TRY_SHAPE(64, 4)
    MOE_TRY_SHAPE(16, 1) MOE_TRY_SHAPE(16, 2) MOE_TRY_SHAPE(16, 3) MOE_TRY_SHAPE(16, 4)
    MOE_TRY_SHAPE(8, 1) MOE_TRY_SHAPE(4, 1)
#undef MOE_TRY_SHAPE
    // other sizes: 64 lanes per row, guarded blocks
    if (nblk <= 64) return launch_one<64, 1, GATEUP, FMT>(a, R, K, n_groups, max_m, s);
    if (nblk <= 128) return launch_one<64, 2, GATEUP, FMT>(a, R, K, n_groups, max_m, s);
    if (nblk <= 256) return launch_one<64, 4, GATEUP, FMT>(a, R, K, n_groups, max_m, s);
    if (nblk <= 512) return launch_one<64, 8, GATEUP, FMT>(a, R, K, n_groups, max_m, s);
    return moe::fail(MOE_E_SHAPE, "expert_ffn: K=%d too large (max 16384)", K);
}

}  // namespace

namespace moe {

template <bool GATEUP>
int gemv_phase(const FfnArgs &a, int max_m, hipStream_t s) {
    const int n_groups = a.n_routed_groups + (a.shared ? 1 : 0);
    if (n_groups == 0) return MOE_OK;
    switch (a.fmt) {
        case 0: return launch_phase<GATEUP, 0>(a, n_groups, max_m, s);
        case 1: return launch_phase<GATEUP, 1>(a, n_groups, max_m, s);
        case 2: return launch_phase<GATEUP, 2>(a, n_groups, max_m, s);
    }
    return fail(MOE_E_ARG, "grouped GEMV: weight format %d", a.fmt);
}

int ffn_gemv_gate_up(const FfnArgs &a, int max_m, hipStream_t s) { return gemv_phase<true>(a, max_m, s); }
int ffn_gemv_down(const FfnArgs &a, int max_m, hipStream_t s) { return gemv_phase<false>(a, max_m, s); }

}  // namespace moe
