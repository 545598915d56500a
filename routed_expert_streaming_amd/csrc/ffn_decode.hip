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
#include "router.h"
#include "topk.h"
#include "ffn.h"

#include <type_traits>

namespace {

// Build-time tuning knobs (defaults are the tuned values).
#ifndef MOE_DECODE_WG_PER_CU
#define MOE_DECODE_WG_PER_CU 2  // target workgroups per compute unit
#endif
#ifndef MOE_DECODE_D_GU
#define MOE_DECODE_D_GU 5  // gate/up units in flight per lane group (H = 4096)
#endif
#ifndef MOE_DECODE_D_DN
#define MOE_DECODE_D_DN 4  // down units in flight per lane group (I = 1536)
#endif

// s_waitcnt immediate that waits until at most n vector-memory loads are in
// flight (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at
// their no-wait maxima)
constexpr int kWaitVm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }

#ifndef MOE_DECODE1_EARLY
#define MOE_DECODE1_EARLY 1  // one-token gate/up: request a shared-expert unit before routing
#endif

constexpr int kMaxTok = 4;      // tokens per launch on this path
constexpr int kMaxGroups = 64;  // T*k + 1

// Permute one 32-column activation block (4 x 16 B of bf16, natural order) into
// the dot2 pair order of dequant.h and return its fp32 sum (in index order).
__device__ __forceinline__ float block_pairs(const uint4 (&d)[4], uint4 (&X)[4]) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        X[j].x = (d[j].x & 0xFFFFu) | (d[j].z << 16);
        X[j].y = (d[j].x >> 16) | (d[j].z & 0xFFFF0000u);
        X[j].z = (d[j].y & 0xFFFFu) | (d[j].w << 16);
        X[j].w = (d[j].y >> 16) | (d[j].w & 0xFFFF0000u);
        const uint32_t v[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            s += bf16_bits_to_f32(v[q] & 0xFFFFu);
            s += bf16_bits_to_f32(v[q] >> 16);
        }
    }
    return s;
}

// Stage n activation rows (K columns, bf16) into LDS in dot2 pair order plus
// the fp32 block sums (same layout as the general kernels).
__device__ __forceinline__ void stage_all(const uint16_t *__restrict__ act, int K, int n, uint4 *X, float *S) {
    const int nblk = K >> 5;
    for (int id = threadIdx.x; id < n * nblk; id += blockDim.x) {
        const int m = id / nblk, b = id - m * nblk;
        const uint4 *src = reinterpret_cast<const uint4 *>(act + (size_t)m * K + 32 * b);
        uint4 d[4], p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = src[j];  // the whole block in one round trip
        S[m * nblk + b] = block_pairs(d, p);
#pragma unroll
        for (int j = 0; j < 4; ++j) X[(m * 4 + j) * nblk + b] = p[j];
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

// The weight loads of the register ring are issued unconditionally (tail units
// and masked groups re-read a valid row and skip the compute), so the compiler
// can count outstanding loads exactly and wait only for the oldest unit instead
// of draining the whole ring.
// ---------------------------------------------------------------- gate/up
template <int LPR, int BPL, int D, bool XREG>
__global__ __launch_bounds__(256) void decode_gate_up_kernel(moe::FfnArgs a, int units_per_sg) {
    constexpr int RPW = 64 / LPR;
    const int H = a.H, I = a.I, T = a.T, nblk = H >> 5;
    const int G = a.n_routed_groups + (a.shared ? 1 : 0);
    const long long Q = (long long)G * I;
    extern __shared__ uint4 lds[];
    uint4 *Xs = lds;
    float *Ss = reinterpret_cast<float *>(lds + (size_t)T * 4 * nblk);
    __shared__ const uint8_t *gslab[kMaxGroups];
    __shared__ const uint8_t *any_slab;
    load_group_slabs(a, gslab, G);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint8_t *p = nullptr;
        for (int g = 0; g < G && !p; ++g) p = gslab[g];
        any_slab = p;
    }

    const uint32_t magic = moe_magic_vgpr();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPR, c = lane % LPR;
    const long long sg = ((long long)blockIdx.x * 4 + wave) * RPW + sub;
    const long long q0 = sg * units_per_sg;
    const int n = (int)max(0LL, min(q0 + units_per_sg, Q) - q0);  // units of this lane group
    const size_t rs = moe::slab_row_bytes(H);  // W1 row r at slab + 2*rs*r, W3 row r right after it

    // one token: the lane's activation blocks go straight to registers
    uint4 xd[XREG ? BPL : 1][4];
    if (XREG) {
#pragma unroll
        for (int b = 0; b < BPL; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) xd[b][j] = load_global_u4(a.x + 32 * (c + b * LPR) + 8 * j);
    }
    __syncthreads();  // any_slab
    const uint8_t *fallback = any_slab;
    if (!fallback) return;  // every group masked off

    uint4 c0[D][BPL], c1[D][BPL];
    uint32_t p0[D][BPL], p1[D][BPL];
    // issue cursor (unit index, group, row) walks ahead of the compute cursor
    int ui = 0, gi = (int)(q0 / I), ri = (int)(q0 - (long long)gi * I);
    auto issue = [&](int j) {
        const uint8_t *slab = (ui < n) ? gslab[gi] : nullptr;
        const size_t row = slab ? (size_t)ri : 0;
        if (!slab) slab = fallback;
        const uint8_t *w1 = slab + 2 * rs * row, *w3 = w1 + rs;
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
            const int blk = c + b * LPR;
            c0[j][b] = load_stream_u4(w1 + 16 * blk);
            p0[j][b] = load_stream_u32(w1 + H / 2 + 4 * blk);
            c1[j][b] = load_stream_u4(w3 + 16 * blk);
            p1[j][b] = load_stream_u32(w3 + H / 2 + 4 * blk);
        }
        ++ui;
        if (++ri == I) {
            ri = 0;
            ++gi;
        }
    };
#pragma unroll
    for (int j = 0; j < D; ++j) issue(j);

    uint4 Xr[XREG ? BPL : 1][4];
    float Sr[XREG ? BPL : 1];
    if (XREG) {
#pragma unroll
        for (int b = 0; b < BPL; ++b) Sr[b] = block_pairs(xd[b], Xr[b]);
    } else {
        stage_all(a.x, H, T, Xs, Ss);
        __syncthreads();
    }

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
                        if (XREG) {
                            v0 += moe_block_value(p0[j][b], moe_block_dot(c0[j][b], Xr[b], 1, magic), Sr[b]);
                            v1 += moe_block_value(p1[j][b], moe_block_dot(c1[j][b], Xr[b], 1, magic), Sr[b]);
                        } else {
                            const uint4 *xb = Xs + (size_t)(t * 4) * nblk + blk;
                            const float Sb = Ss[t * nblk + blk];
                            v0 += moe_block_value(p0[j][b], moe_block_dot(c0[j][b], xb, nblk, magic), Sb);
                            v1 += moe_block_value(p1[j][b], moe_block_dot(c1[j][b], xb, nblk, magic), Sb);
                        }
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

// ---------------------------------------------------------------- gate/up, one token
// A 64-bit pointer that is the same in every lane, moved to scalar registers so
// that address arithmetic on it runs on the scalar unit.
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint8_t *)(((uint64_t)hi << 32) | lo);
}

// One token, H = 64*32*BPL: a whole wave covers one weight row (lane l owns
// blocks l, l+64, ...), so the unit cursor is wave-uniform and every weight load
// is a scalar row base plus the lane's fixed offset.  Units (group, row) are
// dealt to the waves round-robin (wave w takes units w, w+W, w+2W, ...), so the
// loads in flight across the chip at any moment cover one contiguous window of
// each weight matrix instead of one scattered run per wave.  The token's
// activation blocks stay in registers for the whole launch.
//
// Routing: with PER = 0 the k slots come from a.topk_idx; with PER > 0 every
// wave finishes the router itself from the per-slice fp64 partial logits
// (same fp32 logits, same top-k and softmax as the router entry point) and
// one wave publishes idx / weights / logits for the down kernel and the
// caller.  The expert table is loaded alongside the partials, so resolving a
// slot's slab is a lane shuffle rather than another trip to memory.
//
// Groups: the shared expert (when present) is group 0 and slot s is group
// s+1, so most waves start on the shared expert, whose slab is known before
// routing: they request their first unit before the top-k.  Lane g holds the
// slab of group g and a group's slab is read with v_readlane (no LDS, no
// barrier).
template <int BPL, int D, int PER, int FMT = 0>
__global__ __launch_bounds__(256) void decode1_gate_up_kernel(moe::FfnArgs a, moe::RouteArgs ra, int n_waves) {
    const int H = a.H, I = a.I, nblk = H >> 5, k = a.k;
    const int hs = a.shared ? 1 : 0;
    const int G = k + hs;
    const int Q = G * I;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint4 xd[BPL][4];
#pragma unroll
    for (int b = 0; b < BPL; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) xd[b][j] = load_global_u4(a.x + 32 * (lane + 64 * b) + 8 * j);

    const uint8_t *shared_slab = (const uint8_t *)a.shared;
    const uint32_t magic = moe_magic_vgpr();
    const int w0 = blockIdx.x * 4 + wave;
    const int n = w0 < Q ? (Q - w0 + n_waves - 1) / n_waves : 0;  // units of this wave
    const int dg = n_waves / I, dr = n_waves - dg * I;              // cursor step in (group, row)
    const uint32_t rs = (uint32_t)moe::row_bytes_fmt<FMT>(H);  // W1 row r at slab + 2*rs*r, W3 row r right after it
    // block lane + 64b: its codes at 16 bytes per block, its record (4 bytes; an
    // MXFP4 scale: 1 byte) after the row's codes
    // (format 2: the 16-byte header of the lane's super-block, block lane % 8 of it)
    constexpr uint32_t RB = FMT == 1 ? 1u : 4u;
    const uint32_t code_off = 16u * lane,
                   rec_off = (uint32_t)(H / 2) + (FMT == 2 ? 2u * (uint32_t)(lane & ~7) : RB * lane);
    using Rec = std::conditional_t<FMT == 2, uint4, uint32_t>;

    uint4 c0[D][BPL], c1[D][BPL];
    Rec p0[D][BPL], p1[D][BPL];
    int ui = 0, gi = w0 / I, ri = w0 - gi * I;  // issue cursor, D units ahead
    auto load_unit = [&](int j, const uint8_t *slab, int row) {
        const uint8_t *w1 = slab + (size_t)row * (2 * rs);
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
            c0[j][b] = load_stream_u4(w1 + (code_off + 1024u * b));
            c1[j][b] = load_stream_u4(w1 + (rs + code_off + 1024u * b));
            if constexpr (FMT == 2) {
                p0[j][b] = load_stream_u4(w1 + (rec_off + 128u * b));
                p1[j][b] = load_stream_u4(w1 + (rs + rec_off + 128u * b));
            } else if constexpr (FMT == 1) {
                p0[j][b] = load_stream_u8(w1 + (rec_off + 64u * b));
                p1[j][b] = load_stream_u8(w1 + (rs + rec_off + 64u * b));
            } else {
                p0[j][b] = load_stream_u32(w1 + (rec_off + 256u * b));
                p1[j][b] = load_stream_u32(w1 + (rs + rec_off + 256u * b));
            }
        }
    };
    auto advance_issue = [&]() {
        ++ui;
        gi += dg;
        ri += dr;
        if (ri >= I) {
            ri -= I;
            ++gi;
        }
    };
    // routing loads first (branch-free, indices clamped into range), so that
    // waiting for them never waits for weight loads issued after them
    int slot_e;  // lane s < k: expert of slot s
    uint64_t tab[PER > 0 ? PER : 1];
    moe_u32x4 pv[PER > 0 ? PER : 1][2];
    float bv[PER > 0 ? PER : 1];
    if constexpr (PER > 0) {
        typedef __attribute__((address_space(1))) const moe_u32x4 gvec;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int ec = min(lane + 64 * j, ra.E - 1);
            const double *pp = ra.partial + (size_t)ec * moe::kMaxSlices;
            pv[j][0] = *(gvec *)pp;
            pv[j][1] = *(gvec *)(pp + 2);
            tab[j] = (uint64_t)a.table[ec];
            // no branch around the load: without a bias read any valid float and drop it
            const float braw = (ra.bias ? ra.bias : (const float *)ra.partial)[ec];
            bv[j] = ra.bias ? braw : 0.0f;
        }
    } else {
        slot_e = lane < k ? a.topk_idx[lane] : 0;
    }
    // the first unit of a wave that starts on the shared expert goes out now
    const bool early = MOE_DECODE1_EARLY && hs && n > 0 && gi == 0;
    if (early) {
        load_unit(0, shared_slab, ri);
        advance_issue();
    }
    if constexpr (PER > 0) {
        // wait for the routing loads only: the early unit's 4*BPL loads are younger
        // (explicit counts, since the two paths leave different loads in flight)
        if (early)
            __builtin_amdgcn_s_waitcnt(kWaitVm(4 * BPL));
        else
            __builtin_amdgcn_s_waitcnt(kWaitVm(0));
        // the grid's last wave (one of those with the fewest units) publishes the
        // routing; only it needs the softmax
        const bool publish = w0 == n_waves - 1;
        uint32_t ord[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int e = lane + 64 * j;
            const double q[4] = {__hiloint2double(pv[j][0].y, pv[j][0].x), __hiloint2double(pv[j][0].w, pv[j][0].z),
                                 __hiloint2double(pv[j][1].y, pv[j][1].x), __hiloint2double(pv[j][1].w, pv[j][1].z)};
            const float l = moe::router_logit4(q, ra.nslices, bv[j]);
            ord[j] = e < ra.E ? moe::topk_ord(l) : 0u;
            if (publish && e < ra.E) ra.logits[e] = l;
        }
        float slot_logit;
        moe::topk_select(ord, k, slot_logit, slot_e);
        if (publish) {
            const float w = moe::topk_softmax(slot_logit, k);
            if (lane < k) {
                ra.idx_out[lane] = slot_e;
                ra.w_out[lane] = w;
            }
        }
    }
    // lane g: the slab of group g
    // (shuffles read only active lanes, so they run before any lane diverges)
    const int src = min(max(lane - hs, 0), 63);
    const int ge = __shfl(slot_e, src, 64);  // expert of group g (g >= hs)
    uint64_t ge_slab = 0;
    if constexpr (PER > 0) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)tab[j], ge & 63, 64);
            const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(tab[j] >> 32), ge & 63, 64);
            if ((ge >> 6) == j) ge_slab = ((uint64_t)hi << 32) | lo;
        }
    }
    const uint8_t *mine = nullptr;
    if (lane < hs) {
        mine = shared_slab;
    } else if (lane < G) {
        if constexpr (PER > 0) {
            mine = (const uint8_t *)ge_slab;
        } else {
            if (!a.mask || a.mask[ge]) mine = (const uint8_t *)a.table[ge];
        }
    }
    const uint64_t mv = (uint64_t)mine;
    const int mlo = (int)(uint32_t)mv, mhi = (int)(uint32_t)(mv >> 32);
    auto group_slab = [&](int g) {
        return (const uint8_t *)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(mhi, g) << 32) |
                                 (uint32_t)__builtin_amdgcn_readlane(mlo, g));
    };
    if (a.pair_slab && w0 == n_waves - 1 && lane < G)  // pair order: slots, then shared
        a.pair_slab[lane < hs ? k : lane - hs] = mine;
    // tail units and masked groups re-read row 0 of the first present slab
    const uint64_t present = __ballot(mine != nullptr);
    if (present == 0) return;  // every group masked off
    const uint8_t *fallback = group_slab(__ffsll((long long)present) - 1);

    auto issue = [&](int j) {
        const uint8_t *slab = fallback;
        int row = 0;
        if (ui < n) {
            const uint8_t *p = group_slab(gi);
            if (p) {
                slab = p;
                row = ri;
            }
        }
        load_unit(j, slab, row);
        advance_issue();
    };
    if (!early) issue(0);
#pragma unroll
    for (int j = 1; j < D; ++j) issue(j);
    __builtin_amdgcn_sched_barrier(0);  // the ring requests go out before waiting for x

    uint4 X[BPL][4];
    float S[BPL];
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
        if constexpr (FMT == 1) {  // natural column order, no block sums
#pragma unroll
            for (int j = 0; j < 4; ++j) X[b][j] = xd[b][j];
            S[b] = 0.0f;
        } else {
            S[b] = block_pairs(xd[b], X[b]);
        }
    }

    // Each unit's two sums go to lane (unit index mod 64); SiLU, rounding and the
    // store then run once for up to 64 units in parallel instead of once per unit
    // in a single lane (same arithmetic, so the same bits).
    float sg = 0.0f, su = 0.0f;
    int hoff = -1;  // h element of this lane's pending unit, -1: none
    auto flush = [&]() {
        if (hoff >= 0) a.h[hoff] = (uint16_t)f32_to_bf16_bits(sg / (1.0f + expf(-sg)) * su);
        hoff = -1;
    };
    int g = w0 / I, r = w0 - g * I;  // compute cursor
    for (int base = 0; base < n; base += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int u = base + j;
            if (u >= n) break;
            if (group_slab(g)) {
                float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
                for (int b = 0; b < BPL; ++b) {
                    if constexpr (FMT == 2) {
                        v0 += moe_sb_block_value(p0[j][b], lane & 7, moe_block_dot(c0[j][b], X[b], 1, magic), S[b]);
                        v1 += moe_sb_block_value(p1[j][b], lane & 7, moe_block_dot(c1[j][b], X[b], 1, magic), S[b]);
                    } else if constexpr (FMT == 1) {
                        v0 += moe_mx_block_value(p0[j][b], moe_mx_block_dot(c0[j][b], X[b]));
                        v1 += moe_mx_block_value(p1[j][b], moe_mx_block_dot(c1[j][b], X[b]));
                    } else {
                        v0 += moe_block_value(p0[j][b], moe_block_dot(c0[j][b], X[b], 1, magic), S[b]);
                        v1 += moe_block_value(p1[j][b], moe_block_dot(c1[j][b], X[b], 1, magic), S[b]);
                    }
                }
                v0 = moe_group_sum<64>(v0);
                v1 = moe_group_sum<64>(v1);
                const float t0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v0), 63));
                const float t1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v1), 63));
                if (lane == (u & 63)) {  // h row: slot g - hs, or the shared row k
                    sg = t0;
                    su = t1;
                    hoff = (g < hs ? k : g - hs) * I + r;
                }
            }
            issue(j);  // slot j is free again: request the unit D ahead
            if ((u & 63) == 63) flush();
            g += dg;
            r += dr;
            if (r >= I) {
                r -= I;
                ++g;
            }
        }
    }
    flush();
}

// ---------------------------------------------------------------- down (+ combine)
template <int LPR, int BPL, int D, bool COMBINE>
__global__ __launch_bounds__(256) void decode_down_kernel(moe::FfnArgs a, const float *__restrict__ topk_w,
                                                          uint16_t *__restrict__ out, int n_sg) {
    constexpr int RPW = 64 / LPR;
    constexpr int kStagePerThread = 2;  // (row, block) items of h requested ahead of the ring
    const int H = a.H, I = a.I, T = a.T, k = a.k, nblk = I >> 5;
    const int G = a.n_routed_groups + (a.shared ? 1 : 0);
    const int P = T * k + (a.shared ? T : 0);
    extern __shared__ uint4 lds[];
    uint4 *X = lds;
    float *S = reinterpret_cast<float *>(lds + (size_t)P * 4 * nblk);
    __shared__ const uint8_t *gslab[kMaxGroups];
    __shared__ float wts[kMaxGroups];
    __shared__ const uint8_t *any_slab;
    load_group_slabs(a, gslab, G);
    if (COMBINE)
        for (int i = threadIdx.x; i < T * k; i += blockDim.x) wts[i] = topk_w[i];
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint8_t *p = nullptr;
        for (int g = 0; g < G && !p; ++g) p = gslab[g];
        any_slab = p;
    }

    const uint32_t magic = moe_magic_vgpr();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPR, c = lane % LPR;
    const long long sg = ((long long)blockIdx.x * 4 + wave) * RPW + sub;
    // rows are dealt round-robin (lane group s takes rows s, s+n_sg, ...) so that
    // the loads in flight cover one contiguous window of every expert's W2
    const int r_first = (int)sg;
    const int n_rows = r_first < H ? (H - r_first + n_sg - 1) / n_sg : 0;
    const int n_units = n_rows * G;  // (row, pair) units, pairs innermost
    const size_t w2off = (size_t)I * 2 * moe::slab_row_bytes(H), rs2 = moe::slab_row_bytes(I);  // W2 row r

    // h blocks to stage: issued before the weight ring so that waiting for them
    // does not wait for the ring (items past the end re-read item 0)
    const int n_items = P * nblk;
    uint4 hd[kStagePerThread][4];
#pragma unroll
    for (int i = 0; i < kStagePerThread; ++i) {
        int item = threadIdx.x + i * 256;
        if (item >= n_items) item = 0;
        const int m = item / nblk, b = item - m * nblk;
#pragma unroll
        for (int j = 0; j < 4; ++j) hd[i][j] = load_global_u4(a.h + (size_t)m * I + 32 * b + 8 * j);
    }
    __syncthreads();  // any_slab
    const uint8_t *fallback = any_slab;

    uint4 cw[D][BPL];
    uint32_t pw[D][BPL];
    int ui = 0, ri = r_first, gi = 0;
    auto issue = [&](int j) {
        const uint8_t *slab = (ui < n_units) ? gslab[gi] : nullptr;
        const size_t row = slab ? (size_t)ri : 0;
        if (!slab) slab = fallback;
        const uint8_t *w2 = slab + w2off + row * rs2;
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
            const int blk = c + b * LPR;
            cw[j][b] = load_stream_u4(w2 + 16 * blk);
            pw[j][b] = load_stream_u32(w2 + I / 2 + 4 * blk);
        }
        ++ui;
        if (++gi == G) {
            gi = 0;
            ri += n_sg;
        }
    };
    if (fallback) {
#pragma unroll
        for (int j = 0; j < D; ++j) issue(j);
    }
#pragma unroll
    for (int i = 0; i < kStagePerThread; ++i) {
        const int item = threadIdx.x + i * 256;
        if (item < n_items) {
            const int m = item / nblk, b = item - m * nblk;
            uint4 Xb[4];
            S[m * nblk + b] = block_pairs(hd[i], Xb);
#pragma unroll
            for (int j = 0; j < 4; ++j) X[(m * 4 + j) * nblk + b] = Xb[j];
        }
    }
    // larger P: the remaining items the plain way (this wait also covers the ring)
    for (int item = threadIdx.x + kStagePerThread * 256; item < n_items; item += 256) {
        const int m = item / nblk, b = item - m * nblk;
        uint4 d[4], Xb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = load_global_u4(a.h + (size_t)m * I + 32 * b + 8 * j);
        S[m * nblk + b] = block_pairs(d, Xb);
#pragma unroll
        for (int j = 0; j < 4; ++j) X[(m * 4 + j) * nblk + b] = Xb[j];
    }
    __syncthreads();
    if (!fallback) return;

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
                rr += n_sg;
            }
        }
    }
}

// ---------------------------------------------------------------- down (+ combine), one token
// One token, I = 16*32*BPL: wave p of a workgroup owns pair p of the token
// (routed slots 0..k-1, then the shared expert) and keeps that pair's h row in
// registers; its four 16-lane groups take rows r0+s, r0+s+4, ... of the
// workgroup's row range in W2 of the pair's expert.  Per-(row, pair) results
// meet in LDS and one thread per row combines them in slot order (fmaf with
// the routing weight, then + shared), so the fused output matches the
// two-kernel path bit for bit.  Every SIMD gets several independent waves
// instead of one wave walking all pairs of a row.
constexpr int kDown1MaxRows = 64;  // rows per workgroup
constexpr int kDown1MaxPairs = moe::kDown1MaxPairs;

template <int BPL, int D, bool COMBINE, int FMT = 0, int ROWS = 16>
__global__ __launch_bounds__(1024) void decode1_down_kernel(moe::FfnArgs a, const float *__restrict__ topk_w,
                                                            uint16_t *__restrict__ out) {
    static_assert(ROWS % 4 == 0 && ROWS <= kDown1MaxRows && D >= 1, "rows per workgroup, units in flight");
    constexpr int rows_per_wg = ROWS;
    constexpr int U = ROWS / 4;  // rows per 16-lane group
    const int H = a.H, I = a.I, k = a.k;
    const int P = k + (a.shared ? 1 : 0);
    __shared__ float part[kDown1MaxRows][kDown1MaxPairs + 1];
    __shared__ int present[kDown1MaxPairs];
    __shared__ float wts[kDown1MaxPairs];
    const int lane = threadIdx.x & 63, sub = lane >> 4, c = lane & 15;
    const int p = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r0 = blockIdx.x * rows_per_wg;
    // routing weights requested now, stored to LDS just before the barrier
    const float my_w = (COMBINE && lane < k) ? topk_w[lane] : 0.0f;

    uint4 hd[BPL][4];
#pragma unroll
    for (int b = 0; b < BPL; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) hd[b][j] = load_global_u4(a.h + (size_t)p * I + 32 * (c + 16 * b) + 8 * j);
    // the prefetch hint: 1 KB per wave, requested with the loads of the wave's
    // last batch of rows (so that it is still in the L2 when the next call reads
    // it; with a single batch, with the first loads) and looked at only after
    // the rows are done, so nothing waits for it.  The
    // hint is read in 16 KB units, unit u on XCD u % 8 (workgroups are dealt to
    // the XCDs round-robin, and XCD x's waves take units x, x + 8, ...): the
    // router kernel's workgroup u, which reads one 16 KB slice of weights, then
    // finds it in its own XCD's L2.
    const int pf_x = blockIdx.x % 8, pf_j = (blockIdx.x / 8) * P + p;
    const size_t pf_off = ((size_t)(pf_x + 8 * (pf_j >> 4)) * 16 + (pf_j & 15)) * 1024 + 16 * lane;
    const bool pf = a.prefetch && pf_off + 16 <= a.prefetch_bytes;
    uint4 pfv = make_uint4(0, 0, 0, 0);
    if (pf && U < 2) pfv = load_global_u4(a.prefetch + pf_off);

    // the pair's slab: the shared expert is known up front; a routed slot's slab
    // was published by the gate/up kernel, else it is looked up
    const uint8_t *slab = nullptr;
    if (p >= k) {
        slab = (const uint8_t *)a.shared;
    } else if (a.pair_slab) {
        slab = a.pair_slab[p];
    } else {
        const int e = a.topk_idx[p];
        if (COMBINE || !a.mask || a.mask[e]) slab = (const uint8_t *)a.table[e];  // combine: no mask
    }
    slab = uniform_ptr(slab);
    if (lane == 0) present[p] = slab != nullptr;

    if (slab) {
        const uint32_t magic = moe_magic_vgpr();
        const uint8_t *w2 = slab + (size_t)I * 2 * moe::row_bytes_fmt<FMT>(H);  // W2 row 0
        const uint32_t rs2 = (uint32_t)moe::row_bytes_fmt<FMT>(I);
        constexpr uint32_t RB = FMT == 1 ? 1u : 4u;  // record bytes per block (format 2: a 16-byte header)
        const uint32_t code_off = 16u * c,
                       rec_off = (uint32_t)(I / 2) + (FMT == 2 ? 2u * (uint32_t)(c & ~7) : RB * c);
        uint4 cw[D < U ? D : U][BPL];
        std::conditional_t<FMT == 2, uint4, uint32_t> pw[D < U ? D : U][BPL];
        int ui = 0;
        auto issue = [&](int j) {
            int row = r0 + sub + 4 * ui;
            if (ui >= U || row >= H) row = r0;  // past the end: re-read a valid row
            const uint32_t rrow = (uint32_t)row * rs2;
#pragma unroll
            for (int b = 0; b < BPL; ++b) {
                cw[j][b] = load_stream_u4(w2 + (rrow + code_off + 256u * b));
                if constexpr (FMT == 2)
                    pw[j][b] = load_stream_u4(w2 + (rrow + rec_off + 32u * b));
                else if constexpr (FMT == 1)
                    pw[j][b] = load_stream_u8(w2 + (rrow + rec_off + 16u * b));
                else
                    pw[j][b] = load_stream_u32(w2 + (rrow + rec_off + 64u * b));
            }
            ++ui;
        };
        // a ring of min(D, U) units: every unit's loads are issued once (the unit
        // count is a compile-time constant, so the compiler's wait counts are exact
        // and no load is issued for a unit past the last)
        constexpr int DR = D < U ? D : U;
#pragma unroll
        for (int j = 0; j < DR; ++j) issue(j);
        __builtin_amdgcn_sched_barrier(0);  // the weight requests go out before waiting for h

        uint4 X[BPL][4];
        float S[BPL];
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
            if constexpr (FMT == 1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) X[b][j] = hd[b][j];
                S[b] = 0.0f;
            } else {
                S[b] = block_pairs(hd[b], X[b]);
            }
        }

#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = u % DR;
            const int rl = sub + 4 * u, row = r0 + rl;
            float v = 0.0f;
#pragma unroll
            for (int b = 0; b < BPL; ++b) {
                if constexpr (FMT == 2)
                    v += moe_sb_block_value(pw[j][b], c & 7, moe_block_dot(cw[j][b], X[b], 1, magic), S[b]);
                else if constexpr (FMT == 1)
                    v += moe_mx_block_value(pw[j][b], moe_mx_block_dot(cw[j][b], X[b]));
                else
                    v += moe_block_value(pw[j][b], moe_block_dot(cw[j][b], X[b], 1, magic), S[b]);
            }
            v = moe_group_sum<16>(v);
            if (c == 15 && row < H) {
                if (COMBINE)
                    part[rl][p] = v;
                else
                    a.y[(size_t)p * H + row] = v;
            }
            if (u + DR < U) issue(j);
            if (pf && u == U - 2) pfv = load_global_u4(a.prefetch + pf_off);
        }
    }
    // keeps the prefetch loads (their values are never needed)
    if (pf && pfv.x == 0x2545F491u && pfv.y == 0x9E3779B9u && pfv.z == 0x7F4A7C15u && pfv.w == 0xF39CC060u)
        asm volatile("" ::"v"(pfv.x));
    if (COMBINE) {
        if (p == 0 && lane < k) wts[lane] = my_w;
        __syncthreads();
        const int t = threadIdx.x, row = r0 + t;
        if (t < rows_per_wg && row < H) {
            float acc = 0.0f;
            for (int g = 0; g < P; ++g)
                if (present[g]) acc = g < k ? fmaf(wts[g], part[t][g], acc) : acc + part[t][g];
            out[row] = (uint16_t)f32_to_bf16_bits(acc);
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
    if (a.T == 1) {
        hipLaunchKernelGGL((decode_gate_up_kernel<LPR, BPL, D, true>), dim3(grid), dim3(256), 0, s, a, ups);
    } else {
        const size_t lds = (size_t)a.T * (a.H >> 5) * (4 * 16 + 4);
        int rc = raise_lds(decode_gate_up_kernel<LPR, BPL, D, false>, lds);
        if (rc != MOE_OK) return rc;
        hipLaunchKernelGGL((decode_gate_up_kernel<LPR, BPL, D, false>), dim3(grid), dim3(256), lds, s, a, ups);
    }
    MOE_LAUNCH_CHECK("decode_gate_up_kernel");
    return MOE_OK;
}

#ifndef MOE_DECODE1_WG_PER_CU
#define MOE_DECODE1_WG_PER_CU 2  // workgroups per CU for the one-token gate/up kernel
#endif

template <int BPL, int D, int FMT = 0>
int launch_gate_up1(const moe::FfnArgs &a, const moe::RouteArgs *ra, hipStream_t s) {
    const int G = a.n_routed_groups + (a.shared ? 1 : 0);
    const long long Q = (long long)G * a.I;
    const long long target = (long long)MOE_DECODE1_WG_PER_CU * num_cus() * 4;
    const int grid = (int)((std::min(Q, target) + 3) / 4);
    const moe::RouteArgs none{};
    if (!ra)
        hipLaunchKernelGGL((decode1_gate_up_kernel<BPL, D, 0, FMT>), dim3(grid), dim3(256), 0, s, a, none, grid * 4);
    else if (ra->E <= 64)
        hipLaunchKernelGGL((decode1_gate_up_kernel<BPL, D, 1, FMT>), dim3(grid), dim3(256), 0, s, a, *ra, grid * 4);
    else if (ra->E <= 128)
        hipLaunchKernelGGL((decode1_gate_up_kernel<BPL, D, 2, FMT>), dim3(grid), dim3(256), 0, s, a, *ra, grid * 4);
    else
        hipLaunchKernelGGL((decode1_gate_up_kernel<BPL, D, 4, FMT>), dim3(grid), dim3(256), 0, s, a, *ra, grid * 4);
    MOE_LAUNCH_CHECK("decode1_gate_up_kernel");
    return MOE_OK;
}

template <int LPR, int BPL, int D>
int launch_down(const moe::FfnArgs &a, const float *topk_w, uint16_t *out, hipStream_t s) {
    constexpr int RPW = 64 / LPR;
    const long long target_sg = (long long)MOE_DECODE_WG_PER_CU * num_cus() * 4 * RPW;
    const int grid = (int)((std::min<long long>(a.H, target_sg) + 4 * RPW - 1) / (4 * RPW));
    const int n_sg = grid * 4 * RPW;
    const int P = a.T * a.k + (a.shared ? a.T : 0);
    const size_t lds = (size_t)P * (a.I >> 5) * (4 * 16 + 4);
    if (out) {
        int rc = raise_lds(decode_down_kernel<LPR, BPL, D, true>, lds);
        if (rc != MOE_OK) return rc;
        hipLaunchKernelGGL((decode_down_kernel<LPR, BPL, D, true>), dim3(grid), dim3(256), lds, s, a, topk_w, out,
                           n_sg);
    } else {
        int rc = raise_lds(decode_down_kernel<LPR, BPL, D, false>, lds);
        if (rc != MOE_OK) return rc;
        hipLaunchKernelGGL((decode_down_kernel<LPR, BPL, D, false>), dim3(grid), dim3(256), lds, s, a, topk_w,
                           out, n_sg);
    }
    MOE_LAUNCH_CHECK("decode_down_kernel");
    return MOE_OK;
}

#ifndef MOE_DOWN1_ROWS
// rows per workgroup, one-token down kernel (same measurement: 16 rows 9.5 us,
// 8 rows 9.8 us, 4 rows 12.3 us, one unit in flight)
#define MOE_DOWN1_ROWS 16
#endif
#ifndef MOE_DOWN1_D
// units in flight per lane group, one-token down kernel (measured at H 4096, I 1536,
// 9 pairs, the kernel alone: 1 unit 9.5 us, 2 units 8.9 us, 4 units 9.7 us)
#define MOE_DOWN1_D 2
#endif

template <int BPL, int FMT = 0>
int launch_down1(const moe::FfnArgs &a, const float *topk_w, uint16_t *out, hipStream_t s) {
    const int P = a.k + (a.shared ? 1 : 0);
    const int grid = (a.H + MOE_DOWN1_ROWS - 1) / MOE_DOWN1_ROWS;
    if (out)
        hipLaunchKernelGGL((decode1_down_kernel<BPL, MOE_DOWN1_D, true, FMT, MOE_DOWN1_ROWS>), dim3(grid), dim3(64 * P),
                           0, s, a, topk_w, out);
    else
        hipLaunchKernelGGL((decode1_down_kernel<BPL, MOE_DOWN1_D, false, FMT, MOE_DOWN1_ROWS>), dim3(grid),
                           dim3(64 * P), 0, s, a, topk_w, out);
    MOE_LAUNCH_CHECK("decode1_down_kernel");
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

#ifndef MOE_DECODE1_D
#define MOE_DECODE1_D 1  // units in flight per wave, one-token gate/up (H = 4096)
#endif
#ifndef MOE_DECODE1_D_ROUTED
// the same when the kernel also finishes the routing: a deeper ring keeps more
// weight loads in flight while the top-k runs (measured: 262 vs 264.5 us per
// 8-layer step; without routing the shallower ring is faster, 15.4 vs 15.6 us)
#define MOE_DECODE1_D_ROUTED 2
#endif

bool decode1_routed_supported(const FfnArgs &a, int E) {
    const int nh = a.H >> 5;
    // H <= 4096: at most four router slices, read in one go by the fused prologue
    return a.T == 1 && !a.grouped && a.k + (a.shared ? 1 : 0) <= kMaxGroups && E <= 256 && a.H <= 4 * kSlice &&
           (nh == 128 || nh == 64) && decode_supported(a);
}

bool decode1_publishes_slabs(const FfnArgs &a) {
    const int nh = a.H >> 5;
    return a.T == 1 && !a.grouped && (nh == 128 || nh == 192 || nh == 64) && decode_supported(a);
}

int decode1_routed_gate_up(const FfnArgs &a, const RouteArgs &ra, hipStream_t s) {
    if (ra.nslices > 4) return fail(MOE_E_SHAPE, "routed gate/up: H=%d above 4096", a.H);
    if (a.fmt == 1) {
        switch (a.H >> 5) {
            case 128: return launch_gate_up1<2, MOE_DECODE1_D_ROUTED, 1>(a, &ra, s);
            case 64: return launch_gate_up1<1, 6, 1>(a, &ra, s);
            default: return fail(MOE_E_SHAPE, "routed gate/up (MXFP4): H=%d not supported", a.H);
        }
    }
    if (a.fmt == 2) {
        switch (a.H >> 5) {
            case 128: return launch_gate_up1<2, MOE_DECODE1_D_ROUTED, 2>(a, &ra, s);
            case 64: return launch_gate_up1<1, 6, 2>(a, &ra, s);
            default: return fail(MOE_E_SHAPE, "routed gate/up (super-blocks): H=%d not supported", a.H);
        }
    }
    switch (a.H >> 5) {
        case 128: return launch_gate_up1<2, MOE_DECODE1_D_ROUTED>(a, &ra, s);
        case 64: return launch_gate_up1<1, 6>(a, &ra, s);
        default: return fail(MOE_E_SHAPE, "routed gate/up: H=%d not supported", a.H);
    }
}

int decode_gate_up(const FfnArgs &a, hipStream_t s) {
    if (a.fmt == 1) {
        if (a.T == 1)
            switch (a.H >> 5) {
                case 128: return launch_gate_up1<2, MOE_DECODE1_D, 1>(a, nullptr, s);
                case 192: return launch_gate_up1<3, 3, 1>(a, nullptr, s);
                case 64: return launch_gate_up1<1, 6, 1>(a, nullptr, s);
            }
        return fail(MOE_E_SHAPE, "gate/up (MXFP4): one token with H 2048, 4096 or 6144 only (T=%d, H=%d)", a.T, a.H);
    }
    if (a.fmt == 2) {
        if (a.T == 1)
            switch (a.H >> 5) {
                case 128: return launch_gate_up1<2, MOE_DECODE1_D, 2>(a, nullptr, s);
                case 192: return launch_gate_up1<3, 3, 2>(a, nullptr, s);
                case 64: return launch_gate_up1<1, 6, 2>(a, nullptr, s);
            }
        return fail(MOE_E_SHAPE, "gate/up (super-blocks): one token with H 2048, 4096 or 6144 only (T=%d, H=%d)", a.T,
                    a.H);
    }
    if (a.T == 1) {
        switch (a.H >> 5) {
            case 128: return launch_gate_up1<2, MOE_DECODE1_D>(a, nullptr, s);
            case 192: return launch_gate_up1<3, 3>(a, nullptr, s);
            case 64: return launch_gate_up1<1, 6>(a, nullptr, s);
            default: break;
        }
    }
    switch (a.H >> 5) {
        case 128: return launch_gate_up<64, 2, MOE_DECODE_D_GU>(a, s);
        case 192: return launch_gate_up<64, 3, 3>(a, s);
        case 64: return launch_gate_up<64, 1, 6>(a, s);
        case 8: return launch_gate_up<8, 1, 4>(a, s);
        default: return fail(MOE_E_SHAPE, "decode gate/up: H=%d not supported", a.H);
    }
}

int decode_down(const FfnArgs &a, const float *topk_w, uint16_t *out, hipStream_t s) {
    if (a.fmt == 1) {
        if (a.T == 1 && !a.grouped && a.k + (a.shared ? 1 : 0) <= kDown1MaxPairs)
            switch (a.I >> 5) {
                case 48: return launch_down1<3, 1>(a, topk_w, out, s);
                case 64: return launch_down1<4, 1>(a, topk_w, out, s);
            }
        return fail(MOE_E_SHAPE, "down (MXFP4): one token with I 1536 or 2048 only (T=%d, I=%d)", a.T, a.I);
    }
    if (a.fmt == 2) {
        if (a.T == 1 && !a.grouped && a.k + (a.shared ? 1 : 0) <= kDown1MaxPairs)
            switch (a.I >> 5) {
                case 48: return launch_down1<3, 2>(a, topk_w, out, s);
                case 64: return launch_down1<4, 2>(a, topk_w, out, s);
            }
        return fail(MOE_E_SHAPE, "down (super-blocks): one token with I 1536 or 2048 only (T=%d, I=%d)", a.T, a.I);
    }
    if (a.T == 1 && a.k + (a.shared ? 1 : 0) <= kDown1MaxPairs) {
        switch (a.I >> 5) {
            case 48: return launch_down1<3>(a, topk_w, out, s);
            case 64: return launch_down1<4>(a, topk_w, out, s);
            default: break;
        }
    }
    switch (a.I >> 5) {
        case 48: return launch_down<16, 3, MOE_DECODE_D_DN>(a, topk_w, out, s);
        case 64: return launch_down<64, 1, 8>(a, topk_w, out, s);
        case 128: return launch_down<64, 2, 6>(a, topk_w, out, s);
        case 4: return launch_down<4, 1, 8>(a, topk_w, out, s);
        default: return fail(MOE_E_SHAPE, "decode down: I=%d not supported", a.I);
    }
}

}  // namespace moe
