// Expert FFN for many tokens per expert (prefill): grouped GEMM on MFMA with
// the 4-bit weight tiles dequantised in the kernel.
//
// The multi-token case is a dense contraction per expert: the tokens routed to
// expert e (gathered through the token->expert permutation) form an M_e x H
// activation matrix that meets the expert's W1/W3 (H -> I) and then W2 (I -> H).
// A workgroup owns one expert and one 128-row N tile of the weights and covers
// the expert's tokens in M chunks of up to 96, so at prefill sizes (about 64
// tokens per expert) every weight byte is read from HBM once.
//
// The K dimension streams in chunks of 64 columns through a ring of S LDS
// buffers filled by direct global->LDS loads (global_load_lds_dwordx4), so the
// loads of the next S-1 chunks are in flight while the current chunk is
// multiplied and no registers hold data on its way to LDS.  The (scale, min)
// records come through a ring of their own, RC chunks per load (16 or 32 bytes
// per row): fetched with the codes, 8 bytes per row and chunk, they cost as
// much load bandwidth as the codes, since every row is a separate fetch.  Each wave loads its
// own 32 weight rows; the activation tile is shared and XOR-swizzled in 16-byte
// units so that the A-operand reads hit distinct banks.  One barrier per chunk:
// each wave first waits (exact vmcnt) for its own loads of the chunk, the
// barrier then makes every wave's loads visible and frees the buffer that the
// chunk loads issued next will overwrite.  Each wave owns 32 N columns (of W1
// and of W3 for gate/up): it dequantises its B operand from LDS into bf16
// registers (scale*q + min in fp32, rounded to bf16) and accumulates
// v_mfma_f32_16x16x32_bf16 products in fp32.  Workgroups are numbered so that
// every tile of one expert runs on the same XCD, where the expert's gathered
// activation rows are shared through that XCD's L2.
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (checked on gfx950): lane l holds
// A[l%16][8*(l/16)+j], B[8*(l/16)+j][l%16] for j < 8, and C[4*(l/16)+j][l%16]
// for j < 4.
#include "common.h"
#include "dequant.h"
#include "ffn.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kNT = 128;       // weight rows (N) per workgroup
constexpr int kKC = 64;        // columns (K) per chunk
constexpr int kMaxMT = 6;      // 16-row M tiles per pass
constexpr int kMC = 16 * kMaxMT;
constexpr int kXRow = kKC * 2; // bytes of one activation row of a chunk (8 units of 16 B)
constexpr int kXcds = 8;       // workgroups are dealt to the XCDs round-robin
#ifndef MOE_MFMA_STAGES_GU
#define MOE_MFMA_STAGES_GU 3
#endif
#ifndef MOE_MFMA_STAGES_DN
#define MOE_MFMA_STAGES_DN 4
#endif
constexpr int kStagesGateUp = MOE_MFMA_STAGES_GU;  // ring depth: 3 x 22 KB of LDS, two workgroups per CU
constexpr int kStagesDown = MOE_MFMA_STAGES_DN;    // 4 x 17 KB

// One ring stage: the chunk's activation tile (row r, 16-byte unit u stored at
// unit position u ^ (r & 7)), and per matrix the codes of the 128 rows, wave
// w's 32 rows in its own 1 KB (unit (row, half) at position half*32 + row).
template <int NMAT>
struct __attribute__((aligned(16))) Stage {
    uint8_t x[kMC * kXRow];
    uint8_t w[NMAT][kNT * 32];
};

// Record buffer: per wave 1 KB, the records of RC chunks (2*RC blocks, 8*RC
// bytes) of its 32 rows of each matrix, matrix-major then row-major.  One
// 64-lane 16-byte load fills it (lanes beyond NMAT*RC*16 repeat the first ones
// into the unused rest).
constexpr int kRecWave = 1024;

// Number of multiples of m in [lo, hi].
constexpr int multiples(int lo, int hi, int m) {
    return hi < lo ? 0 : (lo > 0 ? hi / m - (lo - 1) / m : hi / m + 1);
}

// Loads a wave may still have in flight when step c waits, such that chunk c's
// stage and the records of its group are complete.  Issue order: the records of
// group 0, then stages 0 .. S-2; step j issues stage j+S-1 (P loads) and, when
// RC divides j, the records of group j/RC + 1 (NR loads).  The count is the
// number of loads issued after the later of the two.
constexpr int newer_loads(int S, int RC, int P, int NR, int c) {
    const int after_stage = P * (S - 2) + NR * multiples(c - S + 1 > 0 ? c - S + 1 : 0, c - 1, RC);
    const int grp = c / RC;
    const int after_rec = grp == 0 ? (S - 1 + c) * P + NR * multiples(0, c - 1, RC)
                                   : (c - 1 - RC * (grp - 1)) * P + NR * multiples(RC * (grp - 1) + 1, c - 1, RC);
    return after_stage < after_rec ? after_stage : after_rec;
}
// The same for every step at position b of a loop unrolled by U (the pattern
// repeats with period U after the first U steps).
constexpr int vm_allow(int S, int RC, int P, int NR, int U, int b) {
    int m = newer_loads(S, RC, P, NR, b);
    for (int r = 1; r < 4; ++r) {
        const int v = newer_loads(S, RC, P, NR, b + r * U);
        m = v < m ? v : m;
    }
    return m;
}
constexpr int lcm(int a, int b) {
    int x = a, y = b;
    while (y) {
        const int t = x % y;
        x = y;
        y = t;
    }
    return a / x * b;
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Direct global->LDS loads: lane l's 16 (or 4) bytes from g land at LDS byte
// lds + 16*l (4*l); lds must be the same in every lane.  Written as inline asm
// because the compiler, when it sees these loads, makes every later LDS read
// wait for all of them (it cannot tell the ring's stages apart), which would
// drain the ring each chunk; completion is tracked with explicit vmcnt waits
// instead (the instructions have no register results).
__device__ __forceinline__ uint32_t lds_addr(const void *lds) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_u8 *)lds);
}
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds));
}
__device__ __forceinline__ void dma4(const void *g, uint32_t lds) {
    asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds));
}

constexpr int kWaitVm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }

// Workgroup barrier without a memory fence (a fence would wait for every load
// in flight); the asm clobbers keep the compiler from moving memory accesses
// across it, and this wave's LDS reads are complete before it arrives.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 8 consecutive weights of one row (codes dword, its block record) -> bf16x8.
// Byte b of the dword holds column 2b in bits 0-3 and 2b+1 in bits 4-7.  OR-ing
// a nibble into the mantissa of an fp16 constant gives an exact fp16 number:
//   bits 0-3 into 0x6400 (1024, ulp 1)    -> 1024 + q
//   bits 4-7 into 0x5400 (64, ulp 1/16)   ->   64 + q
// so w & 0x000F000F | 0x64006400 holds columns 0 and 4, w & 0x00F000F0 |
// 0x54005400 columns 1 and 5, and the same on w >> 8 columns 2, 6 and 3, 7:
// four extractions for one shift.  v_fma_mix_f32 widens each half and computes
// scale*(base + q) + (min - base*scale) in fp32 with one rounding, which equals
// fmaf(scale, q, min) whenever min - base*scale is exact in fp32 (scale and min
// within 2^12 of each other's magnitude); then round to bf16 in natural order.
__device__ __forceinline__ float fma_half(uint32_t pair, int hi, float sc, float c) {
    const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(hi ? pair >> 16 : pair & 0xFFFFu));
    return fmaf((float)h, sc, c);
}

// Constants of the extraction: masks in SGPRs and the fp16 exponent patterns in
// VGPRs, so that (w & mask) | pattern is one v_and_or_b32 (a VOP3 instruction
// reads at most one scalar operand, and a literal not at all).
struct Dequant {
    uint32_t mask_lo, mask_hi;    // SGPR: 0x000F000F, 0x00F000F0
    uint32_t magic_lo, magic_hi;  // VGPR: 0x64006400, 0x54005400
};

__device__ __forceinline__ Dequant dequant_consts() {
    Dequant d;
    asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(d.mask_lo));
    asm volatile("s_mov_b32 %0, 0x00F000F0" : "=s"(d.mask_hi));
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(d.magic_lo));
    asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(d.magic_hi));
    return d;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int N>
struct IntC {
    static constexpr int value = N;
};

// f(IntC<B>{}), f(IntC<B + 1>{}), ..., f(IntC<E - 1>{})
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(IntC<B>{});
        static_for<B + 1, E>(f);
    }
}

// two floats -> bf16 pair (round to nearest even), lo in bits 0-15
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float __attribute__((ext_vector_type(2)))){lo, hi},
                                                                bf16x2_t));
}

// (a & mask) | pattern as one instruction (the compiler splits it into two)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t pattern) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(pattern));
    return r;
}

__device__ __forceinline__ bf16x8_t dequant8(uint32_t codes, uint32_t rec, const Dequant &d) {
    const float sc = fp16_bits_to_f32(rec & 0xFFFFu);
    const float mn = fp16_bits_to_f32(rec >> 16);
    const float c_lo = fmaf(-1024.0f, sc, mn);
    const float c_hi = fmaf(-64.0f, sc, mn);
    const uint32_t c8 = codes >> 8;
    const uint32_t p0 = and_or(codes, d.mask_lo, d.magic_lo);  // columns 0, 4
    const uint32_t p1 = and_or(codes, d.mask_hi, d.magic_hi);  // columns 1, 5
    const uint32_t p2 = and_or(c8, d.mask_lo, d.magic_lo);     // columns 2, 6
    const uint32_t p3 = and_or(c8, d.mask_hi, d.magic_hi);     // columns 3, 7
    // columns (0,1) (2,3) (4,5) (6,7), each pair rounded to bf16 by one v_cvt_pk_bf16_f32
    const uint32_t w01 = pack_bf16(fma_half(p0, 0, sc, c_lo), fma_half(p1, 0, sc, c_hi));
    const uint32_t w23 = pack_bf16(fma_half(p2, 0, sc, c_lo), fma_half(p3, 0, sc, c_hi));
    const uint32_t w45 = pack_bf16(fma_half(p0, 1, sc, c_lo), fma_half(p1, 1, sc, c_hi));
    const uint32_t w67 = pack_bf16(fma_half(p2, 1, sc, c_lo), fma_half(p3, 1, sc, c_hi));
    return __builtin_bit_cast(bf16x8_t, make_uint4(w01, w23, w45, w67));
}

template <bool GATEUP, int S, int RC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mfma_ffn_kernel(moe::FfnArgs a, int ntiles,
                                                                                           int n_groups) {
    constexpr int NMAT = GATEUP ? 2 : 1;
    static_assert(S >= 2, "the ring needs two stages at least");
    static_assert((RC == 2 || RC == 4) && NMAT * RC <= 4, "one 16-byte load per lane fills a record buffer");
    constexpr int U = lcm(S, RC);       // steps per unrolled loop body
    constexpr int LPR = RC / 2;         // lanes per row of a record load
    const int K = GATEUP ? a.H : a.I;   // reduction length (a multiple of 64 * RC)
    const int R = GATEUP ? a.I : a.H;   // weight rows (output columns)
    // every tile of one expert on the same XCD
    const int xcd = blockIdx.x % kXcds, i = blockIdx.x / kXcds;
    const int g = (i / ntiles) * kXcds + xcd, tile = i % ntiles;
    if (g >= n_groups) return;
    const int n0 = tile * kNT;

    // resolve the group: routed expert g (grouped), or the shared expert
    const uint8_t *slab;
    int M, base = 0;
    const bool routed = g < a.n_routed_groups;
    if (routed) {
        M = __builtin_amdgcn_readfirstlane(a.count[g]);  // uniform: M-tile checks become scalar branches
        if (M == 0 || M < a.min_m || M > a.max_m || (a.mask && a.mask[g] == 0)) return;
        slab = (const uint8_t *)a.table[g];
        base = a.offset[g];
    } else {
        if (!a.shared || a.T < a.min_m || a.T > a.max_m) return;
        slab = (const uint8_t *)a.shared;
        M = a.T;
    }
    const moe::MatRows mat[2] = {GATEUP ? moe::slab_w1(slab, a.H, a.I) : moe::slab_w2(slab, a.H, a.I),
                                 moe::slab_w3(slab, a.H, a.I)};
    const uint16_t *act = GATEUP ? a.x : a.h;

    __shared__ Stage<NMAT> ring[S];
    const uint32_t ring_lds = lds_addr(&ring[0]);
    auto stage_addr = [&](int b) { return ring_lds + (uint32_t)(b * sizeof(Stage<NMAT>)); };
    __shared__ __attribute__((aligned(16))) uint8_t recs_lds[2][4 * kRecWave];
    const uint32_t rec_lds = lds_addr(&recs_lds[0][0]);
    __shared__ int s_src[kMC];  // activation row of each M row
    __shared__ int s_dst[kMC];  // output row of each M row (-1 = padding)
    const Dequant dq = dequant_consts();
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lq = lane >> 4;  // MFMA row-in-tile and k-quarter
    const int nchunks = K / kKC;

    // this lane's global sources, fixed over a pass: weight rows of its wave
    const int wrow = n0 + 32 * wave + (lane & 31);           // codes: lanes 0-31 half 0, 32-63 half 1
    const uint8_t *wsrc[NMAT];
#pragma unroll
    for (int q = 0; q < NMAT; ++q) wsrc[q] = mat[q].row0 + (size_t)wrow * mat[q].stride + (lane >> 5) * 16;
    // records: lane (q, row, part) of the NMAT * 32 * LPR used lanes takes bytes
    // 16*part .. 16*part+15 of the row's records of a group of RC chunks
    const uint8_t *rsrc;
    {
        const int ll = lane % (NMAT * 32 * LPR);
        const int q = ll / (32 * LPR), r = (ll % (32 * LPR)) / LPR, part = ll % LPR;
        const moe::MatRows &m = q ? mat[1] : mat[0];
        rsrc = m.row0 + (size_t)(n0 + 32 * wave + r) * m.stride + K / 2 + part * 16;
    }

    for (int m0 = 0; m0 < M; m0 += kMC) {
        const int mc = min(kMC, M - m0);
        const int mtiles = (mc + 15) >> 4;
        __syncthreads();  // the previous pass is done with s_src / s_dst and the ring
        if (tid < kMC) {
            int src = -1, dst = -1;
            const int m = m0 + (tid < mc ? tid : 0);  // padding rows repeat the first row
            if (routed) {
                const int p = a.pair_of_row[base + m];
                src = GATEUP ? p / a.k : p;
                dst = p;
            } else {
                dst = a.T * a.k + m;
                src = GATEUP ? m : dst;
            }
            s_src[tid] = src;
            s_dst[tid] = tid < mc ? dst : -1;
        }
        __syncthreads();
        // activation loads of this wave: tile units wave + 4j (8 rows each), for
        // j < (MT + 1) / 2 with MT M tiles, so that every wave issues the same
        // number of loads per chunk (rows past the tokens repeat the first row;
        // rows past 16 * MT are loaded for that reason only and never read).
        const uint16_t *xsrc[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int r = 8 * (wave + 4 * j) + (lane >> 3), pos = lane & 7;
            xsrc[j] = act + (size_t)s_src[r] * K + 8 * (pos ^ (r & 7));
        }

        // LDS byte address of stage st (uniform), then constant offsets
        auto issue = [&](uint32_t st, int c, auto mt_count) {
            constexpr int XJ = (decltype(mt_count)::value + 1) / 2;
            const int k0 = c * kKC;
#pragma unroll
            for (int j = 0; j < XJ; ++j) dma16(xsrc[j] + k0, st + (uint32_t)((wave + 4 * j) * 1024));
#pragma unroll
            for (int q = 0; q < NMAT; ++q)
                dma16(wsrc[q] + k0 / 2, st + (uint32_t)(offsetof(Stage<NMAT>, w) + q * kNT * 32 + wave * 1024));
        };
        // the records of chunk group grp into record buffer buf (one load per wave)
        auto issue_rec = [&](int grp, int buf) {
            dma16(rsrc + grp * RC * 8, rec_lds + (uint32_t)(buf * 4 * kRecWave + wave * kRecWave));
        };

        f32x4_t acc[NMAT][kMaxMT][2];
#pragma unroll
        for (int q = 0; q < NMAT; ++q)
#pragma unroll
            for (int mt = 0; mt < kMaxMT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc[q][mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // Byte offsets of matrix q's codes and records in a stage, hidden from the
        // optimiser: otherwise it pairs the reads of the two matrices into one
        // ds_read2st64, whose merged memory operand no longer shows which stage it
        // reads, and then waits for every load in flight before it.
        int wq[NMAT], pq[NMAT];
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {
            wq[q] = (int)(offsetof(Stage<NMAT>, w) + q * kNT * 32) + wave * 1024 + lq * 4;
            pq[q] = q * 32 * LPR * 16 + wave * kRecWave;
            asm volatile("" : "+v"(wq[q]), "+v"(pq[q]));
        }
        // One chunk of MT M tiles: every LDS read of the chunk is issued first (the
        // B codes of both 32-column halves, their records as one 8-byte read per
        // row from rb, the chunk's place in its record buffer, the A tiles), then
        // each half is dequantised and multiplied.
        auto compute = [&](const Stage<NMAT> &st, const uint8_t *rb, auto mt_count) {
            constexpr int MT = decltype(mt_count)::value;
            const uint8_t *sb = reinterpret_cast<const uint8_t *>(&st);
            uint32_t codes[2][NMAT][2];
            uint64_t recs[NMAT][2];
#pragma unroll
            for (int q = 0; q < NMAT; ++q)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int rl = nt * 16 + lr;  // row within the wave's 32
                    recs[q][nt] = *reinterpret_cast<const uint64_t *>(rb + pq[q] + rl * RC * 8);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
                        codes[kb][q][nt] = *reinterpret_cast<const uint32_t *>(sb + wq[q] + (kb * 32 + rl) * 16);
                }
            uint4 av[2][MT];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int r = mt * 16 + lr;
                    av[kb][mt] = *reinterpret_cast<const uint4 *>(&st.x[r * kXRow + (((kb * 4 + lq) ^ (r & 7)) * 16)]);
                }
#pragma unroll
            for (int kb = 0; kb < kKC / 32; ++kb) {
                bf16x8_t bo[NMAT][2];
#pragma unroll
                for (int q = 0; q < NMAT; ++q)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        bo[q][nt] = dequant8(codes[kb][q][nt], (uint32_t)(recs[q][nt] >> (32 * kb)), dq);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, av[kb][mt]);
#pragma unroll
                    for (int q = 0; q < NMAT; ++q)
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt)
                            acc[q][mt][nt] =
                                __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bo[q][nt], acc[q][mt][nt], 0, 0, 0);
                }
            }
        };

        // Step c (at position b of the unrolled loop): wait until chunk c's stage
        // and its records have landed (exact vmcnt, from the fixed issue order),
        // barrier, refill the stage buffer freed by chunk c - 1 with chunk c + S - 1
        // and, at the start of a record group, the record buffer freed by the
        // previous group with the next group's records, then multiply.  Past the
        // last chunk (group) a step re-loads the last one into a buffer that is
        // not read again, so every step issues a fixed number of loads.
        const int ngroups = nchunks / RC;
        auto step = [&](int c, auto b_const, auto mt_count) {
            constexpr int b = decltype(b_const)::value;
            constexpr int P = (decltype(mt_count)::value + 1) / 2 + NMAT;  // loads of one stage
            __builtin_amdgcn_s_waitcnt(kWaitVm(vm_allow(S, RC, P, 1, U, b)));
            ring_barrier();
            issue(stage_addr((b + S - 1) % S), min(c + S - 1, nchunks - 1), mt_count);
            if (b % RC == 0) issue_rec(min(c / RC + 1, ngroups - 1), (c / RC + 1) & 1);
            compute(ring[b % S], &recs_lds[(c / RC) & 1][(b % RC) * 8], mt_count);
        };

        // The K loop, specialised on the pass's M tile count so that the chunk
        // body has no branches, and unrolled by U so that every step names its
        // buffers with constants.
        auto k_loop = [&](auto mt_count) {
            issue_rec(0, 0);
#pragma unroll
            for (int b = 0; b < S - 1; ++b) issue(stage_addr(b), min(b, nchunks - 1), mt_count);
            for (int c0 = 0; c0 < nchunks; c0 += U)
                static_for<0, U>([&](auto b_const) {
                    if (c0 + decltype(b_const)::value < nchunks) step(c0 + decltype(b_const)::value, b_const, mt_count);
                });
        };
        switch (mtiles) {
            case 1: k_loop(IntC<1>{}); break;
            case 2: k_loop(IntC<2>{}); break;
            case 3: k_loop(IntC<3>{}); break;
            case 4: k_loop(IntC<4>{}); break;
            case 5: k_loop(IntC<5>{}); break;
            default: k_loop(IntC<6>{}); break;
        }
        static_assert(kMaxMT == 6, "one k_loop case per M tile count");

        // no load may still be writing LDS when the workgroup moves on or exits
        __builtin_amdgcn_s_waitcnt(kWaitVm(0));

        // epilogue
#pragma unroll
        for (int mt = 0; mt < kMaxMT; ++mt) {
            if (mt >= mtiles) continue;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int n = n0 + wave * 32 + nt * 16 + lr;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int m = mt * 16 + lq * 4 + j;
                    if (m >= mc || n >= R) continue;
                    const int row = s_dst[m];
                    if (GATEUP) {
                        const float gv = acc[0][mt][nt][j], uv = acc[NMAT - 1][mt][nt][j];
                        a.h[(size_t)row * a.I + n] = (uint16_t)f32_to_bf16_bits(gv / (1.0f + expf(-gv)) * uv);
                    } else {
                        a.y[(size_t)row * a.H + n] = acc[0][mt][nt][j];
                    }
                }
            }
        }
    }
}

}  // namespace

namespace moe {

bool mfma_supported(const FfnArgs &a) { return a.grouped && a.H % 128 == 0 && a.I % 128 == 0; }

// Grid: kXcds workgroups per "expert slot" position, so that workgroup b runs on
// XCD b % kXcds and holds tile (b / kXcds) % ntiles of expert
// ((b / kXcds) / ntiles) * kXcds + b % kXcds (padding experts return at once).
template <bool GATEUP, int S, int RC>
int launch_mfma(const FfnArgs &a, hipStream_t s) {
    const int n_groups = a.n_routed_groups + (a.shared ? 1 : 0);
    const int ntiles = ((GATEUP ? a.I : a.H) + kNT - 1) / kNT;
    const unsigned slots = (unsigned)((n_groups + kXcds - 1) / kXcds);
    hipLaunchKernelGGL((mfma_ffn_kernel<GATEUP, S, RC>), dim3(slots * kXcds * ntiles), dim3(256), 0, s, a, ntiles,
                       n_groups);
    MOE_LAUNCH_CHECK(GATEUP ? "mfma_ffn_kernel<gate_up>" : "mfma_ffn_kernel<down>");
    return MOE_OK;
}

// Record groups: 2 chunks (128 columns) for gate/up, whose H is a multiple of
// 128; 4 chunks for the down projection when I is a multiple of 256, else 2.
int mfma_gate_up(const FfnArgs &a, hipStream_t s) { return launch_mfma<true, kStagesGateUp, 2>(a, s); }

int mfma_down(const FfnArgs &a, hipStream_t s) {
    return a.I % 256 == 0 ? launch_mfma<false, kStagesDown, 4>(a, s) : launch_mfma<false, kStagesDown, 2>(a, s);
}

}  // namespace moe
