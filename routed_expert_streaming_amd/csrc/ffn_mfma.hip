// Expert FFN for many tokens per expert (prefill): grouped GEMM on MFMA with
// the 4-bit weights dequantised in registers.
//
// The multi-token case is a dense contraction per expert: the tokens routed to
// expert e (gathered through the token->expert permutation) form an M_e x K
// activation matrix that meets the expert's W1/W3 (K = H -> I) and then W2
// (K = I -> H).  A workgroup (8 waves) owns one expert and 256 rows of W1 and
// of W3 (gate/up) or 512 rows of W2 (down) and covers the expert's tokens in
// passes of up to 96, so at prefill sizes (about 64 tokens per expert) every
// weight byte is read from HBM once and every activation tile read from L2
// serves 512 weight rows.
//
// Weights go from HBM straight into registers, already in the lane order of
// the MFMA B operand, so they need neither LDS nor any synchronisation between
// waves.  v_mfma_f32_16x16x32_bf16 (checked on gfx950: lane l holds
// A[l%16][8*(l/16)+j], B[8*(l/16)+j][l%16] for j < 8, and C[4*(l/16)+j][l%16]
// for j < 4) is fed with the K dimension permuted inside each 128-column group
// (four 32-column blocks): lane quarter q = l/16 owns block q of the group, and
// MFMA step s (of 4) takes the block's columns 8s..8s+7.  So a lane loads the 16
// code bytes of one block of its weight row (one 16-row tile: 16 rows x 64
// contiguous bytes per load instruction), and each of the block's four 8-column
// words is one B operand.  A sum over K is the same in any order of K, and the
// activations (A operand) are read in the same permuted order from LDS.
// The (scale, min) records of 16 blocks (four groups) come in one 16-byte load
// per lane (64 contiguous bytes per row per instruction), lane quarter q taking
// blocks 4q..4q+3, straight into a per-wave LDS area in lane order, where the
// record each lane needs in each of the four groups (that of the block it owns)
// is one 4-byte read away.  Codes run 2 groups ahead in a register ring,
// records one 4-group step ahead.
//
// Activations: the workgroup copies each group's tile (the pass's token rows x
// 128 columns, bf16) into an LDS ring of 3 stages with direct global->LDS loads
// (global_load_lds_dwordx4), 2 groups ahead; row m's 16-byte unit u sits at
// unit position u ^ (m % 16), so that the 16 rows an A-operand read touches hit
// distinct banks.  One barrier per group: each wave first waits (exact vmcnt,
// from the fixed issue order) until its own part of the next group's tile has
// landed; the barrier then makes every wave's part visible and frees the stage
// the next copy overwrites.  Weights are dequantised per 8-column word (scale*q
// + min in fp32, rounded to bf16) and the products accumulate in fp32.
// Workgroups are numbered so that every tile of one expert runs on the same
// XCD, where the expert's gathered activation rows are shared through the L2.
//
// Every load a wave issues in the K loop is SGPR base + 32-bit lane offset, and
// the code ring slot of group g is g % 2, a constant of the 4-group unrolled
// body: no 64-bit per-lane pointers and no register copies of loads in flight,
// either of which made the compiler drain every load in flight once per group.
// Measured at the 2048-token prefill shape (one layer, all 256 experts): the
// weight stream alone runs at 5.7 TB/s in this pattern, the kernel at about
// 2.5 TB/s; counters put the matrix cores at about 22% of SIMD time and the
// dequantisation (about 5 VALU instructions per MFMA) at about 31%, rarely
// co-executing -- the compute issue, not HBM, bounds it.
#include "common.h"
#include "dequant.h"
#include "ffn.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

#ifndef MOE_MFMA_SCHED_BARRIER
#define MOE_MFMA_SCHED_BARRIER 0
#endif
#ifndef MOE_MFMA_MAX_MT
#define MOE_MFMA_MAX_MT 6
#endif
#ifndef MOE_MFMA_CODE_AHEAD
#define MOE_MFMA_CODE_AHEAD 2
#endif
#ifndef MOE_MFMA_WAVES
#define MOE_MFMA_WAVES 8
#endif
constexpr int kWaves = MOE_MFMA_WAVES;   // waves per workgroup (4, 8 or 16: one, two or four per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kTM = 32 / kWaves;         // 16-row weight tiles per wave (512 rows per workgroup)
constexpr int kRowsGateUp = 256;         // rows of W1 (and of W3) per workgroup
constexpr int kRowsDown = 512;           // rows of W2 per workgroup
constexpr int kGK = 128;                 // columns per group (4 blocks of 32)
constexpr int kMaxMT = MOE_MFMA_MAX_MT;  // 16-row M tiles per pass
constexpr int kMC = 16 * kMaxMT;         // tokens per pass
constexpr int kXRow = kGK * 2;           // bytes of one activation row of a group (16 units of 16 B)
constexpr int kStages = 3;               // activation ring stages
constexpr int kAhead = 2;                // activation groups copied ahead (kStages - 1)
constexpr int kCodeAhead = MOE_MFMA_CODE_AHEAD;  // code groups in the register ring
constexpr int kXcds = 8;                 // workgroups are dealt to the XCDs round-robin
static_assert(kAhead == kStages - 1, "the stage a copy overwrites is the one read a step earlier");
static_assert(kCodeAhead == 2 || kCodeAhead == 4, "code ring slots are addressed by the step index mod 4");
static_assert(kWaves == 4 || kWaves == 8 || kWaves == 16, "workgroup of 4, 8 or 16 waves");

struct __attribute__((aligned(16))) XStage {
    uint8_t x[kMC * kXRow];
};

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(1))) const moe_u32x4 gu32x4;

__device__ __forceinline__ uint32_t lds_addr(const void *lds) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_u8 *)lds);
}
// Direct global->LDS load: lane l's 16 bytes from g land at LDS byte lds + 16*l
// (lds uniform).  Written as inline asm because the compiler, seeing these
// loads, would make every later LDS read wait for all of them (it cannot tell
// the ring's stages apart); completion is tracked with explicit vmcnt waits
// instead.  The memory clobber keeps the compiler's own loads in program order
// around it, which the wait counts rely on.
// base (uniform, in SGPRs) + off (this lane's 32-bit byte offset).
// The s_nop gives the 5 wait states a vector memory instruction needs after a
// VALU instruction wrote an SGPR it reads (and the one after an M0 write): the
// compiler inserts these for its own instructions but cannot see into inline
// asm, and under register pressure it restores a spilled base half with
// v_readlane right before the load -- without the wait the load can use the
// stale half and go to a wrong address.
__device__ __forceinline__ void dma16(const void *base, uint32_t off, uint32_t lds) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

constexpr int kWaitVm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }

// Loads a wave may still have in flight at the end of step gstep such that the
// activation tile gstep + 1 has landed (vmcnt counts a wave's loads in issue
// order).  Issue order: the records of step 0 (TM loads); for c < A: tile c (P
// loads) and, for c < D, the codes of group c (TM loads); then per step s:
// [records of step s/4 + 1 when s % 4 == 0], tile s + A, codes of group s + D.
// gstep < 0: the wait before step 0, for tile 0.
constexpr int loads_after_tile(int A, int D, int P, int TM, int gstep) {
    const int t = gstep + 1;
    int count = 0;
    bool seen = false;
    for (int c = 0; c < A; ++c) {
        if (seen) count += P;
        if (c == t) seen = true;
        if (c < D && seen) count += TM;
    }
    for (int s = 0; s <= gstep; ++s) {
        if (s % 4 == 0 && seen) count += TM;
        if (seen) count += P;
        if (s + A == t) seen = true;
        if (seen) count += TM;
    }
    return count;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt %0" ::"n"(kWaitVm(N)) : "memory");
}

// Workgroup barrier without a memory fence (a fence would wait for every load
// in flight); this wave's LDS reads are complete before it arrives.
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
// four extractions for one shift.  Each half is widened and scale*(base + q) +
// (min - base*scale) computed in fp32 with one rounding, which equals
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

// sc = the block's scale, c_lo = min - 1024*scale, c_hi = min - 64*scale (fp32)
__device__ __forceinline__ bf16x8_t dequant8(uint32_t codes, float sc, float c_lo, float c_hi, const Dequant &d) {
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

// MXFP4: 8 consecutive weights of one row (codes dword, the block's scale
// 2^(v-127) as a float) -> bf16x8 in column order: gfx950's scaled convert
// turns byte j of the dword (columns 2j, 2j+1) into two bf16 values, exactly
// (an E2M1 value times a power of two needs two significant bits).
__device__ __forceinline__ bf16x8_t dequant8_mx(uint32_t codes, float scale) {
    const uint32_t w01 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
    const uint32_t w23 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
    const uint32_t w45 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
    const uint32_t w67 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
    return __builtin_bit_cast(bf16x8_t, make_uint4(w01, w23, w45, w67));
}

// E8M0 scale byte -> 2^(v-127) (v = 255: NaN)
__device__ __forceinline__ float e8m0_scale(uint32_t v) {
    return v == 255u ? __builtin_nanf("") : ldexpf(1.0f, (int)v - 127);
}

// Super-block header -> block j's scale d*s_j and min -dmin*m_j (exact in fp32).
__device__ __forceinline__ void sb_block_params(const uint4 hdr, int j, float &sc, float &mn) {
    const float d = fp16_bits_to_f32(hdr.x & 0xFFFFu), dmin = fp16_bits_to_f32(hdr.x >> 16);
    const uint64_t fs = (uint64_t)hdr.y | ((uint64_t)(hdr.z & 0xFFFFu) << 32);
    const uint64_t fm = (uint64_t)(hdr.z >> 16) | ((uint64_t)hdr.w << 16);
    sc = d * (float)(uint32_t)((fs >> (6 * j)) & 63u);
    mn = -dmin * (float)(uint32_t)((fm >> (6 * j)) & 63u);
}

// 16 bytes at base (uniform) + off (this lane's 32-bit byte offset): one load
// with the base in SGPRs, so a lane keeps only its 32-bit offsets
__device__ __forceinline__ uint4 load_u4(const uint8_t *base, uint32_t off) {
    // the empty asm hides that off is loop-invariant: otherwise the compiler
    // hoists base' + off into a 64-bit per-lane pointer (two VGPRs per load, and
    // a 64-bit add per step into registers whose previous load may still be in flight)
    asm volatile("" : "+v"(off));
    const moe_u32x4 v = *(const gu32x4 *)(base + off);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t word(const uint4 &v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// GATEUP: W1 and W3 (tiles 0, 1 of each: the wave's 32 rows), h = bf16(silu(g) * u);
// otherwise W2 (tiles 0..3: the wave's 64 rows), y = W2 h.
// FMT: weight format.  The codes are laid out alike in all three; the block
// parameters of a 4-group step of a row are 64 bytes of (scale, min) records
// (format 0), 16 E8M0 scale bytes (1: every lane quarter loads the same 16) or
// two 16-byte super-block headers (2: quarter q loads header q & 1).
// SCALED (MXFP4 only): the products run on v_mfma_scale_f32_16x16x128_f8f6f4
// with the codes as its FP4 B operand (lane quarter q's 16 code bytes are block
// q of the 128-column group, K = 32q..32q+31: exactly the ring's loads) and the
// block's E8M0 byte as B's scale; the activations are FP8 digit pairs (hi, lo)
// with one E8M0 scale per row (quant_act below), hi and lo each the A operand
// of one product (A lane quarter q: columns 16q..16q+15 and 64+16q..64+16q+15,
// the order quant_act writes).  No dequantisation.
template <bool GATEUP, int FMT, bool SCALED = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4))) void mfma_ffn_kernel(moe::FfnArgs a,
                                                                                                   int ntiles,
                                                                                                   int n_groups) {
    static_assert(!SCALED || FMT == 1, "the block-scaled products take MXFP4 weights");
    const int K = GATEUP ? a.H : a.I;        // reduction length (a multiple of 128)
    const int nrows = GATEUP ? a.I : a.H;    // weight rows (output columns)
    const int wg_rows = GATEUP ? kRowsGateUp : kRowsDown;
    // Which group and tile: by default every tile of one expert on the same XCD
    // (its activation tiles are then fetched into one L2).  Compact (a launch
    // where few groups qualify, the many-token experts of the split path):
    // workgroup b takes tile b % ntiles of the (b / ntiles)-th qualifying group
    // in group order, so each expert's tiles are dealt over all XCDs and the
    // XCDs get equal shares however the qualifying experts are numbered.
    int g, tile;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (a.compact) {
        __shared__ int s_g, s_wcnt[kThreads / 64];
        const int j = blockIdx.x / ntiles;
        tile = blockIdx.x % ntiles;
        if (tid == 0) s_g = -1;
        int before = 0;  // qualifying groups in earlier chunks
        for (int c0 = 0; c0 < a.n_routed_groups; c0 += kThreads) {
            const int gg = c0 + tid;
            bool act = false;
            if (gg < a.n_routed_groups) {
                const int M = a.count[gg];
                act = M > 0 && M >= a.min_m && M <= a.max_m && (!a.mask || a.mask[gg]);
            }
            const uint64_t bal = __ballot(act);
            __syncthreads();  // s_wcnt of the previous chunk has been read
            if (lane == 0) s_wcnt[wave] = __popcll(bal);
            __syncthreads();
            int wb = 0;
            for (int v = 0; v < wave; ++v) wb += s_wcnt[v];
            if (act && before + wb + __popcll(bal & ((1ull << lane) - 1)) == j) s_g = gg;
            for (int v = 0; v < kThreads / 64; ++v) before += s_wcnt[v];
        }
        __syncthreads();
        g = s_g;
        if (g < 0) {  // past the routed groups: the shared expert comes last
            if (!(a.shared && j == before)) return;
            g = a.n_routed_groups;
        }
    } else {
        const int xcd = blockIdx.x % kXcds, i = blockIdx.x / kXcds;
        g = (i / ntiles) * kXcds + xcd;
        tile = i % ntiles;
    }
    // g and tile are uniform over the workgroup; saying so keeps the slab pointer
    // in SGPRs, so every weight load is SGPR base + 32-bit lane offset
    g = __builtin_amdgcn_readfirstlane(g);
    tile = __builtin_amdgcn_readfirstlane(tile);
    if (g >= n_groups) return;
    const int n0 = tile * wg_rows;

    // resolve the group: routed expert g (grouped), or the shared expert
    const uint8_t *slab;
    int M, base = 0;
    const bool routed = g < a.n_routed_groups;
    if (routed) {
        M = __builtin_amdgcn_readfirstlane(a.count[g]);  // uniform: M-tile checks become scalar branches
        if (M == 0 || M < a.min_m || M > a.max_m || (a.mask && a.mask[g] == 0)) return;
        // (the builtin returns a signed int: widen each half through uint32_t,
        // or a low half with bit 31 set would sign-extend over the high half)
        const uint64_t sp = (uint64_t)a.table[g];
        const uint32_t sp_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sp >> 32));
        const uint32_t sp_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sp);
        slab = (const uint8_t *)(((uint64_t)sp_hi << 32) | (uint64_t)sp_lo);
        base = __builtin_amdgcn_readfirstlane(a.offset[g]);
    } else {
        if (!a.shared || a.T < a.min_m || a.T > a.max_m) return;
        slab = (const uint8_t *)a.shared;
        M = a.T;
    }
    const uint16_t *act = GATEUP ? a.x : a.h;

    // This wave's weight tiles: gate/up rows n0 + 8*kTM*wave + 16t of W1 (tm = t)
    // and of W3 (tm = kTM/2 + t); down rows n0 + 16*kTM*wave + 16*tm of W2.  A wave past
    // the last row still issues its loads (from rows 0..15) so that every wave's
    // load counts match the waits below; it skips the products and stores.
    const int wrow0 = GATEUP ? n0 + 8 * kTM * wave : n0 + 16 * kTM * wave;
    const bool active = wrow0 < nrows;
    const int r = lane & 15, q = lane >> 4;
    const int ng = K / kGK;              // groups
    const int nh = (ng + 3) / 4;         // record steps (4 groups each)
    // byte offset in the slab of this lane's row of each tile (< 2^32: a slab is a
    // few tens of MB), plus 16*q: the lane's code bytes of group gg are block
    // 4*gg + q, at base + 64*gg; its records of step hh are those of blocks
    // 16*hh + 4q .. + 3, at base + K/2 + 64*hh (a lane whose blocks lie past the
    // row's last group reads the step's first ones instead; they go unused)
    uint32_t woff[kTM];
#pragma unroll
    for (int tm = 0; tm < kTM; ++tm) {
        const moe::MatRows m = GATEUP ? (tm < kTM / 2 ? moe::slab_w1<FMT>(slab, a.H, a.I)
                                                       : moe::slab_w3<FMT>(slab, a.H, a.I))
                                      : moe::slab_w2<FMT>(slab, a.H, a.I);
        const int row = active ? (GATEUP ? wrow0 + 16 * (tm % (kTM / 2)) : wrow0 + 16 * tm) + r : r;
        woff[tm] = (uint32_t)(m.row0 - slab) + (uint32_t)row * (uint32_t)m.stride + 16 * q;
    }
    constexpr int kStepRec = FMT == 0 ? 64 : FMT == 1 ? 16 : 32;  // parameter bytes of a row per step
    auto code_base = [&](int gg) { return slab + 64 * min(gg, ng - 1); };
    auto rec_base = [&](int hh) { return slab + K / 2 + kStepRec * min(hh, nh - 1); };
    auto rec_off = [&](int tm, int hh) -> uint32_t {
        if constexpr (FMT == 0)  // lanes whose four blocks lie past the last group read the step's first
            return 4 * min(hh, nh - 1) + q < ng ? woff[tm] : woff[tm] - 16 * q;
        else if constexpr (FMT == 1)
            return woff[tm] - 16 * q;
        else  // header 2*hh + (q & 1), or header 2*hh where that is the row's last
            return 2 * min(hh, nh - 1) + (q & 1) < ng / 2 ? woff[tm] - 16 * q + 16 * (q & 1) : woff[tm] - 16 * q;
    };

    __shared__ XStage ring[kStages];
    // records: [step parity][wave][tile] 1 KB, lane l's 16 bytes at 16*l
    __shared__ __attribute__((aligned(16))) uint8_t rring[2][kWaves][kTM][1024];
    __shared__ int s_src[kMC];  // activation row of each M row
    __shared__ int s_dst[kMC];  // output row of each M row (-1 = padding)
    __shared__ int s_asc[kMC];  // SCALED: E8M0 scale of each M row's activation row
    const uint32_t ring_lds = lds_addr(&ring[0]);
    const Dequant dq = SCALED ? Dequant{} : dequant_consts();

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
            if constexpr (SCALED) s_asc[tid] = a.act_scale[src];
            s_dst[tid] = tid < mc ? dst : -1;
        }
        __syncthreads();

        auto k_loop = [&](auto mt_count) {
            constexpr int MT = decltype(mt_count)::value;
            constexpr int RPI = 4 * kWaves;                // rows one copy instruction of every wave covers
            constexpr int P = (16 * MT + RPI - 1) / RPI;  // activation copy instructions per wave and group
            // activation copy: instruction j of this wave covers rows RPI*j + 4*wave .. + 3
            // (when those lie past the stage's kMC rows, the wave copies its rows of
            // instruction 0 again: the same bytes to the same place, so that every
            // wave issues the same number of loads); lane l takes row ... + l/16,
            // unit (l % 16) ^ (row % 16)
            static_assert(RPI <= kMC, "the first copy instruction stays inside a stage");
            uint32_t xoff[P], xrow[P];  // byte offsets in the activations (rows of K bf16); LDS row
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const int r0 = RPI * j + 4 * wave < kMC ? RPI * j + 4 * wave : 4 * wave;
                const int m = r0 + (lane >> 4);
                xrow[j] = (uint32_t)r0;
                xoff[j] = (uint32_t)s_src[m] * (uint32_t)(2 * K) + 16 * ((lane & 15) ^ (m & 15));
            }
            auto issue_x = [&](int gg) {  // group gg's tile into its stage
                const uint8_t *xb = (const uint8_t *)act + 2 * kGK * min(gg, ng - 1);
                const uint32_t st = ring_lds + (uint32_t)((gg % kStages) * sizeof(XStage));
#pragma unroll
                for (int j = 0; j < P; ++j) dma16(xb, xoff[j], st + xrow[j] * kXRow);
            };
            f32x4_t acc[kTM][MT];
#pragma unroll
            for (int tm = 0; tm < kTM; ++tm)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[tm][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

            // issue order (the waits below count on it): records of step 0; then
            // tiles 0 .. kAhead-1, each followed (for the first kCodeAhead) by
            // its group's codes; then per group g: [records of step g/4 + 1 when
            // g % 4 == 0], tile g + kAhead, products of group g, codes of group
            // g + kCodeAhead, wait for tile g + 1, barrier.  Group g's codes sit
            // in ring slot g % kCodeAhead, a constant in the 4-step unrolled body
            // (no register copies of loads in flight).
            uint4 cring[kCodeAhead][kTM];
            // records of step hh (4 groups) into their LDS area
            auto issue_r = [&](int hh) {
                const uint8_t *rb = rec_base(hh);
#pragma unroll
                for (int tm = 0; tm < kTM; ++tm) dma16(rb, rec_off(tm, hh), lds_addr(&rring[hh & 1][wave][tm][0]));
            };
            issue_r(0);
#pragma unroll
            for (int c = 0; c < kAhead; ++c) {
                issue_x(c);
                if (c < kCodeAhead)
#pragma unroll
                    for (int tm = 0; tm < kTM; ++tm) cring[c][tm] = load_u4(code_base(c), woff[tm]);
            }
            // tile 0 has landed once the loads issued after it are the only ones left
            wait_vm<loads_after_tile(kAhead, kCodeAhead, P, kTM, -1)>();
            ring_barrier();

            auto step = [&](int gg, auto b_const) {
                constexpr int b = decltype(b_const)::value;  // gg % 4
                // records of this step: loaded 4 groups ago (complete since the
                // wait for an activation tile issued after them)
                const uint8_t *rbuf = &rring[(gg / 4) & 1][wave][0][0];
                if (b == 0) issue_r(gg / 4 + 1);
                issue_x(gg + kAhead);
                constexpr int slot = b % kCodeAhead;
                // loads and waits run in every step of the unrolled body (past the
                // last group they re-read it), so that the compiler's own load
                // counts never meet a path that skipped them; only the products
                // are skipped
                if (SCALED && active && gg < ng) {
                    // B: the group's codes as loaded; its scale the block's E8M0 byte
                    // (byte 4b + q of the row's 16, quarter 0's copy)
                    const uint8_t *st = &ring[gg % kStages].x[0];
                    i32x8_t bv[kTM];
                    int bsc[kTM];
#pragma unroll
                    for (int tm = 0; tm < kTM; ++tm) {
                        const uint4 c = cring[slot][tm];
                        bv[tm] = i32x8_t{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
                        bsc[tm] = rbuf[tm * 1024 + r * 16 + 4 * b + q];
                    }
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        // A: row m's hi digits in units 2q, 2q+1 and lo digits in units
                        // 8+2q, 9+2q of its 16 (stored at unit ^ (m % 16), m % 16 = r)
                        const int m = 16 * mt + r;
                        const uint8_t *row = st + m * kXRow;
                        const uint4 h0 = *reinterpret_cast<const uint4 *>(row + 16 * ((2 * q) ^ r));
                        const uint4 h1 = *reinterpret_cast<const uint4 *>(row + 16 * ((2 * q + 1) ^ r));
                        const uint4 l0 = *reinterpret_cast<const uint4 *>(row + 16 * ((8 + 2 * q) ^ r));
                        const uint4 l1 = *reinterpret_cast<const uint4 *>(row + 16 * ((9 + 2 * q) ^ r));
                        const i32x8_t ahi{(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w,
                                          (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
                        const i32x8_t alo{(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w,
                                          (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
                        const int asc = s_asc[m];
#pragma unroll
                        for (int tm = 0; tm < kTM; ++tm) {
                            // cbsz 0: A is FP8 E4M3; blgp 4: B is FP4 E2M1
                            acc[tm][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                ahi, bv[tm], acc[tm][mt], 0, 4, 0, asc, 0, bsc[tm]);
                            acc[tm][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                alo, bv[tm], acc[tm][mt], 0, 4, 0, asc, 0, bsc[tm]);
                        }
                    }
                }
                if (!SCALED && active && gg < ng) {
                    const uint8_t *st = &ring[gg % kStages].x[0];
                    // each tile's block parameters (block 16h + 4b + q of this lane's
                    // row): scale and the two extraction offsets, or the MXFP4 scale
                    float sc[kTM], clo[kTM], chi[kTM];
#pragma unroll
                    for (int tm = 0; tm < kTM; ++tm) {
                        const uint8_t *rt = rbuf + tm * 1024;
                        if constexpr (FMT == 1) {  // byte 4b + q of the row's 16 (quarter 0's copy)
                            sc[tm] = e8m0_scale(rt[r * 16 + 4 * b + q]);
                            clo[tm] = chi[tm] = 0.0f;
                        } else {
                            float mn;
                            if constexpr (FMT == 0) {  // lane (row r, quarter b)'s word q
                                const uint32_t rec = *reinterpret_cast<const uint32_t *>(rt + (16 * b + r) * 16 + 4 * q);
                                sc[tm] = fp16_bits_to_f32(rec & 0xFFFFu);
                                mn = fp16_bits_to_f32(rec >> 16);
                            } else {  // header b / 2 of the step (quarter b / 2's copy), block 4 (b % 2) + q of it
                                const uint4 hdr = *reinterpret_cast<const uint4 *>(rt + (16 * (b >> 1) + r) * 16);
                                sb_block_params(hdr, 4 * (b & 1) + q, sc[tm], mn);
                            }
                            clo[tm] = fmaf(-1024.0f, sc[tm], mn);
                            chi[tm] = fmaf(-64.0f, sc[tm], mn);
                        }
                    }
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        bf16x8_t bo[kTM];
#pragma unroll
                        for (int tm = 0; tm < kTM; ++tm) {
                            if constexpr (FMT == 1)
                                bo[tm] = dequant8_mx(word(cring[slot][tm], s), sc[tm]);
                            else
                                bo[tm] = dequant8(word(cring[slot][tm], s), sc[tm], clo[tm], chi[tm], dq);
                        }
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            const int m = 16 * mt + r;
                            const bf16x8_t av = __builtin_bit_cast(
                                bf16x8_t, *reinterpret_cast<const uint4 *>(st + m * kXRow + 16 * ((4 * q + s) ^ r)));
#pragma unroll
                            for (int tm = 0; tm < kTM; ++tm)
                                acc[tm][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bo[tm], acc[tm][mt], 0, 0, 0);
                        }
#if MOE_MFMA_SCHED_BARRIER
                        __builtin_amdgcn_sched_barrier(0);
#endif
                    }
                }
                const uint8_t *cb = code_base(gg + kCodeAhead);
#pragma unroll
                for (int tm = 0; tm < kTM; ++tm) cring[slot][tm] = load_u4(cb, woff[tm]);
                // tile gg + 1 has landed once only the loads issued after it remain
                // (the first steps follow the prologue's order, later ones repeat
                // with period 4)
                if (gg < 4)
                    wait_vm<loads_after_tile(kAhead, kCodeAhead, P, kTM, b)>();
                else
                    wait_vm<loads_after_tile(kAhead, kCodeAhead, P, kTM, 4 + b)>();
                ring_barrier();
            };
            for (int g0 = 0; g0 < ng; g0 += 4)
                static_for<0, 4>([&](auto b_const) { step(g0 + decltype(b_const)::value, b_const); });
            // no copy may still be writing LDS when the workgroup moves on or exits
            wait_vm<0>();

            // epilogue
            if (active) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int m = 16 * mt + 4 * q + j;
                        if (m >= mc) continue;
                        const int row = s_dst[m];
                        if (GATEUP) {
#pragma unroll
                            for (int t = 0; t < kTM / 2; ++t) {
                                const int n = wrow0 + 16 * t + r;
                                const float gv = acc[t][mt][j], uv = acc[kTM / 2 + t][mt][j];
                                a.h[(size_t)row * a.I + n] = (uint16_t)f32_to_bf16_bits(gv / (1.0f + expf(-gv)) * uv);
                            }
                        } else {
#pragma unroll
                            for (int tm = 0; tm < kTM; ++tm) a.y[(size_t)row * a.H + wrow0 + 16 * tm + r] = acc[tm][mt][j];
                        }
                    }
            }
        };
        switch (mtiles) {
            case 1: k_loop(IntC<1>{}); break;
            case 2: k_loop(IntC<2>{}); break;
            case 3: k_loop(IntC<3>{}); break;
            case 4: k_loop(IntC<4>{}); break;
#if MOE_MFMA_MAX_MT >= 6
            case 5: k_loop(IntC<5>{}); break;
            default: k_loop(IntC<6>{}); break;
#else
            default: k_loop(IntC<5>{}); break;
#endif
        }
        static_assert(kMaxMT == 5 || kMaxMT == 6, "one k_loop case per M tile count");
    }
}

// ---------------------------------------------------------------- activations for the scaled products
// A bf16 row x becomes FP8 (E4M3) digit pairs with one E8M0 scale 2^u per row:
// u = e - 8 for the row's largest magnitude f * 2^e (f in [0.5, 1)), so every
// |x| / 2^u < 256; hi = x / 2^u truncated to E4M3 (3 mantissa bits; below 2^-6,
// E4M3's subnormals, to a multiple of 2^-9) and lo = x / 2^u - hi (exact in
// fp32) rounded to nearest even E4M3.  hi + lo equals x / 2^u whenever |x| >=
// 2^u / 4 (then lo's last bit is at or above E4M3's 2^-9): every element within
// 2^10 of the row's largest; smaller ones are off by at most 2^u * 2^-10.
// Output row, 2 bytes per element like the input: per 128-column group, 128 hi
// bytes then 128 lo bytes, each as four 32-byte chunks q holding columns
// 16q..16q+15 then 64+16q..64+16q+15 (the A operand of lane quarter q).
constexpr int kQuantThreads = 256;

// E4M3 byte of a value that E4M3 holds exactly (|v| < 256)
__device__ __forceinline__ uint32_t e4m3_exact(float v) {
    const uint32_t b = __float_as_uint(v), sign = (b >> 24) & 0x80u;
    const float a = fabsf(v);
    if (a < 0.015625f) return sign | (uint32_t)(a * 512.0f);  // subnormal (or zero): m * 2^-9
    const uint32_t e = ((b >> 23) & 0xFFu) - 127u + 7u, m = (b >> 20) & 7u;
    return sign | (e << 3) | m;
}

// E4M3 byte of v rounded to nearest, ties to even (|v| < 16 here)
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
    const uint32_t b = __float_as_uint(v), sign = (b >> 24) & 0x80u;
    const float a = fabsf(v);
    if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);  // 8 (rounded up) is the encoding of 2^-6
    const uint32_t ab = __float_as_uint(a);
    const uint32_t rb = ab + 0x7FFFFu + ((ab >> 20) & 1u);  // round the mantissa to 3 bits
    const uint32_t e = ((rb >> 23) & 0xFFu) - 127u + 7u, m = (rb >> 20) & 7u;
    return sign | (e << 3) | m;
}

__global__ __launch_bounds__(kQuantThreads) void quant_act_kernel(const uint16_t *x, int K, uint8_t *out,
                                                                  int32_t *scale) {
    extern __shared__ uint4 srow4[];  // the row, K bf16
    __shared__ float wmax[kQuantThreads / 64];
    const uint16_t *srow = reinterpret_cast<const uint16_t *>(srow4);
    const int row = blockIdx.x, tid = threadIdx.x;
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + (size_t)row * K);
    float mx = 0.0f;
    for (int i = tid; i < K / 8; i += kQuantThreads) {
        const uint4 v = xr[i];
        srow4[i] = v;
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            mx = fmaxf(mx, fmaxf(fabsf(bf16_bits_to_f32(w[j] & 0xFFFFu)), fabsf(bf16_bits_to_f32(w[j] >> 16))));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if ((tid & 63) == 0) wmax[tid >> 6] = mx;
    __syncthreads();  // also: the whole row is read before anything is written (out may alias x)
#pragma unroll
    for (int w = 0; w < kQuantThreads / 64; ++w) mx = fmaxf(mx, wmax[w]);
    int e = 0;
    (void)frexpf(mx, &e);
    const int u = mx > 0.0f ? max(-127, min(127, e - 8)) : -127;
    if (tid == 0) scale[row] = u + 127;
    uint32_t *orow = reinterpret_cast<uint32_t *>(out + (size_t)row * K * 2);
    for (int d = tid; d < K / 4; d += kQuantThreads) {  // hi dword d: group d/32, chunk (d%32)/8, bytes 4(d%8)..
        const int g = d >> 5, dd = d & 31, q = dd >> 3, j0 = 4 * (dd & 7);
        const int c0 = 128 * g + (j0 < 16 ? 16 * q + j0 : 64 + 16 * q + j0 - 16);
        uint32_t hi = 0, lo = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float y = ldexpf(bf16_bits_to_f32(srow[c0 + j]), -u);
            const float ay = fabsf(y);
            float h = ay < 0.015625f ? truncf(ay * 512.0f) * 0.001953125f
                                     : __uint_as_float(__float_as_uint(ay) & 0xFFF00000u);
            h = copysignf(h, y);
            hi |= e4m3_exact(h) << (8 * j);
            lo |= e4m3_rne(y - h) << (8 * j);
        }
        orow[64 * g + dd] = hi;
        orow[64 * g + 32 + dd] = lo;
    }
}

}  // namespace

namespace moe {

bool mfma_supported(const FfnArgs &a) {
    const int mult = a.fmt == 2 ? 256 : 128;  // super-blocks: whole headers per 4-group step pair
    return a.grouped && a.H % mult == 0 && a.I % mult == 0 && a.fmt >= 0 && a.fmt <= 2;
}

// Grid: kXcds workgroups per "expert slot" position, so that workgroup b runs on
// XCD b % kXcds and holds tile (b / kXcds) % ntiles of expert
// ((b / kXcds) / ntiles) * kXcds + b % kXcds (padding experts return at once).
template <bool GATEUP, int FMT, bool SCALED = false>
int launch_mfma(const FfnArgs &a, hipStream_t s) {
    const int n_groups = a.n_routed_groups + (a.shared ? 1 : 0);
    const int rows = GATEUP ? a.I : a.H, per = GATEUP ? kRowsGateUp : kRowsDown;
    const int ntiles = (rows + per - 1) / per;
    unsigned grid;
    if (a.compact)
        grid = (unsigned)(n_groups * ntiles);
    else
        grid = (unsigned)((n_groups + kXcds - 1) / kXcds * kXcds * ntiles);
    hipLaunchKernelGGL((mfma_ffn_kernel<GATEUP, FMT, SCALED>), dim3(grid), dim3(kThreads), 0, s, a, ntiles, n_groups);
    MOE_LAUNCH_CHECK(GATEUP ? "mfma_ffn_kernel<gate_up>" : "mfma_ffn_kernel<down>");
    return MOE_OK;
}

template <bool GATEUP>
int mfma_phase(const FfnArgs &a, hipStream_t s) {
    switch (a.fmt) {
        case 0: return launch_mfma<GATEUP, 0>(a, s);
        case 1: return launch_mfma<GATEUP, 1>(a, s);
        case 2: return launch_mfma<GATEUP, 2>(a, s);
    }
    return fail(MOE_E_ARG, "MFMA FFN: weight format %d", a.fmt);
}

int mfma_gate_up(const FfnArgs &a, hipStream_t s) { return mfma_phase<true>(a, s); }
int mfma_down(const FfnArgs &a, hipStream_t s) { return mfma_phase<false>(a, s); }

int mfma_gate_up_scaled(const FfnArgs &a, hipStream_t s) {
    if (a.fmt != 1 || !a.act_scale) return fail(MOE_E_ARG, "scaled MFMA gate/up: MXFP4 slabs and row scales needed");
    return launch_mfma<true, 1, true>(a, s);
}
int mfma_down_scaled(const FfnArgs &a, hipStream_t s) {
    if (a.fmt != 1 || !a.act_scale) return fail(MOE_E_ARG, "scaled MFMA down: MXFP4 slabs and row scales needed");
    return launch_mfma<false, 1, true>(a, s);
}

int quant_act(const uint16_t *x, int rows, int K, uint8_t *out, int32_t *scale, hipStream_t s) {
    if (rows <= 0) return MOE_OK;
    if (K <= 0 || K % 128 || K > 16384) return fail(MOE_E_SHAPE, "quant_act: K=%d (a multiple of 128, at most 16384)", K);
    const size_t lds = (size_t)K * 2;
    static bool raised = false;
    if (!raised) {
        hipError_t e = hipFuncSetAttribute((const void *)quant_act_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           16384 * 2);
        if (e != hipSuccess) return fail_hip(e, "hipFuncSetAttribute(quant_act_kernel)");
        raised = true;
    }
    hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)rows), dim3(kQuantThreads), lds, s, x, K, out, scale);
    MOE_LAUNCH_CHECK("quant_act_kernel");
    return MOE_OK;
}

}  // namespace moe
