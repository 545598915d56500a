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
// The K dimension streams in chunks of 64 columns.  Direct global->LDS loads
// (global_load_lds_dwordx4) fill two rings: the activation tiles, one chunk per
// stage, S stages deep; and the weights (codes and (scale, min) records), G
// chunks per buffer, two buffers, so that each row's codes come as one G*32-byte
// piece and its records as one G*8-byte piece (every row is a separate access,
// and small per-row pieces bound the kernel well before HBM does).  While a
// chunk is multiplied the next S-1 activation chunks and the next weight group
// are in flight, and no registers hold data on its way to LDS.  Each wave loads its
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
#ifndef MOE_EXP_SCHED
#define MOE_EXP_SCHED 0
#endif

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kNT = 128;       // weight rows (N) of each matrix per workgroup
constexpr int kKC = 64;        // columns (K) per chunk
constexpr int kMaxMT = 6;      // 16-row M tiles per pass
constexpr int kMC = 16 * kMaxMT;
constexpr int kXRow = kKC * 2; // bytes of one activation row of a chunk (8 units of 16 B)
constexpr int kXcds = 8;       // workgroups are dealt to the XCDs round-robin
#ifndef MOE_MFMA_STAGES
#define MOE_MFMA_STAGES 2
#endif
#ifndef MOE_MFMA_REC_GROUP
#define MOE_MFMA_REC_GROUP 4
#endif
// Activation ring depth (12 KB stages; the tiles are L2 hits, shared by all
// tiles of an expert, so one chunk of lead hides them) and the record group of
// two-matrix workgroups; with the weight rings two workgroups fit a CU.
constexpr int kStagesGateUp = MOE_MFMA_STAGES;
constexpr int kStagesDown = MOE_MFMA_STAGES;
constexpr int kRecGroup = MOE_MFMA_REC_GROUP;

// Activation ring stage: one chunk's tile, row r's 16-byte unit u stored at unit
// position u ^ (r & 7).
struct __attribute__((aligned(16))) XStage {
    uint8_t x[kMC * kXRow];
};

// Weight rings, per wave (32 rows of each of NMAT matrices) a block in each:
//   codes   [NMAT][32 rows][G*32 B], one group of G chunks per buffer: row r's
//           16-byte unit u at unit position u ^ swz(r), so that the B-operand
//           reads of 16 rows hit distinct banks
//   records [NMAT][32 rows][R*8 B], one group of R chunks per buffer, at least
//           1 KB: every 64-lane 16-byte load fills 1 KB (with one matrix and
//           R = 2, lanes beyond 32 repeat the first ones into the rest)
// A row's G*32 code bytes (R*8 record bytes) are fetched by adjacent lanes as
// one piece: the memory pipeline tracks a bounded number of requests per CU, and
// a request carries one row's piece of at most 64 bytes, so bytes per row and
// fetch set the kernel's load bandwidth well below HBM's.
template <int NMAT, int G, int R>
struct WLayout {
    static constexpr int row_code = G * 32;                  // code bytes of one row and group
    static constexpr int codes = NMAT * 32 * row_code;        // per wave
    static constexpr int code_loads = codes / 1024;           // 16-byte loads per wave and group
    static constexpr int row_rec = R * 8;                     // record bytes of one row and group
    static constexpr int recs = NMAT * 32 * row_rec < 1024 ? 1024 : NMAT * 32 * row_rec;
    static constexpr int rec_loads = recs / 1024;
    static constexpr int rec_lanes = NMAT * 32 * row_rec / 16;  // lanes with distinct data
    // unit swizzle of row r (2G units per row): for any one unit, 16 rows that
    // start at a multiple of 16 land in 16 distinct 16-byte slots of a 256-byte
    // bank window
    __device__ static int swz(int r) { return (r >> (G == 2 ? 2 : 1)) & (2 * G - 1); }
};

// Loads a wave may still have in flight when step c waits, such that chunk c's
// activations, its code group and its record group have all landed (vmcnt
// counts a wave's loads in issue order).  Issue order: records of group 0 (NR
// loads), codes of group 0 (NC), activation stages 0 .. S-2 (P each); then step
// j issues stage j+S-1, the codes of group j/G + 1 when G divides j and the
// records of group j/R + 1 when R divides j.  The count is the number of loads
// issued, before step c, after the last of the three it needs.
constexpr int newer_loads(int S, int P, int G, int NC, int R, int NR, int c) {
    int total = NR + NC, pos_x = 0, pos_code = NR + NC, pos_rec = NR;
    for (int b = 0; b < S - 1; ++b) {
        total += P;
        if (b == c) pos_x = total;
    }
    for (int j = 0; j < c; ++j) {
        total += P;
        if (j + S - 1 == c) pos_x = total;
        if (j % G == 0) {
            total += NC;
            if (j / G + 1 == c / G) pos_code = total;
        }
        if (j % R == 0) {
            total += NR;
            if (j / R + 1 == c / R) pos_rec = total;
        }
    }
    int need = pos_x > pos_code ? pos_x : pos_code;
    need = need > pos_rec ? need : pos_rec;
    return total - need;
}
// The same for every step at position b of a loop unrolled by U (a multiple of
// S, G and R: the pattern repeats with period U after the first U steps).
constexpr int vm_allow(int S, int P, int G, int NC, int R, int NR, int U, int b) {
    int m = newer_loads(S, P, G, NC, R, NR, b);
    for (int r = 1; r < 4; ++r) {
        const int v = newer_loads(S, P, G, NC, R, NR, b + r * U);
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

// Direct global->LDS load: lane l's 16 bytes from g land at LDS byte lds + 16*l;
// lds must be the same in every lane.  Written as inline asm
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

// NMAT weight matrices of 128 rows per workgroup: W1 and W3 for gate/up; for
// the down projection two 128-row tiles of W2 (PAIR, H a multiple of 256, so
// that every activation tile loaded serves 256 weight rows) or one.
template <bool GATEUP, int S, int G, int R, bool PAIR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mfma_ffn_kernel(moe::FfnArgs a, int ntiles,
                                                                                           int n_groups) {
    constexpr int NMAT = GATEUP || PAIR ? 2 : 1;
    constexpr int kTileN = GATEUP ? kNT : NMAT * kNT;  // output columns per workgroup
    using WL = WLayout<NMAT, G, R>;
    static_assert(S >= 2, "the activation ring needs two stages at least");
    static_assert((G == 2 || G == 4) && (R == 2 || R == 4 || R == 8), "weight group sizes");
    static_assert(S * sizeof(XStage) + 2 * 4 * (WL::codes + WL::recs) + 2 * kMC * sizeof(int) <= 80 * 1024,
                  "two workgroups per CU");
    constexpr int U = lcm(lcm(S, G), R);  // steps per unrolled loop body
    const int K = GATEUP ? a.H : a.I;   // reduction length (a multiple of 64 * G and 64 * R)
    const int nrows = GATEUP ? a.I : a.H;  // weight rows (output columns)
    // Which group and tile: by default every tile of one expert on the same XCD
    // (its activation tiles are then fetched into one L2).  Compact (a launch
    // where few groups qualify, the many-token experts of the split path):
    // workgroup b takes tile b % ntiles of the (b / ntiles)-th qualifying group
    // in group order, so each expert's tiles are dealt over all XCDs and the
    // XCDs get equal shares however the qualifying experts are numbered.
    int g, tile;
    if (a.compact) {
        __shared__ int s_g, s_wcnt[4];
        const int j = blockIdx.x / ntiles;
        tile = blockIdx.x % ntiles;
        const int t = threadIdx.x, ln = t & 63, w = t >> 6;
        if (t == 0) s_g = -1;
        int before = 0;  // qualifying groups in earlier chunks
        for (int c0 = 0; c0 < a.n_routed_groups; c0 += 256) {
            const int gg = c0 + t;
            bool act = false;
            if (gg < a.n_routed_groups) {
                const int M = a.count[gg];
                act = M > 0 && M >= a.min_m && M <= a.max_m && (!a.mask || a.mask[gg]);
            }
            const uint64_t bal = __ballot(act);
            __syncthreads();  // s_wcnt of the previous chunk has been read
            if (ln == 0) s_wcnt[w] = __popcll(bal);
            __syncthreads();
            int wb = 0;
            for (int v = 0; v < w; ++v) wb += s_wcnt[v];
            if (act && before + wb + __popcll(bal & ((1ull << ln) - 1)) == j) s_g = gg;
            before += s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
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
    if (g >= n_groups) return;
    const int n0 = tile * kTileN;

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
    moe::MatRows mat[2] = {GATEUP ? moe::slab_w1(slab, a.H, a.I) : moe::slab_w2(slab, a.H, a.I),
                           moe::slab_w3(slab, a.H, a.I)};
    if (!GATEUP) {  // matrix 1 of a pair: the W2 rows 128 further on
        mat[1] = mat[0];
        mat[1].row0 += (size_t)kNT * mat[0].stride;
    }
    const uint16_t *act = GATEUP ? a.x : a.h;

    __shared__ XStage ring[S];
    __shared__ __attribute__((aligned(16))) uint8_t cring[2][4 * WL::codes];
    __shared__ __attribute__((aligned(16))) uint8_t rring[2][4 * WL::recs];
    const uint32_t ring_lds = lds_addr(&ring[0]);
    const uint32_t cring_lds = lds_addr(&cring[0][0]), rring_lds = lds_addr(&rring[0][0]);
    auto stage_addr = [&](int b) { return ring_lds + (uint32_t)(b * sizeof(XStage)); };
    __shared__ int s_src[kMC];  // activation row of each M row
    __shared__ int s_dst[kMC];  // output row of each M row (-1 = padding)
    const Dequant dq = dequant_consts();
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lq = lane >> 4;  // MFMA row-in-tile and k-quarter
    const int nchunks = K / kKC, ncgroups = nchunks / G, nrgroups = nchunks / R;
    const int wrow0 = n0 + 32 * wave;  // first weight row of this wave

    // This lane's weight sources, fixed over the kernel (a group adds grp*G*32
    // to the codes, grp*G*8 to the records).  Code load j = q*G + h covers rows
    // h*32/G .. of matrix q: lane l takes row h*32/G + l/(2G), unit (l % 2G) ^ swz.
    const uint8_t *csrc[NMAT * G];
#pragma unroll
    for (int j = 0; j < NMAT * G; ++j) {
        const int q = j / G, h = j % G;
        const int r = h * (32 / G) + lane / (2 * G), u = (lane % (2 * G)) ^ WL::swz(r);
        csrc[j] = mat[q].row0 + (size_t)(wrow0 + r) * mat[q].stride + u * 16;
    }
    // records: load j, lane l takes piece f = (64j + l) mod rec_lanes, 16 bytes
    // (part f % LPR) of row (f / LPR) % 32 of matrix f / (32 LPR)
    const uint8_t *rsrc[WL::rec_loads];
#pragma unroll
    for (int j = 0; j < WL::rec_loads; ++j) {
        constexpr int LPR = R / 2;  // lanes per row
        const int f = (64 * j + lane) % WL::rec_lanes;
        const int q = f / (32 * LPR), r = (f % (32 * LPR)) / LPR, part = f % LPR;
        const moe::MatRows &m = q ? mat[1] : mat[0];
        rsrc[j] = m.row0 + (size_t)(wrow0 + r) * m.stride + K / 2 + part * 16;
    }
    // code group grp into code buffer buf, record group grp into record buffer buf
    auto issue_c = [&](int grp, int buf) {
        const uint32_t wb = cring_lds + (uint32_t)(buf * 4 * WL::codes + wave * WL::codes);
#pragma unroll
        for (int j = 0; j < WL::code_loads; ++j) dma16(csrc[j] + grp * G * 32, wb + (uint32_t)(j * 1024));
    };
    auto issue_r = [&](int grp, int buf) {
        const uint32_t wb = rring_lds + (uint32_t)(buf * 4 * WL::recs + wave * WL::recs);
#pragma unroll
        for (int j = 0; j < WL::rec_loads; ++j) dma16(rsrc[j] + grp * R * 8, wb + (uint32_t)(j * 1024));
    };

    // B-operand read offsets in a wave block: row rl = nt*16 + lr of matrix q,
    // the k-quarter's dword; the unit position is XORed with swz(rl) per read
    int cq[NMAT][2], swz16[2], rq[NMAT][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int rl = nt * 16 + lr;
        swz16[nt] = WL::swz(rl) * 16;
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {
            cq[q][nt] = wave * WL::codes + q * 32 * WL::row_code + rl * WL::row_code + lq * 4;
            rq[q][nt] = wave * WL::recs + q * 32 * WL::row_rec + rl * WL::row_rec;
        }
    }

    for (int m0 = 0; m0 < M; m0 += kMC) {
        const int mc = min(kMC, M - m0);
        const int mtiles = (mc + 15) >> 4;
        __syncthreads();  // the previous pass is done with s_src / s_dst and the rings
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
        // chunk c's activation tile into the stage at LDS address st
        auto issue_x = [&](uint32_t st, int c, auto mt_count) {
            constexpr int XJ = (decltype(mt_count)::value + 1) / 2;
            const int k0 = c * kKC;
#pragma unroll
            for (int j = 0; j < XJ; ++j) dma16(xsrc[j] + k0, st + (uint32_t)((wave + 4 * j) * 1024));
        };

        f32x4_t acc[NMAT][kMaxMT][2];
#pragma unroll
        for (int q = 0; q < NMAT; ++q)
#pragma unroll
            for (int mt = 0; mt < kMaxMT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc[q][mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // One chunk (chunk cg of its code group in code buffer cb, chunk cr of its
        // record group in record buffer rb) of MT M tiles: every LDS read of the
        // chunk is issued first (the B codes of both 32-column halves, their
        // records as one 8-byte read per row, the A tiles), then each half is
        // dequantised and multiplied.
        auto compute = [&](const XStage &st, const uint8_t *cb, auto cg_const, const uint8_t *rb, auto cr_const,
                           auto mt_count) {
            constexpr int MT = decltype(mt_count)::value;
            constexpr int cg = decltype(cg_const)::value, cr = decltype(cr_const)::value;
            uint32_t codes[2][NMAT][2];
            uint64_t recs[NMAT][2];
#pragma unroll
            for (int q = 0; q < NMAT; ++q)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    recs[q][nt] = *reinterpret_cast<const uint64_t *>(rb + rq[q][nt] + cr * 8);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
                        codes[kb][q][nt] =
                            *reinterpret_cast<const uint32_t *>(cb + cq[q][nt] + (((2 * cg + kb) * 16) ^ swz16[nt]));
                }
            uint4 av[2][MT];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int r = mt * 16 + lr;
                    av[kb][mt] = *reinterpret_cast<const uint4 *>(&st.x[r * kXRow + (((kb * 4 + lq) ^ (r & 7)) * 16)]);
                }
#if MOE_EXP_SCHED
            // one B tile at a time: its dequantisation, then its MT products, so
            // that the products of one tile run while the next is dequantised
#pragma unroll
            for (int kb = 0; kb < kKC / 32; ++kb)
#pragma unroll
                for (int q = 0; q < NMAT; ++q)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const bf16x8_t B = dequant8(codes[kb][q][nt], (uint32_t)(recs[q][nt] >> (32 * kb)), dq);
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            acc[q][mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, av[kb][mt]), B, acc[q][mt][nt], 0, 0, 0);
#if MOE_EXP_SCHED == 2
                        __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, MT, 0);
#endif
                    }
#else
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
#endif
        };

        // Step c (at position b of the unrolled loop): wait until chunk c's
        // activations, codes and records have landed (exact vmcnt, from the fixed
        // issue order), barrier, refill the stage freed by chunk c - 1 with chunk
        // c + S - 1 and, at the start of a code (record) group, the buffer freed by
        // the previous group with the next group, then multiply.  Past the last
        // chunk (group) a step re-loads the last one into a buffer that is not
        // read again, so every step issues a fixed number of loads.
        auto step = [&](int c, auto b_const, auto mt_count) {
            constexpr int b = decltype(b_const)::value;
            constexpr int P = (decltype(mt_count)::value + 1) / 2;  // activation loads of one stage
            __builtin_amdgcn_s_waitcnt(
                kWaitVm(vm_allow(S, P, G, WL::code_loads, R, WL::rec_loads, U, b)));
            ring_barrier();
            issue_x(stage_addr((b + S - 1) % S), min(c + S - 1, nchunks - 1), mt_count);
            if (b % G == 0) issue_c(min(c / G + 1, ncgroups - 1), (c / G + 1) & 1);
            if (b % R == 0) issue_r(min(c / R + 1, nrgroups - 1), (c / R + 1) & 1);
            compute(ring[b % S], &cring[(c / G) & 1][0], IntC<b % G>{}, &rring[(c / R) & 1][0], IntC<b % R>{},
                    mt_count);
        };

        // The K loop, specialised on the pass's M tile count so that the chunk
        // body has no branches, and unrolled by U so that every step names its
        // buffers with constants.
        auto k_loop = [&](auto mt_count) {
            issue_r(0, 0);
            issue_c(0, 0);
#pragma unroll
            for (int b = 0; b < S - 1; ++b) issue_x(stage_addr(b), min(b, nchunks - 1), mt_count);
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
                    if (m >= mc || n >= nrows) continue;
                    const int row = s_dst[m];
                    if (GATEUP) {
                        const float gv = acc[0][mt][nt][j], uv = acc[1][mt][nt][j];
                        a.h[(size_t)row * a.I + n] = (uint16_t)f32_to_bf16_bits(gv / (1.0f + expf(-gv)) * uv);
                    } else {
#pragma unroll
                        for (int q = 0; q < NMAT; ++q) a.y[(size_t)row * a.H + n + q * kNT] = acc[q][mt][nt][j];
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
template <bool GATEUP, int S, int G, int R, bool PAIR = false>
int launch_mfma(const FfnArgs &a, hipStream_t s) {
    const int n_groups = a.n_routed_groups + (a.shared ? 1 : 0);
    const int ntiles = GATEUP ? a.I / kNT : a.H / (PAIR ? 2 * kNT : kNT);
    const unsigned slots = (unsigned)((n_groups + kXcds - 1) / kXcds);
    hipLaunchKernelGGL((mfma_ffn_kernel<GATEUP, S, G, R, PAIR>), dim3(slots * kXcds * ntiles), dim3(256), 0, s, a,
                       ntiles, n_groups);
    MOE_LAUNCH_CHECK(GATEUP ? "mfma_ffn_kernel<gate_up>" : "mfma_ffn_kernel<down>");
    return MOE_OK;
}

// Two matrices per workgroup (gate/up, and the down projection when H is a
// multiple of 256): code groups of 2 chunks (64 bytes per row), record groups
// of 4 chunks (32 bytes per row) when the reduction length is a multiple of 256,
// else 2.  One matrix: code and record groups of 4 chunks (a 128-byte line of
// codes per row) when I is a multiple of 256, else 2.
int mfma_gate_up(const FfnArgs &a, hipStream_t s) {
    return a.H % 256 == 0 ? launch_mfma<true, kStagesGateUp, 2, kRecGroup>(a, s)
                          : launch_mfma<true, kStagesGateUp, 2, 2>(a, s);
}

int mfma_down(const FfnArgs &a, hipStream_t s) {
    if (a.H % (2 * kNT) == 0)
        return a.I % 256 == 0 ? launch_mfma<false, kStagesDown, 2, kRecGroup, true>(a, s)
                              : launch_mfma<false, kStagesDown, 2, 2, true>(a, s);
    return a.I % 256 == 0 ? launch_mfma<false, kStagesDown, 4, 4>(a, s) : launch_mfma<false, kStagesDown, 2, 2>(a, s);
}

}  // namespace moe
