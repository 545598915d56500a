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
// The K dimension streams in chunks of 64 columns through two LDS buffers: the
// next chunk's global loads (gathered activations, weight codes, (scale, min)
// records) are in flight in registers while the current chunk is multiplied,
// then land in the other buffer behind one barrier per chunk.  Each wave owns
// 32 N columns (of W1 and of W3 for gate/up): it dequantises its B operand from
// LDS into bf16 registers (scale*q + min in fp32, rounded to bf16) and
// accumulates v_mfma_f32_16x16x32_bf16 products in fp32.  Workgroups are
// numbered so that every tile of one expert runs on the same XCD, where the
// expert's gathered activation rows are shared through that XCD's L2.
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (checked on gfx950): lane l holds
// A[l%16][8*(l/16)+j], B[8*(l/16)+j][l%16] for j < 8, and C[4*(l/16)+j][l%16]
// for j < 4.
#include "common.h"
#include "ffn.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kNT = 128;       // weight rows (N) per workgroup
constexpr int kKC = 64;        // columns (K) per LDS chunk
constexpr int kMaxMT = 6;      // 16-row M tiles per chunk
constexpr int kMC = 16 * kMaxMT;
constexpr int kXStride = 144;  // bytes per staged activation row (128 + 16 pad)
constexpr int kWStride = 40;   // bytes per staged code row (32 + 8 pad: conflict-free B reads)
constexpr int kXcds = 8;       // workgroups are dealt to the XCDs round-robin
static_assert(kMC * (kKC * 2 / 16) % 256 == 0, "activation tile loads must divide over the workgroup");

struct MfmaBuf {
    __attribute__((aligned(16))) uint8_t x[kMC * kXStride];  // activation tile, bf16, natural column order
    uint8_t w[2][kNT * kWStride]; // code tiles (W1, W3) or (W2, -)
    uint2 p[2][kNT];              // (scale, min) records of the chunk's 2 blocks per row
};
struct __attribute__((aligned(16))) MfmaLds {  // 16-byte aligned: A operands load with ds_read_b128
    MfmaBuf buf[2];
    int src[kMC];                 // activation row of each M row (-1 = padding)
    int dst[kMC];                 // output row of each M row
};

// 8 consecutive weights of one row (codes dword, its block record) -> bf16x8.
// (w >> 4s) & 0x000F000F | 0x64006400 holds the fp16 values 1024 + q of columns
// s and s+4; v_fma_mix_f32 widens each half and computes
// scale*(1024+q) + (min - 1024*scale) in fp32 with one rounding, which equals
// fmaf(scale, q, min) whenever min - 1024*scale is exact in fp32 (scale and min
// within 2^12 of each other's magnitude); then round to bf16 in natural order.
__device__ __forceinline__ float fma_half(uint32_t pair, int hi, float sc, float c) {
    const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(hi ? pair >> 16 : pair & 0xFFFFu));
    return fmaf((float)h, sc, c);
}

// The fp16 exponent pattern 0x6400 in both halves, held in a VGPR so that
// (w & mask) | magic is one v_and_or_b32 (the mask goes in an SGPR).
__device__ __forceinline__ uint32_t fp16_magic_vgpr() {
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
    return m;
}

__device__ __forceinline__ bf16x8_t dequant8(uint32_t codes, uint32_t rec, uint32_t magic) {
    const float sc = fp16_bits_to_f32(rec & 0xFFFFu);
    const float mn = fp16_bits_to_f32(rec >> 16);
    const float c = fmaf(-1024.0f, sc, mn);
    const uint32_t mask = 0x000F000Fu;
    float f[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t p = ((codes >> (4 * s)) & mask) | (magic & ~mask);
        f[s] = fma_half(p, 0, sc, c);
        f[s + 4] = fma_half(p, 1, sc, c);
    }
    bf16x8_t v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (__bf16)f[j];
    return v;
}

template <bool GATEUP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mfma_ffn_kernel(moe::FfnArgs a, int ntiles,
                                                                                           int n_groups) {
    constexpr int NMAT = GATEUP ? 2 : 1;
    const int K = GATEUP ? a.H : a.I;   // reduction length
    const int R = GATEUP ? a.I : a.H;   // weight rows (output columns)
    const int nblk = K >> 5;
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
        if (M == 0 || (a.mask && a.mask[g] == 0)) return;
        slab = (const uint8_t *)a.table[g];
        base = a.offset[g];
    } else {
        if (!a.shared) return;
        slab = (const uint8_t *)a.shared;
        M = a.T;
    }
    const size_t m13 = (size_t)a.I * a.H * 5 / 8;
    const uint8_t *mat[2] = {slab + (GATEUP ? 0 : 2 * m13), slab + m13};
    const size_t cbytes = (size_t)R * K / 2;
    const uint16_t *act = GATEUP ? a.x : a.h;

    __shared__ MfmaLds s;
    const uint32_t magic = fp16_magic_vgpr();
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;  // MFMA row-in-tile and k-quarter
    const int nchunks = K / kKC;

    // per-thread share of one chunk's global loads
    constexpr int kXLoads = kMC * (kKC * 2 / 16) / 256;  // 16-byte activation loads per thread
    uint4 xr[kXLoads], wr[NMAT];
    uint2 pr = make_uint2(0u, 0u);
    auto load_chunk = [&](int c) {
        const int k0 = c * kKC;
#pragma unroll
        for (int q = 0; q < kXLoads; ++q) {  // activations: kMC rows x 128 B, 16 B per load
            const int idx = tid + 256 * q, row = idx >> 3, ch = idx & 7;
            const int src = s.src[row];
            xr[q] = src >= 0 ? load_global_u4(act + (size_t)src * K + k0 + ch * 8) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {  // codes: 128 rows x 32 B per matrix
            const int row = tid >> 1, ch = tid & 1, n = n0 + row;
            wr[q] = n < R ? load_stream_u4(mat[q] + (size_t)n * (K / 2) + k0 / 2 + ch * 16) : make_uint4(0u, 0u, 0u, 0u);
        }
        if (tid < NMAT * kNT) {  // records: 2 blocks x 4 B per row
            const int q = tid / kNT, row = tid - q * kNT, n = n0 + row;
            if (n < R) {
                const uint8_t *rp = mat[q] + cbytes + ((size_t)n * nblk + (k0 >> 5)) * 4;
                pr = make_uint2(load_stream_u32(rp), load_stream_u32(rp + 4));
            } else {
                pr = make_uint2(0u, 0u);
            }
        }
    };
    auto store_chunk = [&](int b) {
        MfmaBuf &B = s.buf[b];
#pragma unroll
        for (int q = 0; q < kXLoads; ++q) {
            const int idx = tid + 256 * q, row = idx >> 3, ch = idx & 7;
            *reinterpret_cast<uint4 *>(&B.x[row * kXStride + ch * 16]) = xr[q];
        }
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {
            const int row = tid >> 1, ch = tid & 1;
            *reinterpret_cast<uint4 *>(&B.w[q][row * kWStride + ch * 16]) = wr[q];
        }
        if (tid < NMAT * kNT) {
            const int q = tid / kNT, row = tid - q * kNT;
            B.p[q][row] = pr;
        }
    };

    for (int m0 = 0; m0 < M; m0 += kMC) {
        const int mc = min(kMC, M - m0);
        const int mtiles = (mc + 15) >> 4;
        __syncthreads();  // previous chunk done with s.src / s.dst and the buffers
        if (tid < kMC) {
            int src = -1, dst = -1;
            if (tid < mc) {
                const int m = m0 + tid;
                if (routed) {
                    const int p = a.pair_of_row[base + m];
                    dst = p;
                    src = GATEUP ? p / a.k : p;
                } else {
                    dst = a.T * a.k + m;
                    src = GATEUP ? m : dst;
                }
            }
            s.src[tid] = src;
            s.dst[tid] = dst;
        }
        __syncthreads();
        f32x4_t acc[NMAT][kMaxMT][2];
#pragma unroll
        for (int q = 0; q < NMAT; ++q)
#pragma unroll
            for (int mt = 0; mt < kMaxMT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc[q][mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        load_chunk(0);
        store_chunk(0);
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            const int cur = c & 1;
            if (c + 1 < nchunks) load_chunk(c + 1);  // in flight during this chunk's products
            const MfmaBuf &B = s.buf[cur];
#pragma unroll
            for (int kb = 0; kb < kKC / 32; ++kb) {
                // B operands: this wave's 2 N tiles of each matrix
                bf16x8_t bo[NMAT][2];
#pragma unroll
                for (int q = 0; q < NMAT; ++q)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const int row = wave * 32 + nt * 16 + lr;
                        const uint32_t codes =
                            *reinterpret_cast<const uint32_t *>(&B.w[q][row * kWStride + kb * 16 + lq * 4]);
                        const uint2 rec2 = B.p[q][row];
                        bo[q][nt] = dequant8(codes, kb == 0 ? rec2.x : rec2.y, magic);
                    }
#pragma unroll
                for (int mt = 0; mt < kMaxMT; ++mt) {
                    if (mt < mtiles) {
                        const uint4 av =
                            *reinterpret_cast<const uint4 *>(&B.x[(mt * 16 + lr) * kXStride + kb * 64 + lq * 16]);
                        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
                        for (int q = 0; q < NMAT; ++q)
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt)
                                acc[q][mt][nt] =
                                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bo[q][nt], acc[q][mt][nt], 0, 0, 0);
                    }
                }
            }
            if (c + 1 < nchunks) store_chunk(cur ^ 1);
            __syncthreads();
        }
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
                    const int row = s.dst[m];
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
int mfma_gate_up(const FfnArgs &a, hipStream_t s) {
    const int n_groups = a.n_routed_groups + (a.shared ? 1 : 0);
    const int ntiles = (a.I + kNT - 1) / kNT;
    const unsigned slots = (unsigned)((n_groups + kXcds - 1) / kXcds);
    hipLaunchKernelGGL(mfma_ffn_kernel<true>, dim3(slots * kXcds * ntiles), dim3(256), 0, s, a, ntiles, n_groups);
    MOE_LAUNCH_CHECK("mfma_ffn_kernel<gate_up>");
    return MOE_OK;
}

int mfma_down(const FfnArgs &a, hipStream_t s) {
    const int n_groups = a.n_routed_groups + (a.shared ? 1 : 0);
    const int ntiles = (a.H + kNT - 1) / kNT;
    const unsigned slots = (unsigned)((n_groups + kXcds - 1) / kXcds);
    hipLaunchKernelGGL(mfma_ffn_kernel<false>, dim3(slots * kXcds * ntiles), dim3(256), 0, s, a, ntiles, n_groups);
    MOE_LAUNCH_CHECK("mfma_ffn_kernel<down>");
    return MOE_OK;
}

}  // namespace moe
