// Expert FFN for many tokens per expert (prefill): grouped GEMM on MFMA with
// the 4-bit weight tiles dequantised in the kernel.
//
// The multi-token case is a dense contraction per expert: the tokens routed to
// expert e (gathered through the token->expert permutation) form an M_e x H
// activation matrix that meets the expert's W1/W3 (H -> I) and then W2 (I -> H).
// Each workgroup owns one expert and one 128-wide N tile and covers all of that
// expert's tokens (M chunks of 128), so every weight byte is read from HBM once.
//
// Per K chunk of 128 columns the workgroup stages in LDS: the gathered bf16
// activation tile [128 x 128] and the raw weight codes [128 x 64 B] plus the
// (scale, min) records of the tile's rows.  Each wave then owns 32 N columns (of
// W1 and of W3 for gate/up): it dequantises its B operand from LDS into bf16
// registers (scale*q + min in fp32, rounded to bf16) and accumulates
// v_mfma_f32_16x16x32_bf16 products in fp32.
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (checked on gfx950): lane l holds
// A[l%16][8*(l/16)+j], B[8*(l/16)+j][l%16] for j < 8, and C[4*(l/16)+j][l%16]
// for j < 4.
#include "common.h"
#include "ffn.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMT = 128;        // tokens per M chunk
constexpr int kNT = 128;        // weight rows (N) per workgroup
constexpr int kKC = 128;        // columns (K) per LDS chunk
constexpr int kXStride = 272;   // bytes per staged activation row (256 + 16 pad)
constexpr int kWStride = 80;    // bytes per staged code row (64 + 16 pad)

struct MfmaLds {
    uint8_t x[kMT * kXStride];        // activation tile, bf16
    uint8_t w[2][kNT * kWStride];     // code tiles (W1, W3) or (W2, -)
    uint4 p[2][kNT];                  // (scale, min) records of 4 blocks per row
    int src[kMT];                     // activation row of each M row (-1 = padding)
    int dst[kMT];                     // output row of each M row
};

// 8 consecutive weights of one row (codes dword, its block record) -> bf16x8
__device__ __forceinline__ bf16x8_t dequant8(uint32_t codes, uint32_t rec) {
    const float sc = fp16_bits_to_f32(rec & 0xFFFFu);
    const float mn = fp16_bits_to_f32(rec >> 16);
    bf16x8_t v;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float q = (float)((codes >> (4 * j)) & 0xFu);
        v[j] = (__bf16)fmaf(sc, q, mn);
    }
    return v;
}

template <bool GATEUP>
__global__ __launch_bounds__(256) void mfma_ffn_kernel(moe::FfnArgs a, int ntiles) {
    const int K = GATEUP ? a.H : a.I;   // reduction length
    const int R = GATEUP ? a.I : a.H;   // weight rows (output columns)
    const int nblk = K >> 5;
    const int g = blockIdx.x / ntiles, tile = blockIdx.x - g * ntiles;
    const int n0 = tile * kNT;

    // resolve the group: routed expert g (grouped), or the shared expert
    const uint8_t *slab;
    int M, base = 0;
    const bool routed = g < a.n_routed_groups;
    if (routed) {
        M = a.count[g];
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
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;  // MFMA row-in-tile and k-quarter
    constexpr int NMAT = GATEUP ? 2 : 1;

    for (int m0 = 0; m0 < M; m0 += kMT) {
        const int mc = min(kMT, M - m0);
        const int mtiles = (mc + 15) >> 4;
        __syncthreads();  // previous chunk done with s.src / s.dst
        if (tid < kMT) {
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
        f32x4_t acc[NMAT][8][2];
#pragma unroll
        for (int q = 0; q < NMAT; ++q)
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc[q][mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        for (int k0 = 0; k0 < K; k0 += kKC) {
            __syncthreads();  // LDS tiles free (and s.src visible)
            // activations: 128 rows x 256 B, 8 x 16 B per thread
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int idx = tid + 256 * i, row = idx >> 4, ch = idx & 15;
                const int src = s.src[row];
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (src >= 0) v = load_global_u4(act + (size_t)src * K + k0 + ch * 8);
                *reinterpret_cast<uint4 *>(&s.x[row * kXStride + ch * 16]) = v;
            }
            // codes: 128 rows x 64 B per matrix, 2 x 16 B per thread per matrix
#pragma unroll
            for (int q = 0; q < NMAT; ++q)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int idx = tid + 256 * i, row = idx >> 2, ch = idx & 3;
                    const int n = n0 + row;
                    uint4 v = make_uint4(0u, 0u, 0u, 0u);
                    if (n < R) v = load_stream_u4(mat[q] + (size_t)n * (K / 2) + k0 / 2 + ch * 16);
                    *reinterpret_cast<uint4 *>(&s.w[q][row * kWStride + ch * 16]) = v;
                }
            // block records: 4 blocks x 4 B per row
            if (tid < NMAT * kNT) {
                const int q = tid / kNT, row = tid - q * kNT, n = n0 + row;
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (n < R) v = load_stream_u4(mat[q] + cbytes + ((size_t)n * nblk + (k0 >> 5)) * 4);
                s.p[q][row] = v;
            }
            __syncthreads();
#pragma unroll
            for (int kb = 0; kb < kKC / 32; ++kb) {
                // B operands: this wave's 2 N tiles of each matrix
                bf16x8_t b[NMAT][2];
#pragma unroll
                for (int q = 0; q < NMAT; ++q)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const int row = wave * 32 + nt * 16 + lr;
                        const uint32_t codes =
                            *reinterpret_cast<const uint32_t *>(&s.w[q][row * kWStride + kb * 16 + lq * 4]);
                        const uint4 rec4 = s.p[q][row];
                        const uint32_t rec = kb == 0 ? rec4.x : kb == 1 ? rec4.y : kb == 2 ? rec4.z : rec4.w;
                        b[q][nt] = dequant8(codes, rec);
                    }
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    if (mt < mtiles) {
                        const uint4 av =
                            *reinterpret_cast<const uint4 *>(&s.x[(mt * 16 + lr) * kXStride + kb * 64 + lq * 16]);
                        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
                        for (int q = 0; q < NMAT; ++q)
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt)
                                acc[q][mt][nt] =
                                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, b[q][nt], acc[q][mt][nt], 0, 0, 0);
                    }
                }
            }
        }
        // epilogue
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
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

bool mfma_supported(const FfnArgs &a) { return a.grouped && a.H % kKC == 0 && a.I % kKC == 0; }

int mfma_gate_up(const FfnArgs &a, hipStream_t s) {
    const int n_groups = a.n_routed_groups + (a.shared ? 1 : 0);
    const int ntiles = (a.I + kNT - 1) / kNT;
    hipLaunchKernelGGL(mfma_ffn_kernel<true>, dim3((unsigned)n_groups * ntiles), dim3(256), 0, s, a, ntiles);
    MOE_LAUNCH_CHECK("mfma_ffn_kernel<gate_up>");
    return MOE_OK;
}

int mfma_down(const FfnArgs &a, hipStream_t s) {
    const int n_groups = a.n_routed_groups + (a.shared ? 1 : 0);
    const int ntiles = (a.H + kNT - 1) / kNT;
    hipLaunchKernelGGL(mfma_ffn_kernel<false>, dim3((unsigned)n_groups * ntiles), dim3(256), 0, s, a, ntiles);
    MOE_LAUNCH_CHECK("mfma_ffn_kernel<down>");
    return MOE_OK;
}

}  // namespace moe
