// 4-bit block dequant + dot product helpers shared by every expert-FFN kernel,
// so all kernel families compute each (token, expert) result with the same
// operations in the same order (their outputs are bit-identical).
//
// Weight block: 32 codes q in 16 bytes (byte b: column 2b in bits 0-3, 2b+1 in
// bits 4-7) plus one (fp16 scale, fp16 min) record; value = scale*q + min.
// Activations are bf16, pre-arranged per 8-column word as the pairs
// (x0,x4) (x1,x5) (x2,x6) (x3,x7) that the nibble extraction below produces:
// (w >> 4s) & 0x000F000F puts columns s and s+4 of the word in the two halves,
// OR-ing 0x4300 makes each half the bf16 value 128 + q (exponent 2^7, ulp 1).
// v_dot2_f32_bf16 then accumulates (128+q)*x exactly per product in fp32, and
//   sum (scale*q + min) * x = scale * sum((128+q) x) + (min - 128*scale) * sum x.
#pragma once
#include "common.h"

// Expert slab layout.  A row of a matrix with K columns is K/2 code bytes followed
// by the K/32 four-byte records of its 32-column blocks (then zero padding to a
// multiple of 16 bytes); the slab holds, for each
// r < I, the pair (W1 row r, W3 row r), then the H rows of W2.  So every (expert,
// row) unit of a kernel -- the gate and up rows together, or one down row -- is
// one contiguous stretch of memory.
namespace moe {
// codes and records of a K-column row, padded to a multiple of 16 bytes (no
// padding when K % 128 == 0), so every row starts 16-byte aligned
__host__ __device__ constexpr size_t slab_row_bytes(int K) { return ((size_t)K / 2 + (size_t)K / 8 + 15) / 16 * 16; }

// Rows of one matrix of a slab: row r starts at row0 + r * stride (codes), its
// records at + K/2.
struct MatRows {
    const uint8_t *row0;
    size_t stride;
};
// MXFP4 rows (weight format 1): K/2 E2M1 code bytes then K/32 E8M0 scale bytes,
// padded to a multiple of 16 bytes; same slab arrangement.
__host__ __device__ constexpr size_t mx_row_bytes(int K) { return ((size_t)K / 2 + (size_t)K / 32 + 15) / 16 * 16; }
// Super-block rows (weight format 2, K % 256 == 0): K/2 code bytes then one
// 16-byte header per 256 columns (fp16 d, fp16 dmin, eight 6-bit scale codes,
// eight 6-bit min codes).
__host__ __device__ constexpr size_t sb_row_bytes(int K) { return (size_t)K / 2 + (size_t)K / 16; }
template <int FMT>
__host__ __device__ constexpr size_t row_bytes_fmt(int K) {
    return FMT == 1 ? mx_row_bytes(K) : FMT == 2 ? sb_row_bytes(K) : slab_row_bytes(K);
}

// The three matrices of a slab of weight format FMT.
template <int FMT = 0>
__device__ __forceinline__ MatRows slab_w1(const uint8_t *slab, int H, int) {
    return {slab, 2 * row_bytes_fmt<FMT>(H)};
}
template <int FMT = 0>
__device__ __forceinline__ MatRows slab_w3(const uint8_t *slab, int H, int) {
    return {slab + row_bytes_fmt<FMT>(H), 2 * row_bytes_fmt<FMT>(H)};
}
template <int FMT = 0>
__device__ __forceinline__ MatRows slab_w2(const uint8_t *slab, int H, int I) {
    return {slab + (size_t)I * 2 * row_bytes_fmt<FMT>(H), row_bytes_fmt<FMT>(I)};
}
}  // namespace moe

// The bf16 exponent pattern 0x4300 in both halves, held in a VGPR: gfx9 VOP3
// instructions read at most one scalar/constant operand, so keeping this one in
// a vector register (the mask goes in an SGPR) lets the extraction below compile
// to a single bitfield insert per word.
__device__ __forceinline__ uint32_t moe_magic_vgpr() {
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(m));
    return m;
}

// (a & mask) | magic, written as a bitfield select (magic has no bits inside the
// mask) so that it becomes one v_bfi_b32 that the compiler can schedule freely.
__device__ __forceinline__ uint32_t moe_and_or(uint32_t a, uint32_t mask, uint32_t magic) {
    return (a & mask) | (magic & ~mask);
}

// sum over one block of (128 + q) * x; two interleaved accumulators shorten the
// dependency chain (fixed order: words 0,2 in acc0, words 1,3 in acc1).
__device__ __forceinline__ float moe_block_dot(const uint4 c, const uint4 *xb, int stride, uint32_t magic) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    const uint32_t mask = 0x000F000Fu;
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 X = xb[j * stride];
        float a = acc[j & 1];
        a = dot2_bf16(moe_and_or(w[j], mask, magic), X.x, a);
        a = dot2_bf16(moe_and_or(w[j] >> 4, mask, magic), X.y, a);
        a = dot2_bf16(moe_and_or(w[j] >> 8, mask, magic), X.z, a);
        a = dot2_bf16(moe_and_or(w[j] >> 12, mask, magic), X.w, a);
        acc[j & 1] = a;
    }
    return acc[0] + acc[1];
}

// sum over the block of (scale*q + min) * x from acc = sum (128+q) x and S = sum x
__device__ __forceinline__ float moe_block_value(uint32_t rec, float acc, float S) {
    const float sc = fp16_bits_to_f32(rec & 0xFFFFu);
    const float mn = fp16_bits_to_f32(rec >> 16);
    return fmaf(sc, acc, fmaf(-128.0f, sc, mn) * S);  // min - 128*scale is exact in fp32
}

// Sum over groups of W consecutive lanes.  W = 16 and 64 use DPP row shifts and
// row broadcasts (no LDS traffic); the total is valid in the LAST lane of each
// group.  Other W use a butterfly and every lane holds the total.  The order of
// additions is fixed, so results are reproducible.
template <int W>
__device__ __forceinline__ float moe_group_sum(float v) {
    if constexpr (W == 16 || W == 64) {
        // inclusive scan inside each 16-lane row: lane 15 of a row holds its sum
        v += __builtin_amdgcn_update_dpp(0.0f, v, 0x111, 0xF, 0xF, false);  // row_shr:1
        v += __builtin_amdgcn_update_dpp(0.0f, v, 0x112, 0xF, 0xF, false);  // row_shr:2
        v += __builtin_amdgcn_update_dpp(0.0f, v, 0x114, 0xF, 0xF, false);  // row_shr:4
        v += __builtin_amdgcn_update_dpp(0.0f, v, 0x118, 0xF, 0xF, false);  // row_shr:8
        if constexpr (W == 64) {
            v += __builtin_amdgcn_update_dpp(0.0f, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1,3
            v += __builtin_amdgcn_update_dpp(0.0f, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2,3
        }
        return v;
    } else {
#pragma unroll
        for (int o = W / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
        return v;
    }
}

// lane of a W-lane group that holds moe_group_sum's result
template <int W>
__device__ __forceinline__ bool moe_group_sum_owner(int lane_in_group) {
    return (W == 16 || W == 64) ? lane_in_group == W - 1 : lane_in_group == 0;
}

// MXFP4 block: sum over 32 columns of E2M1(q) * x, with x in natural column
// order (xb[j] holds columns 8j .. 8j+7 as bf16 pairs).  Each code byte becomes
// two bf16 values (low nibble first) through gfx950's scaled FP4 convert with
// scale 1 (exact: an E2M1 value has two significant bits), then
// v_dot2_f32_bf16; two interleaved accumulators as in moe_block_dot.
// (stride: distance in uint4 between the block's consecutive 8-column words)
__device__ __forceinline__ float moe_mx_block_dot(const uint4 c, const uint4 *xb, int stride = 1) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 X = xb[j * stride];
        float a = acc[j & 1];
        a = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], 1.0f, 0)), X.x, a);
        a = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], 1.0f, 1)), X.y, a);
        a = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], 1.0f, 2)), X.z, a);
        a = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], 1.0f, 3)), X.w, a);
        acc[j & 1] = a;
    }
    return acc[0] + acc[1];
}

// block value from the E8M0 scale byte v: acc * 2^(v - 127) (v = 255: NaN)
__device__ __forceinline__ float moe_mx_block_value(uint32_t v, float acc) {
    return v == 255u ? __builtin_nanf("") : ldexpf(acc, (int)v - 127);
}

// Super-block value of block j (0..7) of a header: scale d*s_j and min
// -dmin*m_j (both exact in fp32), then the format-0 identity
//   sum (scale*q + min) * x = scale * sum((128+q) x) + (min - 128*scale) * sum x.
__device__ __forceinline__ float moe_sb_block_value(const uint4 hdr, int j, float acc, float S) {
    const float d = fp16_bits_to_f32(hdr.x & 0xFFFFu), dmin = fp16_bits_to_f32(hdr.x >> 16);
    const uint64_t fs = (uint64_t)hdr.y | ((uint64_t)(hdr.z & 0xFFFFu) << 32);
    const uint64_t fm = (uint64_t)(hdr.z >> 16) | ((uint64_t)hdr.w << 16);
    const float sc = d * (float)(uint32_t)((fs >> (6 * j)) & 63u);
    const float mn = -dmin * (float)(uint32_t)((fm >> (6 * j)) & 63u);
    return fmaf(sc, acc, fmaf(-128.0f, sc, mn) * S);
}
