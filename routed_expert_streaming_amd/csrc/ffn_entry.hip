// Entry points around the expert FFN: token->expert permutation, the FFN
// dispatcher, the weighted combine and the dequantisation debug hook.
#include <mutex>

#include "common.h"
#include "dequant.h"
#include "ffn.h"
#include "router.h"
#include "topk.h"

namespace {

constexpr int kPermMaxPairs = 16384;
constexpr int kPermMaxE = 1024;

// Counting sort of pairs p = t*k+i by expert, stable in p, in one workgroup:
// histogram, exclusive scan, scatter with LDS cursors, then each expert's
// segment is put in ascending pair order by rank counting (pair ids are
// distinct, so the result does not depend on the scatter order).
__global__ __launch_bounds__(1024) void permute_kernel(const int32_t *__restrict__ idx, int n, int E,
                                                       int32_t *__restrict__ count, int32_t *__restrict__ offset,
                                                       int32_t *__restrict__ pair_of_row) {
    __shared__ int cnt[kPermMaxE];
    __shared__ int off[kPermMaxE + 1];
    __shared__ int cur[kPermMaxE];
    extern __shared__ int rows[];  // n entries
    const int tid = threadIdx.x, nt = blockDim.x;
    // this thread's experts, pairs tid, tid + 1024, ... (n <= 16384: at most 16),
    // all requested before any is used
    constexpr int kPer = kPermMaxPairs / 1024;
    int ex[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) ex[i] = tid + 1024 * i < n ? idx[tid + 1024 * i] : -1;
    for (int e = tid; e < E; e += nt) cnt[e] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (ex[i] >= 0) atomicAdd(&cnt[ex[i]], 1);
    __syncthreads();
    {  // exclusive scan of the counts, one expert per thread (E <= 1024 = blockDim.x):
       // inclusive scan inside each wave, then over the wave totals
        __shared__ int wsum[1024 / 64];
        const int wv = tid >> 6, ln = tid & 63;
        const int v = tid < E ? cnt[tid] : 0;
        int incl = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(incl, o, 64);
            if (ln >= o) incl += u;
        }
        if (ln == 63) wsum[wv] = incl;
        __syncthreads();
        if (wv == 0) {
            const int nw = nt >> 6;
            const int t0 = ln < nw ? wsum[ln] : 0;
            int ti = t0;
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                const int u = __shfl_up(ti, o, 64);
                if (ln >= o) ti += u;
            }
            if (ln < nw) wsum[ln] = ti - t0;  // exclusive over the waves
        }
        __syncthreads();
        const int excl = incl - v + wsum[wv];
        if (tid < E) off[tid] = excl;
        if (tid == E - 1) off[E] = excl + v;
    }
    __syncthreads();
    for (int e = tid; e < E; e += nt) {
        cur[e] = off[e];
        count[e] = cnt[e];
        offset[e] = off[e];
    }
    if (tid == 0) offset[E] = off[E];
    __syncthreads();
    int slot[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) slot[i] = ex[i] >= 0 ? atomicAdd(&cur[ex[i]], 1) : -1;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (slot[i] >= 0) rows[slot[i]] = tid + 1024 * i;
    __syncthreads();
    // one wavefront per expert segment
    const int wave = tid >> 6, lane = tid & 63, nwaves = nt >> 6;
    for (int e = wave; e < E; e += nwaves) {
        const int base = off[e], len = cnt[e];
        for (int j = lane; j < len; j += 64) {
            const int v = rows[base + j];
            // rank among the segment, 8 independent reads at a time
            int rank = 0, l = 0;
            for (; l + 8 <= len; l += 8) {
                int r[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) r[u] = rows[base + l + u];
#pragma unroll
                for (int u = 0; u < 8; ++u) rank += r[u] < v;
            }
            for (; l < len; ++l) rank += rows[base + l] < v;
            pair_of_row[base + rank] = v;
        }
    }
}

// dst row rows[i] = src row i (H floats), one workgroup per (row group, column block)
__global__ __launch_bounds__(256) void scatter_rows_kernel(const float *__restrict__ src, const int32_t *__restrict__ rows,
                                                           int n, int H, float *__restrict__ dst) {
    const int i = blockIdx.y;
    const int j = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n || j >= H) return;
    const float4 v = *reinterpret_cast<const float4 *>(src + (size_t)i * H + j);
    *reinterpret_cast<float4 *>(dst + (size_t)rows[i] * H + j) = v;
}

__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y, const float *__restrict__ w, int T,
                                                      int k, int H, int has_shared, uint16_t *__restrict__ out) {
    const int t = blockIdx.y;
    const int j = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (j >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = 0; i < k; ++i) {
        const float wi = w[(size_t)t * k + i];
        const float4 v = *reinterpret_cast<const float4 *>(y + ((size_t)t * k + i) * H + j);
        acc.x = fmaf(wi, v.x, acc.x);
        acc.y = fmaf(wi, v.y, acc.y);
        acc.z = fmaf(wi, v.z, acc.z);
        acc.w = fmaf(wi, v.w, acc.w);
    }
    if (has_shared) {
        const float4 v = *reinterpret_cast<const float4 *>(y + ((size_t)T * k + t) * H + j);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    uint2 o;
    o.x = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
    o.y = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
    *reinterpret_cast<uint2 *>(out + (size_t)t * H + j) = o;
}

// row r of the matrix starts at row0 + r * stride: K/2 code bytes, then the records
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ row0, size_t stride, int R, int K,
                                                      float *__restrict__ out) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)R * K) return;
    const size_t r = i / K, col = i - r * K;
    const uint8_t *row = row0 + r * stride;
    const uint8_t byte = row[col / 2];
    const uint32_t q = (col & 1) ? (byte >> 4) : (byte & 0xF);
    const uint32_t rec = *reinterpret_cast<const uint32_t *>(row + K / 2 + (col / 32) * 4);
    out[i] = fmaf(fp16_bits_to_f32(rec & 0xFFFFu), (float)q, fp16_bits_to_f32(rec >> 16));
}

}  // namespace

namespace moe {

int permute_launch(const int32_t *topk_idx, int T, int k, int E, int32_t *count, int32_t *offset,
                   int32_t *pair_of_row, hipStream_t s) {
    const int n = T * k;
    const size_t lds = (size_t)(n > 0 ? n : 1) * sizeof(int);
    static bool raised = false;
    if (!raised) {
        hipError_t e = hipFuncSetAttribute((const void *)permute_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           kPermMaxPairs * (int)sizeof(int));
        if (e != hipSuccess) return fail_hip(e, "hipFuncSetAttribute(permute_kernel)");
        raised = true;
    }
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), lds, s, topk_idx, n, E, count, offset, pair_of_row);
    MOE_LAUNCH_CHECK("permute_kernel");
    return MOE_OK;
}

}  // namespace moe

extern "C" int moe_permute(const int32_t *topk_idx, int T, int k, int E, int32_t *count, int32_t *offset,
                           int32_t *pair_of_row, void *stream) {
    if (T < 0 || k < 1 || E < 1) return moe::fail(MOE_E_ARG, "permute: T=%d k=%d E=%d", T, k, E);
    if (!count || !offset || (T > 0 && (!topk_idx || !pair_of_row))) return moe::fail(MOE_E_ARG, "permute: NULL");
    if ((long long)T * k > kPermMaxPairs || E > kPermMaxE || k > E)
        return moe::fail(MOE_E_SHAPE, "permute: T*k=%lld (max %d), E=%d (max %d), k=%d", (long long)T * k,
                         kPermMaxPairs, E, kPermMaxE, k);
    return moe::permute_launch(topk_idx, T, k, E, count, offset, pair_of_row, (hipStream_t)stream);
}

namespace {

struct FfnLayout {
    size_t h, count, offset, pairs, y, slabs, scale, total;
};

FfnLayout ffn_layout(int T, int H, int I, int E, int k, int has_shared) {
    FfnLayout L{};
    const size_t P = (size_t)T * k + (has_shared ? (size_t)T : 0);
    size_t o = 0;
    L.h = o;
    o += moe::align_up(P * I * sizeof(uint16_t), 256);
    L.count = o;
    o += moe::align_up((size_t)E * sizeof(int32_t), 256);
    L.offset = o;
    o += moe::align_up((size_t)(E + 1) * sizeof(int32_t), 256);
    L.pairs = o;
    o += moe::align_up((size_t)T * k * sizeof(int32_t), 256);
    L.y = o;
    o += moe::align_up(P * H * sizeof(float), 256);
    L.slabs = o;
    o += moe::align_up(P * sizeof(void *), 256);
    L.scale = o;  // MXFP4 on the scaled matrix cores: the E8M0 scales of x's T rows and h's P rows
    o += moe::align_up(((size_t)T + P) * sizeof(int32_t), 256);
    L.total = o;
    return L;
}

}  // namespace

extern "C" size_t moe_expert_ffn_workspace_bytes(int T, int H, int I, int E, int k, int has_shared) {
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0) return 0;
    return ffn_layout(T, H, I, E, k, has_shared).total;
}

namespace {

int validate_ffn(const void *act, int T, int H, int I, int E, const int32_t *topk_idx, int k,
                 const void *const *expert_table, const void *out, int path, const char *who, int fmt = 0) {
    if (!act || !topk_idx || !expert_table || !out) return moe::fail(MOE_E_ARG, "%s: NULL pointer", who);
    if (fmt < 0 || fmt > 2) return moe::fail(MOE_E_ARG, "%s: weight format %d (0, 1 or 2)", who, fmt);
    if (H <= 0 || I <= 0 || H % 32 || I % 32)
        return moe::fail(MOE_E_SHAPE, "%s: H=%d and I=%d must be positive multiples of 32", who, H, I);
    if (fmt == 2 && (H % 256 || I % 256))
        return moe::fail(MOE_E_SHAPE, "%s: super-block slabs need H, I multiples of 256 (H=%d I=%d)", who, H, I);
    if (H > 16384 || I > 16384) return moe::fail(MOE_E_SHAPE, "%s: H=%d I=%d above 16384", who, H, I);
    if (E < 1 || E > kPermMaxE || k < 1 || k > E) return moe::fail(MOE_E_SHAPE, "%s: E=%d k=%d", who, E, k);
    if (path < MOE_FFN_AUTO || path > MOE_FFN_SPLIT) return moe::fail(MOE_E_ARG, "%s: path=%d", who, path);
    return MOE_OK;
}

// Fills the kernel arguments; grouped iff a permutation is given.
int make_args(moe::FfnArgs &a, const uint16_t *x, uint16_t *h, float *y, int T, int H, int I, int E,
              const int32_t *topk_idx, int k, const int32_t *count, const int32_t *offset, const int32_t *pair_of_row,
              const void *const *table, const void *shared, const uint8_t *mask, int path, int *max_m,
              const char *who, int fmt = 0) {
    const bool have_perm = count && offset && pair_of_row;
    if ((count || offset || pair_of_row) && !have_perm)
        return moe::fail(MOE_E_ARG, "%s: count, offset and pair_of_row go together", who);
    if ((path == MOE_FFN_GROUPED || path == MOE_FFN_MFMA || path == MOE_FFN_SPLIT) && !have_perm)
        return moe::fail(MOE_E_ARG, "%s: grouped, MFMA and split paths need a permutation", who);
    const bool grouped = (path == MOE_FFN_GROUPED) || (path == MOE_FFN_MFMA) || (path == MOE_FFN_SPLIT) ||
                         (path == MOE_FFN_AUTO && have_perm);
    a = moe::FfnArgs{};
    a.x = x;
    a.h = h;
    a.y = y;
    a.T = T;
    a.H = H;
    a.I = I;
    a.E = E;
    a.k = k;
    a.topk_idx = topk_idx;
    a.table = table;
    a.shared = shared;
    a.mask = mask;
    a.grouped = grouped ? 1 : 0;
    a.n_routed_groups = grouped ? E : T * k;
    a.count = count;
    a.offset = offset;
    a.pair_of_row = pair_of_row;
    a.fmt = fmt;
    a.min_m = 0;
    a.max_m = 1 << 30;
    *max_m = grouped ? T : (shared ? T : 1);
    return MOE_OK;
}

// Grouped dequant-GEMV call.  With split (when the shapes allow the MFMA
// kernels and some group may hold more tokens than one GEMV pass stages) the
// GEMV takes the groups of up to kGemvOnePass tokens (each weight read once,
// dotted with every token) and the MFMA kernel the larger ones (each weight
// dequantised once for all its tokens) -- rather than re-reading weights or
// re-staging activations for every pass.
// Per-device helper stream of the split path (default priority, non-blocking).
std::mutex g_aux_mu;
hipStream_t g_aux[64] = {};

int aux_stream(hipStream_t *out) {
    int dev = 0;
    MOE_TRY_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64) return moe::fail(MOE_E_STATE, "split path: device %d", dev);
    std::lock_guard<std::mutex> lk(g_aux_mu);
    if (!g_aux[dev]) MOE_TRY_HIP(hipStreamCreateWithFlags(&g_aux[dev], hipStreamNonBlocking));
    *out = g_aux[dev];
    return MOE_OK;
}

template <bool GATEUP>
int grouped_gemv(moe::FfnArgs a, int max_m, bool split, bool use_fork, hipStream_t s) {
    if (!split || !a.grouped || !moe::mfma_supported(a) || max_m <= moe::kGemvOnePass)
        return GATEUP ? moe::ffn_gemv_gate_up(a, max_m, s) : moe::ffn_gemv_down(a, max_m, s);
    moe::FfnArgs b = a;
    b.min_m = moe::kGemvOnePass + 1;
    b.max_m = 1 << 30;
    b.compact = 1;  // few experts have that many tokens: deal their tiles over all XCDs
    a.max_m = moe::kGemvOnePass;
    if (!use_fork) {  // both parts in order on the caller's stream (no helper stream, no events)
        int rc = GATEUP ? moe::mfma_gate_up(b, s) : moe::mfma_down(b, s);
        if (rc != MOE_OK) return rc;
        return GATEUP ? moe::ffn_gemv_gate_up(a, moe::kGemvOnePass, s) : moe::ffn_gemv_down(a, moe::kGemvOnePass, s);
    }
    // The MFMA part (few experts, few workgroups) runs on a helper stream beside
    // the GEMV part, forked from and joined back into the caller's stream by
    // events; the two write disjoint rows of h (y).
    hipStream_t aux = nullptr;
    int rc = aux_stream(&aux);
    if (rc != MOE_OK) return rc;
    hipEvent_t fork = nullptr, join = nullptr;
    MOE_TRY_HIP(hipEventCreateWithFlags(&fork, hipEventDisableTiming));
    hipError_t e = hipEventCreateWithFlags(&join, hipEventDisableTiming);
    if (e != hipSuccess) {
        (void)hipEventDestroy(fork);
        return moe::fail_hip(e, "hipEventCreateWithFlags(join)");
    }
    e = hipEventRecord(fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(aux, fork, 0);
    if (e == hipSuccess) {
        rc = GATEUP ? moe::mfma_gate_up(b, aux) : moe::mfma_down(b, aux);
        if (rc == MOE_OK) {
            e = hipEventRecord(join, aux);
            if (e == hipSuccess) {
                rc = GATEUP ? moe::ffn_gemv_gate_up(a, moe::kGemvOnePass, s)
                            : moe::ffn_gemv_down(a, moe::kGemvOnePass, s);
                const hipError_t e2 = hipStreamWaitEvent(s, join, 0);  // join even if the GEMV launch failed
                if (rc == MOE_OK && e2 != hipSuccess) e = e2;
            }
        }
    }
    (void)hipEventDestroy(fork);
    (void)hipEventDestroy(join);
    if (e != hipSuccess) return moe::fail_hip(e, "split path fork/join");
    return rc;
}

// Kernel family for a grouped call: MFMA when forced, or automatically for many tokens.
bool use_mfma(const moe::FfnArgs &a, int path) {
    if (!moe::mfma_supported(a)) return false;
    return path == MOE_FFN_MFMA || (path == MOE_FFN_AUTO && a.T >= moe::kMfmaMinTokens);
}

// Automatic path of the one-call entry points: pairs for few (token, slot)
// pairs, MFMA for many tokens, split in between; the MFMA and split paths need
// H and I multiples of 128, other shapes take the grouped GEMV.
int auto_path(int T, int k, int H, int I, int fmt = 0) {
    if ((long long)T * k <= 64) return MOE_FFN_PAIRS;
    const int mult = fmt == 2 ? 256 : 128;
    if (H % mult || I % mult) return MOE_FFN_GROUPED;
    return T >= moe::kMfmaMinTokens ? MOE_FFN_MFMA : MOE_FFN_SPLIT;
}

// The pair-grouped decode kernels as separate gate/up and down calls: format 0
// (the other formats run them only through their one-call entry points, for
// one token; here they take the grouped GEMV, which covers every shape).
bool decode_ok(const moe::FfnArgs &a) { return moe::decode_supported(a) && a.fmt == 0; }

// Split grouped dispatch for an explicit split path, or automatic with a permutation.
bool use_split(const moe::FfnArgs &a, int path) {
    return a.grouped && (path == MOE_FFN_SPLIT || path == MOE_FFN_AUTO);
}

}  // namespace

namespace {
int gate_up_impl(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx, int k, const int32_t *count,
                 const int32_t *offset, const int32_t *pair_of_row, const void *const *expert_table,
                 const void *shared_slab, const uint8_t *expert_mask, uint16_t *h, int path, bool fork, void *stream,
                 int fmt = 0) {
    if (T < 0) return moe::fail(MOE_E_ARG, "expert_gate_up: T=%d < 0", T);
    if (T == 0) return MOE_OK;
    int rc = validate_ffn(x, T, H, I, E, topk_idx, k, expert_table, h, path, "expert_gate_up", fmt);
    if (rc != MOE_OK) return rc;
    moe::FfnArgs a;
    int max_m = 1;
    rc = make_args(a, x, h, nullptr, T, H, I, E, topk_idx, k, count, offset, pair_of_row, expert_table, shared_slab,
                   expert_mask, path, &max_m, "expert_gate_up", fmt);
    if (rc != MOE_OK) return rc;
    if (use_mfma(a, path)) return moe::mfma_gate_up(a, (hipStream_t)stream);
    if (path == MOE_FFN_MFMA)
        return moe::fail(MOE_E_SHAPE, "expert_gate_up: MFMA path needs H, I multiples of %d", fmt == 2 ? 256 : 128);
    if (decode_ok(a)) return moe::decode_gate_up(a, (hipStream_t)stream);
    return grouped_gemv<true>(a, max_m, use_split(a, path), fork, (hipStream_t)stream);
}

int down_impl(const uint16_t *h, int T, int H, int I, int E, const int32_t *topk_idx, int k, const int32_t *count,
              const int32_t *offset, const int32_t *pair_of_row, const void *const *expert_table,
              const void *shared_slab, const uint8_t *expert_mask, float *y, int path, bool fork, void *stream,
              int fmt = 0) {
    if (T < 0) return moe::fail(MOE_E_ARG, "expert_down: T=%d < 0", T);
    if (T == 0) return MOE_OK;
    int rc = validate_ffn(h, T, H, I, E, topk_idx, k, expert_table, y, path, "expert_down", fmt);
    if (rc != MOE_OK) return rc;
    moe::FfnArgs a;
    int max_m = 1;
    rc = make_args(a, nullptr, const_cast<uint16_t *>(h), y, T, H, I, E, topk_idx, k, count, offset, pair_of_row,
                   expert_table, shared_slab, expert_mask, path, &max_m, "expert_down", fmt);
    if (rc != MOE_OK) return rc;
    if (use_mfma(a, path)) return moe::mfma_down(a, (hipStream_t)stream);
    if (path == MOE_FFN_MFMA)
        return moe::fail(MOE_E_SHAPE, "expert_down: MFMA path needs H, I multiples of %d", fmt == 2 ? 256 : 128);
    if (decode_ok(a)) return moe::decode_down(a, nullptr, nullptr, (hipStream_t)stream);
    return grouped_gemv<false>(a, max_m, use_split(a, path), fork, (hipStream_t)stream);
}

int ffn_impl(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx, int k,
             const void *const *expert_table, const void *shared_slab, const uint8_t *expert_mask, float *y,
             void *workspace, size_t workspace_bytes, int path, bool fork, void *stream, int fmt = 0) {
    if (T < 0) return moe::fail(MOE_E_ARG, "expert_ffn: T=%d < 0", T);
    if (T == 0) return MOE_OK;
    if (!workspace) return moe::fail(MOE_E_ARG, "expert_ffn: NULL workspace");
    int rc = validate_ffn(x, T, H, I, E, topk_idx, k, expert_table, y, path, "expert_ffn", fmt);
    if (rc != MOE_OK) return rc;
    const int has_shared = shared_slab != nullptr;
    const FfnLayout Ly = ffn_layout(T, H, I, E, k, has_shared);
    if (workspace_bytes < Ly.total)
        return moe::fail(MOE_E_NOMEM, "expert_ffn: workspace %zu < %zu bytes", workspace_bytes, Ly.total);
    if (path == MOE_FFN_AUTO) path = auto_path(T, k, H, I, fmt);
    if (path != MOE_FFN_PAIRS && (long long)T * k > kPermMaxPairs)
        return moe::fail(MOE_E_SHAPE, "expert_ffn: grouped paths need T*k <= %d", kPermMaxPairs);
    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    uint16_t *h = (uint16_t *)(ws + Ly.h);
    int32_t *count = nullptr, *offset = nullptr, *pairs = nullptr;
    if (path == MOE_FFN_GROUPED || path == MOE_FFN_MFMA || path == MOE_FFN_SPLIT) {
        count = (int32_t *)(ws + Ly.count);
        offset = (int32_t *)(ws + Ly.offset);
        pairs = (int32_t *)(ws + Ly.pairs);
        rc = moe::permute_launch(topk_idx, T, k, E, count, offset, pairs, s);
        if (rc != MOE_OK) return rc;
    }
    if (fmt == 1 && path == MOE_FFN_MFMA && H % 128 == 0 && I % 128 == 0) {
        // MXFP4 on the block-scaled FP4 matrix cores: x's rows as FP8 digit pairs
        // in the y area (y is written only by the down projection, after the
        // gate/up products are done with them), then h's rows in place
        const int P = T * k + (shared_slab ? T : 0);
        uint8_t *xq = (uint8_t *)(ws + Ly.y);
        int32_t *xs = (int32_t *)(ws + Ly.scale), *hs = xs + T;
        rc = moe::quant_act(x, T, H, xq, xs, s);
        if (rc != MOE_OK) return rc;
        moe::FfnArgs a;
        int max_m = 1;
        rc = make_args(a, (const uint16_t *)xq, h, nullptr, T, H, I, E, topk_idx, k, count, offset, pairs,
                       expert_table, shared_slab, expert_mask, MOE_FFN_MFMA, &max_m, "expert_ffn", fmt);
        if (rc != MOE_OK) return rc;
        a.act_scale = xs;
        rc = moe::mfma_gate_up_scaled(a, s);
        if (rc != MOE_OK) return rc;
        rc = moe::quant_act(h, P, I, (uint8_t *)h, hs, s);
        if (rc != MOE_OK) return rc;
        rc = make_args(a, nullptr, h, y, T, H, I, E, topk_idx, k, count, offset, pairs, expert_table, shared_slab,
                       expert_mask, MOE_FFN_MFMA, &max_m, "expert_ffn", fmt);
        if (rc != MOE_OK) return rc;
        a.act_scale = hs;
        return moe::mfma_down_scaled(a, s);
    }
    rc = gate_up_impl(x, T, H, I, E, topk_idx, k, count, offset, pairs, expert_table, shared_slab, expert_mask, h, path,
                      fork, stream, fmt);
    if (rc != MOE_OK) return rc;
    return down_impl(h, T, H, I, E, topk_idx, k, count, offset, pairs, expert_table, shared_slab, expert_mask, y, path,
                     fork, stream, fmt);
}

int ffn_combine_impl(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx, const float *topk_w,
                     int k, const void *const *expert_table, const void *shared_slab, uint16_t *out, void *workspace,
                     size_t workspace_bytes, int path, bool fork, void *stream, int fmt = 0) {
    if (T < 0) return moe::fail(MOE_E_ARG, "expert_ffn_combine: T=%d < 0", T);
    if (T == 0) return MOE_OK;
    if (!workspace || !topk_w) return moe::fail(MOE_E_ARG, "expert_ffn_combine: NULL pointer");
    int rc = validate_ffn(x, T, H, I, E, topk_idx, k, expert_table, out, path, "expert_ffn_combine", fmt);
    if (rc != MOE_OK) return rc;
    const int has_shared = shared_slab != nullptr;
    const FfnLayout Ly = ffn_layout(T, H, I, E, k, has_shared);
    if (workspace_bytes < Ly.total)
        return moe::fail(MOE_E_NOMEM, "expert_ffn_combine: workspace %zu < %zu bytes", workspace_bytes, Ly.total);
    if (path == MOE_FFN_AUTO) path = auto_path(T, k, H, I, fmt);
    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    uint16_t *h = (uint16_t *)(ws + Ly.h);
    if (path == MOE_FFN_PAIRS) {
        moe::FfnArgs a;
        int max_m = 1;
        rc = make_args(a, x, h, nullptr, T, H, I, E, topk_idx, k, nullptr, nullptr, nullptr, expert_table,
                       shared_slab, nullptr, MOE_FFN_PAIRS, &max_m, "expert_ffn_combine", fmt);
        if (rc != MOE_OK) return rc;
        if (decode_ok(a)) {
            if (moe::decode1_publishes_slabs(a)) a.pair_slab = (const uint8_t **)(ws + Ly.slabs);
            rc = moe::decode_gate_up(a, s);
            if (rc != MOE_OK) return rc;
            return moe::decode_down(a, topk_w, out, s);
        }
    }
    float *y = (float *)(ws + Ly.y);
    rc = ffn_impl(x, T, H, I, E, topk_idx, k, expert_table, shared_slab, nullptr, y, workspace, workspace_bytes, path,
                  fork, stream, fmt);
    if (rc != MOE_OK) return rc;
    return moe_combine(y, topk_w, T, k, H, has_shared, out, stream);
}
}  // namespace

extern "C" int moe_expert_gate_up(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx, int k,
                                  const int32_t *count, const int32_t *offset, const int32_t *pair_of_row,
                                  const void *const *expert_table, const void *shared_slab,
                                  const uint8_t *expert_mask, uint16_t *h, int path, void *stream) {
    return gate_up_impl(x, T, H, I, E, topk_idx, k, count, offset, pair_of_row, expert_table, shared_slab,
                        expert_mask, h, path, true, stream);
}

extern "C" int moe_expert_down(const uint16_t *h, int T, int H, int I, int E, const int32_t *topk_idx, int k,
                               const int32_t *count, const int32_t *offset, const int32_t *pair_of_row,
                               const void *const *expert_table, const void *shared_slab, const uint8_t *expert_mask,
                               float *y, int path, void *stream) {
    return down_impl(h, T, H, I, E, topk_idx, k, count, offset, pair_of_row, expert_table, shared_slab, expert_mask,
                     y, path, true, stream);
}

extern "C" int moe_expert_gate_up_fmt(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx, int k,
                                      const int32_t *count, const int32_t *offset, const int32_t *pair_of_row,
                                      const void *const *expert_table, const void *shared_slab,
                                      const uint8_t *expert_mask, uint16_t *h, int path, int format, void *stream) {
    return gate_up_impl(x, T, H, I, E, topk_idx, k, count, offset, pair_of_row, expert_table, shared_slab,
                        expert_mask, h, path, true, stream, format);
}

extern "C" int moe_expert_down_fmt(const uint16_t *h, int T, int H, int I, int E, const int32_t *topk_idx, int k,
                                   const int32_t *count, const int32_t *offset, const int32_t *pair_of_row,
                                   const void *const *expert_table, const void *shared_slab,
                                   const uint8_t *expert_mask, float *y, int path, int format, void *stream) {
    return down_impl(h, T, H, I, E, topk_idx, k, count, offset, pair_of_row, expert_table, shared_slab, expert_mask,
                     y, path, true, stream, format);
}

extern "C" int moe_expert_ffn(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx, int k,
                              const void *const *expert_table, const void *shared_slab, const uint8_t *expert_mask,
                              float *y, void *workspace, size_t workspace_bytes, int path, void *stream) {
    return ffn_impl(x, T, H, I, E, topk_idx, k, expert_table, shared_slab, expert_mask, y, workspace,
                    workspace_bytes, path, true, stream);
}

extern "C" int moe_expert_ffn_fmt(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx, int k,
                                  const void *const *expert_table, const void *shared_slab, const uint8_t *expert_mask,
                                  float *y, void *workspace, size_t workspace_bytes, int path, int format,
                                  void *stream) {
    return ffn_impl(x, T, H, I, E, topk_idx, k, expert_table, shared_slab, expert_mask, y, workspace,
                    workspace_bytes, path, true, stream, format);
}

extern "C" int moe_expert_ffn_combine(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx,
                                      const float *topk_w, int k, const void *const *expert_table,
                                      const void *shared_slab, uint16_t *out, void *workspace, size_t workspace_bytes,
                                      int path, void *stream) {
    return ffn_combine_impl(x, T, H, I, E, topk_idx, topk_w, k, expert_table, shared_slab, out, workspace,
                            workspace_bytes, path, true, stream);
}

extern "C" size_t moe_route_ffn_combine_workspace_bytes(int T, int H, int I, int E, int k, int has_shared) {
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0) return 0;
    return moe::align_up(moe_router_workspace_bytes(T, E), 256) + ffn_layout(T, H, I, E, k, has_shared).total;
}

namespace moe {
int route_ffn_combine_impl(const uint16_t *x, int T, int H, int I, const float *w_router, const float *bias, int E,
                           int k, const void *const *expert_table, const void *shared_slab, int32_t *topk_idx,
                           float *topk_w, uint16_t *out, void *workspace, size_t workspace_bytes,
                           const void *prefetch, size_t prefetch_bytes, bool fork, void *stream) {
    const char *who = "route_ffn_combine";
    if (T < 0) return moe::fail(MOE_E_ARG, "%s: T=%d < 0", who, T);
    if (!prefetch && prefetch_bytes) return moe::fail(MOE_E_ARG, "%s: %zu prefetch bytes at NULL", who, prefetch_bytes);
    if (T == 0) return MOE_OK;
    if (!workspace || !w_router || !topk_w) return moe::fail(MOE_E_ARG, "%s: NULL pointer", who);
    int rc = validate_ffn(x, T, H, I, E, topk_idx, k, expert_table, out, MOE_FFN_AUTO, who);
    if (rc != MOE_OK) return rc;
    const int has_shared = shared_slab != nullptr;
    const size_t need = moe_route_ffn_combine_workspace_bytes(T, H, I, E, k, has_shared);
    if (workspace_bytes < need) return moe::fail(MOE_E_NOMEM, "%s: workspace %zu < %zu bytes", who, workspace_bytes, need);
    const size_t rbytes = moe::align_up(moe_router_workspace_bytes(T, E), 256);
    char *rws = (char *)workspace;
    char *fws = rws + rbytes;
    hipStream_t s = (hipStream_t)stream;

    moe::FfnArgs a;
    int max_m = 1;
    const FfnLayout Ly = ffn_layout(T, H, I, E, k, has_shared);
    rc = make_args(a, x, (uint16_t *)(fws + Ly.h), nullptr, T, H, I, E, topk_idx, k, nullptr, nullptr, nullptr,
                   expert_table, shared_slab, nullptr, MOE_FFN_PAIRS, &max_m, who);
    if (rc != MOE_OK) return rc;
    if (k <= moe::kTopkMaxK && H <= moe::kSlice * moe::kMaxSlices && moe::decode1_routed_supported(a, E)) {
        double *partial = moe::router_partials_buf(rws, T, E);
        rc = moe::router_partials(x, T, H, w_router, E, partial, s);
        if (rc != MOE_OK) return rc;
        const moe::RouteArgs ra{partial, bias, E, (H + moe::kSlice - 1) / moe::kSlice, moe::router_logits(rws),
                                topk_idx, topk_w};
        a.pair_slab = (const uint8_t **)(fws + Ly.slabs);
        rc = moe::decode1_routed_gate_up(a, ra, s);
        if (rc != MOE_OK) return rc;
        a.prefetch = (const uint8_t *)prefetch;
        a.prefetch_bytes = prefetch_bytes;
        return moe::decode_down(a, topk_w, out, s);
    }
    rc = moe_router_topk(x, T, H, w_router, bias, E, k, topk_idx, topk_w, rws, rbytes, stream);
    if (rc != MOE_OK) return rc;
    return ffn_combine_impl(x, T, H, I, E, topk_idx, topk_w, k, expert_table, shared_slab, out, fws,
                            workspace_bytes - rbytes, MOE_FFN_AUTO, fork, stream);
}
}  // namespace moe

extern "C" int moe_route_ffn_combine(const uint16_t *x, int T, int H, int I, const float *w_router, const float *bias,
                                     int E, int k, const void *const *expert_table, const void *shared_slab,
                                     int32_t *topk_idx, float *topk_w, uint16_t *out, void *workspace,
                                     size_t workspace_bytes, const void *prefetch, size_t prefetch_bytes,
                                     void *stream) {
    return moe::route_ffn_combine_impl(x, T, H, I, w_router, bias, E, k, expert_table, shared_slab, topk_idx, topk_w,
                                       out, workspace, workspace_bytes, prefetch, prefetch_bytes, true, stream);
}

// ---------------------------------------------------------------- other weight formats
// One-token decode with MXFP4 (format 1) or super-block (format 2) expert slabs:
// the same kernels specialised for the format (pairs path, fused combine).
namespace {
// One token: the fused one-token kernels when they cover the shape (true in *fused).
int fmt_ffn_args(moe::FfnArgs &a, const uint16_t *x, uint16_t *h, int T, int H, int I, int E, const int32_t *topk_idx,
                 int k, const void *const *table, const void *shared, const char *who, int fmt, bool *fused) {
    *fused = false;
    if (T != 1) return MOE_OK;
    int max_m = 1;
    int rc = make_args(a, x, h, nullptr, T, H, I, E, topk_idx, k, nullptr, nullptr, nullptr, table, shared, nullptr,
                       MOE_FFN_PAIRS, &max_m, who, fmt);
    if (rc != MOE_OK) return rc;
    const int ni = I >> 5;
    *fused = moe::decode_supported(a) && moe::decode1_publishes_slabs(a) && (ni == 48 || ni == 64) &&
             a.k + (a.shared ? 1 : 0) <= moe::kDown1MaxPairs;
    return MOE_OK;
}

int fmt_expert_ffn_combine(int fmt, const char *who, const uint16_t *x, int T, int H, int I, int E,
                           const int32_t *topk_idx, const float *topk_w, int k, const void *const *expert_table,
                           const void *shared_slab, uint16_t *out, void *workspace, size_t workspace_bytes,
                           void *stream) {
    if (T < 0) return moe::fail(MOE_E_ARG, "%s: T=%d < 0", who, T);
    if (T == 0) return MOE_OK;
    if (!workspace || !topk_w) return moe::fail(MOE_E_ARG, "%s: NULL pointer", who);
    int rc = validate_ffn(x, T, H, I, E, topk_idx, k, expert_table, out, MOE_FFN_AUTO, who, fmt);
    if (rc != MOE_OK) return rc;
    const FfnLayout Ly = ffn_layout(T, H, I, E, k, shared_slab != nullptr);
    if (workspace_bytes < Ly.total)
        return moe::fail(MOE_E_NOMEM, "%s: workspace %zu < %zu bytes", who, workspace_bytes, Ly.total);
    char *ws = (char *)workspace;
    moe::FfnArgs a;
    bool fused = false;
    rc = fmt_ffn_args(a, x, (uint16_t *)(ws + Ly.h), T, H, I, E, topk_idx, k, expert_table, shared_slab, who, fmt,
                      &fused);
    if (rc != MOE_OK) return rc;
    if (!fused)  // several tokens (or a shape the one-token kernels do not cover): the grouped paths
        return ffn_combine_impl(x, T, H, I, E, topk_idx, topk_w, k, expert_table, shared_slab, out, workspace,
                                workspace_bytes, MOE_FFN_AUTO, true, stream, fmt);
    a.pair_slab = (const uint8_t **)(ws + Ly.slabs);
    rc = moe::decode_gate_up(a, (hipStream_t)stream);
    if (rc != MOE_OK) return rc;
    return moe::decode_down(a, topk_w, out, (hipStream_t)stream);
}

int fmt_route_ffn_combine(int fmt, const char *who, const uint16_t *x, int T, int H, int I, const float *w_router,
                          const float *bias, int E, int k, const void *const *expert_table, const void *shared_slab,
                          int32_t *topk_idx, float *topk_w, uint16_t *out, void *workspace, size_t workspace_bytes,
                          const void *prefetch, size_t prefetch_bytes, void *stream) {
    if (T < 0) return moe::fail(MOE_E_ARG, "%s: T=%d < 0", who, T);
    if (!prefetch && prefetch_bytes) return moe::fail(MOE_E_ARG, "%s: %zu prefetch bytes at NULL", who, prefetch_bytes);
    if (T == 0) return MOE_OK;
    if (!workspace || !w_router || !topk_w) return moe::fail(MOE_E_ARG, "%s: NULL pointer", who);
    int rc = validate_ffn(x, T, H, I, E, topk_idx, k, expert_table, out, MOE_FFN_AUTO, who, fmt);
    if (rc != MOE_OK) return rc;
    const int has_shared = shared_slab != nullptr;
    const size_t need = moe_route_ffn_combine_workspace_bytes(T, H, I, E, k, has_shared);
    if (workspace_bytes < need) return moe::fail(MOE_E_NOMEM, "%s: workspace %zu < %zu bytes", who, workspace_bytes, need);
    const size_t rbytes = moe::align_up(moe_router_workspace_bytes(T, E), 256);
    char *rws = (char *)workspace;
    char *fws = rws + rbytes;
    hipStream_t s = (hipStream_t)stream;
    moe::FfnArgs a;
    const FfnLayout Ly = ffn_layout(T, H, I, E, k, has_shared);
    bool fused = false;
    rc = fmt_ffn_args(a, x, (uint16_t *)(fws + Ly.h), T, H, I, E, topk_idx, k, expert_table, shared_slab, who, fmt,
                      &fused);
    if (rc != MOE_OK) return rc;
    if (fused && k <= moe::kTopkMaxK && H <= moe::kSlice * moe::kMaxSlices && moe::decode1_routed_supported(a, E)) {
        double *partial = moe::router_partials_buf(rws, T, E);
        rc = moe::router_partials(x, T, H, w_router, E, partial, s);
        if (rc != MOE_OK) return rc;
        const moe::RouteArgs ra{partial, bias, E, (H + moe::kSlice - 1) / moe::kSlice, moe::router_logits(rws),
                                topk_idx, topk_w};
        a.pair_slab = (const uint8_t **)(fws + Ly.slabs);
        rc = moe::decode1_routed_gate_up(a, ra, s);
        if (rc != MOE_OK) return rc;
        a.prefetch = (const uint8_t *)prefetch;
        a.prefetch_bytes = prefetch_bytes;
        return moe::decode_down(a, topk_w, out, s);
    }
    rc = moe_router_topk(x, T, H, w_router, bias, E, k, topk_idx, topk_w, rws, rbytes, stream);
    if (rc != MOE_OK) return rc;
    return fmt_expert_ffn_combine(fmt, who, x, T, H, I, E, topk_idx, topk_w, k, expert_table, shared_slab, out, fws,
                                  workspace_bytes - rbytes, stream);
}
}  // namespace

extern "C" int moe_mx_expert_ffn_combine(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx,
                                         const float *topk_w, int k, const void *const *expert_table,
                                         const void *shared_slab, uint16_t *out, void *workspace,
                                         size_t workspace_bytes, void *stream) {
    return fmt_expert_ffn_combine(1, "mx_expert_ffn_combine", x, T, H, I, E, topk_idx, topk_w, k, expert_table,
                                  shared_slab, out, workspace, workspace_bytes, stream);
}

extern "C" int moe_mx_route_ffn_combine(const uint16_t *x, int T, int H, int I, const float *w_router,
                                        const float *bias, int E, int k, const void *const *expert_table,
                                        const void *shared_slab, int32_t *topk_idx, float *topk_w, uint16_t *out,
                                        void *workspace, size_t workspace_bytes, const void *prefetch,
                                        size_t prefetch_bytes, void *stream) {
    return fmt_route_ffn_combine(1, "mx_route_ffn_combine", x, T, H, I, w_router, bias, E, k, expert_table,
                                 shared_slab, topk_idx, topk_w, out, workspace, workspace_bytes, prefetch,
                                 prefetch_bytes, stream);
}

extern "C" int moe_sb_expert_ffn_combine(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx,
                                         const float *topk_w, int k, const void *const *expert_table,
                                         const void *shared_slab, uint16_t *out, void *workspace,
                                         size_t workspace_bytes, void *stream) {
    return fmt_expert_ffn_combine(2, "sb_expert_ffn_combine", x, T, H, I, E, topk_idx, topk_w, k, expert_table,
                                  shared_slab, out, workspace, workspace_bytes, stream);
}

extern "C" int moe_sb_route_ffn_combine(const uint16_t *x, int T, int H, int I, const float *w_router,
                                        const float *bias, int E, int k, const void *const *expert_table,
                                        const void *shared_slab, int32_t *topk_idx, float *topk_w, uint16_t *out,
                                        void *workspace, size_t workspace_bytes, const void *prefetch,
                                        size_t prefetch_bytes, void *stream) {
    return fmt_route_ffn_combine(2, "sb_route_ffn_combine", x, T, H, I, w_router, bias, E, k, expert_table,
                                 shared_slab, topk_idx, topk_w, out, workspace, workspace_bytes, prefetch,
                                 prefetch_bytes, stream);
}

extern "C" int moe_quant_act_mx(const uint16_t *x, int rows, int K, uint8_t *out, int32_t *scales, void *stream) {
    if (rows < 0) return moe::fail(MOE_E_ARG, "quant_act_mx: rows=%d < 0", rows);
    if (rows == 0) return MOE_OK;
    if (!x || !out || !scales) return moe::fail(MOE_E_ARG, "quant_act_mx: NULL pointer");
    return moe::quant_act(x, rows, K, out, scales, (hipStream_t)stream);
}

extern "C" int moe_combine(const float *y, const float *topk_w, int T, int k, int H, int has_shared, uint16_t *out,
                           void *stream) {
    if (T < 0 || k < 1 || H <= 0) return moe::fail(MOE_E_ARG, "combine: T=%d k=%d H=%d", T, k, H);
    if (T == 0) return MOE_OK;
    if (!y || !topk_w || !out) return moe::fail(MOE_E_ARG, "combine: NULL pointer");
    if (H % 4) return moe::fail(MOE_E_SHAPE, "combine: H=%d must be a multiple of 4", H);
    dim3 grid((H / 4 + 255) / 256, T);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, (hipStream_t)stream, y, topk_w, T, k, H, has_shared, out);
    MOE_LAUNCH_CHECK("combine_kernel");
    return MOE_OK;
}

extern "C" int moe_scatter_rows(const float *src, const int32_t *rows, int n, int H, float *dst, void *stream) {
    if (n < 0 || H <= 0) return moe::fail(MOE_E_ARG, "scatter_rows: n=%d H=%d", n, H);
    if (n == 0) return MOE_OK;
    if (!src || !rows || !dst) return moe::fail(MOE_E_ARG, "scatter_rows: NULL pointer");
    if (H % 4) return moe::fail(MOE_E_SHAPE, "scatter_rows: H=%d must be a multiple of 4", H);
    if (n > 65535) return moe::fail(MOE_E_SHAPE, "scatter_rows: n=%d above 65535 rows per call", n);
    dim3 grid((H / 4 + 255) / 256, n);
    hipLaunchKernelGGL(scatter_rows_kernel, grid, dim3(256), 0, (hipStream_t)stream, src, rows, n, H, dst);
    MOE_LAUNCH_CHECK("scatter_rows_kernel");
    return MOE_OK;
}

extern "C" int moe_debug_dequant(const void *slab, int H, int I, int which, float *out, void *stream) {
    if (!slab || !out) return moe::fail(MOE_E_ARG, "debug_dequant: NULL pointer");
    if (H <= 0 || I <= 0 || H % 32 || I % 32) return moe::fail(MOE_E_SHAPE, "debug_dequant: H=%d I=%d", H, I);
    if (which < 0 || which > 2) return moe::fail(MOE_E_ARG, "debug_dequant: which=%d", which);
    const int R = which < 2 ? I : H, K = which < 2 ? H : I;
    const size_t gate_row = moe::slab_row_bytes(H);
    const uint8_t *row0 = (const uint8_t *)slab + (which == 0 ? 0 : which == 1 ? gate_row : (size_t)I * 2 * gate_row);
    const size_t stride = which < 2 ? 2 * gate_row : moe::slab_row_bytes(I);
    const size_t n = (size_t)R * K;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, row0,
                       stride, R, K, out);
    MOE_LAUNCH_CHECK("dequant_kernel");
    return MOE_OK;
}
