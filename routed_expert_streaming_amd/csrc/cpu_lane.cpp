// CPU lane: routed experts computed on host cores straight from the pinned host
// expert pool, in parallel with the GPU, instead of being streamed over PCIe.
//
// The pages name this as a direction of their own system (LayerStoRm README,
// "Status and limitations": CPU hybrid decode among the active work) and
// describe it in a related one (glm-flash-lite page, "How it works": two lanes
// run side by side, the GPU computing the experts held in VRAM while the CPU
// computes those held in system RAM).  Here an expert that misses the HBM cache
// goes either to the copy engine (streamed, then computed by the GPU kernels) or
// to this lane, which computes its SwiGLU FFN for the expert's tokens and hands
// back one fp32 row y = W2 h per (token, expert) pair; the caller uploads those
// rows next to the GPU's and combines as usual.  Which misses take which lane is
// the caller's cost model.
//
// Arithmetic, per token x (bf16) and expert slab (4-bit codes q, per 32-column
// block an fp16 scale s and min m, so W = s*q + m):
//   g[r] = sum_b ( s_b * sum_{c in b} q_c x_c  +  m_b * sum_{c in b} x_c )   (fp32)
//   and likewise u[r] with W3; h[r] = bf16_rne( g / (1 + exp(-g)) * u )     (fp32, rounded once)
//   y[r] = the same block sum over W2's row r and h                          (fp32)
// Within a block the 32 products are taken as 16 lanes (lane j: the even
// column 2j and the odd column 2j+1 of the block: p_j = fma(q_odd, x_odd,
// q_even * x_even)), each lane accumulates fma(s_b, p_j, acc_j) over the even
// blocks and, separately, over the odd blocks (then the two are added), the min
// terms fma(m_b, sum_b, .) likewise, and the 16 lanes are summed in a fixed tree.  Every output row is computed by one thread in that order, so the
// results do not depend on the thread count or on the instruction set that runs
// (the AVX-512, AVX2 and scalar versions perform the same IEEE operations).
//
// Threads: a pool of workers takes the queued jobs (one expert and its tokens)
// in submission order; all workers share a job, first its gate/up rows in chunks,
// then, once every gate/up chunk is done, its down rows.  Jobs complete in
// order, so waiting on a ticket covers every earlier job.
#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <deque>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include "moe.h"

namespace moe {
int fail(int status, const char *fmt, ...);
}

namespace {

constexpr int kBlock = 32;     // columns per scale/min record
constexpr int kMaxGroup = 8;   // tokens per pass over a row
constexpr int kRowsA = 16;     // gate/up rows per chunk
constexpr int kRowsB = 32;     // down rows per chunk

size_t row_bytes(int K) { return ((size_t)K / 2 + (size_t)K / 8 + 15) / 16 * 16; }

float bits_to_float(uint32_t u) {
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// IEEE binary16 -> binary32, exact (subnormals scaled by 2^-24).
float half_to_float(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t e = (h >> 10) & 31u, m = h & 0x3FFu;
    if (e == 0) {
        const float f = std::ldexp((float)m, -24);
        return sign ? -f : f;
    }
    if (e == 31) return bits_to_float(sign | 0x7F800000u | (m << 13));
    return bits_to_float(sign | ((e + 112u) << 23) | (m << 13));
}

float bf16_to_float(uint16_t b) { return bits_to_float((uint32_t)b << 16); }

uint16_t float_to_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// A vector of K columns laid out for the block dot: per block, the 16 even
// columns then the 16 odd ones (fp32), and per block the sum of its 32 values in
// column order.
void to_block_layout(const float *v, int K, float *perm, float *bsum) {
    for (int b = 0; b < K / kBlock; ++b) {
        float s = 0.0f;
        for (int j = 0; j < kBlock; ++j) s += v[b * kBlock + j];
        bsum[b] = s;
        for (int j = 0; j < 16; ++j) {
            perm[b * kBlock + j] = v[b * kBlock + 2 * j];
            perm[b * kBlock + 16 + j] = v[b * kBlock + 2 * j + 1];
        }
    }
}

float lane_total(const float *acc, float accm) {
    float s8[8], s4[4];
    for (int j = 0; j < 8; ++j) s8[j] = acc[j] + acc[j + 8];
    for (int j = 0; j < 4; ++j) s4[j] = s8[j] + s8[j + 4];
    return ((s4[0] + s4[2]) + (s4[1] + s4[3])) + accm;
}

// Scale and min of blocks b .. b+3 as fp32 (s0 m0 s1 m1 ... s3 m3): F16C's
// conversion is exact, so it gives the values half_to_float gives.
__attribute__((target("avx2,f16c"))) inline void records4(const uint8_t *r16, float *sm) {
    _mm256_storeu_ps(sm, _mm256_cvtph_ps(_mm_loadu_si128((const __m128i *)r16)));
}

// out[t] = dot(row, token t) for nt <= kMaxGroup tokens (perm/bsum rows of
// stride K and K/32).  Three versions with identical per-lane arithmetic: even
// and odd blocks accumulate separately (two independent fma chains), then add.
#define MOE_LANE_RECORDS(b)                                                                                    \
    if (((b) & 3) == 0) {                                                                                      \
        if ((b) + 4 <= nb) {                                                                                   \
            records4(rec + 4 * (b), sm);                                                                       \
        } else {                                                                                               \
            for (int i = 0; (b) + i < nb; ++i) {                                                               \
                sm[2 * i] = half_to_float((uint16_t)(rec[4 * ((b) + i)] | (rec[4 * ((b) + i) + 1] << 8)));    \
                sm[2 * i + 1] = half_to_float((uint16_t)(rec[4 * ((b) + i) + 2] | (rec[4 * ((b) + i) + 3] << 8))); \
            }                                                                                                  \
        }                                                                                                      \
    }

template <int NT>
__attribute__((target("avx512f,avx512bw,avx2,fma,f16c"))) void row_dots_avx512_n(const uint8_t *row, int K,
                                                                                  const float *perm,
                                                                                  const float *bsum, float *out) {
    const int nb = K / kBlock;
    const uint8_t *rec = row + K / 2;
    __m512 acc[2][NT];
    float accm[2][NT];
    for (int e = 0; e < 2; ++e)
        for (int t = 0; t < NT; ++t) {
            acc[e][t] = _mm512_setzero_ps();
            accm[e][t] = 0.0f;
        }
    const __m512i fifteen = _mm512_set1_epi32(15);
    alignas(32) float sm[8];
#define MOE_LANE_STEP512(b, e)                                                                                 \
    {                                                                                                          \
        MOE_LANE_RECORDS(b)                                                                                    \
        const __m512i c = _mm512_cvtepu8_epi32(_mm_loadu_si128((const __m128i *)(row + 16 * (b))));          \
        const __m512 lo = _mm512_cvtepi32_ps(_mm512_and_si512(c, fifteen));                                   \
        const __m512 hi = _mm512_cvtepi32_ps(_mm512_srli_epi32(c, 4));                                        \
        const __m512 sv = _mm512_set1_ps(sm[2 * ((b) & 3)]);                                                  \
        const float m = sm[2 * ((b) & 3) + 1];                                                                \
        for (int t = 0; t < NT; ++t) {                                                                         \
            const float *xe = perm + (size_t)t * K + kBlock * (b);                                            \
            const __m512 p = _mm512_fmadd_ps(hi, _mm512_loadu_ps(xe + 16), _mm512_mul_ps(lo, _mm512_loadu_ps(xe))); \
            acc[e][t] = _mm512_fmadd_ps(sv, p, acc[e][t]);                                                    \
            accm[e][t] = std::fma(m, bsum[(size_t)t * nb + (b)], accm[e][t]);                                 \
        }                                                                                                      \
    }
    int b = 0;
    for (; b + 2 <= nb; b += 2) {
        MOE_LANE_STEP512(b, 0)
        MOE_LANE_STEP512(b + 1, 1)
    }
    if (b < nb) MOE_LANE_STEP512(b, 0)
#undef MOE_LANE_STEP512
    for (int t = 0; t < NT; ++t) {
        alignas(64) float a[16];
        _mm512_store_ps(a, _mm512_add_ps(acc[0][t], acc[1][t]));
        out[t] = lane_total(a, accm[0][t] + accm[1][t]);
    }
}

template <int NT>
__attribute__((target("avx2,fma,f16c"))) void row_dots_avx2_n(const uint8_t *row, int K, const float *perm,
                                                               const float *bsum, float *out) {
    const int nb = K / kBlock;
    const uint8_t *rec = row + K / 2;
    __m256 acc[2][NT][2];
    float accm[2][NT];
    for (int e = 0; e < 2; ++e)
        for (int t = 0; t < NT; ++t) {
            acc[e][t][0] = acc[e][t][1] = _mm256_setzero_ps();
            accm[e][t] = 0.0f;
        }
    const __m256i fifteen = _mm256_set1_epi32(15);
    alignas(32) float sm[8];
#define MOE_LANE_STEP256(b, e)                                                                                 \
    {                                                                                                          \
        MOE_LANE_RECORDS(b)                                                                                    \
        __m256 lo[2], hi[2];                                                                                   \
        for (int h = 0; h < 2; ++h) {                                                                          \
            const __m256i c = _mm256_cvtepu8_epi32(_mm_loadl_epi64((const __m128i *)(row + 16 * (b) + 8 * h))); \
            lo[h] = _mm256_cvtepi32_ps(_mm256_and_si256(c, fifteen));                                         \
            hi[h] = _mm256_cvtepi32_ps(_mm256_srli_epi32(c, 4));                                              \
        }                                                                                                      \
        const __m256 sv = _mm256_set1_ps(sm[2 * ((b) & 3)]);                                                  \
        const float m = sm[2 * ((b) & 3) + 1];                                                                \
        for (int t = 0; t < NT; ++t) {                                                                         \
            const float *xe = perm + (size_t)t * K + kBlock * (b);                                            \
            for (int h = 0; h < 2; ++h) {                                                                      \
                const __m256 p = _mm256_fmadd_ps(hi[h], _mm256_loadu_ps(xe + 16 + 8 * h),                    \
                                                 _mm256_mul_ps(lo[h], _mm256_loadu_ps(xe + 8 * h)));         \
                acc[e][t][h] = _mm256_fmadd_ps(sv, p, acc[e][t][h]);                                          \
            }                                                                                                  \
            accm[e][t] = std::fma(m, bsum[(size_t)t * nb + (b)], accm[e][t]);                                 \
        }                                                                                                      \
    }
    int b = 0;
    for (; b + 2 <= nb; b += 2) {
        MOE_LANE_STEP256(b, 0)
        MOE_LANE_STEP256(b + 1, 1)
    }
    if (b < nb) MOE_LANE_STEP256(b, 0)
#undef MOE_LANE_STEP256
    for (int t = 0; t < NT; ++t) {
        alignas(32) float a[16];
        _mm256_store_ps(a, _mm256_add_ps(acc[0][t][0], acc[1][t][0]));
        _mm256_store_ps(a + 8, _mm256_add_ps(acc[0][t][1], acc[1][t][1]));
        out[t] = lane_total(a, accm[0][t] + accm[1][t]);
    }
}
#undef MOE_LANE_RECORDS

#define MOE_LANE_DISPATCH(name)                                                                                  \
    void name(const uint8_t *row, int K, const float *perm, const float *bsum, int nt, float *out) {          \
        switch (nt) {                                                                                          \
            case 1: name##_n<1>(row, K, perm, bsum, out); break;                                               \
            case 2: name##_n<2>(row, K, perm, bsum, out); break;                                               \
            case 3: name##_n<3>(row, K, perm, bsum, out); break;                                               \
            case 4: name##_n<4>(row, K, perm, bsum, out); break;                                               \
            case 5: name##_n<5>(row, K, perm, bsum, out); break;                                               \
            case 6: name##_n<6>(row, K, perm, bsum, out); break;                                               \
            case 7: name##_n<7>(row, K, perm, bsum, out); break;                                               \
            default: name##_n<8>(row, K, perm, bsum, out); break;                                              \
        }                                                                                                      \
    }
MOE_LANE_DISPATCH(row_dots_avx512)
MOE_LANE_DISPATCH(row_dots_avx2)
#undef MOE_LANE_DISPATCH
static_assert(kMaxGroup == 8, "one case per token count");

void row_dots_scalar(const uint8_t *row, int K, const float *perm, const float *bsum, int nt, float *out) {
    const int nb = K / kBlock;
    const uint8_t *rec = row + K / 2;
    for (int t = 0; t < nt; ++t) {
        float acc[2][16] = {};
        float accm[2] = {0.0f, 0.0f};
        for (int b = 0; b < nb; ++b) {
            const uint8_t *r4 = rec + 4 * b;
            const float s = half_to_float((uint16_t)(r4[0] | (r4[1] << 8)));
            const float m = half_to_float((uint16_t)(r4[2] | (r4[3] << 8)));
            const float *xe = perm + (size_t)t * K + kBlock * b;
            const int e = b & 1;
            for (int j = 0; j < 16; ++j) {
                const uint8_t c = row[16 * b + j];
                const float p = std::fma((float)(c >> 4), xe[16 + j], (float)(c & 15) * xe[j]);
                acc[e][j] = std::fma(s, p, acc[e][j]);
            }
            accm[e] = std::fma(m, bsum[(size_t)t * nb + b], accm[e]);
        }
        float a[16];
        for (int j = 0; j < 16; ++j) a[j] = acc[0][j] + acc[1][j];
        out[t] = lane_total(a, accm[0] + accm[1]);
    }
}

using RowDots = void (*)(const uint8_t *, int, const float *, const float *, int, float *);

RowDots pick_row_dots() {
    __builtin_cpu_init();
    const bool avx2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") && __builtin_cpu_supports("f16c");
    if (avx2 && __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw")) return row_dots_avx512;
    if (avx2) return row_dots_avx2;
    return row_dots_scalar;
}

// One expert and its M tokens.
struct Job {
    uint64_t ticket = 0;
    const uint8_t *slab = nullptr;
    int H = 0, I = 0, M = 0;
    std::vector<float *> y;        // [M] caller-owned output rows (H fp32 each)
    std::vector<float> xperm, xsum;  // [M][H], [M][H/32]
    std::vector<float> hval;       // [M][I] h after its bf16 rounding
    std::vector<float> hperm, hsum;  // [M][I], [M][I/32]
    int chunks_a = 0, chunks_b = 0;
    std::atomic<int> next_a{0}, done_a{0}, next_b{0}, done_b{0};
    std::atomic<bool> ready_b{false};
};

}  // namespace

struct moe_cpu_lane {
    std::mutex mu;
    std::condition_variable cv_work, cv_done;
    std::deque<std::shared_ptr<Job>> queue;
    std::vector<std::thread> workers;
    uint64_t submitted = 0, completed = 0;
    bool stop = false;
    RowDots row_dots = nullptr;

    void run(Job &j);
    void finish(Job &j);
    void worker_loop();
};

void moe_cpu_lane::finish(Job &j) {
    std::lock_guard<std::mutex> lk(mu);
    completed = j.ticket;
    queue.pop_front();
    cv_done.notify_all();
    cv_work.notify_all();
}

void moe_cpu_lane::run(Job &j) {
    const int H = j.H, I = j.I, M = j.M;
    const size_t gate_row = row_bytes(H), down_row = row_bytes(I);
    const uint8_t *w2 = j.slab + (size_t)I * 2 * gate_row;
    float g[kMaxGroup], u[kMaxGroup];
    // gate/up rows (W1 row r and W3 row r sit side by side in the slab)
    for (int c; (c = j.next_a.fetch_add(1, std::memory_order_relaxed)) < j.chunks_a;) {
        const int r1 = std::min(I, (c + 1) * kRowsA);
        for (int r = c * kRowsA; r < r1; ++r) {
            const uint8_t *w1 = j.slab + (size_t)r * 2 * gate_row;
            for (int t0 = 0; t0 < M; t0 += kMaxGroup) {
                const int nt = std::min(kMaxGroup, M - t0);
                const float *xp = j.xperm.data() + (size_t)t0 * H, *xs = j.xsum.data() + (size_t)t0 * (H / kBlock);
                row_dots(w1, H, xp, xs, nt, g);
                row_dots(w1 + gate_row, H, xp, xs, nt, u);
                for (int t = 0; t < nt; ++t)
                    j.hval[(size_t)(t0 + t) * I + r] = bf16_to_float(float_to_bf16(g[t] / (1.0f + std::exp(-g[t])) * u[t]));
            }
        }
        if (j.done_a.fetch_add(1, std::memory_order_acq_rel) + 1 == j.chunks_a) {
            // the last gate/up chunk: lay h out for the down rows
            for (int t = 0; t < M; ++t)
                to_block_layout(j.hval.data() + (size_t)t * I, I, j.hperm.data() + (size_t)t * I,
                                j.hsum.data() + (size_t)t * (I / kBlock));
            j.ready_b.store(true, std::memory_order_release);
        }
    }
    while (!j.ready_b.load(std::memory_order_acquire)) std::this_thread::yield();
    float yv[kMaxGroup];
    for (int c; (c = j.next_b.fetch_add(1, std::memory_order_relaxed)) < j.chunks_b;) {
        const int r1 = std::min(H, (c + 1) * kRowsB);
        for (int r = c * kRowsB; r < r1; ++r)
            for (int t0 = 0; t0 < M; t0 += kMaxGroup) {
                const int nt = std::min(kMaxGroup, M - t0);
                row_dots(w2 + (size_t)r * down_row, I, j.hperm.data() + (size_t)t0 * I,
                         j.hsum.data() + (size_t)t0 * (I / kBlock), nt, yv);
                for (int t = 0; t < nt; ++t) j.y[t0 + t][r] = yv[t];
            }
        if (j.done_b.fetch_add(1, std::memory_order_acq_rel) + 1 == j.chunks_b) finish(j);
    }
}

void moe_cpu_lane::worker_loop() {
    uint64_t last = 0;
    for (;;) {
        std::shared_ptr<Job> j;
        {
            std::unique_lock<std::mutex> lk(mu);
            cv_work.wait(lk, [&] { return stop || (!queue.empty() && queue.front()->ticket > last); });
            if (queue.empty() || queue.front()->ticket <= last) return;  // stop with nothing left
            j = queue.front();
        }
        last = j->ticket;
        run(*j);
    }
}

extern "C" int moe_cpu_lane_create(int threads, moe_cpu_lane **out) {
    if (!out) return moe::fail(MOE_E_ARG, "cpu_lane_create: NULL out");
    *out = nullptr;
    if (threads < 1 || threads > 256) return moe::fail(MOE_E_ARG, "cpu_lane_create: threads=%d outside [1, 256]", threads);
    auto *lane = new moe_cpu_lane();
    lane->row_dots = pick_row_dots();
    lane->workers.reserve(threads);
    for (int i = 0; i < threads; ++i) lane->workers.emplace_back([lane] { lane->worker_loop(); });
    *out = lane;
    return MOE_OK;
}

extern "C" int moe_cpu_lane_submit(moe_cpu_lane *lane, const void *slab, int H, int I, int M,
                                   const uint16_t *const *x_rows, float *const *y_rows, uint64_t *ticket) {
    if (!lane || !ticket) return moe::fail(MOE_E_ARG, "cpu_lane_submit: NULL lane or ticket");
    if (H <= 0 || I <= 0 || H % kBlock || I % kBlock)
        return moe::fail(MOE_E_SHAPE, "cpu_lane_submit: H=%d I=%d (positive multiples of 32)", H, I);
    if (M < 0) return moe::fail(MOE_E_ARG, "cpu_lane_submit: M=%d < 0", M);
    if (M == 0) {  // nothing to compute: the ticket of the last job submitted
        std::lock_guard<std::mutex> lk(lane->mu);
        *ticket = lane->submitted;
        return MOE_OK;
    }
    if (!slab || !x_rows || !y_rows) return moe::fail(MOE_E_ARG, "cpu_lane_submit: NULL pointer");
    for (int t = 0; t < M; ++t)
        if (!x_rows[t] || !y_rows[t]) return moe::fail(MOE_E_ARG, "cpu_lane_submit: NULL row %d", t);
    auto j = std::make_shared<Job>();
    j->slab = (const uint8_t *)slab;
    j->H = H;
    j->I = I;
    j->M = M;
    j->y.assign(y_rows, y_rows + M);
    j->xperm.resize((size_t)M * H);
    j->xsum.resize((size_t)M * (H / kBlock));
    j->hval.resize((size_t)M * I);
    j->hperm.resize((size_t)M * I);
    j->hsum.resize((size_t)M * (I / kBlock));
    std::vector<float> xf(H);
    for (int t = 0; t < M; ++t) {
        for (int c = 0; c < H; ++c) xf[c] = bf16_to_float(x_rows[t][c]);
        to_block_layout(xf.data(), H, j->xperm.data() + (size_t)t * H, j->xsum.data() + (size_t)t * (H / kBlock));
    }
    j->chunks_a = (I + kRowsA - 1) / kRowsA;
    j->chunks_b = (H + kRowsB - 1) / kRowsB;
    {
        std::lock_guard<std::mutex> lk(lane->mu);
        if (lane->stop) return moe::fail(MOE_E_STATE, "cpu_lane_submit: lane is shutting down");
        j->ticket = ++lane->submitted;
        *ticket = j->ticket;
        lane->queue.push_back(std::move(j));
    }
    lane->cv_work.notify_all();
    return MOE_OK;
}

extern "C" int moe_cpu_lane_wait(moe_cpu_lane *lane, uint64_t ticket) {
    if (!lane) return moe::fail(MOE_E_ARG, "cpu_lane_wait: NULL lane");
    std::unique_lock<std::mutex> lk(lane->mu);
    if (ticket > lane->submitted)
        return moe::fail(MOE_E_ARG, "cpu_lane_wait: ticket %llu not issued (last %llu)", (unsigned long long)ticket,
                         (unsigned long long)lane->submitted);
    lane->cv_done.wait(lk, [&] { return lane->completed >= ticket; });
    return MOE_OK;
}

extern "C" int moe_cpu_lane_destroy(moe_cpu_lane *lane) {
    if (!lane) return MOE_OK;
    {
        std::unique_lock<std::mutex> lk(lane->mu);
        lane->cv_done.wait(lk, [&] { return lane->completed >= lane->submitted; });
        lane->stop = true;
    }
    lane->cv_work.notify_all();
    for (auto &w : lane->workers) w.join();
    delete lane;
    return MOE_OK;
}

extern "C" int moe_cpu_lane_isa(void) {
    const RowDots f = pick_row_dots();
    return f == row_dots_avx512 ? 512 : f == row_dots_avx2 ? 256 : 0;
}

extern "C" int moe_cpu_lane_force_isa(moe_cpu_lane *lane, int isa) {
    if (!lane) return moe::fail(MOE_E_ARG, "cpu_lane_force_isa: NULL lane");
    const int best = moe_cpu_lane_isa();
    if ((isa != 0 && isa != 256 && isa != 512) || isa > best)
        return moe::fail(MOE_E_ARG, "cpu_lane_force_isa: %d not one of 0, 256, 512 up to this CPU's %d", isa, best);
    std::lock_guard<std::mutex> lk(lane->mu);
    if (lane->completed != lane->submitted) return moe::fail(MOE_E_STATE, "cpu_lane_force_isa: jobs in flight");
    lane->row_dots = isa == 512 ? row_dots_avx512 : isa == 256 ? row_dots_avx2 : row_dots_scalar;
    return MOE_OK;
}
