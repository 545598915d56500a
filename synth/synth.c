/*
 * synth.c -- seeded, counter-based synthetic inputs for the routed-expert FFN step.
 *
 * This module only produces input bytes: hidden states, router weights, router
 * bias and 4-bit expert slabs.  It holds none of the method's arithmetic
 * (no routing, no dequantisation, no FFN), so both the CPU oracle and the GPU
 * path may consume what it writes.
 *
 * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), keyed by the 64-bit config seed, with
 * the 128-bit counter holding (index, expert, layer|kind|matrix, step).  Every
 * element is therefore addressable on its own and the fill is parallel and
 * order independent.  Normals use the Box-Muller transform.
 *
 * Expert slab byte layout (one contiguous slab per expert):
 *   matrix 0 = W1 (gate) [I rows x H cols], matrix 1 = W3 (up) [I x H],
 *   matrix 2 = W2 (down) [H rows x I cols].  A row of a matrix with K cols is
 *   K/2 code bytes (byte b holds column 2b in bits 0-3 and column 2b+1 in bits
 *   4-7; codes are 0..15), then K/32 records of 4 bytes, one per 32-column
 *   block: fp16 scale (bytes 0-1) then fp16 min (bytes 2-3); 0.625*K bytes,
 *   padded with zeros to a multiple of 16 (no padding when K % 128 == 0).
 *   slab = I row pairs [W1 row r | W3 row r], then the H rows of W2; for H and I
 *   multiples of 128 that is 1.875*H*I bytes.
 * Value distributions: x ~ N(0,1) rounded to bf16; router W ~ N(0, 0.02^2)
 * rounded to fp32; codes uniform on 0..15; scale = fp16(|N(0, 0.02^2)|);
 * min = -8*scale (exact in fp16).  The scale of block b is drawn from Philox
 * call b/2 (cosine branch for even b, sine branch for odd b).
 *
 * Weight format 1 (MXFP4, the *_fmt functions): the same slab arrangement, a
 * K-column row being K/2 code bytes (same nibble order; a code is an E2M1
 * value: sign bit 3, exponent bits 2-1, mantissa bit 0) then K/32 one-byte
 * E8M0 block scales, zero-padded to a multiple of 16 bytes (17/32 byte per
 * weight when K % 512 == 0).  Codes uniform on 0..15; scale byte of block b =
 * 120 + (byte b%16 of Philox call b/16) mod 3, i.e. 2^-7, 2^-6 or 2^-5.
 *
 * Weight format 2 (super-blocks of 256 columns, k-quant style): a K-column row
 * (K % 256 == 0) is K/2 code bytes (same nibble order), then one 16-byte header
 * per 256-column super-block: fp16 d (bytes 0-1), fp16 dmin (bytes 2-3), eight
 * 6-bit scale codes (bytes 4-9, code j in bits 6j..6j+5 of that little-endian
 * 48-bit field) and eight 6-bit min codes (bytes 10-15, likewise); 0.5625*K
 * bytes.  Codes uniform on 0..15; d = fp16(0.0002 * (1 + |N(0,1)|)), dmin =
 * fp16(4 * d); scale codes uniform on 16..63, min codes uniform on 0..63.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { KIND_X = 1, KIND_WR = 2, KIND_BIAS = 3, KIND_CODES = 4, KIND_PARAMS = 5, KIND_MX_CODES = 6, KIND_MX_SCALES = 7 };

/* ---------------- Philox4x32-10 ---------------- */
static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t *hi, uint32_t *lo) {
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

static inline void philox_core(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo32(0xD2511F53u, c0, &hi0, &lo0);
        mulhilo32(0xCD9E8D57u, c2, &hi1, &lo1);
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    philox_core(ctr_in, key_in, out);
}

static inline void draw(uint64_t seed, uint32_t kind, uint32_t step, uint32_t layer,
                        uint32_t expert, uint32_t matrix, uint32_t index, uint32_t out[4]) {
    uint32_t ctr[4] = { index, expert, (layer << 16) | (kind << 8) | (matrix & 0xFFu), step };
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    philox_core(ctr, key, out);
}

/* Standard normal from two 32-bit words (Box-Muller, cosine branch). */
static inline double normal_from(uint32_t a, uint32_t b) {
    const double two32 = 4294967296.0;
    double u1 = ((double)a + 0.5) / two32; /* (0,1) */
    double u2 = ((double)b + 0.5) / two32;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

/* Two standard normals from two 32-bit words (Box-Muller, cosine and sine branch). */
static inline void normal_pair_from(uint32_t a, uint32_t b, double *z0, double *z1) {
    const double two32 = 4294967296.0;
    double u1 = ((double)a + 0.5) / two32;
    double u2 = ((double)b + 0.5) / two32;
    double rad = sqrt(-2.0 * log(u1)), ang = 6.283185307179586476925286766559 * u2;
    *z0 = rad * cos(ang);
    *z1 = rad * sin(ang);
}

/* ---------------- input rounding (round to nearest, ties to even) ---------------- */
/* Round a finite double to a float with `mant` explicit significand bits and the
   exponent range of the target format, returning the rounded value as double. */
static double round_to_format(double v, int sig_bits, int emin) {
    if (v == 0.0 || !isfinite(v)) return v;
    int e = ilogb(v);          /* v = m * 2^e, 1 <= |m| < 2 */
    if (e < emin) e = emin;    /* subnormal range: fixed quantum */
    double q = ldexp(v, sig_bits - 1 - e);
    q = nearbyint(q);          /* default rounding mode: to nearest, ties to even */
    return ldexp(q, e - (sig_bits - 1));
}

uint16_t synth_double_to_bf16(double v) {
    double r = round_to_format(v, 8, -126);
    float f = (fabs(r) > 3.4028234663852886e38) ? (r > 0 ? INFINITY : -INFINITY)
                                                 : (float)r; /* exact: <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* double -> fp16 bits, round to nearest even, on the integer significand. */
uint16_t synth_double_to_fp16(double v) {
    uint64_t u;
    memcpy(&u, &v, 8);
    uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    int e = (int)((u >> 52) & 0x7FF) - 1023;
    uint64_t frac = u & ((1ull << 52) - 1);
    if (e == 1024) return sign | (frac ? 0x7E00u : 0x7C00u);   /* inf / nan */
    if (e < -26) return sign;                                      /* below half the min subnormal */
    uint64_t m = frac | (1ull << 52);                              /* significand, value m * 2^(e-52) */
    int shift = (e >= -14) ? 42 : 42 + (-14 - e);                  /* keep 10 fraction bits (normal) */
    uint64_t half = 1ull << (shift - 1);
    uint64_t q = m >> shift, rem = m & ((1ull << shift) - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    if (e >= -14) {
        int ee = e;
        if (q == 2048) { q = 1024; ++ee; }
        if (ee > 15) return sign | 0x7C00u;
        return sign | (uint16_t)(((uint32_t)(ee + 15) << 10) | (uint32_t)(q - 1024));
    }
    return sign | (uint16_t)q;  /* subnormal; q == 1024 rolls into the smallest normal */
}

static int clamp_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
    return nthreads < 1 ? 1 : nthreads;
}

/* ---------------- generators ---------------- */
/* x[t, h] for one (step, layer): N(0,1) rounded to bf16. */
void synth_x_bf16(uint64_t seed, uint32_t step, uint32_t layer, int64_t T, int64_t H,
                  uint16_t *out, int nthreads) {
    int64_t n = T * H;
    nthreads = clamp_threads(nthreads);
    #pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint32_t r[4];
        draw(seed, KIND_X, step, layer, 0, 0, (uint32_t)i, r);
        out[i] = synth_double_to_bf16(normal_from(r[0], r[1]));
    }
}

/* router weight Wr[e, h] for one layer: N(0, 0.02^2) rounded to fp32. */
void synth_router_w(uint64_t seed, uint32_t layer, int64_t E, int64_t H, float *out, int nthreads) {
    int64_t n = E * H;
    nthreads = clamp_threads(nthreads);
    #pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint32_t r[4];
        draw(seed, KIND_WR, 0, layer, 0, 0, (uint32_t)i, r);
        out[i] = (float)(0.02 * normal_from(r[0], r[1]));
    }
}

/* Seeded permutation rank[e] in 1..E (Fisher-Yates driven by Philox words). */
void synth_rank_permutation(uint64_t seed, uint32_t layer, int64_t E, int32_t *rank) {
    for (int64_t e = 0; e < E; ++e) rank[e] = (int32_t)(e + 1);
    for (int64_t i = E - 1; i > 0; --i) {
        uint32_t r[4];
        draw(seed, KIND_BIAS, 0, layer, 0, 0, (uint32_t)i, r);
        uint64_t wide = ((uint64_t)r[0] << 32) | r[1];
        int64_t j = (int64_t)(wide % (uint64_t)(i + 1));
        int32_t t = rank[i]; rank[i] = rank[j]; rank[j] = t;
    }
}

/* Zipf-popularity router bias: bias[e] = -s * ln(rank[e]), rounded to fp32. */
void synth_zipf_bias(uint64_t seed, uint32_t layer, int64_t E, double s, float *out) {
    int32_t *rank = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    synth_rank_permutation(seed, layer, E, rank);
    for (int64_t e = 0; e < E; ++e) out[e] = (float)(-s * log((double)rank[e]));
    free(rank);
}

/* Bytes of one row of a matrix with `cols` columns: codes and records, rounded up
   to 16 so that every row starts on a 16-byte boundary. */
static int64_t row_bytes(int64_t cols) { return (cols / 2 + (cols / 32) * 4 + 15) / 16 * 16; }
int64_t synth_matrix_bytes(int64_t rows, int64_t cols) { return rows * row_bytes(cols); }
int64_t synth_slab_bytes(int64_t H, int64_t I) { return 2 * synth_matrix_bytes(I, H) + synth_matrix_bytes(H, I); }

/* Where row r of matrix m starts in a slab, and the distance between its rows. */
static int64_t matrix_start(int64_t H, int64_t I, uint32_t m) {
    return m == 0 ? 0 : m == 1 ? row_bytes(H) : 2 * I * row_bytes(H);
}
static int64_t matrix_row_stride(int64_t H, int64_t I, uint32_t m) {
    return m < 2 ? 2 * row_bytes(H) : row_bytes(I);
}

static inline void write_params(double z, uint8_t *rec) {
    uint16_t sc = synth_double_to_fp16(fabs(0.02 * z));
    /* min = -8 * scale: decode the fp16 scale exactly, scale by -8 (exact in fp16). */
    uint32_t ex = (sc >> 10) & 0x1F, mt = sc & 0x3FF;
    double sv = ex ? ldexp((double)(mt | 0x400), (int)ex - 25) : ldexp((double)mt, -24);
    uint16_t mn = synth_double_to_fp16(-8.0 * sv);
    rec[0] = (uint8_t)(sc & 0xFF);
    rec[1] = (uint8_t)(sc >> 8);
    rec[2] = (uint8_t)(mn & 0xFF);
    rec[3] = (uint8_t)(mn >> 8);
}

/* Record of global block B (row-major over (row, block)) of a matrix. */
static inline uint8_t *record_at(uint8_t *base, int64_t stride, int64_t cols, int64_t B) {
    int64_t nblk = cols / 32, row = B / nblk, blk = B - row * nblk;
    return base + row * stride + cols / 2 + 4 * blk;
}

/* Scale of block b comes from Philox call b/2: the cosine branch for even b, the
   sine branch for odd b (b counts the matrix's blocks row-major). */
static inline void params_for_pair(uint64_t seed, uint32_t layer, uint32_t expert, uint32_t m,
                                   int64_t pair, int64_t nblocks, uint8_t *base, int64_t stride, int64_t cols) {
    uint32_t r[4];
    double z0, z1;
    draw(seed, KIND_PARAMS, 0, layer, expert, m, (uint32_t)pair, r);
    normal_pair_from(r[0], r[1], &z0, &z1);
    write_params(z0, record_at(base, stride, cols, 2 * pair));
    if (2 * pair + 1 < nblocks) write_params(z1, record_at(base, stride, cols, 2 * pair + 1));
}

/* Fill part `part` of `nparts` of one matrix: its 16-byte code chunks c (row-major,
   K/32 per row) and its records; base = the matrix's row 0, stride = between rows. */
static void fill_matrix_part(uint64_t seed, uint32_t layer, uint32_t expert, uint32_t m,
                             int64_t rows, int64_t cols, uint8_t *base, int64_t stride, int64_t part,
                             int64_t nparts) {
    int64_t chunks_per_row = cols / 32;
    int64_t nchunks = rows * chunks_per_row;
    int64_t nblocks = rows * (cols / 32);
    int64_t c0 = nchunks * part / nparts, c1 = nchunks * (part + 1) / nparts;
    const int64_t used = cols / 2 + (cols / 32) * 4, pad = row_bytes(cols) - used;
    for (int64_t c = c0; c < c1; ++c) {
        uint32_t r[4];
        int64_t row = c / chunks_per_row, ch = c - row * chunks_per_row;
        draw(seed, KIND_CODES, 0, layer, expert, m, (uint32_t)c, r);
        memcpy(base + row * stride + 16 * ch, r, 16);
        if (ch == 0 && pad > 0) memset(base + row * stride + used, 0, (size_t)pad);  /* row padding */
    }
    int64_t npairs = (nblocks + 1) / 2;
    int64_t b0 = npairs * part / nparts, b1 = npairs * (part + 1) / nparts;
    for (int64_t b = b0; b < b1; ++b) params_for_pair(seed, layer, expert, m, b, nblocks, base, stride, cols);
}

/* Many slabs in parallel: outs[i] receives expert experts[i] of `layer`.  Expert
   ids >= E may be used for shared experts; they select another Philox stream. */
void synth_expert_slabs(uint64_t seed, uint32_t layer, const uint32_t *experts, int64_t n,
                        int64_t H, int64_t I, uint8_t *const *outs, int nthreads) {
    nthreads = clamp_threads(nthreads);
    /* Split every matrix into parts so a handful of slabs still keeps all threads busy. */
    const int64_t nparts = 16;
    int64_t njobs = n * 3 * nparts;
    #pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int64_t job = 0; job < njobs; ++job) {
        int64_t i = job / (3 * nparts);
        uint32_t m = (uint32_t)((job / nparts) % 3);
        int64_t part = job % nparts;
        int64_t rows = (m < 2) ? I : H, cols = (m < 2) ? H : I;
        fill_matrix_part(seed, layer, experts[i], m, rows, cols, outs[i] + matrix_start(H, I, m),
                         matrix_row_stride(H, I, m), part, nparts);
    }
}

void synth_expert_slab(uint64_t seed, uint32_t layer, uint32_t expert, int64_t H, int64_t I, uint8_t *out) {
    uint8_t *outs[1] = { out };
    synth_expert_slabs(seed, layer, &expert, 1, H, I, outs, 1);
}

/* ---------------- weight format 1: MXFP4 ---------------- */
static int64_t row_bytes_fmt(int64_t cols, int fmt) {
    return fmt == 1 ? (cols / 2 + cols / 32 + 15) / 16 * 16 : row_bytes(cols);
}
int64_t synth_slab_bytes_sb(int64_t H, int64_t I);
int64_t synth_slab_bytes_fmt(int64_t H, int64_t I, int fmt) {
    if (fmt == 2) return (H % 256 || I % 256) ? 0 : synth_slab_bytes_sb(H, I);
    return 2 * I * row_bytes_fmt(H, fmt) + H * row_bytes_fmt(I, fmt);
}

static void fill_matrix_part_mx(uint64_t seed, uint32_t layer, uint32_t expert, uint32_t m, int64_t rows,
                                int64_t cols, uint8_t *base, int64_t stride, int64_t part, int64_t nparts) {
    const int64_t cpr = cols / 32, used = cols / 2 + cols / 32, pad = row_bytes_fmt(cols, 1) - used;
    const int64_t r0 = rows * part / nparts, r1 = rows * (part + 1) / nparts;
    for (int64_t row = r0; row < r1; ++row) {
        uint8_t *rp = base + row * stride;
        for (int64_t ch = 0; ch < cpr; ++ch) {
            uint32_t r[4];
            draw(seed, KIND_MX_CODES, 0, layer, expert, m, (uint32_t)(row * cpr + ch), r);
            memcpy(rp + 16 * ch, r, 16);
        }
        for (int64_t b = 0; b < cpr; ++b) {
            int64_t B = row * cpr + b;
            uint32_t r[4];
            draw(seed, KIND_MX_SCALES, 0, layer, expert, m, (uint32_t)(B / 16), r);
            uint8_t bytes[16];
            memcpy(bytes, r, 16);
            rp[cols / 2 + b] = (uint8_t)(120 + bytes[B % 16] % 3);
        }
        if (pad > 0) memset(rp + used, 0, (size_t)pad);
    }
}

static void fill_matrix_part_sb(uint64_t, uint32_t, uint32_t, uint32_t, int64_t, int64_t, uint8_t *, int64_t,
                                int64_t, int64_t);
static int64_t row_bytes_sb(int64_t cols);

void synth_expert_slabs_fmt(uint64_t seed, uint32_t layer, const uint32_t *experts, int64_t n, int64_t H,
                            int64_t I, uint8_t *const *outs, int nthreads, int fmt) {
    if (fmt != 1 && fmt != 2) {
        synth_expert_slabs(seed, layer, experts, n, H, I, outs, nthreads);
        return;
    }
    nthreads = clamp_threads(nthreads);
    const int64_t nparts = 16, njobs = n * 3 * nparts;
    const int64_t rh = fmt == 2 ? row_bytes_sb(H) : row_bytes_fmt(H, 1), ri = fmt == 2 ? row_bytes_sb(I) : row_bytes_fmt(I, 1);
    #pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int64_t job = 0; job < njobs; ++job) {
        int64_t i = job / (3 * nparts);
        uint32_t m = (uint32_t)((job / nparts) % 3);
        int64_t part = job % nparts;
        int64_t rows = (m < 2) ? I : H, cols = (m < 2) ? H : I;
        int64_t start = m == 0 ? 0 : m == 1 ? rh : 2 * I * rh, stride = m < 2 ? 2 * rh : ri;
        if (fmt == 2)
            fill_matrix_part_sb(seed, layer, experts[i], m, rows, cols, outs[i] + start, stride, part, nparts);
        else
            fill_matrix_part_mx(seed, layer, experts[i], m, rows, cols, outs[i] + start, stride, part, nparts);
    }
}

/* ---------------- weight format 2: 256-column super-blocks ---------------- */
enum { KIND_SB_CODES = 8, KIND_SB_HEAD = 9 };
static int64_t row_bytes_sb(int64_t cols) { return cols / 2 + cols / 16; }
int64_t synth_slab_bytes_sb(int64_t H, int64_t I) { return 2 * I * row_bytes_sb(H) + H * row_bytes_sb(I); }

static void put6(uint8_t *field, int j, unsigned v) {   /* 6-bit code j into a 48-bit little-endian field */
    uint64_t f = 0;
    for (int b = 0; b < 6; ++b) f |= (uint64_t)field[b] << (8 * b);
    f = (f & ~((uint64_t)63 << (6 * j))) | ((uint64_t)(v & 63) << (6 * j));
    for (int b = 0; b < 6; ++b) field[b] = (uint8_t)(f >> (8 * b));
}

static void fill_matrix_part_sb(uint64_t seed, uint32_t layer, uint32_t expert, uint32_t m, int64_t rows,
                                int64_t cols, uint8_t *base, int64_t stride, int64_t part, int64_t nparts) {
    const int64_t cpr = cols / 32, nsb = cols / 256;
    const int64_t r0 = rows * part / nparts, r1 = rows * (part + 1) / nparts;
    for (int64_t row = r0; row < r1; ++row) {
        uint8_t *rp = base + row * stride;
        for (int64_t ch = 0; ch < cpr; ++ch) {
            uint32_t r[4];
            draw(seed, KIND_SB_CODES, 0, layer, expert, m, (uint32_t)(row * cpr + ch), r);
            memcpy(rp + 16 * ch, r, 16);
        }
        for (int64_t sb = 0; sb < nsb; ++sb) {
            uint32_t r[4], r2[4];
            draw(seed, KIND_SB_HEAD, 0, layer, expert, m, (uint32_t)(2 * (row * nsb + sb)), r);
            draw(seed, KIND_SB_HEAD, 0, layer, expert, m, (uint32_t)(2 * (row * nsb + sb) + 1), r2);
            uint8_t *h = rp + cols / 2 + 16 * sb;
            memset(h, 0, 16);
            uint16_t d = synth_double_to_fp16(0.0002 * (1.0 + fabs(normal_from(r[0], r[1]))));
            uint32_t ex = (d >> 10) & 0x1F, mt = d & 0x3FF;
            double dv = ex ? ldexp((double)(mt | 0x400), (int)ex - 25) : ldexp((double)mt, -24);
            uint16_t dmin = synth_double_to_fp16(4.0 * dv);
            h[0] = (uint8_t)(d & 0xFF);
            h[1] = (uint8_t)(d >> 8);
            h[2] = (uint8_t)(dmin & 0xFF);
            h[3] = (uint8_t)(dmin >> 8);
            uint8_t bytes[16];
            memcpy(bytes, r2, 16);
            for (int j = 0; j < 8; ++j) {
                put6(h + 4, j, 16u + bytes[j] % 48u);
                put6(h + 10, j, bytes[8 + j] % 64u);
            }
        }
    }
}
