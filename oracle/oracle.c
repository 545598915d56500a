/*
 * oracle.c -- plain, slow, fp64 CPU reference of the routed-expert FFN step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this code; the GPU library never does.
 * It shares no code with the GPU path (its own format decoding, rounding,
 * selection and arithmetic), and it is deliberately unblocked and unfused.
 *
 * What it computes (LayerStoRm README, "TL;DR": the router tells which few
 * experts each token activates; those experts' FFNs run and their outputs are
 * combined; glm-flash-lite page, "How it works": 8 experts per layer per token):
 *   1. logits  L[e] = fp32( sum_h x[h]*Wr[e,h] + b[e] ), summed in fp64 in index
 *      order and rounded once to fp32 (round to nearest even);
 *   2. top-k   the k largest logits, ties to the lower expert index, emitted in
 *      order of descending logit then ascending index;
 *   3. weights softmax over the k selected logits, in fp64;
 *   4. expert FFN (SwiGLU):  g = W1 x, u = W3 x, h = silu(g) * u,
 *      silu(z) = z / (1 + exp(-z)), y = W2 h, with every weight dequantised as
 *      W = scale * q + min from its 4-bit code q and its block's fp16 scale/min;
 *   5. combine out = sum_i w_i * y_{idx_i} + y_shared, in slot order i = 0..k-1,
 *      then the shared expert with weight 1; reported in fp64 and rounded to bf16.
 * Slab layout: see the header of the input generator (synth/synth.c); this file
 * decodes it on its own from that description.
 *
 * Weight format 1, MXFP4 (the pages name MXFP4 decode paths among the sources
 * of their kernels: LayerStoRm README, "License and attributions"; the element
 * and scale encodings are those of the OCP Microscaling Formats specification
 * v1.0): per 32-column block one E8M0 scale byte v (2^(v-127), v = 255 NaN) and
 * 32 E2M1 codes q (sign bit 3, exponent bits 2-1 with bias 1, mantissa bit 0;
 * exponent 0 is subnormal: 0 or 0.5), W = E2M1(q) * 2^(v-127).  A K-column row
 * is K/2 code bytes (same nibble order) then K/32 scale bytes, padded to 16.
 *
 * Weight format 2, k-quant-style super-blocks (the pages' own weights are a
 * 4-bit k-quant GGUF variant: LayerStoRm README, "TL;DR" and "Serve"): per
 * 256-column super-block an fp16 d and fp16 dmin and, for each of its eight
 * 32-column blocks j, a 6-bit scale code s_j and a 6-bit min code m_j;
 * W = d*s_j*q - dmin*m_j.  A K-column row (K % 256 == 0) is K/2 code bytes then
 * one 16-byte header per super-block: d, dmin, then the eight s_j (bytes 4-9)
 * and the eight m_j (bytes 10-15), code j in bits 6j..6j+5 of each 48-bit
 * little-endian field.
 * The *_fmt functions take the format; the others are format 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------- scalar formats ---------------- */
double oracle_bf16_to_double(uint16_t b) {
    /* bf16 is the upper half of an IEEE binary32 */
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

double oracle_fp16_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int mt = h & 0x3FF;
    double v;
    if (ex == 0) v = ldexp((double)mt, -24);                      /* subnormal */
    else if (ex == 31) v = mt ? NAN : INFINITY;                    /* inf / nan */
    else v = ldexp((double)(1024 + mt), ex - 25);                  /* normal */
    return sign ? -v : v;
}

/* double -> bf16 bits, round to nearest, ties to even (8 significant bits,
   binary32 exponent range including subnormals). */
uint16_t oracle_double_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);              /* a = f * 2^e, 0.5 <= f < 1, i.e. unbiased exponent e-1 */
    int ue = e - 1;
    if (ue < -126) ue = -126;  /* subnormal: quantum 2^-133 */
    double quantum = ldexp(1.0, ue - 7);
    double n = a / quantum;    /* exact: power-of-two scaling */
    double fl = floor(n);
    double rem = n - fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = fl * quantum;
    if (r > 3.3895313892515355e38) return sign | 0x7F80;  /* beyond the largest bf16 */
    float f = (float)r;        /* exact: at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

/* ---------------- slab decoding ---------------- */
/* A row of K columns: K/2 code bytes, K/32 records of 4 bytes, zero padding to a multiple of 16. */
static int g_fmt = 0; /* weight format of the call in progress (set by the *_fmt entry points) */
static int64_t row_bytes_f(int64_t cols, int fmt) {
    if (fmt == 2) return cols / 2 + cols / 16;
    return fmt == 1 ? (cols / 2 + cols / 32 + 15) / 16 * 16 : (cols / 2 + (cols / 32) * 4 + 15) / 16 * 16;
}

/* 6-bit code j of a 48-bit little-endian field. */
static unsigned field6(const uint8_t *f, int j) {
    uint64_t v = 0;
    for (int b = 0; b < 6; ++b) v |= (uint64_t)f[b] << (8 * b);
    return (unsigned)((v >> (6 * j)) & 63);
}
static int64_t row_bytes(int64_t cols) { return row_bytes_f(cols, g_fmt); }

int64_t oracle_slab_bytes(int64_t H, int64_t I) { return 2 * I * row_bytes_f(H, 0) + H * row_bytes_f(I, 0); }
int64_t oracle_slab_bytes_fmt(int64_t H, int64_t I, int fmt) {
    if (fmt == 2 && (H % 256 || I % 256)) return 0;
    return 2 * I * row_bytes_f(H, fmt) + H * row_bytes_f(I, fmt);
}

/* OCP MX v1.0 FP4 (E2M1) element value. */
double oracle_e2m1_to_double(int q) {
    const int sign = (q >> 3) & 1, e = (q >> 1) & 3, m = q & 1;
    const double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}
/* OCP MX v1.0 E8M0 scale value. */
double oracle_e8m0_to_double(uint8_t v) { return v == 255 ? NAN : ldexp(1.0, (int)v - 127); }

/* Row r of matrix `which` (0 = W1 gate [I x H], 1 = W3 up [I x H], 2 = W2 down
   [H x I]); the slab holds the I row pairs (W1 row, W3 row), then the H rows of W2. */
static const uint8_t *matrix_row(const uint8_t *slab, int64_t H, int64_t I, int which, int64_t r) {
    const int64_t gate_row = row_bytes(H), down_row = row_bytes(I);
    if (which < 2) return slab + r * 2 * gate_row + (which == 1 ? gate_row : 0);
    return slab + I * 2 * gate_row + r * down_row;
}

/* Dequantise one row (K = cols columns, starting at `row`) into out[cols]. */
static void dequant_row(const uint8_t *row, int64_t cols, double *out) {
    if (g_fmt == 2) {
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = row[c / 2];
            int q = (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
            const uint8_t *h = row + cols / 2 + 16 * (c / 256);
            const int j = (int)((c / 32) % 8);
            double d = oracle_fp16_to_double((uint16_t)(h[0] | (h[1] << 8)));
            double dmin = oracle_fp16_to_double((uint16_t)(h[2] | (h[3] << 8)));
            out[c] = d * field6(h + 4, j) * q - dmin * field6(h + 10, j);
        }
        return;
    }
    if (g_fmt == 1) {
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = row[c / 2];
            int q = (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
            out[c] = oracle_e2m1_to_double(q) * oracle_e8m0_to_double(row[cols / 2 + c / 32]);
        }
        return;
    }
    const uint8_t *codes = row;
    const uint8_t *params = row + cols / 2;
    for (int64_t c = 0; c < cols; ++c) {
        uint8_t byte = codes[c / 2];
        int q = (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
        const uint8_t *rec = params + (c / 32) * 4;
        double scale = oracle_fp16_to_double((uint16_t)(rec[0] | (rec[1] << 8)));
        double mn = oracle_fp16_to_double((uint16_t)(rec[2] | (rec[3] << 8)));
        out[c] = scale * (double)q + mn;
    }
}

/* Full dequantised matrix `which` of a slab, row-major. */
void oracle_dequant(const uint8_t *slab, int64_t H, int64_t I, int which, double *out) {
    int64_t rows = (which < 2) ? I : H, cols = (which < 2) ? H : I;
    for (int64_t r = 0; r < rows; ++r) dequant_row(matrix_row(slab, H, I, which, r), cols, out + r * cols);
}

/* ---------------- expert FFN ---------------- */
/* One token through one expert.  g, u, h may be NULL (then scratch is used). */
void oracle_expert_ffn(const uint8_t *slab, int64_t H, int64_t I, const double *x,
                       double *g_out, double *u_out, double *h_out, double *y) {
    double *row = (double *)malloc(sizeof(double) * (size_t)(H > I ? H : I));
    double *g = g_out ? g_out : (double *)malloc(sizeof(double) * (size_t)I);
    double *u = u_out ? u_out : (double *)malloc(sizeof(double) * (size_t)I);
    double *h = h_out ? h_out : (double *)malloc(sizeof(double) * (size_t)I);
    for (int64_t r = 0; r < I; ++r) {
        double acc = 0.0;
        dequant_row(matrix_row(slab, H, I, 0, r), H, row);
        for (int64_t c = 0; c < H; ++c) acc += row[c] * x[c];
        g[r] = acc;
        acc = 0.0;
        dequant_row(matrix_row(slab, H, I, 1, r), H, row);
        for (int64_t c = 0; c < H; ++c) acc += row[c] * x[c];
        u[r] = acc;
        h[r] = g[r] / (1.0 + exp(-g[r])) * u[r];
    }
    for (int64_t r = 0; r < H; ++r) {
        double acc = 0.0;
        dequant_row(matrix_row(slab, H, I, 2, r), I, row);
        for (int64_t c = 0; c < I; ++c) acc += row[c] * h[c];
        y[r] = acc;
    }
    free(row);
    if (!g_out) free(g);
    if (!u_out) free(u);
    if (!h_out) free(h);
}

/* Down projection alone: y = W2 h (h has I entries, y has H). */
void oracle_expert_down(const uint8_t *slab, int64_t H, int64_t I, const double *h, double *y) {
    double *row = (double *)malloc(sizeof(double) * (size_t)I);
    for (int64_t r = 0; r < H; ++r) {
        double acc = 0.0;
        dequant_row(matrix_row(slab, H, I, 2, r), I, row);
        for (int64_t c = 0; c < I; ++c) acc += row[c] * h[c];
        y[r] = acc;
    }
    free(row);
}

/* ---------------- router ---------------- */
/* logits[e] for one token (x is bf16 bits, Wr is [E x H] fp32, bias may be NULL). */
static void token_logits(const uint16_t *x, int64_t H, const float *Wr, const float *bias, int64_t E,
                         float *logits) {
    for (int64_t e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int64_t h = 0; h < H; ++h) acc += oracle_bf16_to_double(x[h]) * (double)Wr[e * H + h];
        if (bias) acc += (double)bias[e];
        logits[e] = (float)acc;  /* one rounding, to nearest even */
    }
}

/* k largest logits, ties to the lower index, by repeated selection. */
static void token_topk(const float *logits, int64_t E, int k, int32_t *idx) {
    unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
    for (int i = 0; i < k; ++i) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || logits[e] > logits[best]) best = e;  /* strict: equal keeps the lower index */
        }
        idx[i] = (int32_t)best;
        taken[best] = 1;
    }
    free(taken);
}

/* Softmax restricted to the k selected logits, in fp64. */
static void token_weights(const float *logits, const int32_t *idx, int k, double *w) {
    double top = (double)logits[idx[0]];
    double sum = 0.0;
    for (int i = 0; i < k; ++i) {
        w[i] = exp((double)logits[idx[i]] - top);
        sum += w[i];
    }
    for (int i = 0; i < k; ++i) w[i] /= sum;
}

static int clamp_threads(int n) {
#ifdef _OPENMP
    if (n <= 0) n = omp_get_max_threads();
#else
    n = 1;
#endif
    return n < 1 ? 1 : n;
}

/* Routing for T tokens: logits [T x E] (may be NULL), idx [T x k], w [T x k]. */
void oracle_router(const uint16_t *x, int64_t T, int64_t H, const float *Wr, const float *bias, int64_t E,
                   int k, float *logits_out, int32_t *idx, double *w, int nthreads) {
    nthreads = clamp_threads(nthreads);
    #pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        float *lg = (float *)malloc(sizeof(float) * (size_t)E);
        token_logits(x + t * H, H, Wr, bias, E, lg);
        token_topk(lg, E, k, idx + t * k);
        token_weights(lg, idx + t * k, k, w + t * k);
        if (logits_out) memcpy(logits_out + t * E, lg, sizeof(float) * (size_t)E);
        free(lg);
    }
}

/* ---------------- expert FFNs and combine for a given routing ---------------- */
/* Steps 4 and 5 above for routing that is already known: token t's slot i runs
   expert idx[t*k+i] with gate weight w[t*k+i]; then the shared expert (if any)
   with weight 1.  slabs[e] = host slab of routed expert e; shared = host slab of
   the always-on shared expert or NULL.  Tokens listed in `rows` (n_rows of them;
   NULL = all T) are the only ones computed; out64/out_bf16 are [T x H] and only
   those rows are written. */
void oracle_moe_ffn_routed(const uint16_t *x, int64_t T, int64_t H, int64_t I, int k, const int32_t *idx,
                           const double *w, const uint8_t *const *slabs, const uint8_t *shared,
                           const int32_t *rows, int64_t n_rows, int nthreads, double *out64, uint16_t *out_bf16) {
    nthreads = clamp_threads(nthreads);
    int64_t nt = rows ? n_rows : T;
    int per = k + (shared ? 1 : 0);
    int64_t npairs = nt * per;
    double *y = (double *)malloc(sizeof(double) * (size_t)(npairs * H));
    /* every (token, expert) pair independently */
    #pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int64_t p = 0; p < npairs; ++p) {
        int64_t j = p / per, i = p % per;
        int64_t t = rows ? rows[j] : j;
        double *xd = (double *)malloc(sizeof(double) * (size_t)H);
        for (int64_t h = 0; h < H; ++h) xd[h] = oracle_bf16_to_double(x[t * H + h]);
        const uint8_t *slab = (i < k) ? slabs[idx[t * k + i]] : shared;
        oracle_expert_ffn(slab, H, I, xd, NULL, NULL, NULL, y + p * H);
        free(xd);
    }
    /* combine in slot order, then the shared expert */
    #pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t j = 0; j < nt; ++j) {
        int64_t t = rows ? rows[j] : j;
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int i = 0; i < k; ++i) acc += w[t * k + i] * y[(j * per + i) * H + h];
            if (shared) acc += y[(j * per + k) * H + h];
            out64[t * H + h] = acc;
            out_bf16[t * H + h] = oracle_double_to_bf16(acc);
        }
    }
    free(y);
}

/* ---------------- one MoE layer ---------------- */
/* Steps 1-5: the router for every token (idx/w are computed for all T), then the
   expert FFNs and the combine for the tokens in `rows` (NULL = all). */
void oracle_moe_layer(const uint16_t *x, int64_t T, int64_t H, int64_t I, int64_t E, int k,
                      const float *Wr, const float *bias, const uint8_t *const *slabs, const uint8_t *shared,
                      const int32_t *rows, int64_t n_rows, int nthreads,
                      int32_t *idx, double *w, double *out64, uint16_t *out_bf16) {
    nthreads = clamp_threads(nthreads);
    oracle_router(x, T, H, Wr, bias, E, k, NULL, idx, w, nthreads);
    oracle_moe_ffn_routed(x, T, H, I, k, idx, w, slabs, shared, rows, n_rows, nthreads, out64, out_bf16);
}

/* ---------------- residual stream between chained layers ----------------
 * The pages describe no block around the MoE layers; when layers are chained
 * (layer l+1's input depends on layer l's output, which predictive expert
 * prefetching needs: LayerStoRm README, "Status and limitations" and
 * "References", gating lookahead) the plainest pre-norm residual step stands in
 * for the rest of the block, per token row:
 *   resid += add            (fp32 values; the sum taken exactly, rounded once to fp32)
 *   x_next = bf16( resid / sqrt(mean(resid^2) + eps) )   in fp64, rounded once
 * add may be NULL (resid unchanged). */
void oracle_residual_norm(const uint16_t *add, float *resid, int64_t T, int64_t H, double eps, uint16_t *x_next) {
    for (int64_t t = 0; t < T; ++t) {
        float *r = resid + t * H;
        if (add)
            for (int64_t h = 0; h < H; ++h) r[h] = (float)((double)r[h] + oracle_bf16_to_double(add[t * H + h]));
        double ss = 0.0;
        for (int64_t h = 0; h < H; ++h) ss += (double)r[h] * (double)r[h];
        const double den = sqrt(ss / (double)H + eps);
        for (int64_t h = 0; h < H; ++h) x_next[t * H + h] = oracle_double_to_bf16((double)r[h] / den);
    }
}

/* ---------------- weight format selection ----------------
 * The same computations for a slab of weight format `fmt` (0 or 1).  Not
 * reentrant across formats: callers run one format at a time. */
void oracle_dequant_fmt(const uint8_t *slab, int64_t H, int64_t I, int which, double *out, int fmt) {
    g_fmt = fmt;
    oracle_dequant(slab, H, I, which, out);
    g_fmt = 0;
}
void oracle_expert_ffn_fmt(const uint8_t *slab, int64_t H, int64_t I, const double *x, double *g, double *u,
                           double *h, double *y, int fmt) {
    g_fmt = fmt;
    oracle_expert_ffn(slab, H, I, x, g, u, h, y);
    g_fmt = 0;
}
void oracle_moe_layer_fmt(const uint16_t *x, int64_t T, int64_t H, int64_t I, int64_t E, int k, const float *Wr,
                          const float *bias, const uint8_t *const *slabs, const uint8_t *shared, const int32_t *rows,
                          int64_t n_rows, int nthreads, int32_t *idx, double *w, double *out64, uint16_t *out_bf16,
                          int fmt) {
    g_fmt = fmt;
    oracle_moe_layer(x, T, H, I, E, k, Wr, bias, slabs, shared, rows, n_rows, nthreads, idx, w, out64, out_bf16);
    g_fmt = 0;
}
void oracle_moe_ffn_routed_fmt(const uint16_t *x, int64_t T, int64_t H, int64_t I, int k, const int32_t *idx,
                               const double *w, const uint8_t *const *slabs, const uint8_t *shared,
                               const int32_t *rows, int64_t n_rows, int nthreads, double *out64, uint16_t *out_bf16,
                               int fmt) {
    g_fmt = fmt;
    oracle_moe_ffn_routed(x, T, H, I, k, idx, w, slabs, shared, rows, n_rows, nthreads, out64, out_bf16);
    g_fmt = 0;
}
