/*
 * moe_oracle.c -- plain, slow CPU oracle of the routed sparse-MoE expert FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library.  It shares no code, header, table or helper with the HIP library;
 * both only consume the same seeded input tensors.
 *
 * What it computes is the plain definition of one MoE layer, evaluated token by token:
 *   route   : each token keeps the k experts with the largest router score and gets
 *             normalised gate weights (sparse MoE FFN: one big FFN split into many small
 *             experts of which a few are active per token -- CMU 11-868 appendix A2 lecture
 *             notes (semidirectx.com), section 4.1; DeepSeek-V3: 256 routed experts, 8 per
 *             token, plus one shared expert -- KTransformers article (chenxutan.com), 1.2).
 *   permute : expert histogram, exclusive prefix sum and the stable order of the (token, slot)
 *             assignments by expert ("gating and sorting" before expert compute in the
 *             expert-parallel MoE flow -- Xingyun OSDI'26 hybrid-inference article
 *             (xingyun.xin), DSLP / expert-parallel section).
 *   expert  : gate and up projections, activation times up, then down (the article's
 *             "CPU fine-grained parallelism" section: each expert is gate, up and down, and
 *             down consumes the activated product of gate and up).  Weights are E4M3FN FP8
 *             with one fp32 scale per 128x128 block that multiplies the code (the article's
 *             "native FP8 GEMV" section), or plain bf16.  Activations are bf16.
 *   combine : weighted sum of the token's expert outputs plus the shared expert ("weighted
 *             reduction" after combine in the same DSLP / expert-parallel section).
 *
 * Precision: every sum is accumulated in double.  Dequantised weights are exact in double
 * (a 4-bit significand times a 24-bit scale).  The two roundings the method fixes are
 * modelled: the intermediate h = SiLU(gate) * up is rounded to bf16 (round to nearest even),
 * and the layer output is rounded to bf16.  Router weights are computed in double and
 * rounded to fp32, the type the layer hands between steps.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - the selection key is the raw fp32 score (softmax and sigmoid are monotone); ties go to
 *     the lower expert id; slots are stored in descending order of that key;
 *   - softmax weights are normalised over the selected k (renorm=1) or over all E (renorm=0);
 *     sigmoid weights are divided by their sum over the selected k (renorm=1) or used as is;
 *   - the activation is SiLU(g) = g / (1 + exp(-g));
 *   - the permutation is stable: within an expert, assignments keep ascending flat index t*k+j.
 *
 * Optional FP8 activations (act_fp8 != 0; the FP8 MFMA mode).  The pages quantise weights in
 * 128-blocks with a scale per block (the article's "native FP8 GEMV" section); activations are
 * quantised the same way along the input dimension: per token, per 128 consecutive channels, a
 * power-of-two scale 2^e with e the smallest integer such that the block's largest magnitude is
 * at most 448 * 2^e (e clamped to [-127, 127]), codes = E4M3FN round-to-nearest-even of
 * x * 2^-e computed in fp32.  The gate/up input x and the bf16-rounded h feeding down are both
 * quantised; everything after dequantisation is exact in double as above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR 1

/* ---------------------------------------------------------------- number formats ---------- */

/* E4M3FN as defined by the OCP 8-bit floating point specification: sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN and
 * there is no infinity.  The article's "native FP8 GEMV" section names this encoding. */
double oracle_fp8_e4m3fn_to_double(uint8_t code) {
    int sign = code >> 7, expo = (code >> 3) & 15, mant = code & 7;
    double v;
    if (expo == 15 && mant == 7) return NAN;
    if (expo == 0)
        v = ldexp((double)mant, -9);
    else
        v = ldexp(1.0 + mant / 8.0, expo - 7);
    return sign ? -v : v;
}

/* OCP microscaling FP4 (E2M1): sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0
 * encodes the subnormals m * 0.5.  The format has no infinity and no NaN; its largest magnitude
 * is 6.  (The 4-bit weight codec of this library: its groups of 32 values share one E8M0 scale.) */
double oracle_fp4_e2m1_to_double(uint8_t code) {
    int sign = (code >> 3) & 1, expo = (code >> 1) & 3, mant = code & 1;
    double v = expo == 0 ? 0.5 * mant : ldexp(1.0 + 0.5 * mant, expo - 1);
    return sign ? -v : v;
}

/* OCP E8M0 scale: 2^(s - 127); s = 255 is NaN. */
double oracle_e8m0_to_double(uint8_t s) { return s == 255 ? NAN : ldexp(1.0, (int)s - 127); }

/* bf16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, in one step.
 * bf16 keeps 8 significant bits; its normal range starts at 2^-126 and its subnormals are
 * multiples of 2^-133.  For |v| in [2^(e-1), 2^e) the spacing of bf16 values is 2^(e-8), and
 * 2^-133 below the normal range. */
uint16_t oracle_double_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    int e;
    frexp(v, &e);
    if (v == 0.0) e = -125;
    int q = (e > -125 ? e : -125) - 8;
    double r = ldexp(rint(ldexp(v, -q)), q); /* rint: round half to even (default mode) */
    float f;
    if (fabs(r) >= ldexp(1.0, 128))
        f = (r > 0) ? INFINITY : -INFINITY;
    else
        f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* ---------------------------------------------------------------- routing ------------------ */

/* Top-k routing of T tokens over E experts.  scores [T][E] fp32 row-major.
 * Outputs ids [T][k] (descending key, ties to the lower id) and weights w [T][k] fp32.
 * score_fn 0 = softmax, 1 = sigmoid. */
/* E4M3FN code of a float with |v| <= 448, round to nearest, ties to even (OCP definition:
 * normals 1.m x 2^E for E in [-6, 8] with 3 mantissa bits, subnormals m x 2^-9).  The sign of a
 * zero is kept (0x80 is -0). */
uint8_t oracle_float_to_e4m3fn(float v) {
    const uint8_t sign = signbit(v) ? 0x80 : 0;
    const double a = fabs((double)v);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);                       /* a in [2^(e2-1), 2^e2) */
    const int E = e2 - 1;
    const double q = E < -6 ? ldexp(1.0, -9) : ldexp(1.0, E - 3); /* grid step of a's binade */
    const double val = rint(a / q) * q;  /* a / q is exact; rint rounds half to even */
    if (val == 0.0) return sign;
    if (val < ldexp(1.0, -6)) return sign | (uint8_t)(val / ldexp(1.0, -9));
    frexp(val, &e2);
    const int Ev = e2 - 1;
    const int mant = (int)(val / ldexp(1.0, Ev - 3)) - 8; /* 8..15 -> 0..7 */
    return sign | (uint8_t)(((Ev + 7) << 3) | mant);
}

/* Exponent e of the power-of-two scale of an activation block with largest magnitude amax:
 * the smallest e with amax <= 448 * 2^e = 1.75 * 2^(8+e), clamped to [-127, 127]; 0 for amax 0. */
int oracle_act_scale_exp(double amax) {
    if (!(amax > 0.0)) return 0;
    int e2;
    const double m = frexp(amax, &e2); /* amax = m 2^e2, m in [0.5, 1) */
    int e = (m <= 0.875) ? e2 - 9 : e2 - 8;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* Quantises n values (exact in fp32) in place to their dequantised FP8 values, one scale for the
 * block; returns the scale's exponent.  codes (optional) receives the n codes. */
static int quantize_block(double* v, int n, uint8_t* codes) {
    double amax = 0.0;
    for (int i = 0; i < n; ++i) amax = fmax(amax, fabs(v[i]));
    const int e = oracle_act_scale_exp(amax);
    for (int i = 0; i < n; ++i) {
        const uint8_t c = oracle_float_to_e4m3fn(ldexpf((float)v[i], -e));
        if (codes) codes[i] = c;
        v[i] = ldexp(oracle_fp8_e4m3fn_to_double(c), e);
    }
    return e;
}

/* Rows of bf16 values [rows][K] (K a multiple of 128) -> E4M3FN codes [rows][K] and scale
 * exponents [rows][K/128] (the activation quantisation above). */
void oracle_quantize_rows(const uint16_t* x, int rows, int K, uint8_t* codes, int8_t* exps) {
    double v[128];
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < K / 128; ++b) {
            for (int i = 0; i < 128; ++i) v[i] = oracle_bf16_to_double(x[(size_t)r * K + b * 128 + i]);
            exps[(size_t)r * (K / 128) + b] =
                (int8_t)quantize_block(v, 128, codes + (size_t)r * K + b * 128);
        }
}

int oracle_route(const float* scores, int T, int E, int k, int score_fn, int renorm,
                 int32_t* ids, float* w) {
    if (k < 1 || k > E) return ORACLE_ERR;
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        const float* s = scores + (size_t)t * E;
        int32_t* id = ids + (size_t)t * k;
        memset(taken, 0, (size_t)E);
        /* selection by repeated search for the largest remaining score */
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || s[e] > s[best])) best = e;
            taken[best] = 1;
            id[j] = best;
        }
        double den = 0.0, num[1024];
        if (k > 1024) { free(taken); return ORACLE_ERR; }
        if (score_fn == 0) {
            double mx = (double)s[id[0]];
            for (int j = 0; j < k; ++j) num[j] = exp((double)s[id[j]] - mx);
            if (renorm)
                for (int j = 0; j < k; ++j) den += num[j];
            else
                for (int e = 0; e < E; ++e) den += exp((double)s[e] - mx);
        } else {
            for (int j = 0; j < k; ++j) num[j] = 1.0 / (1.0 + exp(-(double)s[id[j]]));
            if (renorm)
                for (int j = 0; j < k; ++j) den += num[j];
            else
                den = 1.0;
        }
        for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = (float)(num[j] / den);
    }
    free(taken);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- grouping ----------------- */

/* Histogram, exclusive prefix sum and stable permutation of the T*k assignments by expert.
 * perm[p] = flat index t*k+j of the p-th assignment in expert order; inv[perm[p]] = p. */
int oracle_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                   int32_t* perm, int32_t* inv) {
    long n = (long)T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (long f = 0; f < n; ++f) {
        if (ids[f] < 0 || ids[f] >= E) return ORACLE_ERR;
        counts[ids[f]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    long p = 0;
    for (int e = 0; e < E; ++e)
        for (long f = 0; f < n; ++f)
            if (ids[f] == e) perm[p++] = (int32_t)f;
    for (p = 0; p < n; ++p) inv[perm[p]] = (int32_t)p;
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- expert FFN --------------- */

/* n experts of one layer, nn.Linear layout (output rows, input contiguous):
 * gate, up [n][I][H]; down [n][H][I].  wdtype 0: E4M3FN codes with fp32 scales
 * s_gate, s_up [n][I/128][H/128], s_down [n][H/128][I/128]; wdtype 1: bf16 bits, no scales. */
/* wdtype 0: E4M3FN codes [n][rows][cols] + fp32 scales [n][rows/128][cols/128];
 *        1: bf16 bits [n][rows][cols] (no scales);
 *        2: MXFP4, bytes [n][rows][cols/2] (two codes a byte) + E8M0 bytes [n][rows][cols/32]
 *           (the s_* pointers then point to bytes). */
typedef struct {
    int32_t wdtype, n, H, I;
    const void *gate, *up, *down;
    const float *s_gate, *s_up, *s_down;
} oracle_weights;

/* The 256 E4M3FN values, the 16 E2M1 values and the 256 E8M0 values, tabulated once from
 * oracle_fp8_e4m3fn_to_double, oracle_fp4_e2m1_to_double and oracle_e8m0_to_double (a cache of
 * those functions, so the inner loops do not call ldexp per weight). */
static double fp8_table[256];
static double fp4_table[16];
static double e8m0_table[256];
static int fp8_table_ready = 0;

static void fill_fp8_table(void) {
#ifdef _OPENMP
#pragma omp critical(oracle_fp8_table)
#endif
    {
        if (!fp8_table_ready) {
            for (int i = 0; i < 256; ++i) fp8_table[i] = oracle_fp8_e4m3fn_to_double((uint8_t)i);
            for (int i = 0; i < 16; ++i) fp4_table[i] = oracle_fp4_e2m1_to_double((uint8_t)i);
            for (int i = 0; i < 256; ++i) e8m0_table[i] = oracle_e8m0_to_double((uint8_t)i);
            fp8_table_ready = 1;
        }
    }
}

/* Dequantised weight (row r, column c) of matrix `mat` of expert slot `x`, shape rows x cols. */
static double weight(const oracle_weights* W, const void* mat, const float* sc, int x, int rows,
                     int cols, int r, int c) {
    size_t at = ((size_t)x * rows + r) * cols + c;
    if (W->wdtype == 1) return oracle_bf16_to_double(((const uint16_t*)mat)[at]);
    if (W->wdtype == 2) {  /* MXFP4: two codes a byte (element 2j low nibble), E8M0 per 32 */
        const uint8_t b = ((const uint8_t*)mat)[at / 2];
        const uint8_t code = (c & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
        const uint8_t s = ((const uint8_t*)sc)[at / 32];
        return fp4_table[code] * e8m0_table[s];
    }
    double scale = sc[((size_t)x * (rows / 128) + r / 128) * (cols / 128) + c / 128];
    return fp8_table[((const uint8_t*)mat)[at]] * scale;
}

/* The activated product of one output column: bf16( SiLU(g) * u ), SiLU(g) = g / (1 + e^-g)
 * (the article's "CPU fine-grained parallelism" section: activation of gate, times up). */
static uint16_t silu_mul_bf16(double g, double u) {
    return oracle_double_to_bf16(g / (1.0 + exp(-g)) * u);
}

/* Gate and up of expert slot x on the activations xd (length H, double):
 * h[n] = bf16(SiLU(g_n) * u_n) with g = Wg x, u = Wu x.  Writes the bf16 bits to h_out (if not
 * NULL) and their values to hd. */
static void gate_up_row(const oracle_weights* W, int x, const double* xd, uint16_t* h_out,
                        double* hd) {
    const int H = W->H, I = W->I;
    for (int n = 0; n < I; ++n) {
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; ++c) {
            g += xd[c] * weight(W, W->gate, W->s_gate, x, I, H, n, c);
            u += xd[c] * weight(W, W->up, W->s_up, x, I, H, n, c);
        }
        uint16_t hb = silu_mul_bf16(g, u);
        if (h_out) h_out[n] = hb;
        hd[n] = oracle_bf16_to_double(hb);
    }
}

/* Down projection of expert slot x: y = Wd h (double, length H) for h of length I. */
static void down_row(const oracle_weights* W, int x, const double* hd, double* y_out) {
    const int H = W->H, I = W->I;
    for (int c = 0; c < H; ++c) {
        double y = 0.0;
        for (int n = 0; n < I; ++n) y += hd[n] * weight(W, W->down, W->s_down, x, H, I, c, n);
        y_out[c] = y;
    }
}

/* One expert (slot x) on one token row xrow (bf16 bits, length H): gate_up_row then down_row,
 * with x and h quantised first in the FP8 activation mode. */
static void expert_on_token(const oracle_weights* W, int x, const uint16_t* xrow, uint16_t* h_out,
                            double* y_out, double* xd, double* hd, int act_fp8) {
    const int H = W->H, I = W->I;
    for (int c = 0; c < H; ++c) xd[c] = oracle_bf16_to_double(xrow[c]);
    if (act_fp8)
        for (int b = 0; b < H / 128; ++b) quantize_block(xd + b * 128, 128, NULL);
    gate_up_row(W, x, xd, h_out, hd);
    if (act_fp8)
        for (int b = 0; b < I / 128; ++b) quantize_block(hd + b * 128, 128, NULL);
    down_row(W, x, hd, y_out);
}

/* Expert phase 1 alone on rows p = 0..n_rows-1: h[p] = gate/up of expert slot[p] on the bf16
 * activations x[token[p]] (bits, rows of length H), as in the layer (bf16 activations). */
int oracle_expert_gate_up(const uint16_t* x, int n_tokens, int n_rows, const int32_t* token,
                          const int32_t* slot, const oracle_weights* W, uint16_t* h, int n_threads) {
    fill_fp8_table();
    for (int p = 0; p < n_rows; ++p)
        if (token[p] < 0 || token[p] >= n_tokens || slot[p] < 0 || slot[p] >= W->n) return ORACLE_ERR;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel
#endif
    {
        double* xd = (double*)malloc(sizeof(double) * W->H);
        double* hd = (double*)malloc(sizeof(double) * W->I);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int p = 0; p < n_rows; ++p) {
            const uint16_t* xrow = x + (size_t)token[p] * W->H;
            for (int c = 0; c < W->H; ++c) xd[c] = oracle_bf16_to_double(xrow[c]);
            gate_up_row(W, slot[p], xd, h + (size_t)p * W->I, hd);
        }
        free(xd); free(hd);
    }
    return ORACLE_OK;
}

/* Expert phase 2 alone: y[p] = down projection of expert slot[p] on the bf16 row h[p] (bits,
 * length I), in double. */
int oracle_expert_down(const uint16_t* h, int n_rows, const int32_t* slot, const oracle_weights* W,
                       double* y, int n_threads) {
    fill_fp8_table();
    for (int p = 0; p < n_rows; ++p)
        if (slot[p] < 0 || slot[p] >= W->n) return ORACLE_ERR;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel
#endif
    {
        double* hd = (double*)malloc(sizeof(double) * W->I);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int p = 0; p < n_rows; ++p) {
            for (int n = 0; n < W->I; ++n) hd[n] = oracle_bf16_to_double(h[(size_t)p * W->I + n]);
            down_row(W, slot[p], hd, y + (size_t)p * W->H);
        }
        free(hd);
    }
    return ORACLE_OK;
}

static void set_error(int* err) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
    *err = 1;
}

/* The whole layer for the tokens listed in rows[0..n_rows) (rows == NULL: all T tokens).
 *   scores [T][E], x [T][H] bf16 bits;
 *   routed: the routed experts; expert_slot[e] gives the slot of expert e in `routed`
 *           (NULL: slot = e; -1: expert not provided, an error if selected);
 *   shared: the shared expert (slot 0, gate weight 1) or NULL.
 * Outputs for row i (all optional except out):
 *   ids [i][k], w [i][k], out [i][H] bf16 bits, h [i][k][I] bf16 bits, y [i][k][H] double,
 *   S [i][H] double (shared expert output), hS [i][I] bf16 bits (the shared expert's h).
 * out = bf16( S + sum_j w_j * y_j ), accumulated in double in the order S, j = 0..k-1.
 * Only experts e_begin <= e < e_end are evaluated and summed: one rank's local weighted partial
 * reduction under expert parallelism (OSDI'26 article, SmallEP section); [0, E) is the layer.
 * The h and y of the other assignments are reported as zeros. */
int oracle_moe_layer(const float* scores, const uint16_t* x, int T, int H, int I, int E, int k,
                     int score_fn, int renorm, const oracle_weights* routed,
                     const int32_t* expert_slot, const oracle_weights* shared,
                     const int32_t* rows, int n_rows, int32_t* ids_out, float* w_out,
                     uint16_t* out, uint16_t* h_out, double* y_out, double* S_out,
                     int n_threads, int act_fp8, uint16_t* hS_out, int e_begin, int e_end) {
    if (routed->H != H || routed->I != I) return ORACLE_ERR;
    if (shared && (shared->H != H || shared->I != I)) return ORACLE_ERR;
    if (rows == NULL) n_rows = T;
    fill_fp8_table();
    int err = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel
#endif
    {
        double* xd = (double*)malloc(sizeof(double) * H);
        double* hd = (double*)malloc(sizeof(double) * I);
        double* y = (double*)malloc(sizeof(double) * H * (size_t)(k + 1));
        uint16_t* hb = (uint16_t*)malloc(sizeof(uint16_t) * I);
        int32_t id[1024];
        float wt[1024];
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int i = 0; i < n_rows; ++i) {
            int t = rows ? rows[i] : i;
            if (t < 0 || t >= T || k > 1024 ||
                oracle_route(scores + (size_t)t * E, 1, E, k, score_fn, renorm, id, wt)) {
                set_error(&err);
                continue;
            }
            const uint16_t* xrow = x + (size_t)t * H;
            double* S = y + (size_t)k * H;
            for (int c = 0; c < H; ++c) S[c] = 0.0;
            if (shared)
                expert_on_token(shared, 0, xrow, hS_out ? hS_out + (size_t)i * I : NULL, S, xd, hd,
                                act_fp8);
            for (int j = 0; j < k; ++j) {
                if (id[j] < e_begin || id[j] >= e_end) {  /* not this share's expert */
                    for (int c = 0; c < H; ++c) y[(size_t)j * H + c] = 0.0;
                    if (h_out) memset(h_out + ((size_t)i * k + j) * I, 0, sizeof(uint16_t) * I);
                    continue;
                }
                int slot = expert_slot ? expert_slot[id[j]] : id[j];
                if (slot < 0 || slot >= routed->n) { set_error(&err); break; }
                expert_on_token(routed, slot, xrow, hb, y + (size_t)j * H, xd, hd, act_fp8);
                if (h_out) memcpy(h_out + ((size_t)i * k + j) * I, hb, sizeof(uint16_t) * I);
            }
            for (int c = 0; c < H; ++c) {
                double acc = S[c];
                for (int j = 0; j < k; ++j)
                    if (id[j] >= e_begin && id[j] < e_end) acc += (double)wt[j] * y[(size_t)j * H + c];
                out[(size_t)i * H + c] = oracle_double_to_bf16(acc);
            }
            if (ids_out) memcpy(ids_out + (size_t)i * k, id, sizeof(int32_t) * k);
            if (w_out) memcpy(w_out + (size_t)i * k, wt, sizeof(float) * k);
            if (y_out) memcpy(y_out + (size_t)i * k * H, y, sizeof(double) * (size_t)k * H);
            if (S_out) memcpy(S_out + (size_t)i * H, S, sizeof(double) * H);
        }
        free(xd); free(hd); free(y); free(hb);
    }
    return err ? ORACLE_ERR : ORACLE_OK;
}

/* Number of threads an OpenMP parallel region of this library uses with n_threads requested. */
int oracle_max_threads(int n_threads) {
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
    return omp_get_max_threads();
#else
    (void)n_threads;
    return 1;
#endif
}

/* ---------------------------------------------------------------- batched form ------------
 * The pieces of the same definition for an evaluation that takes each expert's tokens
 * together: the expert's matrices dequantised once (exact doubles), and the element-wise steps
 * over whole arrays.  The sums themselves are formed by a library float64 matrix product; every
 * other step is the code above. */

/* Matrix `which` (0 gate, 1 up, 2 down) of expert slot x, dequantised into out, row-major
 * [rows][cols] = [I][H] (gate, up) or [H][I] (down). */
int oracle_dequantize(const oracle_weights* W, int x, int which, double* out, int n_threads) {
    if (x < 0 || x >= W->n || which < 0 || which > 2) return ORACLE_ERR;
    fill_fp8_table();
    const void* mat = which == 0 ? W->gate : which == 1 ? W->up : W->down;
    const float* sc = which == 0 ? W->s_gate : which == 1 ? W->s_up : W->s_down;
    const int rows = which == 2 ? W->H : W->I, cols = which == 2 ? W->I : W->H;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(static)
#endif
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c)
            out[(size_t)r * cols + c] = weight(W, mat, sc, x, rows, cols, r, c);
    return ORACLE_OK;
}

/* h[i] = bf16( SiLU(g[i]) * u[i] ) for n values. */
void oracle_silu_mul_bf16(const double* g, const double* u, long n, uint16_t* h) {
    for (long i = 0; i < n; ++i) h[i] = silu_mul_bf16(g[i], u[i]);
}

/* bf16 bits of n doubles (round to nearest even, one step). */
void oracle_double_to_bf16_array(const double* v, long n, uint16_t* out) {
    for (long i = 0; i < n; ++i) out[i] = oracle_double_to_bf16(v[i]);
}

/* The FP8 activation mode's quantisation applied in place to rows of values [rows][K] (exact in
 * fp32, K a multiple of 128): each 128-block replaced by its dequantised E4M3FN codes. */
void oracle_quantize_dequantize(double* v, long rows, int K) {
    for (long r = 0; r < rows; ++r)
        for (int b = 0; b < K / 128; ++b) quantize_block(v + r * K + b * 128, 128, NULL);
}
