/* Drives every entry point of the C oracle on small layers in every weight format and both
 * activation modes, for a build with AddressSanitizer and UndefinedBehaviorSanitizer: any
 * out-of-bounds access, use of uninitialised heap memory or undefined arithmetic aborts.
 * The values are only checked for finiteness; their correctness is pinned elsewhere. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t wdtype, n, H, I;
    const void *gate, *up, *down;
    const float *s_gate, *s_up, *s_down;
} oracle_weights;

int oracle_route(const float*, int, int, int, int, int, int32_t*, float*);
int oracle_permute(const int32_t*, int, int, int, int32_t*, int32_t*, int32_t*, int32_t*);
int oracle_moe_layer(const float*, const uint16_t*, int, int, int, int, int, int, int,
                     const oracle_weights*, const int32_t*, const oracle_weights*, const int32_t*,
                     int, int32_t*, float*, uint16_t*, uint16_t*, double*, double*, int, int,
                     uint16_t*, int, int);
void oracle_quantize_rows(const uint16_t*, int, int, uint8_t*, int8_t*);
int oracle_expert_gate_up(const uint16_t*, int, int, const int32_t*, const int32_t*,
                          const oracle_weights*, uint16_t*, int);
int oracle_expert_down(const uint16_t*, int, const int32_t*, const oracle_weights*, double*, int);
int oracle_dequantize(const oracle_weights*, int, int, double*, int);
void oracle_silu_mul_bf16(const double*, const double*, long, uint16_t*);
void oracle_double_to_bf16_array(const double*, long, uint16_t*);
void oracle_quantize_dequantize(double*, long, int);
uint16_t oracle_double_to_bf16(double);
double oracle_bf16_to_double(uint16_t);

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng >> 8; }
static double unif(void) { return (next() & 0xFFFFFF) / 16777216.0; }

static void* fill_bytes(size_t n, int avoid_fp8_nan) {
    uint8_t* p = malloc(n);
    for (size_t i = 0; i < n; ++i) {
        uint8_t b = (uint8_t)next();
        if (avoid_fp8_nan && (b & 0x7F) == 0x7F) b = 0;
        p[i] = b;
    }
    return p;
}

static uint16_t* bf16_normal(size_t n, double scale) {
    uint16_t* p = malloc(n * 2);
    for (size_t i = 0; i < n; ++i) p[i] = oracle_double_to_bf16((unif() - 0.5) * scale);
    return p;
}

static oracle_weights make_weights(int wdtype, int n, int H, int I, void** keep) {
    oracle_weights w = {wdtype, n, H, I, 0, 0, 0, 0, 0, 0};
    size_t mat = (size_t)n * H * I;
    for (int m = 0; m < 3; ++m) {
        if (wdtype == 1) keep[m] = bf16_normal(mat, 0.04);
        else keep[m] = fill_bytes(wdtype == 2 ? mat / 2 : mat, wdtype == 0);
        size_t ns = wdtype == 0 ? (size_t)n * (H / 128) * (I / 128) : wdtype == 2 ? mat / 32 : 0;
        if (wdtype == 0) {
            float* s = malloc(ns * 4);
            for (size_t i = 0; i < ns; ++i) s[i] = (float)(unif() * 0.01);
            keep[3 + m] = s;
        } else if (wdtype == 2) {
            uint8_t* s = malloc(ns);
            for (size_t i = 0; i < ns; ++i) s[i] = (uint8_t)(120 + next() % 10);
            keep[3 + m] = s;
        } else {
            keep[3 + m] = NULL;
        }
    }
    w.gate = keep[0]; w.up = keep[1]; w.down = keep[2];
    w.s_gate = keep[3]; w.s_up = keep[4]; w.s_down = keep[5];
    return w;
}

static int finite_bf16(const uint16_t* v, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(oracle_bf16_to_double(v[i]))) return 0;
    return 1;
}

int main(void) {
    const int T = 12, H = 256, I = 128, E = 6, k = 3;
    int failures = 0;
    for (int wdtype = 0; wdtype < 3; ++wdtype)
        for (int act = 0; act < 2; ++act) {
            if (wdtype == 1 && act) continue;
            void *kr[6], *ks[6];
            oracle_weights W = make_weights(wdtype, E, H, I, kr);
            oracle_weights S = make_weights(wdtype, 1, H, I, ks);
            float* scores = malloc(sizeof(float) * T * E);
            for (int i = 0; i < T * E; ++i) scores[i] = (float)unif();
            uint16_t* x = bf16_normal((size_t)T * H, 4.0);
            int32_t* ids = malloc(sizeof(int32_t) * T * k);
            float* w = malloc(sizeof(float) * T * k);
            uint16_t* out = malloc(2 * (size_t)T * H);
            uint16_t* h = malloc(2 * (size_t)T * k * I);
            uint16_t* hS = malloc(2 * (size_t)T * I);
            double* y = malloc(sizeof(double) * T * k * H);
            double* Sy = malloc(sizeof(double) * T * H);
            int32_t rows[5] = {0, 3, 11, 7, 7};
            if (oracle_route(scores, T, E, k, act, 1, ids, w)) ++failures;
            int32_t counts[6], offsets[7], perm[36], inv[36];
            if (oracle_permute(ids, T, k, E, counts, offsets, perm, inv)) ++failures;
            if (oracle_moe_layer(scores, x, T, H, I, E, k, 1, 1, &W, NULL, &S, NULL, 0, ids, w,
                                 out, h, y, Sy, 1, act, hS, 0, E)) ++failures;
            if (!finite_bf16(out, (size_t)T * H)) ++failures;
            if (oracle_moe_layer(scores, x, T, H, I, E, k, 0, 0, &W, NULL, NULL, rows, 5, ids, w,
                                 out, h, y, Sy, 1, act, NULL, 2, 5)) ++failures;
            int32_t tok[4] = {0, 5, 11, 2}, slot[4] = {0, 5, 3, 3};
            if (oracle_expert_gate_up(x, T, 4, tok, slot, &W, h, 1)) ++failures;
            if (oracle_expert_down(h, 4, slot, &W, y, 1)) ++failures;
            double* d = malloc(sizeof(double) * H * I);
            for (int m = 0; m < 3; ++m)
                if (oracle_dequantize(&S, 0, m, d, 1)) ++failures;
            uint16_t* hb = malloc(2 * (size_t)H * I);
            oracle_silu_mul_bf16(d, d, (long)H * I, hb);
            oracle_double_to_bf16_array(d, (long)H * I, hb);
            oracle_quantize_dequantize(d, I, H);
            uint8_t* codes = malloc((size_t)T * H);
            int8_t* exps = malloc((size_t)T * (H / 128));
            oracle_quantize_rows(x, T, H, codes, exps);
            /* rejected arguments */
            if (oracle_route(scores, T, E, E + 1, 0, 1, ids, w) == 0) ++failures;
            ids[0] = E;
            if (oracle_permute(ids, T, k, E, counts, offsets, perm, inv) == 0) ++failures;
            if (oracle_dequantize(&S, 1, 0, d, 1) == 0) ++failures;
            free(d); free(hb); free(codes); free(exps);
            free(scores); free(x); free(ids); free(w); free(out); free(h); free(hS); free(y); free(Sy);
            for (int m = 0; m < 6; ++m) { free(kr[m]); free(ks[m]); }
        }
    printf("oracle driver: %d failures\n", failures);
    return failures != 0;
}
