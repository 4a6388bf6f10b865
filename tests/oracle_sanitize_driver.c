/* Drives every oracle entry point on small seeded inputs, for a host build
 * of the oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitizers.py).  Exits non-zero if a pack round trip
 * or an overflow flag is wrong; the sanitizers abort on any memory or
 * undefined-behaviour error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_mask(const uint16_t *W, int64_t n_out, int64_t k, int n, int m, uint8_t *mask);
double oracle_gamma(const uint16_t *W, int64_t n_out, int64_t k, int over_masked, const uint8_t *mask);
void oracle_ternary(const uint16_t *W, const uint8_t *mask, double gamma, int64_t n_out, int64_t k,
                    int8_t *T);
void oracle_act_quant(const uint16_t *X, int64_t tokens, int64_t k, int8_t *xq, double *scale);
int oracle_fwd(const int8_t *xq, const double *scale, const int8_t *T, double gamma, int64_t tokens,
               int64_t k, int64_t n_out, int32_t *acc, double *Y, int threads);
void oracle_fwd_pairs(const int8_t *xq, const double *scale, const int8_t *T, double gamma, int64_t k,
                      const int64_t *t_idx, const int64_t *n_idx, int64_t count, int64_t *acc,
                      double *Y);
int oracle_fwd_bf16(const int8_t *xq, const double *scale, const int8_t *T, double gamma,
                    int64_t tokens, int64_t k, int64_t n_out, uint16_t *Y);
void oracle_bwd_dx(const uint16_t *dY, const int8_t *T, double gamma, int64_t tokens, int64_t k,
                   int64_t n_out, double *dX, int threads);
void oracle_bwd_dw(const uint16_t *dY, const int8_t *xq, const double *scale, int64_t tokens,
                   int64_t k, int64_t n_out, double *dW, int threads);
void oracle_bwd_dx_pairs(const uint16_t *dY, const int8_t *T, double gamma, int64_t k, int64_t n_out,
                         const int64_t *t_idx, const int64_t *c_idx, int64_t count, double *out);
void oracle_bwd_dw_pairs(const uint16_t *dY, const int8_t *xq, const double *scale, int64_t tokens,
                         int64_t k, int64_t n_out, const int64_t *r_idx, const int64_t *c_idx,
                         int64_t count, double *out);
int oracle_s_of(int n, int m);
int64_t oracle_packed_bytes(int64_t n_out, int64_t k, int s);
int oracle_pack(const int8_t *T, int64_t n_out, int64_t k, int s, uint8_t *packed);
void oracle_unpack(const uint8_t *packed, int64_t n_out, int64_t k, int s, int8_t *T);
int64_t oracle_sp24_packed_bytes(int64_t n_out, int64_t k);
int oracle_pack_sp24(const int8_t *T, int64_t n_out, int64_t k, uint8_t *packed);
void oracle_unpack_sp24(const uint8_t *packed, int64_t n_out, int64_t k, int8_t *T);
void oracle_latent_update(float *w_master, const float *dw, int64_t count, float lr, uint16_t *w);
void oracle_relu2_gate(const float *G, const float *U, int64_t count, uint16_t *H);
void oracle_relu2_gate_bwd(const float *dH, const float *G, const float *U, int64_t count, uint16_t *dG,
                           uint16_t *dU);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double uniform(void) {  /* splitmix64 -> [0, 1) */
    uint64_t z = (state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return (double)((z ^ (z >> 31)) >> 11) * 0x1.0p-53;
}
static uint16_t bf16_of(float f) {  /* truncation is enough for test data */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void) {
    const int64_t n_out = 72, k = 256, tokens = 5;  /* a ragged strip, two k blocks */
    const int patterns[6][2] = {{8, 8}, {6, 8}, {4, 8}, {2, 4}, {3, 8}, {2, 8}};
    uint16_t *W = malloc(sizeof(uint16_t) * n_out * k), *X = malloc(sizeof(uint16_t) * tokens * k);
    uint16_t *dY = malloc(sizeof(uint16_t) * tokens * n_out);
    for (int64_t i = 0; i < n_out * k; ++i) W[i] = bf16_of((float)(0.04 * (uniform() - 0.5)));
    for (int64_t i = 0; i < tokens * k; ++i) X[i] = bf16_of((float)(4.0 * (uniform() - 0.5)));
    for (int64_t i = 0; i < tokens * n_out; ++i) dY[i] = bf16_of((float)(uniform() - 0.5));
    uint8_t *mask = malloc((size_t)(n_out * k / 8));
    int8_t *T = malloc((size_t)(n_out * k)), *T2 = malloc((size_t)(n_out * k));
    int8_t *xq = malloc((size_t)(tokens * k));
    double *sc = malloc(sizeof(double) * tokens);
    int32_t *acc = malloc(sizeof(int32_t) * tokens * n_out);
    double *Y = malloc(sizeof(double) * tokens * n_out);
    uint16_t *Yb = malloc(sizeof(uint16_t) * tokens * n_out);
    double *dX = malloc(sizeof(double) * tokens * k), *dW = malloc(sizeof(double) * n_out * k);
    oracle_act_quant(X, tokens, k, xq, sc);
    for (int p = 0; p < 6; ++p) {
        const int n = patterns[p][0], m = patterns[p][1], s = oracle_s_of(n, m);
        CHECK(s > 0);
        oracle_mask(W, n_out, k, n, m, mask);
        for (int over = 0; over < 2; ++over) {
            const double g = oracle_gamma(W, n_out, k, over, mask);
            CHECK(g > 0.0);
            oracle_ternary(W, mask, g, n_out, k, T);
        }
        const double g = oracle_gamma(W, n_out, k, 0, mask);
        const int64_t pb = oracle_packed_bytes(n_out, k, s);
        uint8_t *packed = malloc((size_t)pb);
        CHECK(oracle_pack(T, n_out, k, s, packed) == 0);
        oracle_unpack(packed, n_out, k, s, T2);
        CHECK(memcmp(T, T2, (size_t)(n_out * k)) == 0);
        free(packed);
        if (n == 2 && m == 4) {
            uint8_t *sp = malloc((size_t)oracle_sp24_packed_bytes(n_out, k));
            CHECK(oracle_pack_sp24(T, n_out, k, sp) == 0);
            oracle_unpack_sp24(sp, n_out, k, T2);
            CHECK(memcmp(T, T2, (size_t)(n_out * k)) == 0);
            free(sp);
        }
        for (int threads = 1; threads <= 3; threads += 2) {
            CHECK(oracle_fwd(xq, sc, T, g, tokens, k, n_out, acc, Y, threads) == 0);
            oracle_bwd_dx(dY, T, g, tokens, k, n_out, dX, threads);
            oracle_bwd_dw(dY, xq, sc, tokens, k, n_out, dW, threads);
        }
        CHECK(oracle_fwd_bf16(xq, sc, T, g, tokens, k, n_out, Yb) == 0);
        const int64_t ti[3] = {0, 2, tokens - 1}, ni[3] = {0, 5, n_out - 1}, ci[3] = {0, 130, k - 1};
        int64_t pacc[3];
        double py[3], pdx[3], pdw[3];
        oracle_fwd_pairs(xq, sc, T, g, k, ti, ni, 3, pacc, py);
        for (int i = 0; i < 3; ++i) CHECK(pacc[i] == acc[ti[i] * n_out + ni[i]]);
        oracle_bwd_dx_pairs(dY, T, g, k, n_out, ti, ci, 3, pdx);
        oracle_bwd_dw_pairs(dY, xq, sc, tokens, k, n_out, ni, ci, 3, pdw);
        for (int i = 0; i < 3; ++i) {
            CHECK(fabs(pdx[i] - dX[ti[i] * k + ci[i]]) <= 1e-12 * (1.0 + fabs(pdx[i])));
            CHECK(fabs(pdw[i] - dW[ni[i] * k + ci[i]]) <= 1e-12 * (1.0 + fabs(pdw[i])));
        }
    }
    const int64_t cnt = 64;
    float wm[64], dw[64], G[64], U[64], dH[64];
    uint16_t wb[64], H[64], dG[64], dU[64];
    for (int i = 0; i < cnt; ++i) {
        wm[i] = (float)(uniform() - 0.5); dw[i] = (float)(uniform() - 0.5);
        G[i] = (float)(uniform() - 0.5); U[i] = (float)(uniform() - 0.5); dH[i] = (float)(uniform() - 0.5);
    }
    oracle_latent_update(wm, dw, cnt, 1e-3f, wb);
    oracle_relu2_gate(G, U, cnt, H);
    oracle_relu2_gate_bwd(dH, G, U, cnt, dG, dU);
    free(W); free(X); free(dY); free(mask); free(T); free(T2); free(xq); free(sc); free(acc); free(Y);
    free(Yb); free(dX); free(dW);
    puts("oracle entry points ran clean");
    return 0;
}
