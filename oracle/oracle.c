/*
 * oracle.c -- plain, slow CPU reference for the Sparse-BitNet BitLinear path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark do.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * Every function computes the plain definition of one step, element by
 * element, in exact integer arithmetic or in IEEE binary64.  No blocking,
 * no fusion, no reordering beyond what the definition states.  Where the
 * pages leave a step open, the reading taken is stated next to the code.
 *
 * Sources (cited by page title and section; the pages give prose only, no
 * formulas):
 *   [SB]    Sparse-BitNet explainer article (m.top168.com, news 814037),
 *           sections 二 .. 七.
 *   [SBabs] "Sparse-BitNet: 1.58-bit LLMs are Naturally Friendly to
 *           Semi-Structured Sparsity", paper listing, abstract.
 *   [2B4T]  BitNet b1.58 2B4T article (lsdiaocha.cn), sections 一 and 四.
 *
 * Data conventions:
 *   bf16 values arrive as their raw 16-bit patterns (uint16_t).
 *   W is [n_out x k] row-major, X is [tokens x k] row-major,
 *   dY is [tokens x n_out] row-major.
 *   A mask is uint8 [n_out][k/8]; bit (k % 8) of byte k/8 is 1 = kept.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* bf16 decoding (exact: every bf16 value is a binary64 value).        */
/* ------------------------------------------------------------------ */
static double bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------ */
/* Step 1: N:M mask.                                                   */
/* [SB] §三: the mask is recomputed every training step from the        */
/* current weights; §五: within every group of 8 parameters a per-group */
/* threshold keeps 6 and drops 2 (6:8), §四 sweeps 8:8 .. 2:8 and 2:4;  */
/* §六: the ranking uses the full-precision latent weights, not the     */
/* ternary codes.                                                       */
/* Reading: groups are M consecutive entries along the input dimension  */
/* k; entries are ranked by |W| (exact, +0 == -0), larger first, and     */
/* equal magnitudes rank the lower k first; the first N are kept.       */
/* ------------------------------------------------------------------ */
void oracle_mask(const uint16_t *W, int64_t n_out, int64_t k, int n, int m,
                 uint8_t *mask)
{
    memset(mask, 0, (size_t)(n_out * (k / 8)));
    for (int64_t r = 0; r < n_out; ++r) {
        for (int64_t g0 = 0; g0 < k; g0 += m) {
            for (int j = 0; j < m; ++j) {
                double aj = fabs(bf16_value(W[r * k + g0 + j]));
                int rank = 0; /* entries that rank ahead of j */
                for (int i = 0; i < m; ++i) {
                    if (i == j) continue;
                    double ai = fabs(bf16_value(W[r * k + g0 + i]));
                    if (ai > aj || (ai == aj && i < j)) rank++;
                }
                if (rank < n) {
                    int64_t col = g0 + j;
                    mask[r * (k / 8) + col / 8] |= (uint8_t)(1u << (col % 8));
                }
            }
        }
    }
}

static int mask_bit(const uint8_t *mask, int64_t k, int64_t r, int64_t c)
{
    return (mask[r * (k / 8) + c / 8] >> (c % 8)) & 1;
}

/* ------------------------------------------------------------------ */
/* Step 2: absmean scale gamma.                                        */
/* [2B4T] §一: weights map to {-1,0,+1} by absolute-mean quantisation.  */
/* [SB] §六: quantise first, then sparsify -- so the mean runs over the */
/* dense latent tensor (over_masked = 0).  over_masked = 1 is the       */
/* sparsify-first ablation: the sum runs over kept entries only, the    */
/* divisor stays n_out*k.                                              */
/* Reading: the mean is the exact sum of |W| rounded once to binary64   */
/* (round to nearest, ties to even), then divided by the count in       */
/* binary64.  This is order independent.                                */
/*                                                                     */
/* Exact sum: every finite bf16 magnitude is an integer multiple of     */
/* 2^-133 (the smallest subnormal), at most 255 * 2^253 of those units. */
/* The sum is kept as a 320-bit unsigned integer in 32-bit limbs.      */
/* ------------------------------------------------------------------ */
#define BIG_LIMBS 10

typedef struct { uint64_t limb[BIG_LIMBS]; } big_t; /* each limb < 2^32 */

static void big_add_shifted(big_t *b, uint32_t v, int shift)
{
    /* b += v * 2^shift, v < 2^8 */
    uint64_t carry = 0;
    int li = shift / 32, bo = shift % 32;
    uint64_t add = (uint64_t)v << bo; /* < 2^40 */
    for (int i = li; i < BIG_LIMBS; ++i) {
        uint64_t part = (i == li) ? (add & 0xffffffffu) : (i == li + 1 ? (add >> 32) : 0);
        uint64_t s = b->limb[i] + part + carry;
        b->limb[i] = s & 0xffffffffu;
        carry = s >> 32;
        if (i > li + 1 && carry == 0) break;
    }
}

static int big_bit(const big_t *b, int pos)
{
    return (int)((b->limb[pos / 32] >> (pos % 32)) & 1u);
}

/* Round the big integer (in units of 2^-133) to the nearest binary64,
 * ties to even. */
static double big_to_double(const big_t *b)
{
    int top = -1;
    for (int pos = BIG_LIMBS * 32 - 1; pos >= 0; --pos)
        if (big_bit(b, pos)) { top = pos; break; }
    if (top < 0) return 0.0;
    if (top <= 52) {
        uint64_t v = 0;
        for (int pos = top; pos >= 0; --pos) v = (v << 1) | (uint64_t)big_bit(b, pos);
        return ldexp((double)v, -133);
    }
    int low = top - 52; /* lowest bit kept in the 53-bit significand */
    uint64_t sig = 0;
    for (int pos = top; pos >= low; --pos) sig = (sig << 1) | (uint64_t)big_bit(b, pos);
    int half = big_bit(b, low - 1);
    int sticky = 0;
    for (int pos = low - 2; pos >= 0; --pos)
        if (big_bit(b, pos)) { sticky = 1; break; }
    if (half && (sticky || (sig & 1u))) sig += 1; /* may reach 2^53: still exact */
    return ldexp((double)sig, low - 133);
}

/* Exact value of |h| in units of 2^-133: (significand, shift). */
static void bf16_abs_units(uint16_t h, uint32_t *sig, int *shift)
{
    uint32_t e = (h >> 7) & 0xffu, f = h & 0x7fu;
    if (e == 0) { *sig = f; *shift = 0; }           /* subnormal: f * 2^-133 */
    else        { *sig = 0x80u | f; *shift = (int)e - 1; }
}

double oracle_gamma(const uint16_t *W, int64_t n_out, int64_t k,
                    int over_masked, const uint8_t *mask)
{
    big_t sum;
    memset(&sum, 0, sizeof sum);
    for (int64_t r = 0; r < n_out; ++r)
        for (int64_t c = 0; c < k; ++c) {
            if (over_masked && !mask_bit(mask, k, r, c)) continue;
            uint32_t sig; int shift;
            bf16_abs_units(W[r * k + c], &sig, &shift);
            if (sig) big_add_shifted(&sum, sig, shift);
        }
    double s = big_to_double(&sum);
    return s / (double)(n_out * k);
}

/* ------------------------------------------------------------------ */
/* Step 3: masked ternary codes.                                       */
/* [2B4T] §一: ternary {-1,0,+1}; [SB] §六: quantise then sparsify,     */
/* the mask decides which codes survive.                               */
/* Definition: Wq = clip(round_half_even(W / gamma), -1, 1), then zero  */
/* where the mask is 0.  For the exact quotient q = |W|/gamma:          */
/* round_half_even(q) is 0 for q <= 1/2 (q = 1/2 rounds to even 0) and  */
/* >= 1 otherwise, so after the clip the code is sign(W) exactly when   */
/* q > 1/2, i.e. when 2|W| > gamma.  2|W| is exact in binary64, so the  */
/* comparison below is the exact-quotient definition.  gamma == 0 (an   */
/* all-zero tensor) gives all zeros (reading: no epsilon is added).     */
/* ------------------------------------------------------------------ */
void oracle_ternary(const uint16_t *W, const uint8_t *mask, double gamma,
                    int64_t n_out, int64_t k, int8_t *T)
{
    for (int64_t r = 0; r < n_out; ++r)
        for (int64_t c = 0; c < k; ++c) {
            double w = bf16_value(W[r * k + c]);
            int8_t code = 0;
            if (mask_bit(mask, k, r, c) && gamma > 0.0 && 2.0 * fabs(w) > gamma)
                code = (w < 0.0) ? -1 : 1;
            T[r * k + c] = code;
        }
}

/* ------------------------------------------------------------------ */
/* Step 4: per-token absmax int8 activations.                          */
/* [2B4T] §一 and §四: activations are 8-bit integers (W1.58A8).        */
/* Reading: one scale per token, a_t = max_k |x[t,k]|;                  */
/* x_q = clip(round_half_even(127 * x / a_t), -128, 127), s_t = a_t/127. */
/* a_t == 0 gives x_q = 0 and s_t = 0 (no epsilon).                     */
/* 127*x and a_t are exact in binary64.  Both have 8-bit significands,  */
/* so a quotient that is not itself a half-integer lies at least about  */
/* 2^-16 (relative) away from every half-integer; the correctly rounded */
/* binary64 quotient (error 2^-53) therefore rounds like the exact one, */
/* and nearbyint (ties to even, the default mode) gives the exact RHE.  */
/* ------------------------------------------------------------------ */
void oracle_act_quant(const uint16_t *X, int64_t tokens, int64_t k,
                      int8_t *xq, double *scale)
{
    for (int64_t t = 0; t < tokens; ++t) {
        double a = 0.0;
        for (int64_t c = 0; c < k; ++c) {
            double v = fabs(bf16_value(X[t * k + c]));
            if (v > a) a = v;
        }
        scale[t] = a / 127.0;
        for (int64_t c = 0; c < k; ++c) {
            double q = 0.0;
            if (a > 0.0) q = nearbyint(127.0 * bf16_value(X[t * k + c]) / a);
            if (q > 127.0) q = 127.0;
            if (q < -128.0) q = -128.0;
            xq[t * k + c] = (int8_t)q;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Step 5 and 6: contraction and epilogue.                             */
/* [2B4T] §四: ternary weights times int8 activations.                  */
/* acc[t,n] = sum_k x_q[t,k] * T[n,k]   (exact, int64, checked to fit   */
/* int32);  Y[t,n] = acc[t,n] * gamma * a_t / 127   (binary64).         */
/* No bias term ([2B4T] §一: all biases removed).                       */
/* ------------------------------------------------------------------ */
typedef struct {
    const int8_t *xq; const double *scale; const int8_t *T; double gamma;
    int64_t tokens, k, n_out;
    int32_t *acc; double *Y;
    int64_t row0, row1; int overflow;
} fwd_job;

static void *fwd_worker(void *p)
{
    fwd_job *j = (fwd_job *)p;
    for (int64_t t = j->row0; t < j->row1; ++t)
        for (int64_t r = 0; r < j->n_out; ++r) {
            int64_t s = 0;
            for (int64_t c = 0; c < j->k; ++c)
                s += (int64_t)j->xq[t * j->k + c] * (int64_t)j->T[r * j->k + c];
            if (s > INT32_MAX || s < INT32_MIN) j->overflow = 1;
            if (j->acc) j->acc[t * j->n_out + r] = (int32_t)s;
            if (j->Y) j->Y[t * j->n_out + r] = (double)s * j->gamma * j->scale[t];
        }
    return NULL;
}

/* Runs over token rows with `threads` POSIX threads (1 = serial).
 * Returns 0, or 1 if some accumulator left the int32 range. */
int oracle_fwd(const int8_t *xq, const double *scale, const int8_t *T,
               double gamma, int64_t tokens, int64_t k, int64_t n_out,
               int32_t *acc, double *Y, int threads)
{
    if (threads < 1) threads = 1;
    if (threads > tokens) threads = (int)(tokens > 0 ? tokens : 1);
    fwd_job *jobs = calloc((size_t)threads, sizeof *jobs);
    pthread_t *tid = calloc((size_t)threads, sizeof *tid);
    int overflow = 0;
    for (int i = 0; i < threads; ++i) {
        jobs[i] = (fwd_job){xq, scale, T, gamma, tokens, k, n_out, acc, Y,
                            tokens * i / threads, tokens * (i + 1) / threads, 0};
        if (threads == 1) fwd_worker(&jobs[i]);
        else pthread_create(&tid[i], NULL, fwd_worker, &jobs[i]);
    }
    for (int i = 0; i < threads; ++i) {
        if (threads > 1) pthread_join(tid[i], NULL);
        overflow |= jobs[i].overflow;
    }
    free(jobs); free(tid);
    return overflow;
}

/* Selected outputs only: for each (t, n) pair, the same sum and scaling. */
void oracle_fwd_pairs(const int8_t *xq, const double *scale, const int8_t *T,
                      double gamma, int64_t k, const int64_t *t_idx,
                      const int64_t *n_idx, int64_t count, int64_t *acc,
                      double *Y)
{
    for (int64_t i = 0; i < count; ++i) {
        int64_t t = t_idx[i], r = n_idx[i], s = 0;
        for (int64_t c = 0; c < k; ++c)
            s += (int64_t)xq[t * k + c] * (int64_t)T[r * k + c];
        acc[i] = s;
        Y[i] = (double)s * gamma * scale[t];
    }
}

/* ------------------------------------------------------------------ */
/* Step 7 and 8: dual straight-through backward.                       */
/* [SB] §三 and §六: gradients pass straight through both the ternary   */
/* rounding and the sparsification; a masked weight still receives its */
/* gradient, so dW is dense.                                           */
/* Readings: the forward used is Y = (x_q s) (T gamma)^T; the input     */
/* gradient flows through the masked ternary weights (T gamma); the     */
/* activation quantiser passes gradients unchanged; gamma and s_t are   */
/* treated as constants; dW uses the dequantised activation x_q s_t.    */
/*   dX[t,k] = gamma * sum_n dY[t,n] T[n,k]                             */
/*   dW[n,k] = sum_t dY[t,n] * s_t * x_q[t,k]                           */
/* ------------------------------------------------------------------ */
typedef struct {
    const uint16_t *dY; const int8_t *xq; const double *scale; const int8_t *T;
    double gamma; int64_t tokens, k, n_out; double *dX; double *dW;
    int64_t lo, hi;
} bwd_job;

static void *dx_worker(void *p)
{
    bwd_job *j = (bwd_job *)p;
    for (int64_t t = j->lo; t < j->hi; ++t)
        for (int64_t c = 0; c < j->k; ++c) {
            double s = 0.0;
            for (int64_t r = 0; r < j->n_out; ++r)
                s += bf16_value(j->dY[t * j->n_out + r]) * (double)j->T[r * j->k + c];
            j->dX[t * j->k + c] = j->gamma * s;
        }
    return NULL;
}

static void *dw_worker(void *p)
{
    bwd_job *j = (bwd_job *)p;
    for (int64_t r = j->lo; r < j->hi; ++r)
        for (int64_t c = 0; c < j->k; ++c) {
            double s = 0.0;
            for (int64_t t = 0; t < j->tokens; ++t)
                s += bf16_value(j->dY[t * j->n_out + r]) * j->scale[t] *
                     (double)j->xq[t * j->k + c];
            j->dW[r * j->k + c] = s;
        }
    return NULL;
}

static void run_bwd(void *(*fn)(void *), bwd_job base, int64_t rows, int threads)
{
    if (threads < 1) threads = 1;
    if (threads > rows) threads = (int)(rows > 0 ? rows : 1);
    bwd_job *jobs = calloc((size_t)threads, sizeof *jobs);
    pthread_t *tid = calloc((size_t)threads, sizeof *tid);
    for (int i = 0; i < threads; ++i) {
        jobs[i] = base;
        jobs[i].lo = rows * i / threads;
        jobs[i].hi = rows * (i + 1) / threads;
        if (threads == 1) fn(&jobs[i]);
        else pthread_create(&tid[i], NULL, fn, &jobs[i]);
    }
    if (threads > 1)
        for (int i = 0; i < threads; ++i) pthread_join(tid[i], NULL);
    free(jobs); free(tid);
}

void oracle_bwd_dx(const uint16_t *dY, const int8_t *T, double gamma,
                   int64_t tokens, int64_t k, int64_t n_out, double *dX,
                   int threads)
{
    bwd_job b = {dY, NULL, NULL, T, gamma, tokens, k, n_out, dX, NULL, 0, 0};
    run_bwd(dx_worker, b, tokens, threads);
}

void oracle_bwd_dw(const uint16_t *dY, const int8_t *xq, const double *scale,
                   int64_t tokens, int64_t k, int64_t n_out, double *dW,
                   int threads)
{
    bwd_job b = {dY, xq, scale, NULL, 0.0, tokens, k, n_out, NULL, dW, 0, 0};
    run_bwd(dw_worker, b, n_out, threads);
}

/* Selected entries: dX at (t, c) pairs and dW at (r, c) pairs. */
void oracle_bwd_dx_pairs(const uint16_t *dY, const int8_t *T, double gamma,
                         int64_t k, int64_t n_out, const int64_t *t_idx,
                         const int64_t *c_idx, int64_t count, double *out)
{
    for (int64_t i = 0; i < count; ++i) {
        double s = 0.0;
        for (int64_t r = 0; r < n_out; ++r)
            s += bf16_value(dY[t_idx[i] * n_out + r]) * (double)T[r * k + c_idx[i]];
        out[i] = gamma * s;
    }
}

void oracle_bwd_dw_pairs(const uint16_t *dY, const int8_t *xq,
                         const double *scale, int64_t tokens, int64_t k,
                         int64_t n_out, const int64_t *r_idx,
                         const int64_t *c_idx, int64_t count, double *out)
{
    for (int64_t i = 0; i < count; ++i) {
        double s = 0.0;
        for (int64_t t = 0; t < tokens; ++t)
            s += bf16_value(dY[t * n_out + r_idx[i]]) * scale[t] *
                 (double)xq[t * k + c_idx[i]];
        out[i] = s;
    }
}

/* ------------------------------------------------------------------ */
/* Packed storage of the masked ternary codes ("code plus index").     */
/* [2B4T] §四 stores 4 ternary values per int8 (2 bits per weight);     */
/* the Sparse-BitNet operator ([SB] §四, [SBabs]) is not described.     */
/* This format is this project's own; it is defined here in full so    */
/* that the oracle produces the exact bytes independently:              */
/*                                                                     */
/*  S = the largest number of nonzeros an 8-group can hold: 8 for 8:8,  */
/*      6 for 6:8, 4 for 4:8 and 2:4.                                   */
/*  Group field (8+S bits) for the 8 codes t_0..t_7 of one row at k =   */
/*  8g..8g+7:                                                          */
/*     bits [0,4)      nonzero bitmap of t_0..t_3                       */
/*     bits [4,4+S)    sign bits (1 = negative): the i-th nonzero among */
/*                     t_0..t_3 (in increasing position) at bit 4+i;    */
/*                     the i-th nonzero among t_4..t_7 at bit 4+S-1-i;  */
/*                     every other sign bit is 0                        */
/*     bits [4+S,8+S)  nonzero bitmap of t_4..t_7                       */
/*  Chunk: 16 group fields, field f at bit offset f*(8+S) of a          */
/*     little-endian bit string of 2*(8+S) bytes (byte j holds string   */
/*     bits 8j..8j+7, LSB first).                                       */
/*  Order: rows in strips of 64 (the last strip padded with zero rows). */
/*     Superblock (strip p, k-block kb) = 64 chunks, at index           */
/*     p * (k/128) + kb; the buffer is the superblocks in order.        */
/*     Chunk c = r + 16q (r in 0..15, q in 0..3) of a superblock holds, */
/*     as field f = 4i + 2h + e (i in 0..3, h and e in 0..1), the group */
/*     of row 64p + 16i + r at k = kb*128 + 8*(8h + 2q + e) ... +7.     */
/*     (Every (row, group) of the superblock appears exactly once.)     */
/* ------------------------------------------------------------------ */
int oracle_s_of(int n, int m)
{
    if (m == 8 && n == 8) return 8;
    if (m == 8 && n == 6) return 6;
    if (m == 8 && n == 4) return 4;
    if (m == 4 && n == 2) return 4;
    if (m == 8 && n == 3) return 4;
    if (m == 8 && n == 2) return 2;
    return -1;
}

int64_t oracle_packed_bytes(int64_t n_out, int64_t k, int s)
{
    int64_t strips = (n_out + 63) / 64;
    return strips * 64 * (k / 128) * 2 * (8 + s);
}

/* byte offset of the chunk, and bit offset within it, of the field that
 * holds group g (0..15) of row r in k-block kb */
static void field_place(int64_t r, int64_t kb, int g, int64_t nkb, int s, int64_t *chunk_byte,
                        int64_t *bit)
{
    int64_t strip = r / 64;
    int rr = (int)(r % 64);
    int i = rr / 16, r16 = rr % 16;
    int h = g / 8, q = (g % 8) / 2, e = g % 2;
    int64_t chunk = (strip * nkb + kb) * 64 + r16 + 16 * q;
    *chunk_byte = chunk * 2 * (8 + s);
    *bit = (int64_t)(4 * i + 2 * h + e) * (8 + s);
}

static void put_bits(uint8_t *blk, int64_t bitpos, uint32_t value, int width)
{
    for (int b = 0; b < width; ++b)
        if ((value >> b) & 1u) blk[(bitpos + b) / 8] |= (uint8_t)(1u << ((bitpos + b) % 8));
}

static uint32_t get_bits(const uint8_t *blk, int64_t bitpos, int width)
{
    uint32_t v = 0;
    for (int b = 0; b < width; ++b)
        v |= (uint32_t)((blk[(bitpos + b) / 8] >> ((bitpos + b) % 8)) & 1u) << b;
    return v;
}

/* Returns 0, or -1 if some group holds more nonzeros than S allows or a
 * half holds more than 4 (impossible for codes in {-1,0,1}). */
int oracle_pack(const int8_t *T, int64_t n_out, int64_t k, int s, uint8_t *packed)
{
    int64_t nkb = k / 128;
    memset(packed, 0, (size_t)oracle_packed_bytes(n_out, k, s));
    for (int64_t r = 0; r < n_out; ++r)
        for (int64_t kb = 0; kb < nkb; ++kb) {
            for (int g = 0; g < 16; ++g) {
                int64_t cb, base;
                field_place(r, kb, g, nkb, s, &cb, &base);
                uint8_t *blk = packed + cb;
                const int8_t *t = T + r * k + kb * 128 + g * 8;
                uint32_t blo = 0, bhi = 0, sign = 0;
                int nlo = 0, nhi = 0;
                for (int p = 0; p < 4; ++p)
                    if (t[p] != 0) {
                        blo |= 1u << p;
                        if (t[p] < 0) sign |= 1u << nlo;
                        nlo++;
                    }
                for (int p = 0; p < 4; ++p)
                    if (t[4 + p] != 0) {
                        bhi |= 1u << p;
                        if (t[4 + p] < 0) sign |= 1u << (s - 1 - nhi);
                        nhi++;
                    }
                if (nlo + nhi > s) return -1;
                put_bits(blk, base, blo, 4);
                put_bits(blk, base + 4, sign, s);
                put_bits(blk, base + 4 + s, bhi, 4);
            }
        }
    return 0;
}

void oracle_unpack(const uint8_t *packed, int64_t n_out, int64_t k, int s, int8_t *T)
{
    int64_t nkb = k / 128;
    for (int64_t r = 0; r < n_out; ++r)
        for (int64_t kb = 0; kb < nkb; ++kb) {
            for (int g = 0; g < 16; ++g) {
                int64_t cb, base;
                field_place(r, kb, g, nkb, s, &cb, &base);
                const uint8_t *blk = packed + cb;
                uint32_t blo = get_bits(blk, base, 4);
                uint32_t sign = get_bits(blk, base + 4, s);
                uint32_t bhi = get_bits(blk, base + 4 + s, 4);
                int8_t *t = T + r * k + kb * 128 + g * 8;
                int nlo = 0, nhi = 0;
                for (int p = 0; p < 4; ++p) {
                    t[p] = 0;
                    if ((blo >> p) & 1u) { t[p] = ((sign >> nlo) & 1u) ? -1 : 1; nlo++; }
                }
                for (int p = 0; p < 4; ++p) {
                    t[4 + p] = 0;
                    if ((bhi >> p) & 1u) { t[4 + p] = ((sign >> (s - 1 - nhi)) & 1u) ? -1 : 1; nhi++; }
                }
            }
        }
}

/* ------------------------------------------------------------------ */
/* 2:4 codes as "sparse operand + index" (this project's second packed */
/* format, for matrix instructions that take a 2:4-sparse operand:     */
/* the structured-sparsity hardware [SB] 七 describes, here gfx950's   */
/* sparse int8 matrix multiply).  Under a 2:4 mask every quad (4       */
/* consecutive k) holds at most two nonzero codes; each quad is stored */
/* as two (position, value) slots:                                     */
/*   2 nonzeros at positions a < b:  slots (a, T[a]), (b, T[b]);       */
/*   1 nonzero at position a:        a = 0: (0, T[0]), (1, 0);         */
/*                                   a > 0: (0, 0), (a, T[a]);         */
/*   no nonzero:                     (0, 0), (1, 0).                   */
/* (positions ascending and distinct in every case).                   */
/* Layout: rows in strips of 64 (the last padded with zero codes), k   */
/* in blocks of 128; superblock (strip p, block kb) at index           */
/* p*(k/128) + kb, 64 chunks of 32 bytes.  Chunk c = r + 16q holds rows */
/* 64p + 16i + r (i = 0..3) over k = 128kb + 32q ... +31: element      */
/* e = 2u + s (quad u = 0..7 at k = 128kb + 32q + 4u, slot s) of row   */
/* tile i sits in                                                      */
/*   word 2i   (index word):  bits 2e, 2e+1 = the slot's position;     */
/*   word 2i+1 (value word):  bits 8(e%4) + 2(e/4), +1 = its code,     */
/*                            0 for 0, 1 for +1, 3 for -1;             */
/* words little-endian, word w at byte 4w of the chunk.                 */
/* ------------------------------------------------------------------ */
int64_t oracle_sp24_packed_bytes(int64_t n_out, int64_t k)
{
    return (n_out + 63) / 64 * 64 * (k / 128) * 32;
}

static uint8_t *sp24_chunk(uint8_t *packed, int64_t row, int64_t kb, int q, int64_t nkb, int *i)
{
    int64_t strip = row / 64;
    int rr = (int)(row % 64);
    *i = rr / 16;
    return packed + ((strip * nkb + kb) * 64 + rr % 16 + 16 * q) * 32;
}

static void put_word(uint8_t *p, uint32_t w)
{
    for (int b = 0; b < 4; ++b) p[b] = (uint8_t)(w >> (8 * b));
}

static uint32_t get_word(const uint8_t *p)
{
    return (uint32_t)p[0] | (uint32_t)p[1] << 8 | (uint32_t)p[2] << 16 | (uint32_t)p[3] << 24;
}

/* Returns 0, or -1 if a quad holds more than two nonzero codes. */
int oracle_pack_sp24(const int8_t *T, int64_t n_out, int64_t k, uint8_t *packed)
{
    int64_t nkb = k / 128, rows = (n_out + 63) / 64 * 64;
    static const int8_t zero_quad[4] = {0, 0, 0, 0};
    memset(packed, 0, (size_t)oracle_sp24_packed_bytes(n_out, k));
    for (int64_t r = 0; r < rows; ++r)  /* rows past n_out: zero codes */
        for (int64_t kb = 0; kb < nkb; ++kb)
            for (int q = 0; q < 4; ++q) {
                int i;
                uint8_t *ch = sp24_chunk(packed, r, kb, q, nkb, &i);
                uint32_t idx = 0, val = 0;
                for (int u = 0; u < 8; ++u) {
                    const int8_t *t = r < n_out ? T + r * k + kb * 128 + 32 * q + 4 * u : zero_quad;
                    int pos[2], n = 0;
                    for (int a = 0; a < 4; ++a)
                        if (t[a] != 0) {
                            if (n == 2) return -1;
                            pos[n++] = a;
                        }
                    if (n == 0) { pos[0] = 0; pos[1] = 1; }
                    if (n == 1) {
                        if (pos[0] == 0) pos[1] = 1;
                        else { pos[1] = pos[0]; pos[0] = 0; }
                    }
                    for (int sl = 0; sl < 2; ++sl) {
                        int e = 2 * u + sl;
                        int8_t v = t[pos[sl]];
                        uint32_t code = v == 0 ? 0u : (v > 0 ? 1u : 3u);
                        idx |= (uint32_t)pos[sl] << (2 * e);
                        val |= code << (8 * (e % 4) + 2 * (e / 4));
                    }
                }
                put_word(ch + 8 * i, idx);
                put_word(ch + 8 * i + 4, val);
            }
    return 0;
}

/* The codes the format represents: every slot adds its value at its
 * position (so a slot holding 0 contributes nothing), as the sparse
 * matrix instruction multiplies and adds every stored element. */
void oracle_unpack_sp24(const uint8_t *packed, int64_t n_out, int64_t k, int8_t *T)
{
    int64_t nkb = k / 128;
    uint8_t *pk = (uint8_t *)packed;
    for (int64_t r = 0; r < n_out; ++r)
        for (int64_t kb = 0; kb < nkb; ++kb)
            for (int q = 0; q < 4; ++q) {
                int i;
                const uint8_t *ch = sp24_chunk(pk, r, kb, q, nkb, &i);
                uint32_t idx = get_word(ch + 8 * i), val = get_word(ch + 8 * i + 4);
                int8_t *t = T + r * k + kb * 128 + 32 * q;
                for (int a = 0; a < 32; ++a) t[a] = 0;
                for (int e = 0; e < 16; ++e) {
                    int pos = (int)((idx >> (2 * e)) & 3u);
                    uint32_t code = (val >> (8 * (e % 4) + 2 * (e / 4))) & 3u;
                    int v = code == 1u ? 1 : code == 3u ? -1 : 0;
                    t[4 * (e / 2) + pos] = (int8_t)(t[4 * (e / 2) + pos] + v);
                }
            }
}

/* ------------------------------------------------------------------ */
/* Latent-weight update ([SB] 三, 六: the latent full-precision weights */
/* take the dense gradient that both straight-through estimators pass; */
/* the next step re-derives mask, gamma and codes from them).  The     */
/* pages name no optimiser; the reading taken is the plain gradient    */
/* step, with the latent weights held in binary32:                     */
/*   w' = the binary32 nearest to the exact w - lr*g (ties to even),   */
/*        which is what C's fmaf returns (one rounding);               */
/*   W  = the bf16 nearest to w' (ties to even), found by comparing    */
/*        the two bf16 neighbours of w' in exact binary64.             */
/* ------------------------------------------------------------------ */
static uint16_t nearest_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint32_t lo = u & 0xffff0000u;          /* same sign, magnitude rounded down */
    uint32_t hi = lo + 0x00010000u;         /* next magnitude up                  */
    float flo, fhi;
    memcpy(&flo, &lo, 4);
    memcpy(&fhi, &hi, 4);
    double dlo = fabs((double)x - (double)flo);
    double dhi = fabs((double)fhi - (double)x);
    if (dlo < dhi) return (uint16_t)(lo >> 16);
    if (dhi < dlo) return (uint16_t)(hi >> 16);
    return (uint16_t)((((lo >> 16) & 1u) == 0) ? (lo >> 16) : (hi >> 16));
}

void oracle_latent_update(float *w_master, const float *dw, int64_t count, float lr,
                          uint16_t *w)
{
    for (int64_t i = 0; i < count; ++i) {
        w_master[i] = fmaf(-lr, dw[i], w_master[i]);
        w[i] = nearest_bf16(w_master[i]);
    }
}

/* ------------------------------------------------------------------ */
/* Squared-ReLU gating of the feed-forward ([2B4T] 一: squared ReLU in  */
/* place of SwiGLU).  The reading taken: gated like the SwiGLU it      */
/* replaces, h = relu(g)^2 * u, with g and u the gate and up           */
/* BitLinears' fp32 outputs; each product rounded to binary32 in the   */
/* order written, then h rounded to bf16 (the down BitLinear's input,  */
/* quantised per token like any bf16 activation).  The backward is the */
/* derivative of that product (relu'(0) = 0), each product rounded to  */
/* binary32, the results rounded to bf16 (the gate and up BitLinears'  */
/* dY).                                                                */
/* ------------------------------------------------------------------ */
void oracle_relu2_gate(const float *G, const float *U, int64_t count, uint16_t *H)
{
    for (int64_t i = 0; i < count; ++i) {
        float r = G[i] > 0.0f ? G[i] : 0.0f;
        float r2 = r * r;
        float h = r2 * U[i];
        H[i] = nearest_bf16(h);
    }
}

void oracle_relu2_gate_bwd(const float *dH, const float *G, const float *U, int64_t count,
                           uint16_t *dG, uint16_t *dU)
{
    for (int64_t i = 0; i < count; ++i) {
        float r = G[i] > 0.0f ? G[i] : 0.0f;
        float r2 = r * r;
        float du = dH[i] * r2;            /* dL/du = dh * r^2          */
        float dhu = dH[i] * U[i];
        float dg = dhu * (2.0f * r);      /* dL/dg = dh * u * 2r       */
        dU[i] = nearest_bf16(du);
        dG[i] = nearest_bf16(dg);
    }
}

/* ------------------------------------------------------------------ */
/* Step 6 with bf16 outputs: the optional bf16 Y epilogue of the block */
/* glue ([2B4T] 二: the model around the BitLinears runs in bf16).     */
/* No page fixes how a bf16 Y is rounded; the reading taken is the     */
/* binary32 Y of the epilogue, rounded once more:                      */
/*   s32 = the binary32 nearest to a_t / 127 (s_t as stored),          */
/*   g32 = the binary32 nearest to gamma * s32 (binary64 product),     */
/*   Y32 = the binary32 nearest to f(acc) * g32, where f(acc) is the   */
/*         binary32 nearest to acc,                                    */
/*   Y16 = the bf16 nearest to Y32 (ties to even).                     */
/* Returns 0, or 1 if some accumulator left the int32 range.           */
/* ------------------------------------------------------------------ */
int oracle_fwd_bf16(const int8_t *xq, const double *scale, const int8_t *T, double gamma,
                    int64_t tokens, int64_t k, int64_t n_out, uint16_t *Y)
{
    int overflow = 0;
    for (int64_t t = 0; t < tokens; ++t) {
        float s32 = (float)scale[t];
        float g32 = (float)(gamma * (double)s32);
        for (int64_t r = 0; r < n_out; ++r) {
            int64_t s = 0;
            for (int64_t c = 0; c < k; ++c)
                s += (int64_t)xq[t * k + c] * (int64_t)T[r * k + c];
            if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
            float a32 = (float)(int32_t)s;
            float y32 = a32 * g32;
            Y[t * n_out + r] = nearest_bf16(y32);
        }
    }
    return overflow;
}
