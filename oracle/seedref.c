/*
 * seedref.c -- plain, slow, obviously correct CPU oracle for SeedLM seed decoding.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and the
 * benchmark's CPU-baseline leg.  The GPU library never links or calls it.
 *
 * Citations name the page and the section each step follows:
 *   [README]  NanoSeedLM repository README, sections "Highlights" and "How it works".
 *   [P4CARD]  model card "Qwen3.8-Flash-Next-NanoSeedLM-P4", sections "How it works",
 *             "Files" and "The family".
 *   [K2CARD]  model card "K2-Horizon-MoVA-36B-A4B - NanoSeedLM p4mx-q4v", section "This upload".
 *   [BLOG]    barnson.org post on NanoSeedLM, sections "Where this started",
 *             "What I changed: September 2026", "LFSR is free", "Four bits is four bits",
 *             "GPU search == CPU search".
 *   [INDEX]   NanoSeedLM documentation index page, sections "Results" and "Plans".
 *
 * Parity unpinned: the register's tap mask and the basis fill order are readings; the
 * pages print no seed -> weights example to check them against.
 *
 * Build: cc -O2 -std=c99 -ffp-contract=off -fopenmp -shared -fPIC seedref.c -lm
 */
#include "seedref.h"
#include <math.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* [BLOG "LFSR is free"], [README "How it works"]: a 16-bit linear feedback shift
 * register.  Reading: Fibonacci form shifting left; the bit shifted in is the XOR of
 * state bits 15, 13, 12 and 10 (mask 0xB400, x^16 + x^14 + x^13 + x^11 + 1), which
 * gives the single 65,535-state cycle the pages' "all 65,535 seeds" requires. */
uint16_t seedref_lfsr_step(uint16_t s)
{
    unsigned taps = (unsigned)s & 0xB400u;
    unsigned bit = 0;
    while (taps) {              /* parity of the tapped bits, one bit at a time */
        bit ^= taps & 1u;
        taps >>= 1;
    }
    return (uint16_t)((((unsigned)s << 1) | bit) & 0xFFFFu);
}

/* [BLOG "What I changed"]: the seed is the initial register state.  The basis uses the
 * states after steps 1..n (the seed itself is not a basis value). */
void seedref_states(uint16_t seed, int n, uint16_t *out)
{
    uint16_t s = seed;
    for (int t = 0; t < n; ++t) {
        s = seedref_lfsr_step(s);
        out[t] = s;
    }
}

/* [K2CARD "This upload"]: coefficients live in NAME.coefs (U16); [BLOG "LFSR is free"]:
 * a nibble q sign-extends as (q ^ 8) - 8.  Reading: one flat nibble stream, P nibbles
 * per block, nibble n at word n >> 2, bits 4*(n & 3). */
int seedref_coef(const uint16_t *coefs, int64_t b, int P, int j)
{
    int64_t n = b * P + j;
    unsigned q = ((unsigned)coefs[n >> 2] >> (4 * (n & 3))) & 0xFu;
    return (int)(q ^ 8u) - 8;
}

/* [P4CARD "How it works"]: a 4-bit exponent code per block; [K2CARD "This upload"]:
 * NAME.codes (U8).  Reading: two codes per byte, even block in the low nibble (the
 * 4.5 bits/weight total of [P4CARD "The family"] leaves room for no more). */
int seedref_code(const uint8_t *codes, int64_t b)
{
    return ((unsigned)codes[b >> 1] >> (4 * (b & 1))) & 0xFu;
}

/* [BLOG "Where this started"]: the block is "this random basis, times these
 * coefficients" scaled by a shared exponent; [BLOG "Attempt one"]: the power of two
 * multiplies.  Basis value = state - 32768; the 2^-15 that maps it into [-1, 1) is
 * folded into the exponent.  The integer sum is exact (|sum| <= 4*8*32768 = 2^20), so the
 * fp32 weight is exact. */
void seedref_block(uint16_t seed, const int *c, int P, int code, int exp_bias, float *w8)
{
    uint16_t st[32];
    seedref_states(seed, 8 * P, st);
    for (int i = 0; i < 8; ++i) {
        long acc = 0;
        for (int j = 0; j < P; ++j)
            acc += (long)c[j] * ((long)st[i * P + j] - 32768L);   /* row-major basis */
        w8[i] = ldexpf((float)acc, code + exp_bias - 15);
    }
}

/* [BLOG "Four bits is four bits"], [P4CARD "The family"]: (16 + 4P + 4) bits per 8 weights. */
int seedref_stream_bytes(int64_t M, int64_t K, int P, int64_t *seed_bytes,
                         int64_t *coef_bytes, int64_t *code_bytes)
{
    if (M < 0 || K < 0 || K % 8 != 0 || (P != 3 && P != 4))
        return -1;
    int64_t nblk = M * (K / 8);
    *seed_bytes = 2 * nblk;
    *coef_bytes = 2 * ((nblk * P + 3) / 4);
    *code_bytes = (nblk + 1) / 2;
    return 0;
}

static int bad_args(int M, int K, int P)
{
    return M < 0 || K < 0 || K % 8 != 0 || (P != 3 && P != 4);
}

/* Keep every weight a normal fp32 (and bf16): |sum| <= 2^20 and the scale is
 * 2^(code + exp_bias - 15) with code in 0..15, so exp_bias in [-100, 100] is safe. */
static int exponent_in_range(int32_t exp_bias)
{
    return exp_bias >= -100 && exp_bias <= 100;
}

/* Decode one row of an [M][K] matrix into w (K floats). */
static void decode_row(const uint16_t *seeds, const uint16_t *coefs, const uint8_t *codes,
                       int32_t exp_bias, int m, int K, int P, float *w)
{
    int64_t bpr = K / 8;
    for (int64_t kb = 0; kb < bpr; ++kb) {
        int64_t b = (int64_t)m * bpr + kb;
        int c[4];
        for (int j = 0; j < P; ++j)
            c[j] = seedref_coef(coefs, b, P, j);
        seedref_block(seeds[b], c, P, seedref_code(codes, b), exp_bias, w + 8 * kb);
    }
}

int seedref_reconstruct_f32(const uint16_t *seeds, const uint16_t *coefs, const uint8_t *codes,
                            int32_t exp_bias, int M, int K, int P, float *W)
{
    if (bad_args(M, K, P) || !exponent_in_range(exp_bias))
        return -1;
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        decode_row(seeds, coefs, codes, exp_bias, m, K, P, W + (int64_t)m * K);
    return 0;
}

/* Round to nearest, ties to even, of a finite fp32 to bf16 (the top 16 bits). */
uint16_t seedref_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u)          /* inf / nan: keep, quiet nan */
        return (uint16_t)((u >> 16) | ((u & 0x007FFFFFu) ? 0x40u : 0u));
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

int seedref_reconstruct_bf16(const uint16_t *seeds, const uint16_t *coefs, const uint8_t *codes,
                             int32_t exp_bias, int M, int K, int P, uint16_t *W)
{
    if (bad_args(M, K, P) || !exponent_in_range(exp_bias))
        return -1;
#pragma omp parallel
    {
        float *row = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(static)
        for (int m = 0; m < M; ++m) {
            decode_row(seeds, coefs, codes, exp_bias, m, K, P, row);
            for (int k = 0; k < K; ++k)
                W[(int64_t)m * K + k] = seedref_f32_to_bf16(row[k]);
        }
        free(row);
    }
    return 0;
}

/* The product itself: the weights never exist outside this loop [README "Highlights"],
 * so the oracle decodes each row and takes the plain dot product in double. */
int seedref_gemv(const uint16_t *seeds, const uint16_t *coefs, const uint8_t *codes,
                 int32_t exp_bias, const float *x, int ldx, float *y, int ldy,
                 int M, int K, int P, int N)
{
    if (bad_args(M, K, P) || N < 0 || ldx < K || ldy < M || !exponent_in_range(exp_bias))
        return -1;
#pragma omp parallel
    {
        float *row = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(static)
        for (int m = 0; m < M; ++m) {
            decode_row(seeds, coefs, codes, exp_bias, m, K, P, row);
            for (int n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int k = 0; k < K; ++k)
                    acc += (double)row[k] * (double)x[(int64_t)n * ldx + k];
                y[(int64_t)n * ldy + m] = (float)acc;
            }
        }
        free(row);
    }
    return 0;
}

/* y = W v in double for a double input vector (used inside the expert). */
static void matvec_double(const uint16_t *seeds, const uint16_t *coefs, const uint8_t *codes,
                          int32_t exp_bias, int M, int K, int P, const double *v, double *out)
{
#pragma omp parallel
    {
        float *row = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(static)
        for (int m = 0; m < M; ++m) {
            decode_row(seeds, coefs, codes, exp_bias, m, K, P, row);
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += (double)row[k] * v[k];
            out[m] = acc;
        }
        free(row);
    }
}

/* SwiGLU expert (the routed FFN experts are what carry seeds [K2CARD "This upload"]):
 * h = silu(G x) * (U x) with silu(z) = z / (1 + e^-z), then D h; all in double. */
int seedref_expert_accum(const uint16_t *g_seeds, const uint16_t *g_coefs, const uint8_t *g_codes,
                         int32_t g_eb,
                         const uint16_t *u_seeds, const uint16_t *u_coefs, const uint8_t *u_codes,
                         int32_t u_eb,
                         const uint16_t *d_seeds, const uint16_t *d_coefs, const uint8_t *d_codes,
                         int32_t d_eb,
                         const float *x, double scale, double *y, int H, int I, int P)
{
    if (bad_args(I, H, P) || bad_args(H, I, P))
        return -1;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(H > 0 ? H : 1));
    double *g = (double *)malloc(sizeof(double) * (size_t)(I > 0 ? I : 1));
    double *u = (double *)malloc(sizeof(double) * (size_t)(I > 0 ? I : 1));
    double *o = (double *)malloc(sizeof(double) * (size_t)(H > 0 ? H : 1));
    for (int k = 0; k < H; ++k)
        xd[k] = (double)x[k];
    matvec_double(g_seeds, g_coefs, g_codes, g_eb, I, H, P, xd, g);
    matvec_double(u_seeds, u_coefs, u_codes, u_eb, I, H, P, xd, u);
    for (int i = 0; i < I; ++i)
        g[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
    matvec_double(d_seeds, d_coefs, d_codes, d_eb, H, I, P, g, o);
    for (int k = 0; k < H; ++k)
        y[k] += scale * o[k];
    free(xd); free(g); free(u); free(o);
    return 0;
}

/* The routed layer: every token sums its top-k experts' outputs, weighted by the
 * router weights, in slot order k = 0 .. top_k-1.  No shared expert. */
int seedref_moe(const int32_t *topk_ids, const float *topk_w, int T, int top_k,
                const float *x, float *y, int E, int H, int I, int P,
                const uint16_t *g_seeds, const uint16_t *g_coefs, const uint8_t *g_codes, const int32_t *g_eb,
                const uint16_t *u_seeds, const uint16_t *u_coefs, const uint8_t *u_codes, const int32_t *u_eb,
                const uint16_t *d_seeds, const uint16_t *d_coefs, const uint8_t *d_codes, const int32_t *d_eb)
{
    if (T < 0 || top_k < 1 || E < 1 || bad_args(I, H, P) || bad_args(H, I, P))
        return -1;
    for (int64_t n = 0; n < (int64_t)T * top_k; ++n)
        if (topk_ids[n] < 0 || topk_ids[n] >= E)
            return -1;
    /* per-expert stream strides: blocks of one [I][H] (or [H][I]) matrix */
    int64_t nblk = (int64_t)I * (H / 8);
    int64_t coef_words = nblk * P / 4;     /* exact when nblk*P % 4 == 0 */
    int64_t code_bytes = nblk / 2;
    if ((nblk * P) % 4 != 0 || nblk % 2 != 0)
        return -1;
    double *acc = (double *)malloc(sizeof(double) * (size_t)(H > 0 ? H : 1));
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < H; ++k)
            acc[k] = 0.0;
        for (int s = 0; s < top_k; ++s) {
            int e = topk_ids[(int64_t)t * top_k + s];
            double wgt = (double)topk_w[(int64_t)t * top_k + s];
            seedref_expert_accum(g_seeds + e * nblk, g_coefs + e * coef_words, g_codes + e * code_bytes, g_eb[e],
                                 u_seeds + e * nblk, u_coefs + e * coef_words, u_codes + e * code_bytes, u_eb[e],
                                 d_seeds + e * nblk, d_coefs + e * coef_words, d_codes + e * code_bytes, d_eb[e],
                                 x + (int64_t)t * H, wgt, acc, H, I, P);
        }
        for (int k = 0; k < H; ++k)
            y[(int64_t)t * H + k] = (float)acc[k];
    }
    free(acc);
    return 0;
}

/* Mixed packs, P chosen per expert ([INDEX "Results"]: hybrid P3 / P4 packs with a
 * third of the experts in P4; [INDEX "Plans"]: hot experts in P4, the rest in P3):
 * expert e has P_e coefficients per block; its seed and code streams sit at the
 * same strides as in seedref_moe, its coefficient stream follows the streams of experts
 * 0..e-1, i.e. at word sum_{e' < e} nblk * P_e' / 4. */
int seedref_moe_mixed(const int32_t *topk_ids, const float *topk_w, int T, int top_k,
                      const float *x, float *y, int E, int H, int I, const int32_t *Pe,
                      const uint16_t *g_seeds, const uint16_t *g_coefs, const uint8_t *g_codes, const int32_t *g_eb,
                      const uint16_t *u_seeds, const uint16_t *u_coefs, const uint8_t *u_codes, const int32_t *u_eb,
                      const uint16_t *d_seeds, const uint16_t *d_coefs, const uint8_t *d_codes, const int32_t *d_eb)
{
    if (T < 0 || top_k < 1 || E < 1)
        return -1;
    for (int e = 0; e < E; ++e)
        if (bad_args(I, H, Pe[e]) || bad_args(H, I, Pe[e]))
            return -1;
    for (int64_t n = 0; n < (int64_t)T * top_k; ++n)
        if (topk_ids[n] < 0 || topk_ids[n] >= E)
            return -1;
    int64_t nblk = (int64_t)I * (H / 8);
    int64_t code_bytes = nblk / 2;
    if (nblk % 4 != 0)
        return -1;
    int64_t *coff = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
    int64_t off = 0;
    for (int e = 0; e < E; ++e) {
        coff[e] = off;
        off += nblk * Pe[e] / 4;
    }
    double *acc = (double *)malloc(sizeof(double) * (size_t)(H > 0 ? H : 1));
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < H; ++k)
            acc[k] = 0.0;
        for (int s = 0; s < top_k; ++s) {
            int e = topk_ids[(int64_t)t * top_k + s];
            double wgt = (double)topk_w[(int64_t)t * top_k + s];
            seedref_expert_accum(g_seeds + e * nblk, g_coefs + coff[e], g_codes + e * code_bytes, g_eb[e],
                                 u_seeds + e * nblk, u_coefs + coff[e], u_codes + e * code_bytes, u_eb[e],
                                 d_seeds + e * nblk, d_coefs + coff[e], d_codes + e * code_bytes, d_eb[e],
                                 x + (int64_t)t * H, wgt, acc, H, I, Pe[e]);
        }
        for (int k = 0; k < H; ++k)
            y[(int64_t)t * H + k] = (float)acc[k];
    }
    free(acc);
    free(coff);
    return 0;
}

/* Solve the P x P system a x = r by Gaussian elimination with partial pivoting. */
static int solve_small(double a[4][4], double r[4], int P, double x[4])
{
    for (int col = 0; col < P; ++col) {
        int piv = col;
        for (int row = col + 1; row < P; ++row)
            if (fabs(a[row][col]) > fabs(a[piv][col]))
                piv = row;
        if (fabs(a[piv][col]) < 1e-300)
            return -1;
        if (piv != col) {
            for (int k = 0; k < P; ++k) {
                double t = a[col][k]; a[col][k] = a[piv][k]; a[piv][k] = t;
            }
            double t = r[col]; r[col] = r[piv]; r[piv] = t;
        }
        for (int row = col + 1; row < P; ++row) {
            double f = a[row][col] / a[col][col];
            for (int k = col; k < P; ++k)
                a[row][k] -= f * a[col][k];
            r[row] -= f * r[col];
        }
    }
    for (int row = P - 1; row >= 0; --row) {
        double s = r[row];
        for (int k = row + 1; k < P; ++k)
            s -= a[row][k] * x[k];
        x[row] = s / a[row][row];
    }
    return 0;
}

/* [P4CARD "How it works"], [K2CARD "This upload"]: the search tries all 65,535 seeds per
 * block and keeps the one whose basis comes nearest to the original weights; [BLOG
 * "GPU search == CPU search"]: no contraction.  d8 (may be NULL: all ones) weights the
 * squared error of each of the 8 weights, as an activation-importance weighting does:
 *   A_jk = sum_i (d_i U_ij) U_ik,  r_j = sum_i (d_i U_ij) w_i,  err = sum_i d_i (w_i - sc v_i)^2
 * with every sum taken in increasing i. */
int seedref_search_block_w(const double *w8, const double *d8, int exp_bias, int P,
                           uint16_t *seed_out, int *c_out, int *code_out, double *err_out)
{
    if (P != 3 && P != 4)
        return -1;
    double best_err = INFINITY;
    int best_seed = -1, best_code = -1, best_c[4] = {0, 0, 0, 0};
    uint16_t st[32];
    for (int seed = 1; seed <= 65535; ++seed) {
        seedref_states((uint16_t)seed, 8 * P, st);
        double U[8][4];
        for (int i = 0; i < 8; ++i)
            for (int j = 0; j < P; ++j)
                U[i][j] = (double)st[i * P + j] - 32768.0;
        double a[4][4], r[4], alpha[4];
        for (int j = 0; j < P; ++j) {
            r[j] = 0.0;
            for (int i = 0; i < 8; ++i)
                r[j] += (d8 ? d8[i] * U[i][j] : U[i][j]) * w8[i];
            for (int k = 0; k < P; ++k) {
                a[j][k] = 0.0;
                for (int i = 0; i < 8; ++i)
                    a[j][k] += (d8 ? d8[i] * U[i][j] : U[i][j]) * U[i][k];
            }
        }
        if (solve_small(a, r, P, alpha) != 0)
            continue;
        for (int code = 0; code < 16; ++code) {
            double sc = ldexp(1.0, code + exp_bias - 15);
            int c[4];
            for (int j = 0; j < P; ++j) {
                double q = rint(alpha[j] / sc);        /* round half to even */
                if (q < -8.0) q = -8.0;
                if (q > 7.0) q = 7.0;
                c[j] = (int)q;
            }
            double err = 0.0;
            for (int i = 0; i < 8; ++i) {
                double v = 0.0;
                for (int j = 0; j < P; ++j)
                    v += U[i][j] * (double)c[j];
                double d = w8[i] - sc * v;
                err += d8 ? d8[i] * (d * d) : d * d;
            }
            if (err < best_err) {      /* strict: ties keep the lower (seed, code) */
                best_err = err;
                best_seed = seed;
                best_code = code;
                for (int j = 0; j < P; ++j)
                    best_c[j] = c[j];
            }
        }
    }
    if (best_seed < 0)
        return -1;
    *seed_out = (uint16_t)best_seed;
    *code_out = best_code;
    for (int j = 0; j < P; ++j)
        c_out[j] = best_c[j];
    *err_out = best_err;
    return 0;
}

int seedref_search_block(const double *w8, int exp_bias, int P, uint16_t *seed_out,
                         int *c_out, int *code_out, double *err_out)
{
    return seedref_search_block_w(w8, NULL, exp_bias, P, seed_out, c_out, code_out, err_out);
}

/* The search over every block of an [M][K] matrix (K % 8 == 0): seeds, the coefficient
 * nibble stream and the code stream in the layout seedref_reconstruct_f32 reads, and the
 * squared error of every block.  colw: per-column importance (length K) or NULL.
 * Blocks are independent; OpenMP spreads them over threads. */
int seedref_search_matrix(const float *W, const float *colw, int M, int K, int P,
                          int exp_bias, uint16_t *seeds, uint16_t *coefs, uint8_t *codes,
                          double *err)
{
    if (M < 0 || K < 0 || K % 8 != 0 || (P != 3 && P != 4))
        return -1;
    const long nblk = (long)M * (K / 8);
    memset(coefs, 0, sizeof(uint16_t) * (size_t)((nblk * P + 3) / 4));
    memset(codes, 0, (size_t)((nblk + 1) / 2));
    int bad = 0;
    int *cs = (int *)malloc(sizeof(int) * (size_t)(nblk > 0 ? nblk : 1) * 5);
    if (!cs)
        return -1;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long b = 0; b < nblk; ++b) {
        const long m = b / (K / 8), kb = b % (K / 8);
        double w8[8], d8[8];
        for (int i = 0; i < 8; ++i) {
            w8[i] = (double)W[m * K + 8 * kb + i];
            if (colw)
                d8[i] = (double)colw[8 * kb + i];
        }
        uint16_t sd;
        int c[4], code;
        double e;
        if (seedref_search_block_w(w8, colw ? d8 : NULL, exp_bias, P, &sd, c, &code, &e) != 0) {
            bad = 1;
            continue;
        }
        seeds[b] = sd;
        for (int j = 0; j < P; ++j)
            cs[b * 5 + j] = c[j];
        cs[b * 5 + 4] = code;
        if (err)
            err[b] = e;
    }
    if (!bad) {   /* packing is sequential: neighbouring blocks share words and bytes */
        for (long b = 0; b < nblk; ++b) {
            for (int j = 0; j < P; ++j) {
                const long n = b * P + j;
                coefs[n >> 2] |= (uint16_t)(((unsigned)cs[b * 5 + j] & 0xFu) << (4 * (n & 3)));
            }
            codes[b >> 1] |= (uint8_t)(((unsigned)cs[b * 5 + 4] & 0xFu) << (4 * (b & 1)));
        }
    }
    free(cs);
    return bad ? -1 : 0;
}

int seedref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the parallel loops that follow (timing only; results do not depend on
 * it, every row is summed in a fixed order). */
void seedref_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
