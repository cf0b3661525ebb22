/*
 * seedref.h -- CPU oracle for SeedLM seed-decoding matrix products.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link, load or call this code.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg use it.  It shares
 * no code, header, table or constant generator with the GPU implementation.
 *
 * What it computes (source: the pages' description of SeedLM, see each function):
 *   a matrix is cut into blocks of 8 consecutive weights along K; each block is a
 *   16-bit LFSR seed, P (3 or 4) int4 coefficients and a 4-bit exponent code, and
 *   every tensor carries one int32 exp_bias.  A block decodes to
 *       w_i = 2^(code + exp_bias - 15) * sum_j c_j * (s_{iP+j+1} - 32768),  i = 0..7
 *   where s_1, s_2, ... are the successive states of the register started at the seed.
 *
 * Readings of points the pages leave open:
 *   - register: 16-bit Fibonacci, shifts left, new bit = parity(state & 0xB400)
 *     enters bit 0 (polynomial x^16 + x^14 + x^13 + x^11 + 1, period 65,535);
 *   - basis: states after steps 1..8P fill the 8 x P basis row-major;
 *   - basis value: state - 32768, with the 2^-15 folded into the exponent;
 *   - coefficients: a flat nibble stream, P nibbles per block, nibble n at
 *     coefs[n >> 2] bits 4*(n & 3), decoded as (q ^ 8) - 8;
 *   - exponent codes: two per byte, even block in the low nibble;
 *   - block b of an [M][K] matrix covers row m = b / (K/8), columns 8*(b % (K/8)) ...
 *
 * Parity status: every function here is pinned by CPU tests against closed forms,
 * exhaustive invariants, brute force and library reductions.  Parity unpinned: the
 * fill order and the tap mask are readings, and bit-compatibility with the published
 * model files cannot be checked (the pages print no seed -> weights example).
 *
 * Floating point: built with -ffp-contract=off; products accumulate in double.
 */
#ifndef SEEDREF_H
#define SEEDREF_H
#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One register step (SeedLM page, "LFSR is free" / "Stream tables"). */
uint16_t seedref_lfsr_step(uint16_t s);
/* States s_1..s_n after steps 1..n from `seed` (the seed is the initial state). */
void seedref_states(uint16_t seed, int n, uint16_t *out);
/* Coefficient j of block b (nibble stream, P nibbles per block). */
int seedref_coef(const uint16_t *coefs, int64_t b, int P, int j);
/* Exponent code of block b (two 4-bit codes per byte). */
int seedref_code(const uint8_t *codes, int64_t b);
/* Decode one block from its parts: 8 exact fp32 weights. */
void seedref_block(uint16_t seed, const int *c, int P, int code, int exp_bias, float *w8);

/* Stream sizes in bytes of an [M][K] matrix (K % 8 == 0). Returns 0 or -1. */
int seedref_stream_bytes(int64_t M, int64_t K, int P, int64_t *seed_bytes,
                         int64_t *coef_bytes, int64_t *code_bytes);

/* Reconstruct W[M][K] (row-major) exactly in fp32. Returns 0 or -1 on bad args. */
int seedref_reconstruct_f32(const uint16_t *seeds, const uint16_t *coefs, const uint8_t *codes,
                            int32_t exp_bias, int M, int K, int P, float *W);
/* Same, rounded to bf16 (round to nearest, ties to even), as raw uint16 bits. */
int seedref_reconstruct_bf16(const uint16_t *seeds, const uint16_t *coefs, const uint8_t *codes,
                             int32_t exp_bias, int M, int K, int P, uint16_t *W);
/* Round-to-nearest-even fp32 -> bf16 bits. */
uint16_t seedref_f32_to_bf16(float f);

/* y[n][m] = sum_k W[m][k] * x[n][k], double accumulation; x fp32 [N][ldx], y fp32 [N][ldy]. */
int seedref_gemv(const uint16_t *seeds, const uint16_t *coefs, const uint8_t *codes,
                 int32_t exp_bias, const float *x, int ldx, float *y, int ldy,
                 int M, int K, int P, int N);

/* One SwiGLU expert: y = D (silu(G x) * (U x)); G, U are [I][H], D is [H][I].
 * x fp32 [H]; y double [H] (accumulated into: y += scale * result). */
int seedref_expert_accum(const uint16_t *g_seeds, const uint16_t *g_coefs, const uint8_t *g_codes,
                         int32_t g_eb,
                         const uint16_t *u_seeds, const uint16_t *u_coefs, const uint8_t *u_codes,
                         int32_t u_eb,
                         const uint16_t *d_seeds, const uint16_t *d_coefs, const uint8_t *d_codes,
                         int32_t d_eb,
                         const float *x, double scale, double *y, int H, int I, int P);

/* Routed MoE layer: y[t] = sum_k topk_w[t][k] * expert_{topk_ids[t][k]}(x[t]).
 * Expert weights are stacked: expert e's streams follow expert e-1's; exp_bias arrays are [E].
 * x fp32 [T][H], y fp32 [T][H].  Returns 0, or -1 on bad args / out-of-range ids. */
int seedref_moe(const int32_t *topk_ids, const float *topk_w, int T, int top_k,
                const float *x, float *y, int E, int H, int I, int P,
                const uint16_t *g_seeds, const uint16_t *g_coefs, const uint8_t *g_codes, const int32_t *g_eb,
                const uint16_t *u_seeds, const uint16_t *u_coefs, const uint8_t *u_codes, const int32_t *u_eb,
                const uint16_t *d_seeds, const uint16_t *d_coefs, const uint8_t *d_codes, const int32_t *d_eb);

/* The same layer with P chosen per expert (Pe[E], 3 or 4; nblk % 4 == 0): seed and code
 * streams at the uniform strides, expert e's coefficient words after those of experts
 * 0..e-1 (word offset sum_{e' < e} nblk * Pe[e'] / 4). */
int seedref_moe_mixed(const int32_t *topk_ids, const float *topk_w, int T, int top_k,
                      const float *x, float *y, int E, int H, int I, const int32_t *Pe,
                      const uint16_t *g_seeds, const uint16_t *g_coefs, const uint8_t *g_codes, const int32_t *g_eb,
                      const uint16_t *u_seeds, const uint16_t *u_coefs, const uint8_t *u_codes, const int32_t *u_eb,
                      const uint16_t *d_seeds, const uint16_t *d_coefs, const uint8_t *d_codes, const int32_t *d_eb);

/* Exhaustive seed search for one block (the encoder's inner step, unweighted).
 * For every seed 1..65535: least-squares coefficients in double, then for every code
 * 0..15 round-half-even / clamp to [-8,7] and measure the exact squared error; keeps
 * the lexicographic minimum of (error, seed, code). */
int seedref_search_block(const double *w8, int exp_bias, int P, uint16_t *seed_out,
                         int *c_out, int *code_out, double *err_out);

/* The same search with a per-weight importance d8 (NULL = all ones): the normal
 * equations and the error are weighted, A_jk = sum_i (d_i U_ij) U_ik,
 * r_j = sum_i (d_i U_ij) w_i, err = sum_i d_i (w_i - sc v_i)^2, sums in increasing i. */
int seedref_search_block_w(const double *w8, const double *d8, int exp_bias, int P,
                           uint16_t *seed_out, int *c_out, int *code_out, double *err_out);

/* Search every block of W [M][K] (fp32, K % 8 == 0; colw: importance per column, length
 * K, or NULL) and write the seeds, coefficient and code streams, and each block's
 * squared error (err may be NULL).  Returns 0, or -1 on bad arguments. */
int seedref_search_matrix(const float *W, const float *colw, int M, int K, int P,
                          int exp_bias, uint16_t *seeds, uint16_t *coefs, uint8_t *codes,
                          double *err);

/* Threads the OpenMP loops use (1 when built without OpenMP). */
int seedref_num_threads(void);
void seedref_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
