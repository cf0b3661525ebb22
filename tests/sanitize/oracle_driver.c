/* Sanitizer driver for the CPU oracle (test infrastructure): calls every oracle entry
 * point on small ragged inputs, P = 3 and 4, so an AddressSanitizer / UBSan build reports
 * any out-of-bounds access, overflow or undefined shift.  It also checks a few results
 * against plain definitions (bf16 = RNE of fp32, the product against a double sum, the
 * layer against a sum of experts).  Exit status 0 = clean. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/seedref.h"

static uint64_t rng = 0x5EED5A17u;
static uint32_t next32(void) {            /* xorshift64*: test data only */
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (uint32_t)((rng * 2685821657736338717ull) >> 32);
}

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

static int one_shape(int M, int K, int P, int eb) {
    int64_t sb, cb, db;
    CHECK(seedref_stream_bytes(M, K, P, &sb, &cb, &db) == 0);
    const int64_t nblk = (int64_t)M * (K / 8);
    uint16_t *seeds = malloc((size_t)sb), *coefs = malloc((size_t)cb);
    uint8_t *codes = malloc((size_t)db);
    for (int64_t i = 0; i < nblk; ++i) seeds[i] = (uint16_t)(next32() % 65536);   /* seed 0 too */
    for (int64_t i = 0; i < cb / 2; ++i) coefs[i] = (uint16_t)next32();
    for (int64_t i = 0; i < db; ++i) codes[i] = (uint8_t)next32();
    float *W = malloc(sizeof(float) * (size_t)M * K);
    uint16_t *Wb = malloc(sizeof(uint16_t) * (size_t)M * K);
    CHECK(seedref_reconstruct_f32(seeds, coefs, codes, eb, M, K, P, W) == 0);
    CHECK(seedref_reconstruct_bf16(seeds, coefs, codes, eb, M, K, P, Wb) == 0);
    for (int64_t i = 0; i < (int64_t)M * K; ++i) CHECK(Wb[i] == seedref_f32_to_bf16(W[i]));
    const int N = 3;
    float *x = malloc(sizeof(float) * (size_t)N * K), *y = malloc(sizeof(float) * (size_t)N * M);
    for (int i = 0; i < N * K; ++i) x[i] = (float)((int)(next32() % 2001) - 1000) / 1000.0f;
    CHECK(seedref_gemv(seeds, coefs, codes, eb, x, K, y, M, M, K, P, N) == 0);
    for (int n = 0; n < N; ++n)
        for (int m = 0; m < M; ++m) {
            double s = 0.0;
            for (int k = 0; k < K; ++k) s += (double)W[(int64_t)m * K + k] * x[n * K + k];
            CHECK(fabs((double)y[n * M + m] - s) <= 1e-6 * (fabs(s) + 1e-30) + 1e-30);
        }
    free(seeds); free(coefs); free(codes); free(W); free(Wb); free(x); free(y);
    return 0;
}

static int layer(int P) {
    const int E = 5, H = 64, I = 32, T = 4, k = 2;
    const int64_t n = (int64_t)I * (H / 8);
    uint16_t *s[3], *c[3];
    uint8_t *d[3];
    int32_t eb[3][5];
    for (int m = 0; m < 3; ++m) {
        s[m] = malloc(sizeof(uint16_t) * (size_t)(E * n));
        c[m] = malloc(sizeof(uint16_t) * (size_t)(E * n * P / 4));
        d[m] = malloc((size_t)(E * n / 2));
        for (int64_t i = 0; i < E * n; ++i) s[m][i] = (uint16_t)(1 + next32() % 65535);
        for (int64_t i = 0; i < E * n * P / 4; ++i) c[m][i] = (uint16_t)next32();
        for (int64_t i = 0; i < E * n / 2; ++i) d[m][i] = (uint8_t)next32();
        for (int e = 0; e < E; ++e) eb[m][e] = -22 + (int)(next32() % 5);
    }
    int32_t ids[T * k];
    float w[T * k], x[T * H], y[T * H], ym[T * H];
    for (int t = 0; t < T; ++t) {
        ids[t * k] = (int)(next32() % E);
        ids[t * k + 1] = (ids[t * k] + 1 + (int)(next32() % (E - 1))) % E;
        w[t * k] = 0.75f; w[t * k + 1] = 0.25f;
    }
    for (int i = 0; i < T * H; ++i) x[i] = (float)((int)(next32() % 2001) - 1000) / 500.0f;
    CHECK(seedref_moe(ids, w, T, k, x, y, E, H, I, P, s[0], c[0], d[0], eb[0], s[1], c[1], d[1],
                      eb[1], s[2], c[2], d[2], eb[2]) == 0);
    int32_t Pe[5];
    for (int e = 0; e < E; ++e) Pe[e] = P;
    CHECK(seedref_moe_mixed(ids, w, T, k, x, ym, E, H, I, Pe, s[0], c[0], d[0], eb[0], s[1], c[1],
                            d[1], eb[1], s[2], c[2], d[2], eb[2]) == 0);
    for (int i = 0; i < T * H; ++i) CHECK(y[i] == ym[i]);
    ids[0] = E;   /* out of range: rejected */
    CHECK(seedref_moe(ids, w, T, k, x, y, E, H, I, P, s[0], c[0], d[0], eb[0], s[1], c[1], d[1],
                      eb[1], s[2], c[2], d[2], eb[2]) != 0);
    for (int m = 0; m < 3; ++m) { free(s[m]); free(c[m]); free(d[m]); }
    return 0;
}

int main(void) {
    uint16_t st[32];
    seedref_states(1, 32, st);
    seedref_states(0, 32, st);
    for (int i = 0; i < 32; ++i) CHECK(st[i] == 0);
    static const int shapes[][2] = {{1, 8}, {3, 24}, {5, 104}, {16, 512}, {7, 72}};
    for (int P = 3; P <= 4; ++P)
        for (int i = 0; i < 5; ++i)
            for (int eb = -100; eb <= 100; eb += 100)
                if (one_shape(shapes[i][0], shapes[i][1], P, eb)) return 1;
    if (layer(3) || layer(4)) return 1;
    /* one exhaustive block search and a tiny matrix search, both P */
    double w8[8];
    for (int i = 0; i < 8; ++i) w8[i] = ((int)(next32() % 2001) - 1000) * 1e-5;
    for (int P = 3; P <= 4; ++P) {
        uint16_t seed; int cc[4], code; double err;
        CHECK(seedref_search_block(w8, -4, P, &seed, cc, &code, &err) == 0);
        CHECK(err >= 0.0);
        float Wm[2 * 16];
        for (int i = 0; i < 32; ++i) Wm[i] = (float)w8[i % 8] * (float)(1 + i / 8);
        uint16_t ss[4], cf[4]; uint8_t cd[2]; double e4[4];
        memset(cf, 0, sizeof cf);
        CHECK(seedref_search_matrix(Wm, NULL, 2, 16, P, -4, ss, cf, cd, e4) == 0);
    }
    CHECK(seedref_reconstruct_f32(NULL, NULL, NULL, 0, 4, 12, 4, NULL) != 0);   /* K % 8 */
    printf("oracle sanitizer driver: clean\n");
    return 0;
}
