/*
 * selftest.c -- a driver of the oracle for sanitizer builds (test
 * infrastructure only). It runs every multi-threaded oracle routine on small
 * seeded inputs with several threads, and checks invariants that must hold
 * whatever the thread count: the same results on 1 and on 7 threads (the
 * routines write disjoint rows), the quantization bound, the kept-block count,
 * finite outputs. Built and run by the CPU test suite under AddressSanitizer
 * with UndefinedBehaviorSanitizer, and under ThreadSanitizer.
 *
 * Prints "selftest ok" and exits 0 when every check passes.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

/* splitmix64 */
static uint64_t next_u64(void) {
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* roughly normal values (sum of four uniforms), as bf16 bit patterns */
static uint16_t rand_bf16(float scale, float offset) {
    float s = 0.f;
    for (int t = 0; t < 4; ++t) s += (float)(next_u64() >> 40) / (float)(1u << 24);
    return orc_f32_to_bf16((s - 2.0f) * 1.7f * scale + offset);
}

static int g_fail = 0;
#define CHECK(cond, what)                                  \
    do {                                                   \
        if (!(cond)) {                                     \
            fprintf(stderr, "selftest: %s failed\n", what); \
            g_fail = 1;                                    \
        }                                                  \
    } while (0)

int main(void) {
    const int64_t BH = 2, N = 700, D = 128, keep = 3;
    const int64_t nqb = orc_nqb(N), nkb = orc_nkb(N), nel = BH * N * D;
    uint16_t* q = malloc(sizeof(uint16_t) * nel);
    uint16_t* k = malloc(sizeof(uint16_t) * nel);
    uint16_t* v = malloc(sizeof(uint16_t) * nel);
    for (int64_t x = 0; x < nel; ++x) {
        q[x] = rand_bf16(1.f, 0.f);
        k[x] = rand_bf16(1.f, (float)(x % D % 7) - 3.f);
        v[x] = rand_bf16(1.f, 0.f);
    }
    float* mu = malloc(sizeof(float) * BH * D);
    orc_k_mean(k, BH, N, D, mu);

    int8_t* qi[2];
    int8_t* ki[2];
    float* qs[2];
    float* ks[2];
    const int threads[2] = {1, 7};
    for (int r = 0; r < 2; ++r) {
        qi[r] = malloc(nel);
        ki[r] = malloc(nel);
        qs[r] = malloc(sizeof(float) * BH * nqb);
        ks[r] = malloc(sizeof(float) * BH * nkb);
        orc_quant(q, NULL, BH, N, D, ORC_QBLK, qi[r], qs[r], threads[r]);
        orc_quant(k, mu, BH, N, D, ORC_KBLK, ki[r], ks[r], threads[r]);
    }
    CHECK(memcmp(qi[0], qi[1], nel) == 0 && memcmp(ki[0], ki[1], nel) == 0, "quant threads");
    CHECK(memcmp(qs[0], qs[1], sizeof(float) * BH * nqb) == 0, "q scale threads");
    for (int64_t x = 0; x < nel; ++x) {
        const float s = qs[0][(x / D / N) * nqb + (x / D % N) / ORC_QBLK];
        CHECK(fabsf(orc_bf16_to_f32(q[x]) - qi[0][x] * s) <= s * 0.5f * (1.f + 0x1p-15f) + 1e-30f,
              "quant bound");
    }

    /* block mask of head 1 */
    float* qbar = malloc(sizeof(float) * nqb * D);
    float* kbar = malloc(sizeof(float) * nkb * D);
    orc_pool(q, N, D, 1, ORC_QBLK, qbar);
    orc_pool(k, N, D, 1, ORC_KBLK, kbar);
    int64_t* rows = malloc(sizeof(int64_t) * nqb);
    for (int64_t i = 0; i < nqb; ++i) rows[i] = i;
    float* sc = malloc(sizeof(float) * nqb * nkb);
    orc_block_scores(qbar, kbar, nkb, D, rows, nqb, sc);
    int32_t* kidx = malloc(sizeof(int32_t) * nqb * keep);
    uint8_t* mask = malloc((size_t)(nqb * nkb));
    orc_topk(sc, nqb, nkb, keep, kidx, mask);
    for (int64_t i = 0; i < nqb; ++i) {
        int cnt = 0;
        for (int64_t j = 0; j < nkb; ++j) cnt += mask[i * nkb + j];
        CHECK(cnt == keep, "kept count");
        for (int64_t a = 1; a < keep; ++a) CHECK(kidx[i * keep + a] > kidx[i * keep + a - 1], "kidx order");
    }

    /* sparse rows, linear rows and dense rows on 1 and 7 threads */
    const int64_t R = N;
    int64_t* tok = malloc(sizeof(int64_t) * R);
    for (int64_t t = 0; t < R; ++t) tok[t] = t;
    double* od[2];
    double* oe[2];
    double* am[2];
    double* ol[2];
    double* h = malloc(sizeof(double) * nkb * D * D);
    double* z = malloc(sizeof(double) * nkb * D);
    double* h1 = malloc(sizeof(double) * nkb * D * D);
    double* z1 = malloc(sizeof(double) * nkb * D);
    orc_linear_states(k, v, N, D, 1, h, z, 7);
    orc_linear_states(k, v, N, D, 1, h1, z1, 1);
    CHECK(memcmp(h, h1, sizeof(double) * nkb * D * D) == 0, "linear states threads");
    for (int r = 0; r < 2; ++r) {
        od[r] = malloc(sizeof(double) * R * D);
        oe[r] = malloc(sizeof(double) * R * D);
        am[r] = malloc(sizeof(double) * R);
        ol[r] = malloc(sizeof(double) * R * D);
        orc_sparse_rows(qi[0], qs[0], ki[0], ks[0], v, N, D, 1, kidx, keep, 0.f, tok, R, od[r],
                        oe[r], am[r], threads[r]);
        orc_linear_rows(q, N, D, 1, h, z, kidx, keep, tok, R, ol[r], threads[r]);
    }
    CHECK(memcmp(od[0], od[1], sizeof(double) * R * D) == 0, "sparse rows threads");
    CHECK(memcmp(ol[0], ol[1], sizeof(double) * R * D) == 0, "linear rows threads");
    for (int64_t x = 0; x < R * D; ++x) CHECK(isfinite(od[0][x]) && isfinite(ol[0][x]), "finite");
    double* dn = malloc(sizeof(double) * 16 * D);
    orc_dense_rows(q, k, v, N, D, 0, 0.f, tok, 16, dn, 7);
    for (int64_t x = 0; x < 16 * D; ++x) CHECK(isfinite(dn[x]), "dense finite");

    /* backward of head 1 on 1 and 7 threads, both branches */
    {
        uint16_t* dout = malloc(sizeof(uint16_t) * nel);
        for (int64_t x = 0; x < nel; ++x) dout[x] = rand_bf16(1.f, 0.f);
        double* g[2][3];
        for (int r = 0; r < 2; ++r) {
            for (int n = 0; n < 3; ++n) g[r][n] = malloc(sizeof(double) * N * D);
            orc_sagesla_bwd(q, k, v, qi[0], qs[0], ki[0], ks[0], N, D, 1, kidx, keep, 3, 0.f, dout,
                            g[r][0], g[r][1], g[r][2], threads[r]);
        }
        for (int n = 0; n < 3; ++n) {
            CHECK(memcmp(g[0][n], g[1][n], sizeof(double) * N * D) == 0, "backward threads");
            for (int64_t x = 0; x < N * D; ++x) CHECK(isfinite(g[0][n][x]), "backward finite");
        }
        /* sampled rows and keys on 7 threads equal the full computation */
        {
            uint8_t* qsel = calloc((size_t)N, 1);
            uint8_t* ksel = calloc((size_t)N, 1);
            qsel[0] = qsel[130] = qsel[N - 1] = 1;
            ksel[3] = ksel[64] = ksel[N - 1] = 1;
            double* h3[3];
            for (int n = 0; n < 3; ++n) h3[n] = malloc(sizeof(double) * N * D);
            orc_sagesla_bwd_sel(q, k, v, qi[0], qs[0], ki[0], ks[0], N, D, 1, kidx, keep, 3, 0.f,
                                dout, qsel, ksel, h3[0], h3[1], h3[2], 7);
            for (int64_t t = 0; t < N; ++t) {
                if (qsel[t])
                    CHECK(memcmp(h3[0] + t * D, g[0][0] + t * D, sizeof(double) * D) == 0,
                          "sampled dq");
                if (ksel[t])
                    for (int n = 1; n < 3; ++n)
                        CHECK(memcmp(h3[n] + t * D, g[0][n] + t * D, sizeof(double) * D) == 0,
                              "sampled dk, dv");
            }
            for (int n = 0; n < 3; ++n) free(h3[n]);
            free(qsel);
            free(ksel);
        }
        for (int r = 0; r < 2; ++r)
            for (int n = 0; n < 3; ++n) free(g[r][n]);
        free(dout);
    }

    /* W8A8 */
    const int64_t M = 300, K = 256, NO = 128;
    uint16_t* xw = malloc(sizeof(uint16_t) * M * K);
    uint16_t* ww = malloc(sizeof(uint16_t) * NO * K);
    for (int64_t x = 0; x < M * K; ++x) xw[x] = rand_bf16(1.f, 0.f);
    for (int64_t x = 0; x < NO * K; ++x) ww[x] = rand_bf16(0.1f, 0.f);
    int8_t* xq = malloc((size_t)(M * K));
    int8_t* wq = malloc((size_t)(NO * K));
    float* sx = malloc(sizeof(float) * 3 * 2);
    float* sw = malloc(sizeof(float) * 1 * 2);
    orc_w8a8_quant(xw, M, K, xq, sx, 7);
    orc_w8a8_quant(ww, NO, K, wq, sw, 7);
    int64_t* mrows = malloc(sizeof(int64_t) * M);
    for (int64_t m = 0; m < M; ++m) mrows[m] = m;
    float* y1 = malloc(sizeof(float) * M * NO);
    float* y7 = malloc(sizeof(float) * M * NO);
    orc_w8a8_gemm(xq, sx, wq, sw, NULL, M, NO, K, mrows, M, y1, 1);
    orc_w8a8_gemm(xq, sx, wq, sw, NULL, M, NO, K, mrows, M, y7, 7);
    CHECK(memcmp(y1, y7, sizeof(float) * M * NO) == 0, "w8a8 threads");

    free(q); free(k); free(v); free(mu);
    for (int r = 0; r < 2; ++r) {
        free(qi[r]); free(ki[r]); free(qs[r]); free(ks[r]);
        free(od[r]); free(oe[r]); free(am[r]); free(ol[r]);
    }
    free(qbar); free(kbar); free(rows); free(sc); free(kidx); free(mask); free(tok);
    free(h); free(z); free(h1); free(z1); free(dn);
    free(xw); free(ww); free(xq); free(wq); free(sx); free(sw); free(mrows); free(y1); free(y7);
    if (g_fail) return 1;
    printf("selftest ok\n");
    return 0;
}
