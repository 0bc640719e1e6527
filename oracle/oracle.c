/*
 * oracle.c -- plain, slow CPU reference for the SageSLA attention path.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h). Built with gcc -O2
 * -ffp-contract=off and no fast-math, so every fp32 expression below is
 * evaluated exactly as written (IEEE round-to-nearest-even, no reassociation,
 * no fused multiply-add unless fmaf is called).
 *
 * Source of the method: the TurboDiffusion pages, page 5 "Four Technical
 * Pillars" (Pillar One: SageAttention quantizes attention to INT8 and smooths
 * outliers; Pillar Two: SLA keeps the important block interactions, about 10%
 * of them, and a cheap linear-attention term stands in for the others; the
 * two stack as "SageSLA") and page 5 "Hands-On Tutorial" (--attention_type
 * sagesla, --sla_topk = fraction of connections kept). Where the pages are
 * silent the concrete reading is stated at each function.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* block counts                                                              */

int64_t orc_nqb(int64_t N) { return (N + ORC_QBLK - 1) / ORC_QBLK; }
int64_t orc_nkb(int64_t N) { return (N + ORC_KBLK - 1) / ORC_KBLK; }

/* --sla_topk is the fraction of key blocks kept (page 5, "Hands-On Tutorial":
 * 0.1 sets 90% sparsity). Reading: round half up, at least one block. */
int64_t orc_keep(int64_t N, double topk) {
    int64_t nkb = orc_nkb(N);
    int64_t kb = (int64_t)floor(topk * (double)nkb + 0.5);
    if (kb < 1) kb = 1;
    if (kb > nkb) kb = nkb;
    return kb;
}

/* ------------------------------------------------------------------------ */
/* bf16                                                                      */

float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a double to the nearest bf16 value (8 significant bits, exponent range
 * of fp32, subnormal spacing 2^-133), ties to even. Written from the format's
 * definition: scale so the kept bits are the integer part, rint, scale back. */
double orc_round_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    frexp(x, &e);            /* |x| = f * 2^e, f in [0.5, 1) */
    int q = e - 8;           /* weight of the last kept bit */
    if (q < -133) q = -133;  /* bf16 subnormals */
    double r = nearbyint(ldexp(x, -q)); /* default mode: ties to even */
    return ldexp(r, q);
}

uint16_t orc_f32_to_bf16(float x) {
    double r = orc_round_bf16((double)x);
    float f = (float)r; /* exact: r is a bf16 value (or inf) */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* a tiny parallel for (dynamic schedule)                                    */

typedef void (*orc_task)(void* ctx, int64_t idx);
typedef struct {
    orc_task fn;
    void* ctx;
    int64_t n;
    atomic_llong next;
} orc_pool_t;

static void* orc_worker(void* arg) {
    orc_pool_t* p = (orc_pool_t*)arg;
    for (;;) {
        int64_t i = atomic_fetch_add(&p->next, 1);
        if (i >= p->n) break;
        p->fn(p->ctx, i);
    }
    return NULL;
}

static void orc_parallel_for(int64_t n, int nthreads, orc_task fn, void* ctx) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (n < nthreads) nthreads = (int)(n > 0 ? n : 1);
    orc_pool_t p;
    p.fn = fn;
    p.ctx = ctx;
    p.n = n;
    atomic_init(&p.next, 0);
    if (nthreads == 1) {
        orc_worker(&p);
        return;
    }
    pthread_t th[256];
    int started = 0;
    for (int t = 0; t < nthreads - 1; ++t)
        if (pthread_create(&th[t], NULL, orc_worker, &p) == 0) ++started;
    orc_worker(&p);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* K smoothing (page 5, Pillar One: "smoothing" of outliers). Reading: the   */
/* mean of K over all N tokens of the head, per channel, subtracted from K.  */
/* Every score of a query row then shifts by the same q.mu, so softmax is    */
/* unchanged. The fp32 summation order is pinned: per 64-token block in      */
/* token order, then over blocks in block order.                             */

void orc_k_mean(const uint16_t* k, int64_t BH, int64_t N, int64_t D, float* mu) {
    int64_t nkb = orc_nkb(N);
    for (int64_t bh = 0; bh < BH; ++bh) {
        const uint16_t* kh = k + bh * N * D;
        for (int64_t d = 0; d < D; ++d) {
            float tot = 0.0f;
            for (int64_t j = 0; j < nkb; ++j) {
                float part = 0.0f;
                int64_t t1 = (j + 1) * ORC_KBLK < N ? (j + 1) * ORC_KBLK : N;
                for (int64_t t = j * ORC_KBLK; t < t1; ++t) part += orc_bf16_to_f32(kh[t * D + d]);
                tot += part;
            }
            mu[bh * D + d] = tot / (float)N;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Per-block INT8 quantization (page 5, Pillar One: attention in 8-bit      */
/* integers). Reading: one fp32 scale per (head, block) over all channels,  */
/* scale = amax/127, q = rint(x/scale) with ties to even, symmetric range.  */
/* The clamp to +-127 is IEEE minNum/maxNum (C99 fminf/fmaxf), which drops  */
/* a NaN operand: a NaN quotient (a NaN element, or an infinite element    */
/* over its block's infinite scale) becomes -127. The pages do not cover    */
/* non-finite inputs; this is the reading, and it keeps every conversion    */
/* to int8 defined.                                                          */

typedef struct {
    const uint16_t* x;
    const float* mu;
    int64_t N, D, blk, nb;
    int8_t* xq;
    float* scale;
} quant_ctx;

static void quant_task(void* vctx, int64_t idx) {
    quant_ctx* c = (quant_ctx*)vctx;
    int64_t bh = idx / c->nb, b = idx % c->nb;
    int64_t D = c->D, N = c->N;
    int64_t t0 = b * c->blk, t1 = t0 + c->blk < N ? t0 + c->blk : N;
    const uint16_t* xh = c->x + bh * N * D;
    const float* mu = c->mu ? c->mu + bh * D : NULL;
    float amax = 0.0f;
    for (int64_t t = t0; t < t1; ++t)
        for (int64_t d = 0; d < D; ++d) {
            float v = orc_bf16_to_f32(xh[t * D + d]);
            if (mu) v = v - mu[d];
            float a = fabsf(v);
            if (a > amax) amax = a;
        }
    float s = amax / 127.0f;
    c->scale[bh * c->nb + b] = s;
    for (int64_t t = t0; t < t1; ++t)
        for (int64_t d = 0; d < D; ++d) {
            float v = orc_bf16_to_f32(xh[t * D + d]);
            if (mu) v = v - mu[d];
            int8_t q = 0;
            if (s > 0.0f) {
                const float r = fminf(fmaxf(rintf(v / s), -127.0f), 127.0f);
                q = (int8_t)r;
            }
            c->xq[(bh * N + t) * D + d] = q;
        }
}

void orc_quant(const uint16_t* x, const float* mu, int64_t BH, int64_t N, int64_t D,
               int64_t blk, int8_t* xq, float* scale, int nthreads) {
    quant_ctx c = {x, mu, N, D, blk, (N + blk - 1) / blk, xq, scale};
    orc_parallel_for(BH * c.nb, nthreads, quant_task, &c);
}

/* ------------------------------------------------------------------------ */
/* int32 scores of one (query block, key block) tile                        */

void orc_qk_tile(const int8_t* q_i8, const int8_t* k_i8, int64_t N, int64_t D,
                 int64_t bh, int64_t i, int64_t j, int32_t* tile) {
    for (int64_t r = 0; r < ORC_QBLK; ++r)
        for (int64_t c = 0; c < ORC_KBLK; ++c) {
            int64_t t = i * ORC_QBLK + r, u = j * ORC_KBLK + c;
            int32_t acc = 0;
            if (t < N && u < N) {
                const int8_t* qr = q_i8 + (bh * N + t) * D;
                const int8_t* kr = k_i8 + (bh * N + u) * D;
                for (int64_t d = 0; d < D; ++d) acc += (int32_t)qr[d] * (int32_t)kr[d];
            }
            tile[r * ORC_KBLK + c] = acc;
        }
}

/* ------------------------------------------------------------------------ */
/* SLA block mask (page 5, Pillar Two: only the most important interactions, */
/* 10% of them at --sla_topk 0.1). Reading: blocks are scored by the dot     */
/* product of the mean-pooled raw Q block and raw K block; each query block */
/* keeps its top `keep` key blocks, ties going to the lower key block.      */

void orc_pool(const uint16_t* x, int64_t N, int64_t D, int64_t bh, int64_t blk, float* out) {
    int64_t nb = (N + blk - 1) / blk;
    const uint16_t* xh = x + bh * N * D;
    for (int64_t b = 0; b < nb; ++b) {
        int64_t t0 = b * blk, t1 = t0 + blk < N ? t0 + blk : N;
        for (int64_t d = 0; d < D; ++d) {
            float s = 0.0f;
            for (int64_t t = t0; t < t1; ++t) s += orc_bf16_to_f32(xh[t * D + d]);
            out[b * D + d] = s / (float)(t1 - t0);
        }
    }
}

void orc_block_scores(const float* qbar, const float* kbar, int64_t Nkb, int64_t D,
                      const int64_t* qblocks, int64_t R, float* score) {
    for (int64_t r = 0; r < R; ++r) {
        const float* qb = qbar + qblocks[r] * D;
        for (int64_t j = 0; j < Nkb; ++j) {
            const float* kb = kbar + j * D;
            float acc = 0.0f;
            for (int64_t d = 0; d < D; ++d) acc = fmaf(qb[d], kb[d], acc);
            score[r * Nkb + j] = acc;
        }
    }
}

typedef struct {
    float s;
    int32_t j;
} scored_t;

/* (score descending, j ascending); -0.0 and +0.0 compare equal. */
static int cmp_scored(const void* a, const void* b) {
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

static int cmp_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

void orc_topk(const float* score, int64_t R, int64_t Nkb, int64_t keep, int32_t* kidx,
              uint8_t* mask) {
    scored_t* tmp = (scored_t*)malloc(sizeof(scored_t) * (size_t)Nkb);
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t j = 0; j < Nkb; ++j) {
            tmp[j].s = score[r * Nkb + j];
            tmp[j].j = (int32_t)j;
        }
        qsort(tmp, (size_t)Nkb, sizeof(scored_t), cmp_scored);
        int32_t* out = kidx + r * keep;
        for (int64_t c = 0; c < keep; ++c) out[c] = tmp[c].j;
        qsort(out, (size_t)keep, sizeof(int32_t), cmp_i32);
        if (mask) {
            memset(mask + r * Nkb, 0, (size_t)Nkb);
            for (int64_t c = 0; c < keep; ++c) mask[r * Nkb + out[c]] = 1;
        }
    }
    free(tmp);
}

/* ------------------------------------------------------------------------ */
/* Sparse softmax branch over the kept blocks (page 5, Pillar One + Two).    */
/*                                                                           */
/* Declared numerics (o_decl). With sm the softmax scale:                    */
/*   K32 = fl32(sm * log2 e); c_j = fl32(fl32(sq * sk_j) * K32)              */
/*   x_u = fl32(S_u * c_j)                 (base-2 logit of key u)           */
/*   m   = ceil(max_u x_u)                 (integer normalizer)              */
/*   p_u = bf16(2^(S_u * c_j - m))         (exact exponent, one rounding)    */
/*   o   = sum_u p_u v_u / sum_u p_u       (exact)                           */
/* Because m is an integer, p_u does not depend on the order in which a GPU  */
/* visits the blocks (rescaling by powers of two is exact), and the row sum  */
/* uses the same rounded p_u the PV product sees.                            */

/* Which rounded p may legitimately differ on a GPU (reading C12). A GPU      */
/* forms the exponent as one fp32 fma, y = S*c - m', against a running       */
/* integer normalizer m' that may lag the row's m = ceil(max x) by up to     */
/* ORC_NORM_LAG (it raises m' only when a tile's max exceeds it by more than */
/* that), so |y| <= |x| + |m| + ORC_NORM_LAG and the fp32 rounding of y moves */
/* 2^y by at most 2^-24 |y| ln 2 relative; its hardware 2^y adds about one   */
/* fp32 ulp. Both bf16 roundings of p are accepted when 2^(x - m) lies       */
/* within p (2^-20 + 2^-23 (|x| + max|x| + |m| + ORC_NORM_LAG + 2)) of a     */
/* bf16 rounding midpoint, a window at least twice those errors. Returns the */
/* bf16 ulp at p when p is ambiguous, else 0.                                */
double orc_p_ambiguous(double p, double xa, double xabs_max, double m) {
    if (!(p >= 0x1p-126)) return 0.0;
    int ex;
    frexp(p, &ex);
    double ulp = ldexp(1.0, ex - 8);
    double k = p / ulp;
    double dist = fabs(k - floor(k) - 0.5) * ulp;
    double win = p * (0x1p-20 + 0x1p-23 * (xa + xabs_max + fabs(m) + ORC_NORM_LAG + 2.0));
    return dist <= win ? ulp : 0.0;
}

typedef struct {
    const int8_t* q_i8;
    const float* q_scale;
    const int8_t* k_i8;
    const float* k_scale;
    const uint16_t* v;
    int64_t N, D, bh, nqb, nkb, keep;
    const int32_t* kidx;
    float sm;
    float K32;
    const int64_t* tokens;
    double *o_decl, *o_exact, *amb;
} sparse_ctx;

static void sparse_task(void* vctx, int64_t r) {
    sparse_ctx* c = (sparse_ctx*)vctx;
    int64_t N = c->N, D = c->D, t = c->tokens[r];
    int64_t i = t / ORC_QBLK;
    int64_t nsel = c->kidx ? c->keep : c->nkb;
    int64_t cap = nsel * ORC_KBLK;
    int32_t* S = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
    int64_t* U = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    float* C = (float*)malloc(sizeof(float) * (size_t)cap);
    double* se = (double*)malloc(sizeof(double) * (size_t)cap);
    double* acc = (double*)calloc((size_t)D, sizeof(double));
    double* acc2 = (double*)calloc((size_t)D, sizeof(double));
    const int8_t* qr = c->q_i8 + (c->bh * N + t) * D;
    float sq = c->q_scale[c->bh * c->nqb + i];
    int64_t n = 0;
    for (int64_t jj = 0; jj < nsel; ++jj) {
        int64_t j = c->kidx ? c->kidx[i * c->keep + jj] : jj;
        float sk = c->k_scale[c->bh * c->nkb + j];
        float cj = (sq * sk) * c->K32;
        int64_t u1 = (j + 1) * ORC_KBLK < N ? (j + 1) * ORC_KBLK : N;
        for (int64_t u = j * ORC_KBLK; u < u1; ++u) {
            const int8_t* kr = c->k_i8 + (c->bh * N + u) * D;
            int32_t s = 0;
            for (int64_t d = 0; d < D; ++d) s += (int32_t)qr[d] * (int32_t)kr[d];
            S[n] = s;
            U[n] = u;
            C[n] = cj;
            se[n] = (double)s * (double)sq * (double)sk * (double)c->sm;
            ++n;
        }
    }
    const uint16_t* vh = c->v + c->bh * N * D;
    /* declared numerics */
    float xmax = -INFINITY;
    for (int64_t a = 0; a < n; ++a) {
        float x = (float)S[a] * C[a];
        if (x > xmax) xmax = x;
    }
    float m = ceilf(xmax);
    double l = 0.0;
    double* pd = (double*)malloc(sizeof(double) * (size_t)n);
    double* pe = (double*)malloc(sizeof(double) * (size_t)n);
    for (int64_t a = 0; a < n; ++a) {
        double y = (double)S[a] * (double)C[a] - (double)m;
        pe[a] = exp2(y);
        pd[a] = orc_round_bf16(pe[a]);
        l += pd[a];
        const uint16_t* vr = vh + U[a] * D;
        for (int64_t e = 0; e < D; ++e) acc[e] += pd[a] * (double)orc_bf16_to_f32(vr[e]);
    }
    if (c->o_decl)
        for (int64_t e = 0; e < D; ++e) c->o_decl[r * D + e] = acc[e] / l;
    if (c->amb) {
        double xabs_max = 0.0;
        for (int64_t a = 0; a < n; ++a) {
            double xa = fabs((double)((float)S[a] * C[a]));
            if (xa > xabs_max) xabs_max = xa;
        }
        double bound = 0.0;
        for (int64_t a = 0; a < n; ++a) {
            double xa = fabs((double)((float)S[a] * C[a]));
            double ulp = orc_p_ambiguous(pe[a], xa, xabs_max, (double)m);
            if (ulp > 0.0) {
                const uint16_t* vr = vh + U[a] * D;
                double dv = 0.0;
                for (int64_t e = 0; e < D; ++e) {
                    double dd = fabs((double)orc_bf16_to_f32(vr[e]) - acc[e] / l);
                    if (dd > dv) dv = dd;
                }
                bound += ulp * dv / l;
            }
        }
        c->amb[r] = bound;
    }
    /* exact arithmetic */
    if (c->o_exact) {
        double smax = -INFINITY;
        for (int64_t a = 0; a < n; ++a)
            if (se[a] > smax) smax = se[a];
        double l2 = 0.0;
        for (int64_t a = 0; a < n; ++a) {
            double p = exp(se[a] - smax);
            l2 += p;
            const uint16_t* vr = vh + U[a] * D;
            for (int64_t e = 0; e < D; ++e) acc2[e] += p * (double)orc_bf16_to_f32(vr[e]);
        }
        for (int64_t e = 0; e < D; ++e) c->o_exact[r * D + e] = acc2[e] / l2;
    }
    free(pd);
    free(pe);
    free(S);
    free(U);
    free(C);
    free(se);
    free(acc);
    free(acc2);
}

static float default_sm(float sm, int64_t D) {
    return sm > 0.0f ? sm : (float)(1.0 / sqrt((double)D));
}

void orc_sparse_rows(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                     const float* k_scale, const uint16_t* v, int64_t N, int64_t D,
                     int64_t bh, const int32_t* kidx_head, int64_t keep, float sm_scale,
                     const int64_t* tokens, int64_t R, double* o_decl, double* o_exact,
                     double* amb, int nthreads) {
    sparse_ctx c;
    c.q_i8 = q_i8;
    c.q_scale = q_scale;
    c.k_i8 = k_i8;
    c.k_scale = k_scale;
    c.v = v;
    c.N = N;
    c.D = D;
    c.bh = bh;
    c.nqb = orc_nqb(N);
    c.nkb = orc_nkb(N);
    c.keep = keep;
    c.kidx = kidx_head;
    c.sm = default_sm(sm_scale, D);
    c.K32 = (float)((double)c.sm * 1.4426950408889634074);
    c.tokens = tokens;
    c.o_decl = o_decl;
    c.o_exact = o_exact;
    c.amb = amb;
    orc_parallel_for(R, nthreads, sparse_task, &c);
}

/* ------------------------------------------------------------------------ */
/* Linear branch (page 5, "The Four Technical Pillars", Pillar Two: the      */
/* interactions the sparse part skips are covered by a cheap linear         */
/* attention over the whole sequence). Reading: feature                     */
/* map phi = elu + 1, no softmax scale, no learned projection; for a query   */
/* block the states are summed over exactly the key blocks it did not keep. */

static double phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

typedef struct {
    const uint16_t *k, *v;
    int64_t N, D, bh;
    double *h, *z;
} lstate_ctx;

static void lstate_task(void* vctx, int64_t j) {
    lstate_ctx* c = (lstate_ctx*)vctx;
    int64_t N = c->N, D = c->D;
    double* hj = c->h + j * D * D;
    double* zj = c->z + j * D;
    memset(hj, 0, sizeof(double) * (size_t)(D * D));
    memset(zj, 0, sizeof(double) * (size_t)D);
    int64_t u1 = (j + 1) * ORC_KBLK < N ? (j + 1) * ORC_KBLK : N;
    for (int64_t u = j * ORC_KBLK; u < u1; ++u) {
        const uint16_t* kr = c->k + (c->bh * N + u) * D;
        const uint16_t* vr = c->v + (c->bh * N + u) * D;
        for (int64_t d = 0; d < D; ++d) {
            double f = phi((double)orc_bf16_to_f32(kr[d]));
            zj[d] += f;
            for (int64_t e = 0; e < D; ++e) hj[d * D + e] += f * (double)orc_bf16_to_f32(vr[e]);
        }
    }
}

void orc_linear_states(const uint16_t* k, const uint16_t* v, int64_t N, int64_t D,
                       int64_t bh, double* h, double* z, int nthreads) {
    lstate_ctx c = {k, v, N, D, bh, h, z};
    orc_parallel_for(orc_nkb(N), nthreads, lstate_task, &c);
}

typedef struct {
    const uint16_t* q;
    int64_t N, D, bh, nkb, keep;
    const double *h, *z;
    const int32_t* kidx;
    const int64_t* tokens;
    int64_t R;
    const int64_t* blocks; /* distinct query blocks */
    double* o;
} lrows_ctx;

static void lrows_task(void* vctx, int64_t bi) {
    lrows_ctx* c = (lrows_ctx*)vctx;
    int64_t D = c->D, N = c->N, i = c->blocks[bi];
    if (!c->kidx || c->keep >= c->nkb) {
        for (int64_t r = 0; r < c->R; ++r)
            if (c->tokens[r] / ORC_QBLK == i)
                for (int64_t e = 0; e < D; ++e) c->o[r * D + e] = 0.0;
        return;
    }
    uint8_t* kept = (uint8_t*)calloc((size_t)c->nkb, 1);
    for (int64_t a = 0; a < c->keep; ++a) kept[c->kidx[i * c->keep + a]] = 1;
    double* H = (double*)calloc((size_t)(D * D), sizeof(double));
    double* zc = (double*)calloc((size_t)D, sizeof(double));
    for (int64_t j = 0; j < c->nkb; ++j) {
        if (kept[j]) continue;
        const double* hj = c->h + j * D * D;
        for (int64_t x = 0; x < D * D; ++x) H[x] += hj[x];
        for (int64_t d = 0; d < D; ++d) zc[d] += c->z[j * D + d];
    }
    double* fq = (double*)malloc(sizeof(double) * (size_t)D);
    for (int64_t r = 0; r < c->R; ++r) {
        int64_t t = c->tokens[r];
        if (t / ORC_QBLK != i) continue;
        const uint16_t* qr = c->q + (c->bh * N + t) * D;
        for (int64_t d = 0; d < D; ++d) fq[d] = phi((double)orc_bf16_to_f32(qr[d]));
        double den = 0.0;
        for (int64_t d = 0; d < D; ++d) den += fq[d] * zc[d];
        for (int64_t e = 0; e < D; ++e) {
            double num = 0.0;
            for (int64_t d = 0; d < D; ++d) num += fq[d] * H[d * D + e];
            c->o[r * D + e] = num / den;
        }
    }
    free(fq);
    free(H);
    free(zc);
    free(kept);
}

void orc_linear_rows(const uint16_t* q, int64_t N, int64_t D, int64_t bh,
                     const double* h, const double* z, const int32_t* kidx_head,
                     int64_t keep, const int64_t* tokens, int64_t R, double* o_lin,
                     int nthreads) {
    int64_t nqb = orc_nqb(N);
    uint8_t* seen = (uint8_t*)calloc((size_t)nqb, 1);
    int64_t* blocks = (int64_t*)malloc(sizeof(int64_t) * (size_t)(R > 0 ? R : 1));
    int64_t nb = 0;
    for (int64_t r = 0; r < R; ++r) {
        int64_t i = tokens[r] / ORC_QBLK;
        if (!seen[i]) {
            seen[i] = 1;
            blocks[nb++] = i;
        }
    }
    lrows_ctx c = {q, N, D, bh, orc_nkb(N), keep, h, z, kidx_head, tokens, R, blocks, o_lin};
    orc_parallel_for(nb, nthreads, lrows_task, &c);
    free(seen);
    free(blocks);
}

/* ------------------------------------------------------------------------ */
/* fp64 dense softmax attention on the unquantized inputs                   */

typedef struct {
    const uint16_t *q, *k, *v;
    int64_t N, D, bh;
    double sm;
    const int64_t* tokens;
    double* out;
} dense_ctx;

static void dense_task(void* vctx, int64_t r) {
    dense_ctx* c = (dense_ctx*)vctx;
    int64_t N = c->N, D = c->D, t = c->tokens[r];
    const uint16_t* qr = c->q + (c->bh * N + t) * D;
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    double* acc = (double*)calloc((size_t)D, sizeof(double));
    double smax = -INFINITY;
    for (int64_t u = 0; u < N; ++u) {
        const uint16_t* kr = c->k + (c->bh * N + u) * D;
        double a = 0.0;
        for (int64_t d = 0; d < D; ++d)
            a += (double)orc_bf16_to_f32(qr[d]) * (double)orc_bf16_to_f32(kr[d]);
        s[u] = a * c->sm;
        if (s[u] > smax) smax = s[u];
    }
    double l = 0.0;
    for (int64_t u = 0; u < N; ++u) {
        double p = exp(s[u] - smax);
        l += p;
        const uint16_t* vr = c->v + (c->bh * N + u) * D;
        for (int64_t e = 0; e < D; ++e) acc[e] += p * (double)orc_bf16_to_f32(vr[e]);
    }
    for (int64_t e = 0; e < D; ++e) c->out[r * D + e] = acc[e] / l;
    free(s);
    free(acc);
}

void orc_dense_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t N,
                    int64_t D, int64_t bh, float sm_scale, const int64_t* tokens, int64_t R,
                    double* out, int nthreads) {
    dense_ctx c = {q, k, v, N, D, bh, (double)default_sm(sm_scale, D), tokens, out};
    orc_parallel_for(R, nthreads, dense_task, &c);
}

/* ------------------------------------------------------------------------ */
/* W8A8 linear layer (page 5, "Four Technical Pillars", Pillar Three: INT8  */
/* weights and activations, quantized with a block-wise granularity of     */
/* 128x128).                                                                */

typedef struct {
    const uint16_t* x;
    int64_t rows, cols, nrb, ncb;
    int8_t* q;
    float* scale;
} w8_quant_ctx;

/* One 128 x 128 block: the Pillar One rule of orc_quant over the block's
 * valid rows (a partial last row block) and its 128 columns. */
static void w8_quant_task(void* vctx, int64_t idx) {
    w8_quant_ctx* c = (w8_quant_ctx*)vctx;
    int64_t rb = idx / c->ncb, cb = idx % c->ncb;
    int64_t r0 = rb * ORC_W8_BLK, r1 = r0 + ORC_W8_BLK < c->rows ? r0 + ORC_W8_BLK : c->rows;
    int64_t c0 = cb * ORC_W8_BLK;
    float amax = 0.0f;
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t k = c0; k < c0 + ORC_W8_BLK; ++k) {
            float a = fabsf(orc_bf16_to_f32(c->x[r * c->cols + k]));
            if (a > amax) amax = a;
        }
    float s = amax / 127.0f;
    c->scale[rb * c->ncb + cb] = s;
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t k = c0; k < c0 + ORC_W8_BLK; ++k) {
            int8_t q = 0;
            if (s > 0.0f) {
                /* the clamp as in the attention quantizer (NaN -> -127) */
                const float v =
                    fminf(fmaxf(rintf(orc_bf16_to_f32(c->x[r * c->cols + k]) / s), -127.0f), 127.0f);
                q = (int8_t)v;
            }
            c->q[r * c->cols + k] = q;
        }
}

void orc_w8a8_quant(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                    int nthreads) {
    w8_quant_ctx c = {x, rows, cols, (rows + ORC_W8_BLK - 1) / ORC_W8_BLK, cols / ORC_W8_BLK, q,
                      scale};
    orc_parallel_for(c.nrb * c.ncb, nthreads, w8_quant_task, &c);
}

typedef struct {
    const int8_t *xq, *wq;
    const float *sx, *sw, *bias;
    int64_t M, N, K;
    const int64_t* rows;
    float* y;
} w8_gemm_ctx;

/* One output row: for each column n, the exact int32 sum of each 128-wide
 * column block kb of K, then y = fmaf((float)I_kb, s_kb, y) in ascending kb
 * from 0, s_kb = fl32(sx[mb][kb] * sw[nb][kb]); then y = fl32(y + bias[n])
 * when the layer has a bias. */
static void w8_gemm_task(void* vctx, int64_t r) {
    w8_gemm_ctx* c = (w8_gemm_ctx*)vctx;
    int64_t m = c->rows[r], nkb = c->K / ORC_W8_BLK, mb = m / ORC_W8_BLK;
    const int8_t* xr = c->xq + m * c->K;
    for (int64_t n = 0; n < c->N; ++n) {
        const int8_t* wr = c->wq + n * c->K;
        int64_t nb = n / ORC_W8_BLK;
        float y = 0.0f;
        for (int64_t kb = 0; kb < nkb; ++kb) {
            int32_t acc = 0;
            for (int64_t k = kb * ORC_W8_BLK; k < (kb + 1) * ORC_W8_BLK; ++k)
                acc += (int32_t)xr[k] * (int32_t)wr[k];
            float s = c->sx[mb * nkb + kb] * c->sw[nb * nkb + kb];
            y = fmaf((float)acc, s, y);
        }
        if (c->bias) y = y + c->bias[n];
        c->y[r * c->N + n] = y;
    }
}

void orc_w8a8_gemm(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                   const float* bias, int64_t M, int64_t N, int64_t K, const int64_t* rows,
                   int64_t R, float* y, int nthreads) {
    w8_gemm_ctx c = {xq, wq, sx, sw, bias, M, N, K, rows, y};
    orc_parallel_for(R, nthreads, w8_gemm_task, &c);
}

/* The same product with the dequantization carried in fp64 (the plainest
 * exact reading of Pillar Three's block dequantization): y64 = sum over kb of
 * (double)I_kb * (double)sx * (double)sw, plus the bias; yabs = sum over kb of
 * |I_kb| * sx * sw, the scale of the terms (for error bounds). */
typedef struct {
    const int8_t *xq, *wq;
    const float *sx, *sw, *bias;
    int64_t M, N, K;
    const int64_t* rows;
    double *y, *yabs;
} w8_f64_ctx;

static void w8_f64_task(void* vctx, int64_t r) {
    w8_f64_ctx* c = (w8_f64_ctx*)vctx;
    int64_t m = c->rows[r], nkb = c->K / ORC_W8_BLK, mb = m / ORC_W8_BLK;
    const int8_t* xr = c->xq + m * c->K;
    for (int64_t n = 0; n < c->N; ++n) {
        const int8_t* wr = c->wq + n * c->K;
        int64_t nb = n / ORC_W8_BLK;
        double y = 0.0, ya = 0.0;
        for (int64_t kb = 0; kb < nkb; ++kb) {
            int64_t acc = 0;
            for (int64_t k = kb * ORC_W8_BLK; k < (kb + 1) * ORC_W8_BLK; ++k)
                acc += (int64_t)xr[k] * (int64_t)wr[k];
            double s = (double)c->sx[mb * nkb + kb] * (double)c->sw[nb * nkb + kb];
            y += (double)acc * s;
            ya += fabs((double)acc) * s;
        }
        if (c->bias) y += (double)c->bias[n];
        c->y[r * c->N + n] = y;
        c->yabs[r * c->N + n] = ya;
    }
}

void orc_w8a8_gemm_f64(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                       const float* bias, int64_t M, int64_t N, int64_t K, const int64_t* rows,
                       int64_t R, double* y, double* yabs, int nthreads) {
    w8_f64_ctx c = {xq, wq, sx, sw, bias, M, N, K, rows, y, yabs};
    orc_parallel_for(R, nthreads, w8_f64_task, &c);
}

/* ------------------------------------------------------------------------ */
/* SageSLA backward (page 5, "What is TurboDiffusion?" and the training      */
/* guide: the sparse-linear attention is trainable and is fine-tuned). The   */
/* pages do not say how gradients pass the 8-bit quantizer. Reading: the     */
/* quantizer is a straight-through estimator (its derivative is taken as the */
/* identity), the block selection is held fixed (it is piecewise constant),  */
/* and the gradient is the exact derivative of the forward as a function of  */
/* the dequantized operands qh = sq * q_i8, kh = sk * k_i8 (sparse branch)   */
/* and of the raw bf16 Q, K (linear branch), evaluated at the forward's      */
/* values; V enters both branches directly. dQ and dK collect both branches. */
/* The K mean needs no term: moving every key of a row by the same vector    */
/* moves every score of the row by the same amount, so the softmax ignores  */
/* it (the rows of dS sum to zero).                                          */
/* Everything is fp64. Sparse branch, with s = sm * qh . kh over the kept    */
/* keys u of a query t, P = softmax(s), dP_tu = dO_t . v_u,                  */
/* Dt = sum_u P_tu dP_tu, dS_tu = P_tu (dP_tu - Dt):                          */
/*   dq_t += sm sum_u dS_tu kh_u, dk_u += sm sum_t dS_tu qh_t,               */
/*   dv_u += sum_t P_tu dO_t.                                                */
/* Linear branch, with a = phi(q_t), H, z the sums over the non-kept blocks, */
/* den = a . z, o_l = a^T H / den, g = dO_t:                                 */
/*   dnum = g / den, dden = -(g . o_l) / den,                                */
/*   dq_t += (H dnum + z dden) * phi'(q_t),                                  */
/*   G_i = sum_{t in i} a dnum^T, w_i = sum_{t in i} a dden,                 */
/*   for a key u of block j, with Gc, wc the sums of G_i, w_i over the query */
/*   blocks i that did NOT keep j:                                           */
/*   dk_u += (Gc v_u + wc) * phi'(k_u), dv_u += Gc^T phi(k_u);               */
/* phi'(x) = 1 for x > 0, e^x otherwise.                                     */

static double dphi(double x) { return x > 0.0 ? 1.0 : exp(x); }

/* does query block i keep key block j (kidx_head NULL: dense, all kept) */
static int kept_by(const int32_t* kidx, int64_t keep, int64_t i, int64_t j) {
    if (!kidx) return 1;
    for (int64_t a = 0; a < keep; ++a)
        if (kidx[i * keep + a] == j) return 1;
    return 0;
}

typedef struct {
    const int8_t *q_i8, *k_i8;
    const float *q_scale, *k_scale;
    const uint16_t *v, *dout;
    int64_t N, D, bh, nqb, nkb, keep;
    const uint8_t* kept;        /* [nqb][nkb]: 1 where query block i keeps key block j */
    const uint8_t* need_stats;  /* [N]: rows whose statistics are needed */
    const uint8_t *qsel, *ksel; /* [N] or NULL (every row): rows of dq, keys of dk and dv */
    double sm;
    double *rmax, *rsum, *rD; /* per query row */
    double *dq, *dk, *dv;
} sbwd_ctx;

/* exact score s_tu (fp64) */
static double sb_score(const sbwd_ctx* c, int64_t t, int64_t u) {
    const int8_t* qr = c->q_i8 + (c->bh * c->N + t) * c->D;
    const int8_t* kr = c->k_i8 + (c->bh * c->N + u) * c->D;
    int64_t S = 0;
    for (int64_t d = 0; d < c->D; ++d) S += (int64_t)qr[d] * (int64_t)kr[d];
    return (double)S * (double)c->q_scale[c->bh * c->nqb + t / ORC_QBLK] *
           (double)c->k_scale[c->bh * c->nkb + u / ORC_KBLK] * c->sm;
}

static double sb_dp(const sbwd_ctx* c, int64_t t, int64_t u) {
    const uint16_t* gr = c->dout + (c->bh * c->N + t) * c->D;
    const uint16_t* vr = c->v + (c->bh * c->N + u) * c->D;
    double a = 0.0;
    for (int64_t e = 0; e < c->D; ++e)
        a += (double)orc_bf16_to_f32(gr[e]) * (double)orc_bf16_to_f32(vr[e]);
    return a;
}

/* pass 1 (per query row t): softmax statistics, D_t and dq_t. The row's
 * scores and dP over its kept keys are formed once and reused by the later
 * sweeps, which take them in the same order (j, then u, ascending). */
static void sbwd_rows_task(void* vctx, int64_t t) {
    sbwd_ctx* c = (sbwd_ctx*)vctx;
    if (!c->need_stats[t]) return;
    int64_t N = c->N, D = c->D, i = t / ORC_QBLK;
    const uint8_t* kept = c->kept + i * c->nkb;
    int64_t nk = 0;
    for (int64_t j = 0; j < c->nkb; ++j)
        if (kept[j]) nk += ((j + 1) * ORC_KBLK < N ? (j + 1) * ORC_KBLK : N) - j * ORC_KBLK;
    double* sv = (double*)malloc(sizeof(double) * (size_t)(2 * nk));
    double* dpv = sv + nk;
    double m = -INFINITY;
    int64_t x = 0;
    for (int64_t j = 0; j < c->nkb; ++j) {
        if (!kept[j]) continue;
        int64_t u1 = (j + 1) * ORC_KBLK < N ? (j + 1) * ORC_KBLK : N;
        for (int64_t u = j * ORC_KBLK; u < u1; ++u, ++x) {
            sv[x] = sb_score(c, t, u);
            dpv[x] = sb_dp(c, t, u);
            if (sv[x] > m) m = sv[x];
        }
    }
    double l = 0.0, Dt = 0.0;
    for (x = 0; x < nk; ++x) l += exp(sv[x] - m);
    for (x = 0; x < nk; ++x) Dt += exp(sv[x] - m) / l * dpv[x];
    c->rmax[t] = m;
    c->rsum[t] = l;
    c->rD[t] = Dt;
    if (!c->qsel || c->qsel[t]) {
        double* dq = c->dq + t * D;
        x = 0;
        for (int64_t j = 0; j < c->nkb; ++j) {
            if (!kept[j]) continue;
            double sk = (double)c->k_scale[c->bh * c->nkb + j];
            int64_t u1 = (j + 1) * ORC_KBLK < N ? (j + 1) * ORC_KBLK : N;
            for (int64_t u = j * ORC_KBLK; u < u1; ++u, ++x) {
                double P = exp(sv[x] - m) / l;
                double dS = P * (dpv[x] - Dt);
                const int8_t* kr = c->k_i8 + (c->bh * N + u) * D;
                for (int64_t d = 0; d < D; ++d) dq[d] += c->sm * dS * sk * (double)kr[d];
            }
        }
    }
    free(sv);
}

/* pass 2 (per key u): dk_u and dv_u over the queries whose block kept u's */
static void sbwd_keys_task(void* vctx, int64_t u) {
    sbwd_ctx* c = (sbwd_ctx*)vctx;
    if (c->ksel && !c->ksel[u]) return;
    int64_t N = c->N, D = c->D, j = u / ORC_KBLK;
    double* dk = c->dk + u * D;
    double* dv = c->dv + u * D;
    for (int64_t i = 0; i < c->nqb; ++i) {
        if (!c->kept[i * c->nkb + j]) continue;
        double sq = (double)c->q_scale[c->bh * c->nqb + i];
        int64_t t1 = (i + 1) * ORC_QBLK < N ? (i + 1) * ORC_QBLK : N;
        for (int64_t t = i * ORC_QBLK; t < t1; ++t) {
            double P = exp(sb_score(c, t, u) - c->rmax[t]) / c->rsum[t];
            double dS = P * (sb_dp(c, t, u) - c->rD[t]);
            const int8_t* qr = c->q_i8 + (c->bh * N + t) * D;
            const uint16_t* gr = c->dout + (c->bh * N + t) * D;
            for (int64_t d = 0; d < D; ++d) {
                dk[d] += c->sm * dS * sq * (double)qr[d];
                dv[d] += P * (double)orc_bf16_to_f32(gr[d]);
            }
        }
    }
}

typedef struct {
    const uint16_t *q, *k, *v, *dout;
    int64_t N, D, bh, nqb, nkb, keep;
    const uint8_t* kept;   /* [nqb][nkb] */
    const uint8_t* ksel;   /* [N] or NULL: keys of dk and dv */
    const double *h, *z; /* per key block states */
    double *G, *w;       /* per query block [D][D], [D] */
    double *dq, *dk, *dv;
} lbwd_ctx;

/* per query block i: dq (linear part), G_i, w_i */
static void lbwd_q_task(void* vctx, int64_t i) {
    lbwd_ctx* c = (lbwd_ctx*)vctx;
    int64_t N = c->N, D = c->D;
    double* H = (double*)calloc((size_t)(D * D), sizeof(double));
    double* z = (double*)calloc((size_t)D, sizeof(double));
    int64_t ncomp = 0;
    for (int64_t j = 0; j < c->nkb; ++j) {
        if (c->kept[i * c->nkb + j]) continue;
        ++ncomp;
        for (int64_t x = 0; x < D * D; ++x) H[x] += c->h[j * D * D + x];
        for (int64_t d = 0; d < D; ++d) z[d] += c->z[j * D + d];
    }
    double* G = c->G + i * D * D;
    double* w = c->w + i * D;
    memset(G, 0, sizeof(double) * (size_t)(D * D));
    memset(w, 0, sizeof(double) * (size_t)D);
    if (ncomp > 0) {
        double* a = (double*)malloc(sizeof(double) * (size_t)D);
        double* ol = (double*)malloc(sizeof(double) * (size_t)D);
        double* dnum = (double*)malloc(sizeof(double) * (size_t)D);
        int64_t t1 = (i + 1) * ORC_QBLK < N ? (i + 1) * ORC_QBLK : N;
        for (int64_t t = i * ORC_QBLK; t < t1; ++t) {
            const uint16_t* qr = c->q + (c->bh * N + t) * D;
            const uint16_t* gr = c->dout + (c->bh * N + t) * D;
            double den = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                a[d] = phi((double)orc_bf16_to_f32(qr[d]));
                den += a[d] * z[d];
            }
            double go = 0.0;
            for (int64_t e = 0; e < D; ++e) {
                double num = 0.0;
                for (int64_t d = 0; d < D; ++d) num += a[d] * H[d * D + e];
                ol[e] = num / den;
                go += (double)orc_bf16_to_f32(gr[e]) * ol[e];
            }
            double dden = -go / den;
            for (int64_t e = 0; e < D; ++e) dnum[e] = (double)orc_bf16_to_f32(gr[e]) / den;
            for (int64_t d = 0; d < D; ++d) {
                double da = z[d] * dden;
                for (int64_t e = 0; e < D; ++e) da += H[d * D + e] * dnum[e];
                c->dq[t * D + d] += da * dphi((double)orc_bf16_to_f32(qr[d]));
                for (int64_t e = 0; e < D; ++e) G[d * D + e] += a[d] * dnum[e];
                w[d] += a[d] * dden;
            }
        }
        free(a);
        free(ol);
        free(dnum);
    }
    free(H);
    free(z);
}

/* per key block j: dk, dv (linear part) of its keys */
static void lbwd_k_task(void* vctx, int64_t j) {
    lbwd_ctx* c = (lbwd_ctx*)vctx;
    int64_t N = c->N, D = c->D;
    int64_t u0 = j * ORC_KBLK, u1 = (j + 1) * ORC_KBLK < N ? (j + 1) * ORC_KBLK : N;
    if (c->ksel) {
        int any = 0;
        for (int64_t u = u0; u < u1; ++u) any |= c->ksel[u];
        if (!any) return;
    }
    double* Gc = (double*)calloc((size_t)(D * D), sizeof(double));
    double* wc = (double*)calloc((size_t)D, sizeof(double));
    for (int64_t i = 0; i < c->nqb; ++i) {
        if (c->kept[i * c->nkb + j]) continue;
        for (int64_t x = 0; x < D * D; ++x) Gc[x] += c->G[i * D * D + x];
        for (int64_t d = 0; d < D; ++d) wc[d] += c->w[i * D + d];
    }
    double* f = (double*)malloc(sizeof(double) * (size_t)D);
    for (int64_t u = u0; u < u1; ++u) {
        if (c->ksel && !c->ksel[u]) continue;
        const uint16_t* kr = c->k + (c->bh * N + u) * D;
        const uint16_t* vr = c->v + (c->bh * N + u) * D;
        for (int64_t d = 0; d < D; ++d) f[d] = phi((double)orc_bf16_to_f32(kr[d]));
        for (int64_t d = 0; d < D; ++d) {
            double g = wc[d];
            for (int64_t e = 0; e < D; ++e) g += Gc[d * D + e] * (double)orc_bf16_to_f32(vr[e]);
            c->dk[u * D + d] += g * dphi((double)orc_bf16_to_f32(kr[d]));
        }
        for (int64_t e = 0; e < D; ++e) {
            double g = 0.0;
            for (int64_t d = 0; d < D; ++d) g += Gc[d * D + e] * f[d];
            c->dv[u * D + e] += g;
        }
    }
    free(f);
    free(Gc);
    free(wc);
}

void orc_sagesla_bwd_sel(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                         const float* k_scale, int64_t N, int64_t D, int64_t bh,
                         const int32_t* kidx_head, int64_t keep, int branches, float sm_scale,
                         const uint16_t* dout, const uint8_t* qsel, const uint8_t* ksel,
                         double* dq, double* dk, double* dv, int nthreads) {
    int64_t nqb = orc_nqb(N), nkb = orc_nkb(N);
    if (!kidx_head) keep = nkb;
    memset(dq, 0, sizeof(double) * (size_t)(N * D));
    memset(dk, 0, sizeof(double) * (size_t)(N * D));
    memset(dv, 0, sizeof(double) * (size_t)(N * D));
    /* the kept-block table, from kidx (every block when dense) */
    uint8_t* kept = (uint8_t*)malloc((size_t)(nqb * nkb));
    for (int64_t i = 0; i < nqb; ++i)
        for (int64_t j = 0; j < nkb; ++j) kept[i * nkb + j] = (uint8_t)kept_by(kidx_head, keep, i, j);
    if (branches & 1) {
        /* statistics are needed for the selected rows and for every row of a
         * query block that keeps the block of a selected key */
        uint8_t* need = (uint8_t*)malloc((size_t)N);
        uint8_t* kbsel = (uint8_t*)calloc((size_t)nkb, 1);
        for (int64_t u = 0; u < N; ++u)
            if (!ksel || ksel[u]) kbsel[u / ORC_KBLK] = 1;
        for (int64_t i = 0; i < nqb; ++i) {
            uint8_t blk = 0;
            for (int64_t j = 0; j < nkb && !blk; ++j) blk = kept[i * nkb + j] && kbsel[j];
            int64_t t1 = (i + 1) * ORC_QBLK < N ? (i + 1) * ORC_QBLK : N;
            for (int64_t t = i * ORC_QBLK; t < t1; ++t) need[t] = blk || !qsel || qsel[t];
        }
        sbwd_ctx c;
        c.q_i8 = q_i8;
        c.k_i8 = k_i8;
        c.q_scale = q_scale;
        c.k_scale = k_scale;
        c.v = v;
        c.dout = dout;
        c.N = N;
        c.D = D;
        c.bh = bh;
        c.nqb = nqb;
        c.nkb = nkb;
        c.keep = keep;
        c.kept = kept;
        c.need_stats = need;
        c.qsel = qsel;
        c.ksel = ksel;
        c.sm = (double)default_sm(sm_scale, D);
        c.rmax = (double*)malloc(sizeof(double) * (size_t)N);
        c.rsum = (double*)malloc(sizeof(double) * (size_t)N);
        c.rD = (double*)malloc(sizeof(double) * (size_t)N);
        c.dq = dq;
        c.dk = dk;
        c.dv = dv;
        orc_parallel_for(N, nthreads, sbwd_rows_task, &c);
        orc_parallel_for(N, nthreads, sbwd_keys_task, &c);
        free(c.rmax);
        free(c.rsum);
        free(c.rD);
        free(need);
        free(kbsel);
    }
    if ((branches & 2) && kidx_head && keep < nkb) {
        double* h = (double*)malloc(sizeof(double) * (size_t)(nkb * D * D));
        double* z = (double*)malloc(sizeof(double) * (size_t)(nkb * D));
        orc_linear_states(k, v, N, D, bh, h, z, nthreads);
        lbwd_ctx c = {q, k, v, dout, N, D, bh, nqb, nkb, keep, kept, ksel, h, z, NULL, NULL,
                      dq, dk, dv};
        c.G = (double*)malloc(sizeof(double) * (size_t)(nqb * D * D));
        c.w = (double*)malloc(sizeof(double) * (size_t)(nqb * D));
        orc_parallel_for(nqb, nthreads, lbwd_q_task, &c);
        orc_parallel_for(nkb, nthreads, lbwd_k_task, &c);
        free(c.G);
        free(c.w);
        free(h);
        free(z);
    }
    free(kept);
}

void orc_sagesla_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int8_t* q_i8,
                     const float* q_scale, const int8_t* k_i8, const float* k_scale, int64_t N,
                     int64_t D, int64_t bh, const int32_t* kidx_head, int64_t keep, int branches,
                     float sm_scale, const uint16_t* dout, double* dq, double* dk, double* dv,
                     int nthreads) {
    orc_sagesla_bwd_sel(q, k, v, q_i8, q_scale, k_i8, k_scale, N, D, bh, kidx_head, keep, branches,
                        sm_scale, dout, NULL, NULL, dq, dk, dv, nthreads);
}

/* The scalar loss L = sum_{t,e} dO_te O_te of the SageSLA forward written
 * for continuous inputs, fp64: qh, kh feed the sparse branch (exact softmax
 * of sm * qh . kh over the kept keys, no quantization), ql, kl the linear
 * branch, vv both. One head, rows [N][D]. Its central differences pin
 * orc_sagesla_bwd: dQ = dL/dqh + dL/dql at equal positions (the straight-
 * through reading), likewise dK; dV = dL/dvv. */
double orc_sagesla_loss(const double* qh, const double* kh, const double* vv, const double* ql,
                        const double* kl, int64_t N, int64_t D, const int32_t* kidx_head,
                        int64_t keep, int branches, double sm, const double* dout) {
    int64_t nqb = orc_nqb(N), nkb = orc_nkb(N);
    if (!kidx_head) keep = nkb;
    double L = 0.0;
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    double* o = (double*)malloc(sizeof(double) * (size_t)D);
    double* a = (double*)malloc(sizeof(double) * (size_t)D);
    double* H = (double*)malloc(sizeof(double) * (size_t)(D * D));
    double* z = (double*)malloc(sizeof(double) * (size_t)D);
    for (int64_t i = 0; i < nqb; ++i) {
        int64_t t1 = (i + 1) * ORC_QBLK < N ? (i + 1) * ORC_QBLK : N;
        const int lin = (branches & 2) && kidx_head && keep < nkb;
        if (lin) { /* the query block's states: sums over its non-kept keys */
            for (int64_t x = 0; x < D * D; ++x) H[x] = 0.0;
            for (int64_t d = 0; d < D; ++d) z[d] = 0.0;
            for (int64_t u = 0; u < N; ++u) {
                if (kept_by(kidx_head, keep, i, u / ORC_KBLK)) continue;
                for (int64_t d = 0; d < D; ++d) {
                    double f = phi(kl[u * D + d]);
                    z[d] += f;
                    for (int64_t e = 0; e < D; ++e) H[d * D + e] += f * vv[u * D + e];
                }
            }
        }
        for (int64_t t = i * ORC_QBLK; t < t1; ++t) {
            if (branches & 1) {
                double m = -INFINITY;
                for (int64_t u = 0; u < N; ++u) {
                    if (!kept_by(kidx_head, keep, i, u / ORC_KBLK)) continue;
                    double acc = 0.0;
                    for (int64_t d = 0; d < D; ++d) acc += qh[t * D + d] * kh[u * D + d];
                    s[u] = sm * acc;
                    if (s[u] > m) m = s[u];
                }
                double l = 0.0;
                for (int64_t e = 0; e < D; ++e) o[e] = 0.0;
                for (int64_t u = 0; u < N; ++u) {
                    if (!kept_by(kidx_head, keep, i, u / ORC_KBLK)) continue;
                    double p = exp(s[u] - m);
                    l += p;
                    for (int64_t e = 0; e < D; ++e) o[e] += p * vv[u * D + e];
                }
                for (int64_t e = 0; e < D; ++e) L += dout[t * D + e] * o[e] / l;
            }
            if (lin) {
                double den = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    a[d] = phi(ql[t * D + d]);
                    den += a[d] * z[d];
                }
                for (int64_t e = 0; e < D; ++e) {
                    double num = 0.0;
                    for (int64_t d = 0; d < D; ++d) num += a[d] * H[d * D + e];
                    L += dout[t * D + e] * num / den;
                }
            }
        }
    }
    free(s);
    free(o);
    free(a);
    free(H);
    free(z);
    return L;
}
