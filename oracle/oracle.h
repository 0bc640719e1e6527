/*
 * oracle.h -- plain, slow CPU reference for the SageSLA attention path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke entry and the
 * bench's CPU-baseline leg may load this library. The product path (the HIP
 * library under bit_sparse_attention_amd/) never calls it and shares no code
 * with it.
 *
 * What it computes (TurboDiffusion pages; page 5 "Four Technical Pillars",
 * Pillar One (SageAttention: INT8 attention with smoothing of outliers) and
 * Pillar Two (SLA: a small set of important block interactions computed
 * exactly, the others through a cheap linear-attention term, 10% of connections kept
 * at --sla_topk 0.1), and the "Hands-On Tutorial" flags):
 *
 *   K mean smoothing, per-block INT8 quantization of Q (128-token blocks) and
 *   of the smoothed K (64-token blocks) with fp32 scale max|x|/127 and
 *   round-half-even; int32 Q.K^T; the block mask from mean-pooled Q.K block
 *   scores; the sparse softmax branch over the kept blocks; the elu+1 linear
 *   branch over the other blocks; their sum.
 *
 * And, from Pillar Three (INT8 weights and activations in the linear layers,
 * block-wise 128x128): the block quantization of both operands and the
 * block-dequantized INT8 product y = x . w^T.
 *
 * Conventions: bf16 values travel as uint16_t bit patterns. Tensors are
 * row-major [BH][N][D] with D fastest (BH = B*H flattened). Query blocks are
 * 128 tokens, key blocks 64 tokens; the last block of each may be partial.
 * Every floating-point step whose precision the method fixes (fp32 scales,
 * fp32 means and scores) is done in fp32 in a pinned order; everything else
 * is fp64.
 */
#ifndef SSA_ORACLE_H
#define SSA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_QBLK 128
#define ORC_KBLK 64

int64_t orc_nqb(int64_t N);                 /* ceil(N/128) */
int64_t orc_nkb(int64_t N);                 /* ceil(N/64) */
int64_t orc_keep(int64_t N, double topk);   /* clamp(floor(topk*Nkb + 0.5), 1, Nkb) */

/* bf16 helpers (exposed so tests can pin them against an independent
 * conversion). */
float  orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float x);          /* round to nearest, ties to even */
double orc_round_bf16(double x);            /* RNE of a double straight to bf16 */

/* K mean (smoothing): mu[bh][d] = (sum over 64-token blocks j, ascending, of
 * (sum over the tokens of block j, ascending, of fp32 K)) / (float)N, every
 * add in fp32 starting from 0. */
void orc_k_mean(const uint16_t* k, int64_t BH, int64_t N, int64_t D, float* mu);

/* Per-block INT8 quantization. blk = 128 (Q, mu = NULL) or 64 (K, mu = the
 * K mean, subtracted in fp32 first). scale = amax/127 (fp32 division),
 * q = clamp(rint(x/scale), -127, 127); amax = 0 gives scale 0 and q = 0. */
void orc_quant(const uint16_t* x, const float* mu, int64_t BH, int64_t N, int64_t D,
               int64_t blk, int8_t* xq, float* scale, int nthreads);

/* Raw int32 score tile (query block i, key block j) of head bh:
 * tile[r][c] = sum_d q[128i+r][d] * k[64j+c][d], 0 outside valid tokens. */
void orc_qk_tile(const int8_t* q_i8, const int8_t* k_i8, int64_t N, int64_t D,
                 int64_t bh, int64_t i, int64_t j, int32_t* tile /*[128][64]*/);

/* Mean-pooled block means of raw bf16 Q (128-token blocks) or K (64-token
 * blocks): fp32 sequential sum over the block's valid tokens, divided by the
 * valid count. out: [nblocks][D]. */
void orc_pool(const uint16_t* x, int64_t N, int64_t D, int64_t bh, int64_t blk, float* out);

/* Block scores for the listed query blocks of head bh:
 * score[r][j] = fmaf chain over d = 0..D-1 of qbar_i[d] * kbar_j[d], from 0. */
void orc_block_scores(const float* qbar, const float* kbar, int64_t Nkb, int64_t D,
                      const int64_t* qblocks, int64_t R, float* score /*[R][Nkb]*/);

/* Top-keep selection per score row: order by (score descending, j ascending),
 * keep the first `keep`, emit them in ascending j; mask[j] = 1 if kept. */
void orc_topk(const float* score, int64_t R, int64_t Nkb, int64_t keep,
              int32_t* kidx /*[R][keep]*/, uint8_t* mask /*[R][Nkb] or NULL*/);

/* Normalizer lag a GPU may have (reading C12): the GPU keeps an integer     */
/* normalizer that can sit up to this many log2 units below the row's       */
/* ceil(max) while it still yields the same rounded p up to a power of two.  */
#define ORC_NORM_LAG 64.0

/* Flip window of one rounded p (reading C12): p = 2^(x - m) evaluated       */
/* exactly, xa = |x|, xabs_max = max |x| of the row, m = ceil(max x). Returns */
/* the bf16 ulp at p when a GPU's fp32 evaluation may round p the other way, */
/* else 0. */
double orc_p_ambiguous(double p, double xa, double xabs_max, double m);

/* Sparse softmax branch for the listed tokens of head bh.
 * kidx_head: [Nqb][keep] ascending key blocks, or NULL for dense (keep == Nkb).
 * sm_scale <= 0 selects 1/sqrt(D).
 * o_decl: the declared numerics (integer-log2 normalizer, P rounded to bf16,
 *         row sum of the rounded P), everything else exact (fp64).
 * o_exact: fp64 softmax of the dequantized int32 scores, fp64 PV.
 * amb: per-token bound on how far a GPU may legitimately differ from o_decl
 *      because some rounded P sit within fp32 evaluation error of a bf16
 *      rounding midpoint. Any of the three may be NULL. */
void orc_sparse_rows(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                     const float* k_scale, const uint16_t* v, int64_t N, int64_t D,
                     int64_t bh, const int32_t* kidx_head, int64_t keep, float sm_scale,
                     const int64_t* tokens, int64_t R, double* o_decl, double* o_exact,
                     double* amb, int nthreads);

/* Linear-branch states of head bh, fp64: for key block j,
 * h[j][d][e] = sum_u phi(k_u[d]) v_u[e], z[j][d] = sum_u phi(k_u[d]),
 * phi(x) = x + 1 (x > 0) or exp(x) (x <= 0), on raw bf16 K. */
void orc_linear_states(const uint16_t* k, const uint16_t* v, int64_t N, int64_t D,
                       int64_t bh, double* h /*[Nkb][D][D]*/, double* z /*[Nkb][D]*/,
                       int nthreads);

/* Linear branch for the listed tokens: with H, zc the direct sums of h_j, z_j
 * over the key blocks NOT kept for the token's query block,
 * o_l[e] = sum_d phi(q[d]) H[d][e] / sum_d phi(q[d]) zc[d], or 0 when every
 * key block is kept. kidx_head as above (NULL: dense, o_l = 0). */
void orc_linear_rows(const uint16_t* q, int64_t N, int64_t D, int64_t bh,
                     const double* h, const double* z, const int32_t* kidx_head,
                     int64_t keep, const int64_t* tokens, int64_t R, double* o_lin,
                     int nthreads);

/* Plain fp64 dense softmax attention on the unquantized bf16 inputs (sanity
 * reference): o = softmax(q.K^T * sm) V over all N keys. */
void orc_dense_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t N,
                    int64_t D, int64_t bh, float sm_scale, const int64_t* tokens, int64_t R,
                    double* out, int nthreads);

/* SageSLA backward for head bh (page 5: SLA is trainable, fine-tuned in
 * training). Reading: the 8-bit quantizer passes gradients straight through,
 * the block selection is held fixed, and the gradient is the exact fp64
 * derivative of the forward in the dequantized operands (sparse branch:
 * exact softmax of sm * (sq q_i8) . (sk k_i8) over the kept keys) and the raw
 * bf16 Q, K (linear branch, phi = elu + 1 over the non-kept blocks); V feeds
 * both. dout: bf16 dL/dO [BH][N][D]; dq, dk, dv: fp64 [N][D] of head bh.
 * branches: 1 sparse, 2 linear, 3 both (as the forward); kidx_head NULL =
 * dense. sm_scale <= 0 selects 1/sqrt(D). */
void orc_sagesla_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int8_t* q_i8,
                     const float* q_scale, const int8_t* k_i8, const float* k_scale, int64_t N,
                     int64_t D, int64_t bh, const int32_t* kidx_head, int64_t keep, int branches,
                     float sm_scale, const uint16_t* dout, double* dq, double* dk, double* dv,
                     int nthreads);

/* orc_sagesla_bwd restricted to sampled outputs: qsel[N] marks the query rows
 * whose dq is computed, ksel[N] the keys whose dk and dv are (NULL: every row).
 * Selected rows hold exactly what orc_sagesla_bwd gives them; the others are
 * unspecified. Row statistics are formed for the rows the selection needs. */
void orc_sagesla_bwd_sel(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                         const float* k_scale, int64_t N, int64_t D, int64_t bh,
                         const int32_t* kidx_head, int64_t keep, int branches, float sm_scale,
                         const uint16_t* dout, const uint8_t* qsel, const uint8_t* ksel,
                         double* dq, double* dk, double* dv, int nthreads);

/* sum_{t,e} dout[t][e] * O[t][e] of the forward on continuous fp64 inputs of
 * one head: qh, kh (sparse branch, no quantization), ql, kl (linear branch),
 * vv (both); for pinning orc_sagesla_bwd by central differences. */
double orc_sagesla_loss(const double* qh, const double* kh, const double* vv, const double* ql,
                        const double* kl, int64_t N, int64_t D, const int32_t* kidx_head,
                        int64_t keep, int branches, double sm, const double* dout);

/* W8A8 linear layer (page 5, "Four Technical Pillars", Pillar Three: INT8
 * weights and activations, block-wise granularity 128x128).
 * Readings: y = x . w^T with x [M][K] activations and w [N][K] weights (a
 * linear layer's weight layout), no bias; K and N multiples of 128. */
#define ORC_W8_BLK 128

/* Per 128 x 128 block of a row-major [rows][cols] bf16 matrix (cols a
 * multiple of 128, a partial last row block uses its valid rows): the
 * Pillar One rule, scale = max|v|/127 (fp32), q = clamp(rint(v/scale),
 * -127, 127), amax = 0 giving scale 0 and q = 0.
 * scale: [ceil(rows/128)][cols/128]. */
void orc_w8a8_quant(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                    int nthreads);

/* y[r][n] for the listed rows m = rows[r]: per 128-wide column block kb of K
 * the exact int32 I = sum_k xq[m][k] * wq[n][k]; then y = fmaf((float)I, s, y)
 * in ascending kb from 0.0f with s = fl32(sx[m/128][kb] * sw[n/128][kb]);
 * then, if bias is not NULL, y = fl32(y + bias[n]). */
void orc_w8a8_gemm(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                   const float* bias /*[N] or NULL*/, int64_t M, int64_t N, int64_t K,
                   const int64_t* rows, int64_t R, float* y /*[R][N]*/, int nthreads);

/* The same rows with the dequantization in fp64: y = sum over kb of
 * (double)I_kb * (double)sx * (double)sw (+ bias); yabs = sum over kb of
 * |I_kb| * sx * sw. */
void orc_w8a8_gemm_f64(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                       const float* bias, int64_t M, int64_t N, int64_t K, const int64_t* rows,
                       int64_t R, double* y, double* yabs, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
