/*
 * ssa.h -- C ABI of the SageSLA attention library for AMD MI355X (gfx950).
 *
 * The method: TurboDiffusion pages, page 5, "Four Technical Pillars".
 *   Pillar One (SageAttention): attention computed in 8-bit integers, with a
 *   smoothing step that tames outliers.
 *   Pillar Two (SLA): only the most important block interactions are computed
 *   exactly (about 10% of them), a cheap linear-attention term handles the
 *   others; the two stack as "SageSLA".
 *   "Hands-On Tutorial": --attention_type sagesla selects it, --sla_topk is the
 *   fraction of connections kept (0.1 -> 90% sparsity).
 * The concrete numerics (block sizes, scale formula, rounding, block scoring,
 * feature map) are not printed on the pages; the readings used are stated at
 * each entry point below.
 *
 * Conventions shared by every entry point
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Tensor pointers are DEVICE pointers to contiguous row-major [B,H,N,D]
 *     arrays (D fastest), 16-byte aligned; fp32/int32 arrays are 4-byte
 *     aligned. D must be 128. 1 <= N <= SSA_MAX_N, B,H >= 1.
 *   - Query blocks are 128 tokens (Nqb = ceil(N/128)), key blocks 64 tokens
 *     (Nkb = ceil(N/64)); the last block of each may be partial.
 *   - Ownership: the caller owns every buffer, including the workspace whose
 *     size ssa_workspace_bytes() reports. The library never allocates device
 *     memory and keeps no per-call state. Every compute call only enqueues
 *     work on `stream` (a hipStream_t; NULL = the null stream) and returns
 *     without synchronizing; the one call that waits on the device is the
 *     benchmark hook ssa_kernel_timer_read, which waits for the events it reads.
 *   - Errors: argument problems are reported synchronously with nothing
 *     enqueued (SSA_ERR_INVALID / SSA_ERR_UNSUPPORTED / SSA_ERR_WORKSPACE),
 *     shapes whose launch grids the device cannot take included (B*H at most
 *     65535, B*H*Nqb below 2^24, and B*H*258*ceil(Nqb/640) below 2^24 for
 *     the linear branch's state GEMM). A failed HIP launch returns SSA_ERR_HIP; in
 *     a call that enqueues several kernels the launches before the failing
 *     one stay enqueued. Device faults surface at the caller's next
 *     synchronization. ssa_last_error() gives a message for the last failing
 *     call on the calling thread. Nothing is printed.
 *   - Outputs must not overlap inputs (checked).
 */
#ifndef SSA_H
#define SSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssa_status {
    SSA_OK = 0,
    SSA_ERR_INVALID = 1,     /* null / misaligned pointer, bad size, aliasing */
    SSA_ERR_UNSUPPORTED = 2, /* D != 128, N too large, device is not gfx950 */
    SSA_ERR_WORKSPACE = 3,   /* workspace missing or too small */
    SSA_ERR_HIP = 4          /* a HIP runtime call or launch failed */
} ssa_status;

typedef struct ssa_shape {
    int64_t B, H, N, D;
} ssa_shape;

enum { SSA_OP_QUANT = 0, SSA_OP_MASK = 1, SSA_OP_ATTN = 2, SSA_OP_STEP = 3, SSA_OP_BWD = 4 };
enum { SSA_BRANCH_SPARSE = 1, SSA_BRANCH_LINEAR = 2 };

#define SSA_HEAD_DIM 128
#define SSA_QBLK 128
#define SSA_KBLK 64
#define SSA_MAX_N (1 << 19)

int64_t ssa_num_q_blocks(int64_t N); /* ceil(N/128) */
int64_t ssa_num_k_blocks(int64_t N); /* ceil(N/64) */

/* Key blocks kept per query block for a kept fraction `topk` (the meaning of
 * --sla_topk, page 5 "Hands-On Tutorial"): clamp(floor(topk*Nkb + 0.5), 1, Nkb). */
int64_t ssa_keep_blocks(int64_t N, double topk);

/* Bytes of device workspace the entry point `op` needs for shape s (keep and
 * branches only matter for SSA_OP_ATTN and SSA_OP_STEP; pass keep = Nkb for
 * dense). Returns 0 for an invalid shape. */
size_t ssa_workspace_bytes(int op, ssa_shape s, int64_t keep, int branches);

const char* ssa_status_str(ssa_status st);
const char* ssa_last_error(void);

/* ---------------------------------------------------------------------------
 * sage_quant_qk -- K smoothing and per-block INT8 quantization.
 * Page 5, Pillar One (INT8 attention, "smoothing" for outliers).
 * Readings: mu[b,h,d] = mean over all N tokens of K[b,h,:,d], summed in fp32
 * per 64-token block in token order, then over blocks in block order, divided
 * by N (IEEE fp32). K' = fp32(K) - mu. Q in 128-token blocks of raw Q, K' in
 * 64-token blocks; one fp32 scale per (b,h,block) = max|x| / 127 over the
 * block's valid tokens and all channels; q = clamp(rint(x/scale), -127, 127)
 * with the division in IEEE fp32 and ties to even; an all-zero block gets
 * scale 0 and q = 0.
 *   q, k     in : bf16 [B,H,N,D]
 *   q_i8     out: int8 [B,H,N,D]      q_scale out: fp32 [B,H,Nqb]
 *   k_i8     out: int8 [B,H,N,D]      k_scale out: fp32 [B,H,Nkb]
 *   k_mean   out: fp32 [B,H,D]
 *   pool     out: NULL, or ssa_pool_bytes(s) bytes (256-byte aligned) that
 *                 receive the pooled block means sla_block_mask scores with
 *                 (its qbar and kbar, bit-identical, in an internal layout),
 *                 computed in the same passes over Q and K; hand the buffer
 *                 to sla_block_mask so it need not read Q and K again.
 *   ws: ssa_workspace_bytes(SSA_OP_QUANT, s, 0, 0) bytes, 256-byte aligned.
 */
ssa_status sage_quant_qk(const uint16_t* q, const uint16_t* k, ssa_shape s, int8_t* q_i8,
                         float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                         void* pool, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the pooled-means buffer of sage_quant_qk / sla_block_mask for
 * shape s (0 for an invalid shape). */
size_t ssa_pool_bytes(ssa_shape s);

/* ---------------------------------------------------------------------------
 * sage_quant_qk_noalloc -- sage_quant_qk for callers that cannot allocate
 * device memory or hand over a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Same arguments, results
 * and errors as sage_quant_qk, bit for bit, without ws / ws_bytes: the K-mean
 * block partials go to a fixed 32 MiB device array inside the library (one
 * per GPU, held until the process ends). Limit: B*H*Nkb <= 65536 (e.g. 40
 * heads of 75600 tokens); larger shapes return SSA_ERR_UNSUPPORTED with
 * nothing enqueued. The call allocates nothing; its first call on a device
 * looks up that device's array once. Every call on one GPU shares the array,
 * and each call writes every entry it reads: calls on one GPU whose work
 * overlaps in time (other streams, other threads) race and must be ordered
 * by the caller.
 */
ssa_status sage_quant_qk_noalloc(const uint16_t* q, const uint16_t* k, ssa_shape s,
                                 int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                                 float* k_mean, void* pool, void* stream);

/* ---------------------------------------------------------------------------
 * sla_block_mask -- the SLA critical-block selection.
 * Page 5, Pillar Two (only the most important interactions are computed) and
 * "Hands-On Tutorial" (--sla_topk = fraction kept).
 * Readings: qbar_i = fp32 mean of raw bf16 Q over the valid tokens of query
 * block i (sequential sum in token order, IEEE division by the valid count);
 * kbar_j likewise for raw K; score_ij = fmaf chain over d = 0..127 from 0;
 * each query block keeps its `keep` best key blocks under (score descending,
 * j ascending), -0.0 equal to +0.0.
 *   pool in : NULL, or the buffer sage_quant_qk filled for the same Q, K and
 *             shape: the means are then taken from it, and q, k are not read
 *             (they may be NULL) and ws is not used (it may be NULL).
 *   kidx out: int32 [B,H,Nqb,keep], kept key blocks in ascending order
 *   mask out: uint8 [B,H,Nqb,Nkb] (1 = kept) or NULL
 *   ws: ssa_workspace_bytes(SSA_OP_MASK, s, keep, 0) bytes (without pool).
 */
ssa_status sla_block_mask(const uint16_t* q, const uint16_t* k, ssa_shape s, int64_t keep,
                          const void* pool, int32_t* kidx, uint8_t* mask, void* ws,
                          size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * sage_sla_attn_fwd -- SageSLA forward: sparse INT8 softmax attention over the
 * kept blocks plus the elu+1 linear branch over the other blocks.
 * Page 5, Pillars One and Two, "SageSLA".
 * Sparse branch (branches & SSA_BRANCH_SPARSE): for each query token, over the
 * valid keys u of its kept blocks, S_u = int32 q_i8 . k_i8 (exact);
 * K32 = fl32(sm * log2 e); c = fl32(fl32(q_scale * k_scale) * K32);
 * m = ceil(max_u fl32(S_u * c)) (an integer normalizer); p_u = bf16 of
 * 2^(S_u*c - m); o_s = sum p_u v_u / sum p_u with fp32 accumulation (P in
 * bf16 against bf16 V on the matrix cores).
 * Linear branch (branches & SSA_BRANCH_LINEAR): phi(x) = x + 1 (x > 0) or e^x,
 * on raw bf16 Q and K; for query block i, H_i = sum over key blocks j NOT kept
 * of sum_{u in j} phi(k_u) v_u^T and z_i = sum phi(k_u) likewise;
 * o_l = phi(q)^T H_i / phi(q)^T z_i, or 0 when every block is kept.
 * Output: out = o_s + o_l (either term dropped when its branch is off).
 *   q, k, v      in : bf16 [B,H,N,D] (q, k only read by the linear branch)
 *   q_i8..k_scale in : as produced by sage_quant_qk
 *   kidx         in : int32 [B,H,Nqb,keep] ascending, as produced by
 *                     sla_block_mask; NULL = dense (keep must equal Nkb).
 *                     Entries are clamped into [0, Nkb) on the device, so a
 *                     malformed kidx yields wrong values, never a stray access.
 *   sm_scale     in : softmax scale; <= 0 selects 1/sqrt(D) rounded to fp32
 *   out          out: bf16 [B,H,N,D] (round to nearest even of the fp32 result)
 *   out_f32      out: fp32 [B,H,N,D] copy of the result before rounding, or NULL
 *   lse          out: fp32 [B,H,N], each query row's m + log2(sum p) of the
 *                     sparse branch (written when that branch runs), or NULL:
 *                     with out_f32, what sage_sla_attn_bwd needs to skip
 *                     recomputing the forward
 *   ws: ssa_workspace_bytes(SSA_OP_ATTN, s, keep, branches) bytes.
 */
ssa_status sage_sla_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             ssa_shape s, const int8_t* q_i8, const float* q_scale,
                             const int8_t* k_i8, const float* k_scale, const int32_t* kidx,
                             int64_t keep, int branches, float sm_scale, uint16_t* out,
                             float* out_f32, float* lse, void* ws, size_t ws_bytes,
                             void* stream);

/* ---------------------------------------------------------------------------
 * sage_sla_fwd -- the whole SageSLA step in one call (page 5, Pillars One and
 * Two, "SageSLA"): K smoothing and INT8 quantization, the block selection and
 * the attention, with every result bit-identical to sage_quant_qk (with a
 * pool), then sla_block_mask (from that pool), then sage_sla_attn_fwd on the
 * same arguments. Enqueued as one pass, it reads raw K once less: the per-block
 * K sums of the mean and the pooled key means come out of the pass that lays
 * out V (and forms the linear states), which reads K anyway. K is still read
 * twice in all, since K' = K - mu needs the finished mean.
 *   q, k, v         in : bf16 [B,H,N,D]
 *   keep, branches, sm_scale: as for sage_sla_attn_fwd
 *   q_i8..k_mean    out: as sage_quant_qk writes them
 *   kidx            out: int32 [B,H,Nqb,keep] as sla_block_mask writes it, or
 *                        NULL = dense (keep must equal Nkb; no selection runs)
 *   mask            out: uint8 [B,H,Nqb,Nkb] or NULL (needs kidx)
 *   out, out_f32, lse out: as for sage_sla_attn_fwd
 *   ws: ssa_workspace_bytes(SSA_OP_STEP, s, keep, branches) bytes, 256-byte
 *       aligned; its contents on return are unspecified.
 */
ssa_status sage_sla_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, ssa_shape s,
                        int64_t keep, int branches, float sm_scale, int8_t* q_i8, float* q_scale,
                        int8_t* k_i8, float* k_scale, float* k_mean, int32_t* kidx,
                        uint8_t* mask, uint16_t* out, float* out_f32, float* lse, void* ws,
                        size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * sage_sla_attn_bwd -- SageSLA backward: the gradients of a loss L with
 * respect to Q, K and V given dL/dO of sage_sla_attn_fwd's output, for
 * training the sparse-linear attention (page 5: SLA is trainable and is
 * fine-tuned; training guide, "SLA Adaptation Fine-tuning").
 * Readings: the 8-bit quantizer passes gradients straight through and the
 * block selection is held fixed. Sparse branch: with the forward's P over the
 * kept keys (recomputed from the exact int32 scores, normalized with the
 * forward's m + log2(l)) and D = dO . o_s per query row, dS = P (dP - D),
 * dP = dO . v:  dQ = sm dS K', dK = sm dS^T Q', dV = P^T dO, with Q' and K'
 * the dequantized quantized operands (q_scale q_i8, k_scale k_i8); K's mean
 * needs no term (each row of dS sums to zero). Linear branch: the exact
 * gradient of phi(q)^T H_i / phi(q)^T z_i over the non-kept blocks (phi =
 * elu + 1 on raw Q, K). Arithmetic: int8 scores exact; P and dS rounded to
 * bf16 for the bf16 matrix-core products (fp32 accumulation); the linear
 * branch in fp32 (its states summed as the forward's, from a bf16 stack and a
 * stack of each entry's bf16 rest, with an fp32 total). Relative L2 error
 * against the exact gradient ~1e-3.
 *   q, k, v, q_i8..k_scale, kidx, keep, branches, sm_scale: as for
 *                     sage_sla_attn_fwd (the same values the forward used)
 *   dout         in : bf16 [B,H,N,D], dL/d(out)
 *   out_f32, lse in : the forward's out_f32 and lse (from the same inputs and
 *                     branches), or both NULL. Given, the row statistics come
 *                     from them (D = dO . out - dO . o_l, o_l from the linear
 *                     branch's own pass) and the forward is not recomputed;
 *                     NULL, a pass of the forward's sparse branch recomputes
 *                     them. Either way within the same error of the exact
 *                     gradient.
 *   dq, dk, dv   out: fp32 [B,H,N,D] (both branches' gradients summed)
 *   ws: ssa_workspace_bytes(SSA_OP_BWD, s, keep, branches) bytes, 256-byte
 *       aligned (the forward's workspace plus the backward's).
 * Errors as for the entry points above; SSA_ERR_INVALID when only one of
 * out_f32 and lse is given.
 */
ssa_status sage_sla_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             ssa_shape s, const int8_t* q_i8, const float* q_scale,
                             const int8_t* k_i8, const float* k_scale, const int32_t* kidx,
                             int64_t keep, int branches, float sm_scale, const uint16_t* dout,
                             const float* out_f32, const float* lse, float* dq, float* dk,
                             float* dv, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * sage_qk_int32_tiles -- test export of raw int32 score tiles computed by the
 * same device routine the attention kernel uses (INT8 matrix-core product
 * with int32 accumulation, page 5 Pillar One).
 *   tiles in : int32 [T,3] device array of (b*H + h, query block i, key block j)
 *   out   out: int32 [T,128,64]; out[t][r][c] = sum_d q_i8[128i+r][d]*k_i8[64j+c][d],
 *              0 where the row or column is past N.
 * Tile indices are validated on the device: an out-of-range triple yields an
 * all-zero tile.
 */
ssa_status sage_qk_int32_tiles(const int8_t* q_i8, const int8_t* k_i8, ssa_shape s,
                               const int32_t* tiles, int64_t T, int32_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * W8A8 linear layer -- page 5, "Four Technical Pillars", Pillar Three: the
 * linear layers run with INT8 weights and activations, quantized with a
 * block-wise granularity of 128x128.
 * Readings: y = x . w^T for activations x [M][K] and weights w [N][K] (a
 * linear layer's [out][in] layout), no bias; K and N multiples of 128. Each
 * operand is quantized per 128-row x 128-column block with the rule of
 * sage_quant_qk (scale = max|v|/127 in fp32 over the block's valid rows,
 * q = clamp(rint(v/scale), -127, 127), ties to even, scale 0 and q = 0 for an
 * all-zero block).
 *
 * w8a8_quant -- block quantization of a row-major bf16 [rows][cols] matrix
 * (activations or weights; cols a multiple of 128, rows and cols <= 2^20).
 *   x     in : bf16 [rows][cols], 16-byte aligned
 *   q     out: int8 [rows][cols], 16-byte aligned
 *   scale out: fp32 [ceil(rows/128)][cols/128]
 */
ssa_status w8a8_quant(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                      void* stream);

/* w8a8_gemm -- the block-dequantized INT8 product. For each 128-wide block kb
 * of K, I = sum over the block of xq[m][k] * wq[n][k] (exact int32), and
 * y[m][n] = fmaf((float)I, fl32(sx[m/128][kb] * sw[n/128][kb]), y) in
 * ascending kb from 0 (INT8 matrix cores, fp32 accumulation); then, for a
 * layer with a bias, y = fl32(y + bias[n]).
 *   xq, sx in : w8a8_quant of x [M][K];  wq, sw in : w8a8_quant of w [N][K]
 *   bias   in : fp32 [N], or NULL for none (16-byte aligned)
 *   y      out: bf16 [M][N] (round to nearest even of the fp32 result)
 *   y32    out: fp32 [M][N] copy before rounding, or NULL (16-byte aligned)
 * M, N, K <= 2^20; N and K multiples of 128; ceil(M/256) * N/128 below 2^22
 * (the launch grid). Errors as for the entry points above (validation before
 * anything is enqueued, SSA_ERR_HIP on a failed launch).
 */
ssa_status w8a8_gemm(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                     const float* bias, int64_t M, int64_t N, int64_t K, uint16_t* y, float* y32,
                     void* stream);

/* ---------------------------------------------------------------------------
 * Kernel timer (for benchmarks). After ssa_kernel_timer_start(n), each of the
 * next n sage_sla_attn_fwd calls records a pair of HIP events on its stream
 * immediately around its sparse-attention kernel launch (after the linear
 * states / V re-layout launches). ssa_kernel_timer_read waits for the recorded
 * events and writes up to `cap` per-launch durations in milliseconds (-1 for a
 * failed read), returning how many it wrote. ssa_kernel_timer_stop releases
 * the events. The events are host-side runtime objects; no device memory is
 * allocated. The timer is process-wide and guarded by a mutex.
 */
ssa_status ssa_kernel_timer_start(int max_launches);
int ssa_kernel_timer_read(float* ms, int cap);
void ssa_kernel_timer_stop(void);

#ifdef __cplusplus
}
#endif
#endif
