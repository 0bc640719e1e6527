// kernels.hpp -- launchers of the gfx950 kernels (internal, not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

// x / s for many x and one block scale s, correctly rounded like the IEEE
// division, from rs = 1/s (itself an IEEE division): q0 = x*rs, then one fma
// correction with the exact residual x - s*q0 (Markstein's method, 1990: with a
// correctly rounded reciprocal the corrected quotient is correctly rounded as
// long as the residual does not underflow). Callers use it only for finite
// s >= 2^-90; then a residual can underflow only for |x| < s/4, whose quotient
// rounds to the integer 0 either way. (An infinite scale, from an infinite
// element, takes the division: there 1/s = 0 would turn finite x into NaN.)
// Checked against the IEEE division on 1.6e8 (x, s) pairs: every quotient
// with |x| >= s/4 equal bit for bit.
constexpr float FAST_DIV_MIN_SCALE = 0x1p-90f;
constexpr float FAST_DIV_MAX_SCALE = 3.40282347e+38f;  // the largest finite float
__device__ __forceinline__ float div_by_scale(float x, float s, float rs) {
    const float q0 = x * rs;
    return __builtin_fmaf(__builtin_fmaf(-s, q0, x), rs, q0);
}

// quant.hip
// qbar / kbarT (may be null): also write the block mask's pooled means (the
// layouts launch_pool writes), from the same passes over Q and K
hipError_t launch_quant_qk(const uint16_t* q, const uint16_t* k, int64_t BH, int N, int8_t* q_i8,
                           float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                           float* ws_part, float* qbar, float* kbarT, int ldk, hipStream_t st);
// the same minus the K-mean partial pass: ws_part already holds the per-block
// K sums (from launch_linear_states / launch_vt_only with kpart)
hipError_t launch_quant_from_sums(const uint16_t* q, const uint16_t* k, int64_t BH, int N,
                                  int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                                  float* k_mean, const float* ws_part, float* qbar,
                                  hipStream_t st);
hipError_t launch_pool(const uint16_t* q, const uint16_t* k, int64_t BH, int N, float* qbar,
                       float* kbarT, int ldk, hipStream_t st);
// mask.hip
hipError_t launch_score_topk(const float* qbar, const float* kbarT, int ldk, int64_t BH, int nqb,
                             int nkb, int keep, int32_t* kidx, uint8_t* mask, hipStream_t st);

// linear.hip
constexpr int LIN_GROUP = 16;    // key blocks per linear-states workgroup
constexpr int GEMM_KALIGN = 32;  // the complement GEMM's key-block count is padded to this
// kpart (may be null): also write the per-block K sums of the K mean, and
// kbarT (may be null) the pooled key means, from the same pass over K
// hs_lo (may be null): also the bf16 rests of the states (see linear.hip)
hipError_t launch_linear_states(const uint16_t* k, const uint16_t* v, int64_t BH, int N,
                                uint16_t* vt, uint16_t* hs, uint16_t* hs_lo, float* hpart,
                                float* htot, float* kpart, float* kbarT, int ldk, hipStream_t st);
hipError_t launch_vt_only(const uint16_t* k, const uint16_t* v, int64_t BH, int N, uint16_t* vt,
                          float* kpart, float* kbarT, int ldk, hipStream_t st);
// bytes of the complement GEMM's selection rows (msel) for nkbp padded key blocks
size_t msel_bytes(int64_t BH, int64_t nqb, int64_t nkbp);
// workgroups of the complement GEMM per head (256 threads each)
int64_t complement_tiles_per_head(int64_t nqb);
// hs_lo (may be null): a second pass with the states' bf16 rests
hipError_t launch_complement(const int32_t* kidx, int keep, const uint16_t* hs,
                             const uint16_t* hs_lo, const float* htot, int64_t BH, int N,
                             uint32_t* msel, float* hnon, hipStream_t st);

// as launch_complement, with the selection rows taken from lists instead of
// kidx: row r (of nrows) selects the reduction entries lists[bh][r][0..counts)
// (of nred); the stack has nred rows; out gets nrows rows
hipError_t launch_complement_lists(const uint16_t* lists, const int32_t* counts, int nrows,
                                   int nred, int complement, const uint16_t* stack,
                                   const uint16_t* stack_lo, const float* total, int64_t BH,
                                   uint32_t* msel, float* out, hipStream_t st);
// H_total-style sums: out[bh][n] = sum over groups g, in order, of part[bh][g][n]
hipError_t launch_state_total(const float* part, int ngroups, int64_t BH, float* out,
                              hipStream_t st);

// bwd.hip
struct BwdArgs {
    const int8_t* q_i8;
    const float* q_scale;
    const int8_t* k_i8;
    const float* k_scale;
    const uint16_t* v;       // raw bf16 V [BH][N][128]
    const uint16_t* dout;    // bf16 dL/dO [BH][N][128]
    const int32_t* kidx;     // [BH][nqb][keep] or null (dense)
    int keep;
    const uint16_t* lists;   // [BH][nkb][nqb]: query blocks that kept each key block
    const int32_t* counts;   // [BH][nkb]
    int dq_accumulate;       // dq_kernel adds to dq (the linear branch wrote it first)
    int N, nqb, nkb;
    int64_t BH;
    float K32;               // fl32(sm * log2 e)
    float sm;
    const float* mlog;       // [BH][N] m + log2(l) of the forward
    const float* dstat;      // [BH][N] dO . o_s
    float *dq, *dk, *dv;     // fp32 [BH][N][128]
};
// bytes of the bit matrix launch_inv_lists builds the lists from
size_t keep_bits_bytes(int64_t BH, int64_t nqb, int64_t nkb);
hipError_t launch_inv_lists(const int32_t* kidx, int keep, int64_t BH, int nqb, int nkb,
                            uint32_t* bits, uint16_t* lists, int32_t* counts, hipStream_t st);
hipError_t launch_bwd_sparse(const BwdArgs& a, hipStream_t st);
hipError_t launch_lin_bwd_q(const uint16_t* q, const uint16_t* dout, const float* hnon, int64_t BH,
                            int N, float* dq, float* gf, uint16_t* gs, uint16_t* gs_lo, float* dol,
                            hipStream_t st);
hipError_t launch_dstat(const uint16_t* dout, const float* out32, const float* dol, int64_t rows,
                        float* dstat, hipStream_t st);
hipError_t launch_lin_bwd_k(const uint16_t* k, const uint16_t* v, const float* gc, int64_t BH,
                            int N, int accumulate, float* dk, float* dv, hipStream_t st);
hipError_t launch_zero(float* p, int64_t n, hipStream_t st);

// w8a8.hip
hipError_t launch_w8a8_quant(const uint16_t* x, int rows, int cols, int8_t* q, float* scale,
                             hipStream_t st);
// workgroups (1024 threads each) of the product's launch
int64_t w8a8_gemm_workgroups(int64_t M, int64_t N);
hipError_t launch_w8a8_gemm(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                            const float* bias, int M, int N, int K, uint16_t* y, float* y32,
                            hipStream_t st);

// attn.hip
struct AttnArgs {
    const int8_t* q_i8;
    const float* q_scale;
    const int8_t* k_i8;
    const float* k_scale;
    const uint16_t* vt;    // [BH][nkb][128 dv][64 permuted keys]
    const int32_t* kidx;   // [BH][nqb][keep] or null (dense)
    int keep;
    int N, nqb, nkb;
    int64_t BH;
    float K32;             // fl32(sm * log2 e)
    int do_sparse;
    const uint16_t* q;     // raw bf16 Q (linear branch)
    const float* hnon;     // [BH][nqb][HS_ROW] complement states, or null
    uint16_t* out;
    float* out32;
    // backward row statistics (both set: the statistics pass, no output):
    // mlog[bh][t] = m + log2(l), dstat[bh][t] = dO . o_s, from dout
    const uint16_t* dout;
    float* mlog;
    float* dstat;
    // forward: also write lse[bh][t] = m + log2(l) of the sparse branch (or null)
    float* lse;
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);
hipError_t launch_qk_tiles(const int8_t* q_i8, const int8_t* k_i8, int64_t BH, int N,
                           const int32_t* tiles, int64_t T, int32_t* out, hipStream_t st);

}  // namespace ssa
