// kernels.hpp -- launchers of the gfx950 kernels (internal, not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

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
hipError_t launch_linear_states(const uint16_t* k, const uint16_t* v, int64_t BH, int N,
                                uint16_t* vt, uint16_t* hs, float* hpart, float* htot,
                                float* kpart, float* kbarT, int ldk, hipStream_t st);
hipError_t launch_vt_only(const uint16_t* k, const uint16_t* v, int64_t BH, int N, uint16_t* vt,
                          float* kpart, float* kbarT, int ldk, hipStream_t st);
// bytes of the complement GEMM's selection rows (msel) for nkbp padded key blocks
size_t msel_bytes(int64_t BH, int64_t nqb, int64_t nkbp);
hipError_t launch_complement(const int32_t* kidx, int keep, const uint16_t* hs, const float* htot,
                             int64_t BH, int N, uint32_t* msel, float* hnon, hipStream_t st);

// w8a8.hip
hipError_t launch_w8a8_quant(const uint16_t* x, int rows, int cols, int8_t* q, float* scale,
                             hipStream_t st);
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
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);
hipError_t launch_qk_tiles(const int8_t* q_i8, const int8_t* k_i8, int64_t BH, int N,
                           const int32_t* tiles, int64_t T, int32_t* out, hipStream_t st);

}  // namespace ssa
