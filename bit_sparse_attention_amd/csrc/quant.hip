// quant.hip -- K smoothing mean, per-block INT8 quantization, and the
// block column sums the block mask pools with.
//
// TurboDiffusion pages, page 5 "Four Technical Pillars", Pillar One:
// attention inputs quantized to 8-bit integers, with smoothing for outliers.
// Every fp32 operation here is bit-reproducible: sums run in token order
// (then block order), divisions are IEEE (this file is compiled with
// -ffp-contract=off), and round-half-even comes from v_rndne_f32.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ssa {

// Per-block column sums of a bf16 [BH][N][128] tensor.
// One workgroup covers NB consecutive blocks of BLK tokens; thread
// (blk = tid/16, g = tid%16) owns channels 8g..8g+7 of its block and adds the
// block's valid tokens in token order, starting from 0.
//   MODE 0: out[bh][b][d] = sum                    (K mean partials), and, if
//           out2 is given, out2 as MODE 2 (the same sums give the pooled means)
//   MODE 1: out[bh][b][d] = sum / valid            (pooled means)
//   MODE 2: out[bh][d][b] = sum / valid, row pitch ld (pooled means, transposed)
template <int BLK, int MODE>
__global__ __launch_bounds__((1024 / BLK) * 16)
void colsum_kernel(const uint16_t* __restrict__ x, int N, int nb, int ld, float* __restrict__ out,
                   float* __restrict__ out2) {
    constexpr int NB = 1024 / BLK;
    __shared__ float stage[MODE == 1 ? 1 : NB * HD];
    const int tid = threadIdx.x;
    const int bl = tid >> 4, g = tid & 15;
    const int64_t bh = blockIdx.y;
    const int b = blockIdx.x * NB + bl;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int valid = 0;
    if (b < nb) {
        const int t0 = b * BLK;
        valid = min(BLK, N - t0);
        const uint16_t* p = x + (bh * N + t0) * HD + 8 * g;
        int t = 0;
        for (; t + 4 <= valid; t += 4) {
            u16x8 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *(const u16x8*)(p + (int64_t)(t + u) * HD);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += bf2f(v[u][e]);
        }
        for (; t < valid; ++t) {
            u16x8 v = *(const u16x8*)(p + (int64_t)t * HD);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += bf2f(v[e]);
        }
    }
    if (MODE == 0 || MODE == 1) {
        if (b < nb) {
            float r[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) r[e] = MODE == 1 ? acc[e] / (float)valid : acc[e];
            float* o = out + ((bh * nb + b) * HD + 8 * g);
            *(f32x4*)o = f32x4{r[0], r[1], r[2], r[3]};
            *(f32x4*)(o + 4) = f32x4{r[4], r[5], r[6], r[7]};
        }
    }
    float* tout = MODE == 2 ? out : MODE == 0 ? out2 : nullptr;
    if (MODE != 1 && tout) {
        if (b < nb)
#pragma unroll
            for (int e = 0; e < 8; ++e) stage[bl * HD + 8 * g + e] = acc[e] / (float)valid;
        __syncthreads();
        // transpose: NB*HD values, written as runs of NB consecutive blocks per channel
        for (int idx = tid; idx < NB * HD; idx += NB * 16) {
            const int d = idx / NB, bb = idx % NB;
            const int b2 = blockIdx.x * NB + bb;
            if (b2 < nb) tout[(bh * HD + d) * ld + b2] = stage[bb * HD + d];
        }
    }
}

// mu[bh][d] = (sum over key blocks j in order of part[bh][j][d]) / N.
// One workgroup per (head, 32 channels). The partials arrive in chunks of
// KM_CHUNK key blocks, loaded by all threads into LDS (many loads in flight),
// then one thread per channel adds its column of the chunk in block order.
// The sum starts at +0.0 and only existing blocks are added.
constexpr int KM_CH = 32;      // channels per workgroup
constexpr int KM_CHUNK = 256;  // key blocks per LDS chunk
__global__ __launch_bounds__(256) void kmean_final_kernel(const float* __restrict__ part, int nkb,
                                                          int N, float* __restrict__ mu) {
    __shared__ float st[KM_CHUNK][KM_CH + 1];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int d0 = blockIdx.y * KM_CH;
    const float* p = part + bh * nkb * HD + d0;
    float tot = 0.f;
    for (int j0 = 0; j0 < nkb; j0 += KM_CHUNK) {
        const int nj = min(KM_CHUNK, nkb - j0);
        // 8 float4 per thread: row r = idx / 8, channels 4 * (idx % 8) .. + 3
#pragma unroll
        for (int k = 0; k < KM_CHUNK * KM_CH / 4 / 256; ++k) {
            const int idx = tid + 256 * k;
            const int r = idx >> 3, c4 = (idx & 7) * 4;
            if (r < nj) {
                const f32x4 v = *(const f32x4*)(p + (int64_t)(j0 + r) * HD + c4);
                st[r][c4] = v[0];
                st[r][c4 + 1] = v[1];
                st[r][c4 + 2] = v[2];
                st[r][c4 + 3] = v[3];
            }
        }
        __syncthreads();
        if (tid < KM_CH)
            for (int r = 0; r < nj; ++r) tot += st[r][tid];
        __syncthreads();
    }
    if (tid < KM_CH) mu[bh * HD + d0 + tid] = tot / (float)N;
}

// Per-block INT8 quantization of one (head, block): scale = amax/127 over the
// block's valid tokens and all channels, q = clamp(rint(x/scale), +-127).
// SMOOTH subtracts the K mean first (one fp32 subtraction).
// POOL also writes the block's pooled means, pooled[bh][b][d] = (sum of the
// valid tokens of channel d in token order, from 0) / valid: the raw block is
// staged in LDS and thread d adds its column in order, so the result is the
// one colsum_kernel MODE 1 gives.
template <int BLK, bool SMOOTH, bool POOL>
__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ x,
                                                    const float* __restrict__ mu, int N, int nb,
                                                    int8_t* __restrict__ xq,
                                                    float* __restrict__ scale,
                                                    float* __restrict__ pooled) {
    constexpr int IT = BLK * 16 / 256;  // 16-byte chunks per thread
    __shared__ float wmax[4];
    __shared__ __attribute__((aligned(16))) uint16_t raw[POOL ? BLK * HD : 8];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.y;
    const int b = blockIdx.x;
    const int t0 = b * BLK;
    const int valid = min(BLK, N - t0);
    const int g = tid & 15;
    float m8[8];
    if (SMOOTH) {
        const float* mp = mu + bh * HD + 8 * g;
#pragma unroll
        for (int e = 0; e < 8; ++e) m8[e] = mp[e];
    }
    float v[IT][8];
    float amax = 0.f;
    const uint16_t* base = x + (bh * N + t0) * HD;
    // every load is issued before any is used (rows past the block's end
    // re-read its last row and are then dropped), so they are in flight together
    u16x8 r8[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int row = min((tid >> 4) + 16 * it, valid - 1);
        r8[it] = *(const u16x8*)(base + (int64_t)row * HD + 8 * g);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int row = (tid >> 4) + 16 * it;
        if (row < valid) {
            if (POOL) *(u16x8*)(raw + row * HD + 8 * g) = r8[it];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float f = bf2f(r8[it][e]);
                if (SMOOTH) f = f - m8[e];
                v[it][e] = f;
                amax = fmaxf(amax, fabsf(f));
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[it][e] = 0.f;
        }
    }
    amax = wave_max_f32(amax);
    if ((tid & 63) == 0) wmax[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float s = amax / 127.0f;
    if (tid == 0) scale[bh * nb + b] = s;
    if (POOL && tid < HD) {  // the staged rows are visible after the barrier above
        // reads in batches of 32 so they are in flight together; the adds
        // stay in token order over the valid rows
        float sum = 0.f;
        for (int r0 = 0; r0 < valid; r0 += 32) {
            float t[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) t[u] = bf2f(raw[min(r0 + u, BLK - 1) * HD + tid]);
#pragma unroll
            for (int u = 0; u < 32; ++u)
                if (r0 + u < valid) sum += t[u];
        }
        pooled[(bh * nb + b) * HD + tid] = sum / (float)valid;
    }
    int8_t* qbase = xq + (bh * N + t0) * HD;
    // q = clamp(rint(v / s)); the quotient through div_by_scale when the
    // (block-uniform) scale allows, which gives the same bytes
    auto store = [&](auto fast) {
        const float rs = decltype(fast)::value ? 1.0f / s : 0.f;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int row = (tid >> 4) + 16 * it;
            if (row < valid) {
                uint32_t w[2] = {0u, 0u};
                if (s > 0.f) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float qt = decltype(fast)::value ? div_by_scale(v[it][e], s, rs)
                                                               : v[it][e] / s;
                        const float r = fminf(fmaxf(__builtin_rintf(qt), -127.f), 127.f);
                        const uint32_t byte = (uint32_t)(uint8_t)(int8_t)(int)r;
                        w[e >> 2] |= byte << (8 * (e & 3));
                    }
                }
                *(u32x2*)(qbase + (int64_t)row * HD + 8 * g) = u32x2{w[0], w[1]};
            }
        }
    };
    if (s >= FAST_DIV_MIN_SCALE && s <= FAST_DIV_MAX_SCALE)
        store(std::true_type{});
    else
        store(std::false_type{});
}

// ---------------------------------------------------------------------------
// launchers

hipError_t launch_quant_qk(const uint16_t* q, const uint16_t* k, int64_t BH, int N,
                           int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                           float* k_mean, float* ws_part, float* qbar, float* kbarT, int ldk,
                           hipStream_t st) {
    const int nkb = (N + KBLK - 1) / KBLK;
    hipLaunchKernelGGL((colsum_kernel<KBLK, 0>), dim3((nkb + 15) / 16, BH), dim3(256), 0, st, k, N,
                       nkb, ldk, ws_part, kbarT);
    return launch_quant_from_sums(q, k, BH, N, q_i8, q_scale, k_i8, k_scale, k_mean, ws_part, qbar,
                                  st);
}

hipError_t launch_quant_from_sums(const uint16_t* q, const uint16_t* k, int64_t BH, int N,
                                  int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                                  float* k_mean, const float* ws_part, float* qbar,
                                  hipStream_t st) {
    const int nqb = (N + QBLK - 1) / QBLK, nkb = (N + KBLK - 1) / KBLK;
    hipLaunchKernelGGL(kmean_final_kernel, dim3(BH, HD / KM_CH), dim3(256), 0, st, ws_part, nkb, N,
                       k_mean);
    if (qbar)
        hipLaunchKernelGGL((quant_kernel<QBLK, false, true>), dim3(nqb, BH), dim3(256), 0, st, q,
                           nullptr, N, nqb, q_i8, q_scale, qbar);
    else
        hipLaunchKernelGGL((quant_kernel<QBLK, false, false>), dim3(nqb, BH), dim3(256), 0, st, q,
                           nullptr, N, nqb, q_i8, q_scale, nullptr);
    hipLaunchKernelGGL((quant_kernel<KBLK, true, false>), dim3(nkb, BH), dim3(256), 0, st, k,
                       k_mean, N, nkb, k_i8, k_scale, nullptr);
    return hipGetLastError();
}

hipError_t launch_pool(const uint16_t* q, const uint16_t* k, int64_t BH, int N, float* qbar,
                       float* kbarT, int ldk, hipStream_t st) {
    const int nqb = (N + QBLK - 1) / QBLK, nkb = (N + KBLK - 1) / KBLK;
    hipLaunchKernelGGL((colsum_kernel<QBLK, 1>), dim3((nqb + 7) / 8, BH), dim3(128), 0, st, q, N, nqb,
                       0, qbar, nullptr);
    hipLaunchKernelGGL((colsum_kernel<KBLK, 2>), dim3((nkb + 15) / 16, BH), dim3(256), 0, st, k, N,
                       nkb, ldk, kbarT, nullptr);
    return hipGetLastError();
}

}  // namespace ssa
