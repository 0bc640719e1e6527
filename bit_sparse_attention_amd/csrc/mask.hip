// mask.hip -- SLA critical-block selection.
//
// TurboDiffusion pages, page 5 "Four Technical Pillars", Pillar Two (only the
// most important block interactions are computed exactly) and "Hands-On
// Tutorial" (--sla_topk: fraction of key blocks kept). Each query block scores
// every key block by the dot product of their mean-pooled rows (an exact fmaf
// chain over the 128 channels) and keeps the best `keep` under (score
// descending, key block ascending). Selection is an exact 4-pass MSB radix
// select on order-preserving 32-bit keys, so the result is unique and
// bit-identical to a sort.
#include "common.hpp"
#include "kernels.hpp"

namespace ssa {

__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (s == 0.f) u = 0u;  // -0.0 ranks with +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan over a 256-thread workgroup. `wsum` holds 4 ints of LDS.
__device__ __forceinline__ int block_incl_scan(int v, int* wsum) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    __syncthreads();
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    int add = 0;
    for (int u = 0; u < w; ++u) add += wsum[u];
    return v + add;
}

// One workgroup scores R query blocks of one head against every key block and
// selects, per query block, the `keep` best key blocks.
// kbarT: [BH][128][ldk] pooled K means (transposed); qbar: [BH][nqb][128].
template <int R>
__global__ __launch_bounds__(256) void score_topk_kernel(const float* __restrict__ qbar,
                                                         const float* __restrict__ kbarT, int ldk,
                                                         int nqb, int nkb, int keep,
                                                         int32_t* __restrict__ kidx,
                                                         uint8_t* __restrict__ mask) {
    extern __shared__ float dyn[];
    float* sc = dyn;                   // [R][nkb]
    __shared__ float qs[R][HD];
    __shared__ int hist[256];
    __shared__ int wsum[4];
    __shared__ int sel_digit, sel_rem;
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.y;
    const int i0 = blockIdx.x * R;
    for (int idx = tid; idx < R * HD; idx += 256) {
        const int r = idx / HD, d = idx % HD;
        qs[r][d] = (i0 + r < nqb) ? qbar[(bh * nqb + i0 + r) * HD + d] : 0.f;
    }
    __syncthreads();
    const float* kb = kbarT + bh * HD * (int64_t)ldk;
    for (int j = tid; j < nkb; j += 256) {
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll 8
        for (int d = 0; d < HD; ++d) {
            const float kv = kb[(int64_t)d * ldk + j];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = __builtin_fmaf(qs[r][d], kv, acc[r]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r * nkb + j] = acc[r];
    }
    __syncthreads();

    for (int r = 0; r < R; ++r) {
        const int i = i0 + r;
        if (i >= nqb) break;  // uniform across the workgroup
        const float* s = sc + r * nkb;
        // ---- radix select of the keep-th largest key
        uint32_t prefix = 0u, pmask = 0u;
        int rem = keep;
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            hist[tid] = 0;
            __syncthreads();
            for (int j = tid; j < nkb; j += 256) {
                const uint32_t key = order_key(s[j]);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
            }
            __syncthreads();
            // suffix counts from the top digit down: thread t looks at digit 255-t
            const int h = hist[255 - tid];
            const int cum = block_incl_scan(h, wsum);  // count of digits >= 255-tid
            if (cum >= rem && cum - h < rem) {
                sel_digit = 255 - tid;
                sel_rem = rem - (cum - h);
            }
            __syncthreads();
            prefix |= (uint32_t)sel_digit << shift;
            pmask |= 255u << shift;
            rem = sel_rem;
            __syncthreads();
        }
        const uint32_t T = prefix;  // keep-th largest key; take `rem` of the keys equal to T
        // ---- emit kept blocks in ascending j
        int eq_base = 0, out_base = 0;
        int32_t* krow = kidx + (bh * nqb + i) * (int64_t)keep;
        uint8_t* mrow = mask ? mask + (bh * nqb + i) * (int64_t)nkb : nullptr;
        for (int j0 = 0; j0 < nkb; j0 += 256) {
            const int j = j0 + tid;
            uint32_t key = 0u;
            bool inb = j < nkb;
            if (inb) key = order_key(s[j]);
            const int eq = (inb && key == T) ? 1 : 0;
            const int eq_incl = block_incl_scan(eq, wsum);
            const int eq_chunk = wsum[0] + wsum[1] + wsum[2] + wsum[3];
            const int rank_eq = eq_base + eq_incl - eq;  // equal keys before j
            const int sel = (inb && (key > T || (eq && rank_eq < rem))) ? 1 : 0;
            const int sel_incl = block_incl_scan(sel, wsum);
            const int sel_chunk = wsum[0] + wsum[1] + wsum[2] + wsum[3];
            if (sel) krow[out_base + sel_incl - 1] = j;
            if (mrow && inb) mrow[j] = (uint8_t)sel;
            out_base += sel_chunk;
            eq_base += eq_chunk;
        }
        __syncthreads();
    }
}

hipError_t launch_score_topk(const float* qbar, const float* kbarT, int ldk, int64_t BH, int nqb,
                             int nkb, int keep, int32_t* kidx, uint8_t* mask, hipStream_t st) {
    // largest row group whose scores fit in 48 KB of LDS (nkb <= 8192: SSA_MAX_N)
    const size_t per_row = (size_t)nkb * sizeof(float);
    if (4 * per_row <= 48 * 1024) {
        hipLaunchKernelGGL((score_topk_kernel<4>), dim3((nqb + 3) / 4, BH), dim3(256), 4 * per_row,
                           st, qbar, kbarT, ldk, nqb, nkb, keep, kidx, mask);
    } else if (2 * per_row <= 48 * 1024) {
        hipLaunchKernelGGL((score_topk_kernel<2>), dim3((nqb + 1) / 2, BH), dim3(256), 2 * per_row,
                           st, qbar, kbarT, ldk, nqb, nkb, keep, kidx, mask);
    } else {
        hipLaunchKernelGGL((score_topk_kernel<1>), dim3(nqb, BH), dim3(256), per_row, st, qbar,
                           kbarT, ldk, nqb, nkb, keep, kidx, mask);
    }
    return hipGetLastError();
}

}  // namespace ssa
