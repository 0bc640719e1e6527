// mask.hip -- SLA critical-block selection.
//
// TurboDiffusion pages, page 5 "Four Technical Pillars", Pillar Two (only the
// most important block interactions are computed exactly) and "Hands-On
// Tutorial" (--sla_topk: fraction of key blocks kept). Each query block scores
// every key block by the dot product of their mean-pooled rows (an exact fmaf
// chain over the 128 channels) and keeps the best `keep` under (score
// descending, key block ascending). Selection is an exact 4-pass MSB radix
// select on order-preserving 32-bit keys, one wave per query block, so the
// result is unique and bit-identical to a sort.
#include "common.hpp"
#include "kernels.hpp"

namespace ssa {

__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (s == 0.f) u = 0u;  // -0.0 ranks with +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive and exclusive prefix sums across one wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Selection of one score row by one wave: the `keep` best key blocks under
// (score descending, j ascending), written ascending to krow (and the 0/1
// mask row). An exact MSB radix select finds the keep-th largest key T and
// how many keys equal to T are kept (the lowest j first). The leading bits
// that every key of the row shares (sign and top exponent bits, as a rule)
// are skipped: the keys are shifted left by that count, so the first 8-bit
// pass already spreads over the histogram, and ceil(significant bits / 8)
// passes suffice.
__device__ __forceinline__ void wave_select_row(const float* __restrict__ s, int nkb, int keep,
                                                int* __restrict__ hist, int32_t* __restrict__ krow,
                                                uint8_t* __restrict__ mrow) {
    const int lane = threadIdx.x & 63;
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for (int j = lane; j < nkb; j += 64) {
        const uint32_t key = order_key(s[j]);
        kmin = min(kmin, key);
        kmax = max(kmax, key);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
    }
    const int common = kmin == kmax ? 32 : __builtin_clz(kmin ^ kmax);  // shared leading bits
    const int npass = (32 - common + 7) >> 3;
    uint32_t prefix = 0u, pmask = 0u;  // over the shifted keys
    int rem = keep;
    for (int pass = 0; pass < npass; ++pass) {
        const int shift = 24 - 8 * pass;
#pragma unroll
        for (int b = 0; b < 4; ++b) hist[4 * lane + b] = 0;
        __builtin_amdgcn_wave_barrier();
        for (int j = lane; j < nkb; j += 64) {
            const uint32_t key = order_key(s[j]) << common;  // common < 32 here
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        __builtin_amdgcn_wave_barrier();
        // lane l holds digits 255-4l .. 252-4l (descending); counts of digits
        // above its first one come from the scan
        int hb[4], hsum = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            hb[b] = hist[255 - 4 * lane - b];
            hsum += hb[b];
        }
        const int incl = wave_incl_scan(hsum);
        int above = incl - hsum;  // keys with a digit greater than 255 - 4*lane
        int digit = -1, nrem = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (digit < 0 && above + hb[b] >= rem) {
                digit = 255 - 4 * lane - b;
                nrem = rem - above;
            }
            above += hb[b];
        }
        // exactly one lane found the digit: the one where the count crosses rem
        const uint64_t who = __builtin_amdgcn_ballot_w64(digit >= 0 && (incl - hsum) < rem);
        const int src = (int)__builtin_ctzll(who);
        digit = __shfl(digit, src, 64);
        nrem = __shfl(nrem, src, 64);
        prefix |= (uint32_t)digit << shift;
        pmask |= 255u << shift;
        rem = nrem;
        __builtin_amdgcn_wave_barrier();
    }
    // keep-th largest key; keep `rem` of the keys equal to T (with no pass, every
    // key equals kmin)
    const uint32_t T = npass == 0 ? kmin
                                  : (prefix >> common) | (common ? kmin & (~0u << (32 - common)) : 0u);
    // emit in ascending j, 64 blocks per round: lane l looks at j = 64t + l; a
    // key equal to T is kept while fewer than `rem` equal keys come before it,
    // and the kept blocks of a round are compacted by their rank in the ballot
    const uint64_t below = (1ull << lane) - 1ull;
    int out = 0, eq_seen = 0;
    for (int j0 = 0; j0 < nkb; j0 += 64) {
        const int j = j0 + lane;
        const uint32_t key = j < nkb ? order_key(s[j]) : 0u;
        const bool eq = j < nkb && key == T;
        const uint64_t eqm = __builtin_amdgcn_ballot_w64(eq);
        const bool sel = j < nkb && (key > T || (eq && eq_seen + __builtin_popcountll(eqm & below) < rem));
        const uint64_t selm = __builtin_amdgcn_ballot_w64(sel);
        if (sel) krow[out + __builtin_popcountll(selm & below)] = j;
        if (mrow && j < nkb) mrow[j] = (uint8_t)sel;
        out += __builtin_popcountll(selm);
        eq_seen += __builtin_popcountll(eqm);
    }
}

// One workgroup scores R query blocks of one head against every key block (so
// each pooled-K value read feeds R exact fmaf chains), then each wave selects
// for its rows.
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
    __shared__ int hist[4][256];
    const int tid = threadIdx.x, wave = tid >> 6;
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
    for (int r = wave; r < R; r += 4) {
        const int i = i0 + r;
        if (i >= nqb) break;  // uniform across the wave
        wave_select_row(sc + r * nkb, nkb, keep, hist[wave],
                        kidx + (bh * nqb + i) * (int64_t)keep,
                        mask ? mask + (bh * nqb + i) * (int64_t)nkb : nullptr);
    }
}

hipError_t launch_score_topk(const float* qbar, const float* kbarT, int ldk, int64_t BH, int nqb,
                             int nkb, int keep, int32_t* kidx, uint8_t* mask, hipStream_t st) {
    // largest row group whose scores fit in 48 KB of LDS (nkb <= 8192: SSA_MAX_N)
    const size_t per_row = (size_t)nkb * sizeof(float);
    // (eight rows per workgroup would halve the pooled-K reads, but measured
    // about three times slower on the 1182-block rows: kept at four at most)
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
