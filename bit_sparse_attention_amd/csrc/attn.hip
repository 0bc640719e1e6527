// attn.hip -- the SageSLA sparse attention kernel for gfx950.
//
// TurboDiffusion pages, page 5 "Four Technical Pillars": Pillar One
// (attention in 8-bit integers on the integer matrix units) and Pillar Two
// (only the kept block interactions are computed exactly; a linear-attention
// term covers the rest), stacked as SageSLA.
//
// One workgroup = one 128-token query block of one head, 4 waves x 32 query
// rows. For each kept 64-token key block (ascending):
//   S^T = K_j . Q^T        v_mfma_i32_32x32x32_i8, exact int32
//   x = S * c_ij           c_ij = fl32(fl32(sq*sk) * fl32(sm*log2 e))
//   m = running integer max of ceil(x); rescale by exact powers of two
//   p = bf16(2^(S*c - m)), l += p
//   O^T += V_j^T . P^T     v_mfma_f32_32x32x16_bf16, fp32 accumulation
// Computing S^T (keys as MFMA rows) puts one query per lane column, so the
// row max and row sum stay inside a lane pair, and the int32 accumulator
// order is exactly the bf16 B-operand order of the PV product: P never
// leaves registers. V arrives pre-transposed in that key order (linear.hip).
// The linear branch is applied in the epilogue from the complement states
// (phi(Q) . H_i / phi(Q) . z_i, split-bf16 MFMA) and added to the output.
#include "common.hpp"
#include "kernels.hpp"

namespace ssa {

constexpr int KP = 144;  // LDS row pitch in bytes of the K (int8) and V^T (bf16) tiles

// K tile of key block j -> LDS rows [64][KP], int8, zero past N.
__device__ __forceinline__ void load_k_regs(const int8_t* __restrict__ k_i8, int64_t bh, int N,
                                            int j, int tid, i32x4 (&kr)[2]) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int row = (tid >> 3) + 32 * p;
        const int tok = j * KBLK + row;
        kr[p] = tok < N ? *(const i32x4*)(k_i8 + (bh * N + tok) * HD + 16 * (tid & 7)) : i32x4{};
    }
}

__device__ __forceinline__ void store_k_lds(uint8_t* ks, int tid, const i32x4 (&kr)[2]) {
#pragma unroll
    for (int p = 0; p < 2; ++p) *(i32x4*)(ks + ((tid >> 3) + 32 * p) * KP + 16 * (tid & 7)) = kr[p];
}

// Q operand of one wave: lane supplies query (lane & 31), channels
// 32c + 16*(lane>>5) .. +15 for c = 0..3.
__device__ __forceinline__ void load_q_operand(const int8_t* __restrict__ q_i8, int64_t bh, int N,
                                               int t, int hi, i32x4 (&qop)[4]) {
    const bool ok = t < N;
    const int8_t* qp = q_i8 + (bh * N + (ok ? t : 0)) * HD;
#pragma unroll
    for (int c = 0; c < 4; ++c) qop[c] = ok ? *(const i32x4*)(qp + 32 * c + 16 * hi) : i32x4{};
}

// The shared QK^T routine: S^T for keys 0..31 (s0) and 32..63 (s1) of the LDS
// K tile against the wave's 32 queries. Lane (l32, hi), register r of s0 holds
// key 8*(r/4) + 4*hi + r%4 for query l32 (32 + that for s1).
__device__ __forceinline__ void qk_tile_mfma(const uint8_t* ks, const i32x4 (&qop)[4], int l32,
                                             int hi, i32x16& s0, i32x16& s1) {
    s0 = i32x16{};
    s1 = i32x16{};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const i32x4 a0 = *(const i32x4*)(ks + l32 * KP + 32 * c + 16 * hi);
        const i32x4 a1 = *(const i32x4*)(ks + (32 + l32) * KP + 32 * c + 16 * hi);
        s0 = mfma_i8_32x32x32(a0, qop[c], s0);
        s1 = mfma_i8_32x32x32(a1, qop[c], s1);
    }
}

template <bool LIN>
__global__ __launch_bounds__(256, 2) void sagesla_attn_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t ks[2][KBLK * KP];
    __shared__ __attribute__((aligned(16))) uint8_t vs[2][HD * KP];
    const int64_t total = a.BH * a.nqb;
    const int64_t item = xcd_item(blockIdx.x, total);
    if (item >= total) return;
    const int64_t bh = item / a.nqb;
    const int i = (int)(item % a.nqb);
    const int N = a.N, nkb = a.nkb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31,
              hi = lane >> 5;
    const int t = i * QBLK + wave * 32 + l32;  // this lane's query token

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    if (a.do_sparse) {
        i32x4 qop[4];
        load_q_operand(a.q_i8, bh, N, t, hi, qop);
        const float sq = a.q_scale[bh * a.nqb + i];
        const int nsel = a.kidx ? a.keep : nkb;
        const int32_t* krow = a.kidx ? a.kidx + (bh * a.nqb + i) * (int64_t)a.keep : nullptr;
        const uint16_t* vtb = a.vt + bh * (int64_t)nkb * HD * KBLK;

        i32x4 kr[2], vr[4];
        auto gload = [&](int j) {
            load_k_regs(a.k_i8, bh, N, j, tid, kr);
            const uint16_t* vp = vtb + (int64_t)j * HD * KBLK;
#pragma unroll
            for (int p = 0; p < 4; ++p)
                vr[p] = *(const i32x4*)(vp + ((tid >> 3) + 32 * p) * KBLK + 8 * (tid & 7));
        };
        auto lstore = [&](int buf) {
            store_k_lds(ks[buf], tid, kr);
#pragma unroll
            for (int p = 0; p < 4; ++p)
                *(i32x4*)(vs[buf] + ((tid >> 3) + 32 * p) * KP + 16 * (tid & 7)) = vr[p];
        };

        // kept block indices are clamped into [0, nkb): a malformed kidx can
        // give wrong values but never an access outside K or V
        auto blk = [&](int jj) { return krow ? min(max(krow[jj], 0), nkb - 1) : jj; };
        int j = blk(0);
        gload(j);
        lstore(0);
        __syncthreads();
        for (int jj = 0; jj < nsel; ++jj) {
            const int cur = jj & 1;
            const int jn = (jj + 1 < nsel) ? blk(jj + 1) : -1;
            if (jn >= 0) gload(jn);

            i32x16 s0, s1;
            qk_tile_mfma(ks[cur], qop, l32, hi, s0, s1);

            // softmax statistics on the int32 scores (c > 0 is uniform per tile)
            const int kval = min(KBLK, N - j * KBLK);
            int smax = INT_MIN;
            if (kval == KBLK) {
#pragma unroll
                for (int r = 0; r < 16; ++r) smax = max(smax, max(s0[r], s1[r]));
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = mfma32_row(lane, r);
                    if (key < kval) smax = max(smax, s0[r]);
                    if (key + 32 < kval) smax = max(smax, s1[r]);
                }
            }
            smax = max(smax, __shfl_xor(smax, 32, 64));
            const float sk = a.k_scale[bh * nkb + j];
            const float c = (sq * sk) * a.K32;
            const float mt = ceilf((float)smax * c);
            if (mt > m_run) {
                const float alpha =
                    (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_ldexpf(1.0f, (int)(m_run - mt));
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
                l_run *= alpha;
                m_run = mt;
            }
            const float nm = -m_run;
            bf16x8 pb[4];
            float lsum = 0.f;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int r = 8 * (cc & 1) + s;
                    const int sv = (cc < 2) ? s0[r] : s1[r];
                    float p = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sv, c, nm));
                    if (kval < KBLK) {
                        const int key = 16 * cc + 8 * (s >> 2) + 4 * hi + (s & 3);
                        if (key >= kval) p = 0.f;
                    }
                    const __bf16 pbv = (__bf16)p;
                    pb[cc][s] = pbv;
                    lsum += (float)pbv;
                }
            }
            l_run += lsum;

#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const bf16x8 va =
                        *(const bf16x8*)(vs[cur] + (32 * dt + l32) * KP + (16 * cc + 8 * hi) * 2);
                    o[dt] = mfma_bf16_32x32x16(va, pb[cc], o[dt]);
                }

            if (jn >= 0) lstore(cur ^ 1);
            __syncthreads();
            j = jn;
        }
    }

    const float lt = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = a.do_sparse ? 1.0f / lt : 0.f;

    f32x16 ol[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) ol[dt] = f32x16{};
    float linv = 0.f;
    if (LIN) {
        const float* hp = a.hnon + (bh * a.nqb + i) * (int64_t)HS_ROW;
        const bool ok = t < N;
        const uint16_t* qr = a.q + (bh * N + (ok ? t : 0)) * HD;
        float den = 0.f;
#pragma unroll 2
        for (int cd = 0; cd < 8; ++cd) {
            const int d0 = 16 * cd + 8 * hi;
            const u16x8 qv = ok ? *(const u16x8*)(qr + d0) : u16x8{};
            const f32x4 z0 = *(const f32x4*)(hp + HD * HD + d0);
            const f32x4 z1 = *(const f32x4*)(hp + HD * HD + d0 + 4);
            bf16x8 bqh, bql;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const float f = bf2f(qv[s]);
                const float ph = f > 0.f ? f + 1.f : __expf(f);
                __bf16 h, l;
                split_bf16(ph, h, l);
                bqh[s] = h;
                bql[s] = l;
                den = __builtin_fmaf(ph, s < 4 ? z0[s] : z1[s - 4], den);
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const float* hr = hp + (32 * dt + l32) * HD + d0;
                const f32x4 h0 = *(const f32x4*)hr, h1 = *(const f32x4*)(hr + 4);
                bf16x8 ah, al;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    __bf16 x, y;
                    split_bf16(s < 4 ? h0[s] : h1[s - 4], x, y);
                    ah[s] = x;
                    al[s] = y;
                }
                ol[dt] = mfma_bf16_32x32x16(ah, bqh, ol[dt]);
                ol[dt] = mfma_bf16_32x32x16(ah, bql, ol[dt]);
                ol[dt] = mfma_bf16_32x32x16(al, bqh, ol[dt]);
            }
        }
        den += __shfl_xor(den, 32, 64);
        linv = 1.0f / den;
    }

    if (t < N) {
        uint16_t* orow = a.out + (bh * N + t) * HD;
        float* orow32 = a.out32 ? a.out32 + (bh * N + t) * HD : nullptr;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dv = 32 * dt + 8 * g + 4 * hi;
                float r4[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float val = o[dt][4 * g + u] * inv;
                    if (LIN) val += ol[dt][4 * g + u] * linv;
                    r4[u] = val;
                }
                *(u16x4*)(orow + dv) = u16x4{f2bf(r4[0]), f2bf(r4[1]), f2bf(r4[2]), f2bf(r4[3])};
                if (orow32) *(f32x4*)(orow32 + dv) = f32x4{r4[0], r4[1], r4[2], r4[3]};
            }
    }
}

// Raw int32 tiles through the same LDS staging and qk_tile_mfma routine.
__global__ __launch_bounds__(256) void qk_tiles_kernel(const int8_t* __restrict__ q_i8,
                                                       const int8_t* __restrict__ k_i8, int64_t BH,
                                                       int N, const int32_t* __restrict__ tiles,
                                                       int32_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint8_t ks[KBLK * KP];
    const int64_t tix = blockIdx.x;
    const int nqb = (N + QBLK - 1) / QBLK, nkb = (N + KBLK - 1) / KBLK;
    const int64_t bh = tiles[3 * tix];
    const int i = tiles[3 * tix + 1], j = tiles[3 * tix + 2];
    const bool valid = bh >= 0 && bh < BH && i >= 0 && i < nqb && j >= 0 && j < nkb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31,
              hi = lane >> 5;
    int32_t* ot = out + tix * QBLK * KBLK;
    if (!valid) {
        for (int x = tid; x < QBLK * KBLK; x += 256) ot[x] = 0;
        return;
    }
    i32x4 kr[2];
    load_k_regs(k_i8, bh, N, j, tid, kr);
    store_k_lds(ks, tid, kr);
    __syncthreads();
    i32x4 qop[4];
    const int t = i * QBLK + wave * 32 + l32;
    load_q_operand(q_i8, bh, N, t, hi, qop);
    i32x16 s0, s1;
    qk_tile_mfma(ks, qop, l32, hi, s0, s1);
    const int row = wave * 32 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int key = mfma32_row(lane, r);
        ot[row * KBLK + key] = s0[r];
        ot[row * KBLK + key + 32] = s1[r];
    }
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
    const int64_t total = a.BH * a.nqb;
    const int64_t grid = (total + 7) / 8 * 8;
    if (a.hnon)
        hipLaunchKernelGGL((sagesla_attn_kernel<true>), dim3((unsigned)grid), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((sagesla_attn_kernel<false>), dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_qk_tiles(const int8_t* q_i8, const int8_t* k_i8, int64_t BH, int N,
                           const int32_t* tiles, int64_t T, int32_t* out, hipStream_t st) {
    hipLaunchKernelGGL(qk_tiles_kernel, dim3((unsigned)T), dim3(256), 0, st, q_i8, k_i8, BH, N,
                       tiles, out);
    return hipGetLastError();
}

}  // namespace ssa
