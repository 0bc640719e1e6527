// linear.hip -- the linear-attention branch of SageSLA, and the V re-layout
// the sparse kernel reads.
//
// TurboDiffusion pages, page 5 "Four Technical Pillars", Pillar Two: the
// block interactions the sparse part skips are handled by a cheap
// linear-attention term instead. With phi = elu + 1 on raw K, each 64-token key block
// j contributes the state h_j = sum_u phi(k_u) v_u^T (128 x 128) and
// z_j = sum_u phi(k_u). A query block needs the sums over the key blocks it did
// NOT keep. They are formed as H_i = H_total - sum_{j kept} h_j: H_total in
// fp32, the kept-block sum as a dense 0/1 x bf16 matrix-core GEMM, so the bf16
// rounding of h_j only touches the kept ~10% of the blocks. When more than
// half the blocks are kept the GEMM sums the non-kept ones directly instead,
// H_i = sum_{j not kept} h_j, so the rounding always touches the smaller set.
#include <type_traits>

#include "../../include/ssa.h"
#include "common.hpp"
#include "kernels.hpp"

namespace ssa {

constexpr int TP = KBLK + 8;  // LDS pitch (bf16) of a [channel][token] tile: 144 B
// LDS pitch (bf16) of a [token][channel] tile: 288 B, so the four token rows a
// transposing read touches land in disjoint groups of 8 banks
constexpr int RP = HD + 16;
constexpr int LS_THREADS = 512;                       // 8 waves
constexpr int LS_IT = KBLK * HD / 8 / LS_THREADS;     // 16-byte chunks per thread per tile

// Eight consecutive tokens t0 .. t0+7 of channel c0 + (lane & 15), from a
// token-major LDS tile of pitch RP, as one bf16 MFMA operand (element k =
// token t0 + k). t0 and c0 are uniform within each 16-lane group: lane i
// points at token t0 + i/4, channels c0 + 4(i%4) .. +3, and the transposing
// read hands it channel c0 + i at tokens t0 .. t0+3 (then t0+4 .. t0+7).
__device__ __forceinline__ bf16x8 tok8(const uint16_t* tile, int t0, int c0, int lane) {
    const int i = lane & 15;
    const uint16_t* p = tile + (t0 + (i >> 2)) * RP + c0 + 4 * (i & 3);
    const i16x4 a = lds_read_tr16(p), b = lds_read_tr16(p + 4 * RP);
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(bf16x8, i16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
}

// Position p (0..63) of a re-laid V tile row holds key 16*(p/16) + kperm(p%16):
// the order in which one lane of the 32x32 MFMA output holds its keys, so the
// sparse kernel feeds its P registers to the PV product without shuffles.
//   positions 0-3 -> keys 0-3, 4-7 -> 8-11, 8-11 -> 4-7, 12-15 -> 12-15.

// Per 64-token key block: V^T re-laid for the sparse kernel, and (STATES)
// the linear state h_j^T and z_j as one bf16 row of HS_ROW (for the GEMM), and
// an fp32 running sum over the workgroup's LIN_GROUP key blocks. Row e of h^T
// holds d at position 16cd + 8hi + s for d = 16cd + 8(s/4) + 4hi + s%4 (the
// order in which one lane of the 32x32 MFMA output holds its rows), and z
// follows in the same d order; the GEMM and the apply only need a consistent
// order. The h^T rows are staged in LDS and stored as whole rows.
//
// SUMS: the same pass over K also yields what the K mean and the block mask
// need from raw K, so that K is read once before its quantization instead of
// twice: per key block, kpart[bh][j][d] = the fp32 sum of the block's valid
// tokens of channel d, added in token order from 0 (the block partial of the
// K mean), and kbarT[bh][d][j] = kpart / valid (the pooled key mean, stored
// transposed with row pitch ldk; skipped when kbarT is null). Raw K is staged
// token-major in LDS and one thread adds one channel's column in order, so
// both equal what colsum_kernel<64, 0> writes, bit for bit.
//
// LO: also write hs_lo = bf16(state - hs), the bf16 rest of each state entry,
// so that a product taken with both stacks carries ~16 significant bits (the
// backward's states, whose cancellations the bf16 rounding alone would show).
template <bool STATES, bool SUMS, bool LO = false>
__global__ __launch_bounds__(LS_THREADS, 1) void linear_states_kernel(const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v, int N,
                                                            int nkb, int ngroups,
                                                            uint16_t* __restrict__ vt,
                                                            uint16_t* __restrict__ hs,
                                                            uint16_t* __restrict__ hs_lo,
                                                            float* __restrict__ hpart,
                                                            float* __restrict__ kpart,
                                                            float* __restrict__ kbarT, int ldk) {
    constexpr int KBP = HD + 1;  // pitch of the staged pooled means (no bank conflicts)
    // token-major tiles of the block (V; elu+1 of K as bf16 high parts and
    // rests; raw K), written with one 16-byte store per chunk, and V^T
    // channel-major for the re-laid copy
    __shared__ __attribute__((aligned(16))) uint16_t vtok[KBLK * RP];
    __shared__ __attribute__((aligned(16))) uint16_t vtl[HD * TP];
    __shared__ __attribute__((aligned(16))) uint16_t fh[STATES ? KBLK * RP : 8];
    __shared__ __attribute__((aligned(16))) uint16_t fl[STATES ? KBLK * RP : 8];
    __shared__ __attribute__((aligned(16))) uint16_t kraw[SUMS ? KBLK * RP : 8];
    __shared__ float kbs[SUMS ? LIN_GROUP * KBP : 1];
    // the block's state rows h^T (and their bf16 rests), staged so that they
    // leave as whole rows; pitch 272 B, so the 16 rows a 16-lane group writes
    // at one position fall in distinct banks
    constexpr int HP = HD + 8;
    __shared__ __attribute__((aligned(16))) uint16_t hst[STATES ? HD * HP : 8];
    __shared__ __attribute__((aligned(16))) uint16_t hstl[(STATES && LO) ? HD * HP : 8];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31,
              hi = lane >> 5;
    // wave (eg, dh) owns the state columns e = 32eg .. 32eg+31 and rows
    // d = 64dh .. 64dh+63 (row tiles dt = 2dh, 2dh+1); the waves with dh = 0
    // also own z rows d = 32eg .. 32eg+31
    const int eg = wave & 3, dh = wave >> 2;
    const int64_t bh = blockIdx.y;
    const int g = blockIdx.x;
    const int G = (STATES || SUMS) ? LIN_GROUP : 1;
    f32x16 tot[2], totz = f32x16{};
#pragma unroll
    for (int t = 0; t < 2; ++t) tot[t] = f32x16{};
    // raw K and V of one key block in registers: thread tid holds chunk c =
    // tid + 512*it, i.e. token u = c / 16, channels 8ch .. 8ch+7 for ch = c % 16,
    // so each wave reads four whole 256-byte token rows. Two sets, so the loads
    // of blocks j+1 and j+2 are in flight while block j is worked.
    u16x8 va[LS_IT], ka[LS_IT], vb[LS_IT], kb[LS_IT];
    auto load = [&](int j, u16x8 (&vv)[LS_IT], u16x8 (&kk)[LS_IT]) {
#pragma unroll
        for (int it = 0; it < LS_IT; ++it) {
            const int c = tid + LS_THREADS * it;
            const int u = c >> 4, ch = c & 15;
            const int tok = j * KBLK + u;
            const bool ok = tok < N;
            const int64_t off = (bh * N + (ok ? tok : 0)) * HD + 8 * ch;
            vv[it] = ok ? *(const u16x8*)(v + off) : u16x8{};
            if (STATES || SUMS) kk[it] = ok ? *(const u16x8*)(k + off) : u16x8{};
        }
    };
    auto block = [&](int jb, u16x8 (&vv)[LS_IT], u16x8 (&kk)[LS_IT]) {
        const int j = g * G + jb;
        // token-major LDS stores: a 16-lane group writes one 256-byte row
#pragma unroll
        for (int it = 0; it < LS_IT; ++it) {
            const int c = tid + LS_THREADS * it;
            const int u = c >> 4, ch = c & 15;
            const bool ok = j * KBLK + u < N;
            *(u16x8*)(vtok + u * RP + 8 * ch) = vv[it];
            if (SUMS) *(u16x8*)(kraw + u * RP + 8 * ch) = kk[it];
            if (STATES) {
                u16x8 h8, l8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float f = bf2f(kk[it][e]);
                    // elu + 1 without branches: the exp of min(f, 0) is finite and
                    // is selected only for f <= 0; invalid tokens are scaled to 0
                    const float ex = __expf(fminf(f, 0.f));
                    const float ph = (f > 0.f ? f + 1.f : ex) * (ok ? 1.f : 0.f);
                    __bf16 h, l;
                    split_bf16(ph, h, l);
                    h8[e] = __builtin_bit_cast(uint16_t, h);
                    l8[e] = __builtin_bit_cast(uint16_t, l);
                }
                *(u16x8*)(fh + u * RP + 8 * ch) = h8;
                *(u16x8*)(fl + u * RP + 8 * ch) = l8;
            }
        }
        __syncthreads();
        // the registers are free again: block j+2 goes in flight
        if (jb + 2 < G && j + 2 < nkb) load(j + 2, vv, kk);
        // V^T channel-major for the re-laid copy (stored after the block's
        // last barrier): 16 token quads x 8 groups of 16 channels, four per
        // 16-lane group, each a transposing read and one 8-byte store
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int item = (tid >> 4) + 32 * r;
            const int c0 = 16 * (item & 7), t0 = 4 * (item >> 3), i = tid & 15;
            const i16x4 q = lds_read_tr16(vtok + (t0 + (i >> 2)) * RP + c0 + 4 * (i & 3));
            *(i16x4*)(vtl + (c0 + i) * TP + t0) = q;
        }
        // K sums: thread tid adds the column of channel d = tid % 128 in token
        // order, 16 tokens at a time, and waves 4 and 5 store the result. With
        // the states every wave runs the adds, one piece after each step of
        // MFMAs: that measured 40 us faster at 40 x 75600 tokens than adds in
        // waves 4 and 5 only, whose per-lane branch kept the scheduler from
        // overlapping them with the MFMAs.
        const bool sumw = SUMS && tid >= 256 && tid < 256 + HD;
        const int dsum = tid & (HD - 1);
        const int valid = min(KBLK, N - j * KBLK);
        float ksum = 0.f;
        // The full-block / ragged-block choice is uniform; its branch also
        // keeps each piece of adds between its group of MFMAs and the next
        // (without it the compiler moves all 64 adds behind the last MFMA,
        // measured 60 us slower at 40 x 75600 tokens).
        auto sum16 = [&](int uc) {
            // tokens 16uc .. 16uc+15 of channel dsum (= 16*(dsum/16) + lane % 16)
            uint16_t r[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = tid & 15;
                const i16x4 x = lds_read_tr16(kraw + (16 * uc + 4 * q + (i >> 2)) * RP +
                                              (dsum & ~15) + 4 * (i & 3));
#pragma unroll
                for (int e = 0; e < 4; ++e) r[4 * q + e] = (uint16_t)x[e];
            }
            if (valid == KBLK) {
#pragma unroll
                for (int e = 0; e < 16; ++e) ksum += bf2f(r[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (16 * uc + e < valid) ksum += bf2f(r[e]);
            }
        };
        if (SUMS && !STATES && sumw)
#pragma unroll
            for (int uc = 0; uc < 4; ++uc) sum16(uc);
        if (STATES) {
            // (h_j^T)^T[d][e] = sum_u phi(K)[u][d] V[u][e]: A = phi(K)^T rows d (hi and
            // lo parts, two products, fp32 accumulation), B = V columns e. This
            // wave takes columns e = 32eg .. 32eg+31; acc[t] holds rows
            // d = 32(2dh + t) + ...
            f32x16 acc[2], accz = f32x16{};
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[t] = f32x16{};
            bf16x8 ones;
#pragma unroll
            for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
            // operands through transposing reads: lane (l32, hi) takes tokens
            // 16uc + 8hi .. +7 of its row d (or column e); its 16-lane group
            // covers 16 consecutive channels from 32(tile) + 16(l32 / 16)
            const int cq = 16 * (l32 >> 4);
#pragma unroll
            for (int uc = 0; uc < 4; ++uc) {
                const bf16x8 b = tok8(vtok, 16 * uc + 8 * hi, 32 * eg + cq, lane);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int dt = 2 * dh + t;
                    const bf16x8 ah = tok8(fh, 16 * uc + 8 * hi, 32 * dt + cq, lane);
                    const bf16x8 al = tok8(fl, 16 * uc + 8 * hi, 32 * dt + cq, lane);
                    acc[t] = mfma_bf16_32x32x16(ah, b, acc[t]);
                    acc[t] = mfma_bf16_32x32x16(al, b, acc[t]);
                }
                if (SUMS) sum16(uc);
            }
            // z_j[d] for rows d = 32eg + ...: the same product against ones
            if (dh == 0) {
#pragma unroll
                for (int uc = 0; uc < 4; ++uc) {
                    accz = mfma_bf16_32x32x16(tok8(fh, 16 * uc + 8 * hi, 32 * eg + cq, lane), ones, accz);
                    accz = mfma_bf16_32x32x16(tok8(fl, 16 * uc + 8 * hi, 32 * eg + cq, lane), ones, accz);
                }
            }
            // lane (column e = 32eg + l32, hi) holds rows d = 32dt + 8(r/4) + 4hi + r%4:
            // registers 8rb .. 8rb+7 are positions 16(2dt + rb) + 8hi + 0..7 of row e
            uint16_t* hrow = hs + (bh * nkb + j) * (int64_t)HS_ROW;
            const int e = 32 * eg + l32;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int dt = 2 * dh + t;
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    u16x8 o8, l8;
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        o8[x] = f2bf(acc[t][8 * rb + x]);
                        if (LO) l8[x] = f2bf(acc[t][8 * rb + x] - bf2f(o8[x]));
                    }
                    *(u16x8*)(hst + e * HP + 16 * (2 * dt + rb) + 8 * hi) = o8;
                    if (LO) *(u16x8*)(hstl + e * HP + 16 * (2 * dt + rb) + 8 * hi) = l8;
                }
                tot[t] += acc[t];
            }
            if (dh == 0) {
                if (l32 == 0) {  // z rows d = 32eg + ..., every column equal
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        u16x8 o8, l8;
#pragma unroll
                        for (int x = 0; x < 8; ++x) {
                            o8[x] = f2bf(accz[8 * rb + x]);
                            if (LO) l8[x] = f2bf(accz[8 * rb + x] - bf2f(o8[x]));
                        }
                        *(u16x8*)(hrow + HD * HD + 16 * (2 * eg + rb) + 8 * hi) = o8;
                        if (LO)
                            *(u16x8*)(hs_lo + (hrow - hs) + HD * HD + 16 * (2 * eg + rb) + 8 * hi) = l8;
                    }
                }
                totz += accz;
            }
        }
        if (SUMS && sumw) {
            kpart[(bh * nkb + j) * HD + dsum] = ksum;
            kbs[jb * KBP + dsum] = ksum / (float)valid;
        }
        __syncthreads();
        // The state rows from LDS as whole 256-byte rows (a wave stores 1 KB
        // at a time); like vtl below, hst is written again only after the next
        // block's first barrier.
        if (STATES) {
            const int64_t hoff = (bh * nkb + j) * (int64_t)HS_ROW;
#pragma unroll
            for (int c = tid; c < HD * 16; c += LS_THREADS) {
                const int r = c >> 4, q = c & 15;
                *(u16x8*)(hs + hoff + r * HD + 8 * q) = *(const u16x8*)(hst + r * HP + 8 * q);
                if (LO)
                    *(u16x8*)(hs_lo + hoff + r * HD + 8 * q) = *(const u16x8*)(hstl + r * HP + 8 * q);
            }
        }
        // V^T tile in the sparse kernel's key order: 128 rows x 8 chunks of
        // 16 B (the next block writes vtl only after its first barrier, which
        // every thread reaches after these reads)
#pragma unroll
        for (int it = 0; it < LS_IT; ++it) {
            const int c = tid + LS_THREADS * it;
            const int dv = c >> 3, pc = c & 7, cc = pc >> 1, h2 = pc & 1;
            const u16x4 a = *(const u16x4*)(vtl + dv * TP + 16 * cc + 4 * h2);
            const u16x4 b = *(const u16x4*)(vtl + dv * TP + 16 * cc + 8 + 4 * h2);
            *(u16x8*)(vt + ((bh * nkb + j) * HD + dv) * KBLK + 8 * pc) =
                u16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        }
    };
    const int nb = min(G, nkb - g * G);  // key blocks of this workgroup
    if (nb > 0) load(g * G, va, ka);
    if (nb > 1) load(g * G + 1, vb, kb);
    for (int jb = 0; jb < nb; jb += 2) {
        block(jb, va, ka);
        if (jb + 1 < nb) block(jb + 1, vb, kb);
    }
    if (SUMS && kbarT) {
        // the group's pooled means (staged before the last barrier of the
        // block loop) as runs of up to LIN_GROUP consecutive blocks per channel
        for (int idx = tid; idx < HD * LIN_GROUP; idx += LS_THREADS) {
            const int d = idx / LIN_GROUP, i = idx % LIN_GROUP;
            if (i < nb) kbarT[(bh * HD + d) * (int64_t)ldk + g * G + i] = kbs[i * KBP + d];
        }
    }
    if (STATES) {
        float* prow = hpart + (bh * ngroups + g) * (int64_t)HS_ROW;
        const int e = 32 * eg + l32;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                float* dst = prow + e * HD + 16 * (2 * (2 * dh + t) + rb) + 8 * hi;
                *(f32x4*)dst = f32x4{tot[t][8 * rb], tot[t][8 * rb + 1], tot[t][8 * rb + 2],
                                     tot[t][8 * rb + 3]};
                *(f32x4*)(dst + 4) = f32x4{tot[t][8 * rb + 4], tot[t][8 * rb + 5],
                                           tot[t][8 * rb + 6], tot[t][8 * rb + 7]};
            }
        if (dh == 0 && l32 == 0)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                float* dst = prow + HD * HD + 16 * (2 * eg + rb) + 8 * hi;
                *(f32x4*)dst = f32x4{totz[8 * rb], totz[8 * rb + 1], totz[8 * rb + 2], totz[8 * rb + 3]};
                *(f32x4*)(dst + 4) =
                    f32x4{totz[8 * rb + 4], totz[8 * rb + 5], totz[8 * rb + 6], totz[8 * rb + 7]};
            }
    }
}

// H_total[bh][n] = sum over groups, in group order, of the fp32 partials.
__global__ __launch_bounds__(256) void htot_kernel(const float* __restrict__ hpart, int ngroups,
                                                   float* __restrict__ htot) {
    // thread: four consecutive entries n = 4*n4 .. +3, one 16-byte load per group
    const int n4 = blockIdx.x * 256 + threadIdx.x;
    const int64_t bh = blockIdx.y;
    if (n4 >= HS_ROW / 4) return;
    // loads in batches of 16 groups so they are in flight together (the index
    // clamped, so every load is unconditional); the adds stay in group order
    const float* p = hpart + bh * ngroups * (int64_t)HS_ROW + 4 * n4;
    f32x4 s = f32x4{};
    for (int g0 = 0; g0 < ngroups; g0 += 16) {
        f32x4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = *(const f32x4*)(p + (int64_t)min(g0 + u, ngroups - 1) * HS_ROW);
#pragma unroll
        for (int u = 0; u < 16; ++u)
            if (g0 + u < ngroups) s += v[u];
    }
    *(f32x4*)(htot + bh * HS_ROW + 4 * n4) = s;
}

// ---- the 0/1 selection matrix, as offsets into a bf16 expansion table ------
// The complement GEMM multiplies the state stack by each query block's 0/1
// row over the key blocks. That row is kept as bits: bit s of byte b is key
// block 8b + s. A byte becomes one MFMA operand fragment (eight bf16 0/1
// values) by a 16-byte read of a 256-entry table in LDS, so the selection
// costs 1/16 of its bf16 size in memory and in the GEMM's load path.
//
// Table slot of entry e: 16*(e>>4) + ((e & 15) ^ h(e>>4)), h a fixed nibble
// permutation with h(0) = 0. It puts the entries of one-bit bytes (1, 2, 4,
// ..., 128) and 0, the common ones at 10% density, in distinct LDS bank
// groups, so a 16-lane read of such entries has no bank conflict.
__device__ __forceinline__ uint32_t sel_slot(uint32_t e) {
    constexpr uint64_t H = 0x8421FED7CBA69530ull;  // h(0..15) = 0,3,5,9,6,10,11,12,7,13,14,15,1,2,4,8
    return (e & 0xF0u) | ((e & 15u) ^ (uint32_t)((H >> (4 * (e >> 4))) & 15u));
}

// Table entry e: element s (0..7) of the fragment is bf16(1) if bit s of e is
// set, else 0; element pairs (2q, 2q+1) form dword q.
__device__ __forceinline__ u32x4 sel_entry(uint32_t e) {
    u32x4 d;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        d[q] = (((e >> (2 * q)) & 1u) ? 0x3F80u : 0u) | (((e >> (2 * q + 1)) & 1u) ? 0x3F800000u : 0u);
    return d;
}

// Selection rows in the order the GEMM reads them. K step ks covers key
// blocks 32ks .. 32ks+31, bytes b0..b3 of that word. An MFMA lane of k-half
// hi needs bytes hi and 2+hi of each K step, as table slots. Steps are paired
// (kp = ks/2) and a row of a pair is 8 bytes: dword hi holds
// slot(b_hi), slot(b_{2+hi}) of step 2kp, then the same of step 2kp+1, one
// byte each. Layout [bh][kp][i][8 bytes] over an even row count (rows past
// the last one select nothing), so that one 16-byte load takes two rows.
// Key blocks past nkb, and the second step of an unpaired last one, select
// nothing. Rows come from kidx (keep entries each) or, for the backward's
// transposed selection, from lists (counts[bh][row] entries each, row length
// ld).
constexpr int SEL_MAX_WORDS = SSA_MAX_N / KBLK / 32 + 2;
template <bool LISTS>
__global__ __launch_bounds__(256) void msel_kernel(const int32_t* __restrict__ kidx, int keep,
                                                   const uint16_t* __restrict__ lists,
                                                   const int32_t* __restrict__ counts, int ld,
                                                   int nqb, int nkb, int nks, int complement,
                                                   uint32_t* __restrict__ msel) {
    __shared__ uint32_t bits[SEL_MAX_WORDS];
    const int64_t bh = blockIdx.y;
    const int i = blockIdx.x;
    const int nkp = (nks + 1) / 2, nqbp = (nqb + 1) & ~1;
    const bool pad = i >= nqb;
    for (int w = threadIdx.x; w < 2 * nkp; w += 256) bits[w] = 0;
    __syncthreads();
    // kept block indices are clamped into [0, nkb)
    if (pad) {
    } else if (LISTS) {
        const uint16_t* src = lists + (bh * nqb + i) * (int64_t)ld;
        const int n = counts[bh * nqb + i];
        for (int a = threadIdx.x; a < n; a += 256) {
            const int j = min((int)src[a], nkb - 1);
            atomicOr(&bits[j >> 5], 1u << (j & 31));
        }
    } else {
        const int32_t* src = kidx + (bh * nqb + i) * (int64_t)keep;
        for (int a = threadIdx.x; a < keep; a += 256) {
            const int j = min(max(src[a], 0), nkb - 1);
            atomicOr(&bits[j >> 5], 1u << (j & 31));
        }
    }
    __syncthreads();
    if (complement && !pad) {
        // the blocks below nkb that are not kept
        for (int w = threadIdx.x; w < 2 * nkp; w += 256) {
            const int lo = 32 * w;
            const uint32_t valid = lo >= nkb ? 0u : (nkb - lo >= 32 ? ~0u : (1u << (nkb - lo)) - 1u);
            bits[w] = ~bits[w] & valid;
        }
        __syncthreads();
    }
    for (int kp = threadIdx.x; kp < nkp; kp += 256) {
        u32x2 o = u32x2{0u, 0u};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint32_t x = bits[2 * kp + half];
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                const uint32_t lo8 = (x >> (8 * hi)) & 255u, hi8 = (x >> (8 * (2 + hi))) & 255u;
                o[hi] |= (sel_slot(lo8) | sel_slot(hi8) << 8) << (16 * half);
            }
        }
        *(u32x2*)(msel + ((bh * nkp + kp) * nqbp + i) * 2) = o;
    }
}

// Complement GEMM, computed transposed:
//   hnon[bh][i][n] = htot[bh][n] - sum_j hs[bh][j][n] * sel[bh][i][j]
// or, with `complement` (the selection rows then mark the non-kept blocks),
//   hnon[bh][i][n] = sum_j hs[bh][j][n] * sel[bh][i][j]
// for query blocks i < nqb, state entries n < HS_ROW, key blocks j < nkbp.
// With LO the states are given as a bf16 stack and a second stack of each
// entry's bf16 rest, and hs[j][n] is their sum: both products go into the
// same fp32 accumulators.
// C^T = Hs^T . Sel^T on 32x32x16 bf16 MFMAs with fp32 accumulation: the A
// operand is a state fragment, the B operand a selection fragment from the
// table, and each lane of the result holds four consecutive n of one i.
//
// Workgroup tile: 64 n x 640 i (every query block of a head, up to 640).
// Wave w owns rows 160w .. 160w+159 (five 32-row blocks) against both 32-wide
// halves of n: 10 accumulators. The K loop runs over pairs of 32-key-block
// steps; a pair's operands form one stage of a 3-deep LDS ring, fetched by LDS
// DMA two stages ahead:
//   the [64 j][64 n] bf16 state tile (8 KB, 128-byte rows; with LO the rest
//     tile after it), two 1 KB DMAs per wave and tile; 16-byte chunk c of row
//     r sits at chunk c ^ 4*((r >> 1) & 1), and the tile is read with
//     transposing loads (lds_read_tr16) that give a lane 4 consecutive j of
//     one n, the 32 lanes of a half wave hitting distinct 8-byte bank groups;
//   the pair's selection (8 bytes per row), each wave fetching its own 160
//     rows (1280 bytes: one full DMA and a quarter of one).
// The whole state stack is read once.
constexpr int CG_TN = 64;                  // state entries per workgroup
constexpr int CG_IB = 5;                   // 32-row query blocks per wave
constexpr int CG_WROWS = 32 * CG_IB;       // query blocks per wave
constexpr int CG_TM = 4 * CG_WROWS;        // query blocks per workgroup
constexpr int CG_TK = GEMM_KALIGN;         // key blocks per selection word (half a stage)
constexpr int CG_STAGES = 3;
constexpr int CG_TILE = 2 * CG_TK * CG_TN * 2;  // bytes of a stage's state tile [64 j][64 n]
constexpr int CG_SELROW = 8;                    // selection bytes per row and stage
constexpr int CG_SEL = CG_TM * CG_SELROW;       // bytes of a stage's selection
constexpr int CG_LUT = 256 * 16;                // bytes of the expansion table
template <bool LO>
constexpr int cg_stage() { return (LO ? 2 : 1) * CG_TILE + CG_SEL; }
template <bool LO>
constexpr int cg_lds() { return CG_STAGES * cg_stage<LO>() + CG_LUT; }
static_assert(CG_TK == 32, "selection dword per lane per 32 key blocks");
static_assert(HS_ROW % CG_TN == 0, "state rows split into whole column tiles");
static_assert(CG_WROWS * CG_SELROW == 1024 + 16 * 16, "selection DMAs: one of 128 rows and one of 32 per wave");
static_assert(2 * cg_lds<true>() <= 160 * 1024, "two workgroups per CU");

int64_t complement_tiles_per_head(int64_t nqb) {
    return (int64_t)(HS_ROW / CG_TN) * ((nqb + CG_TM - 1) / CG_TM);
}

size_t msel_bytes(int64_t BH, int64_t nqb, int64_t nkbp) {
    const int64_t nkp = (nkbp / CG_TK + 1) / 2;
    return (size_t)BH * nkp * ((nqb + 1) & ~int64_t(1)) * CG_SELROW;
}

template <bool LO>
__global__ __launch_bounds__(256, 2) void complement_gemm_kernel(
    const uint32_t* __restrict__ msel, const uint16_t* __restrict__ hs,
    const uint16_t* __restrict__ hs_lo, const float* __restrict__ htot, int64_t BH, int nqb,
    int nkb, int nkbp, int complement, float* __restrict__ hnon) {
    constexpr int STAGE = cg_stage<LO>();
    constexpr int NT = LO ? 2 : 1;  // state tiles per stage
    constexpr int DMAS = 2 * NT + 2;  // LDS DMAs per wave and stage
    __shared__ __attribute__((aligned(1024))) uint8_t smem[cg_lds<LO>()];
    uint8_t* lut = smem + CG_STAGES * STAGE;
    const int nnt = HS_ROW / CG_TN, nmt = (nqb + CG_TM - 1) / CG_TM;
    const int64_t total = BH * nnt * nmt;
    const int64_t item = xcd_item(blockIdx.x, total);  // i tiles fastest: they share state tiles
    if (item >= total) return;
    const int mt = (int)(item % nmt);
    const int64_t rest = item / nmt;
    const int nt = (int)(rest % nnt);
    const int64_t bh = rest / nnt;
    const int i0 = mt * CG_TM, n0 = nt * CG_TN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31,
              hi = lane >> 5;
    const int nks = nkbp / CG_TK, nkp = (nks + 1) / 2, nqbp = (nqb + 1) & ~1;
    const int iw = i0 + CG_WROWS * wave;  // first query block of this wave (even)

    *(u32x4*)(lut + 16 * sel_slot((uint32_t)tid)) = sel_entry((uint32_t)tid);

    // stage kp: state rows j = 64kp .. 64kp+63 (wave w fills rows 16w .. 16w+15
    // of each tile, two DMAs; lane l row 16w + 8p + l/8 at slot l%8, holding
    // chunk (l%8) ^ 4*((row >> 1) & 1)) and the selection of that K-step pair
    // (lane l of DMA p: rows 2(64p + l), +1 of the wave's, past the padded row
    // count re-reading the last two)
    const int dchunk = (lane & 7) ^ (4 * (((lane >> 3) >> 1) & 1));
    const int64_t sbase0 = (bh * nkb) * (int64_t)HS_ROW + n0;
    auto issue = [&](int kp, int st) {
        uint8_t* T = smem + st * STAGE;
        uint8_t* S = T + NT * CG_TILE;
        const uint32_t* sbase = msel + (bh * nkp + kp) * (int64_t)nqbp * 2;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int c = min((iw >> 1) + 64 * p + lane, (nqbp >> 1) - 1);
            if (p == 0 || lane < 16)
                dma16(sbase, (uint32_t)(c * 16), lds_u32(S + CG_WROWS * CG_SELROW * wave + 1024 * p));
        }
        const int j0 = 2 * CG_TK * kp;
        // rows past nkb (their selection bits are 0) re-read row nkb-1; j0 < nkb
        // because nkbp rounds nkb up by less than one selection word
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int row = 16 * wave + 8 * p + (lane >> 3);
                const int r = min(j0 + row, nkb - 1) - j0;
                dma16((t ? hs_lo : hs) + sbase0 + (int64_t)j0 * HS_ROW,
                      (uint32_t)(r * HS_ROW * 2 + dchunk * 16),
                      lds_u32(T + t * CG_TILE + (16 * wave + 8 * p) * 128));
            }
    };

    f32x16 acc[CG_IB][2];
#pragma unroll
    for (int ib = 0; ib < CG_IB; ++ib) acc[ib][0] = acc[ib][1] = f32x16{};

    auto kstep = [&](auto stage) {
        constexpr int R = decltype(stage)::value;
        const uint8_t* B = smem + R * STAGE;
        const uint8_t* S = B + NT * CG_TILE;
        // byte 2*half + kc of sd[ib]: the table slot of this lane's fragment
        uint32_t sd[CG_IB];
#pragma unroll
        for (int ib = 0; ib < CG_IB; ++ib)
            sd[ib] = *(const uint32_t*)(S + (CG_WROWS * wave + 32 * ib + l32) * CG_SELROW + 4 * hi);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                bf16x8 hf[NT][2];
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) {
                        const int col = 32 * nb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
                        i16x4 part[2];
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int row = 32 * half + 16 * kc + 8 * hi + 4 * u + ((lane & 15) >> 2);
                            const int unit = (col >> 2) ^ (8 * ((row >> 1) & 1));
                            part[u] = lds_read_tr16(B + t * CG_TILE + row * 128 + unit * 8);
                        }
                        const u32x2 w0 = __builtin_bit_cast(u32x2, part[0]);
                        const u32x2 w1 = __builtin_bit_cast(u32x2, part[1]);
                        hf[t][nb] = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
                    }
                bf16x8 sf[CG_IB];
#pragma unroll
                for (int ib = 0; ib < CG_IB; ++ib)
                    sf[ib] = *(const bf16x8*)(lut + 16 * ((sd[ib] >> (8 * (2 * half + kc))) & 0xFFu));
                // the rest tile's products after all of the high tile's, so no
                // accumulator is the input of the next MFMA
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int ib = 0; ib < CG_IB; ++ib) {
                        acc[ib][0] = mfma_bf16_32x32x16(hf[t][0], sf[ib], acc[ib][0]);
                        acc[ib][1] = mfma_bf16_32x32x16(hf[t][1], sf[ib], acc[ib][1]);
                    }
            }
        }
    };

    // Pipeline over K-step pairs: stage kp % 3, two stages ahead. At the end of
    // step kp only stage kp+2's DMAS per wave may stay in flight.
    issue(0, 0);
    if (nkp > 1) issue(1, 1);
    if (nkp > 1) wait_vm<DMAS>(); else wait_vm<0>();
    __syncthreads();  // also publishes the expansion table
    auto step = [&](int kp, auto stage) {
        constexpr int R = decltype(stage)::value;
        if (kp + 2 < nkp) issue(kp + 2, (R + 2) % CG_STAGES);
        kstep(stage);
        if (kp + 1 < nkp) {
            if (kp + 2 < nkp) wait_vm<DMAS>(); else wait_vm<0>();
            __syncthreads();
        }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    static_assert(CG_STAGES == 3, "the K loop is unrolled by the ring depth");
    int kp = 0;
    for (; kp + 3 <= nkp; kp += 3) {
        step(kp, S0{});
        step(kp + 1, S1{});
        step(kp + 2, S2{});
    }
    if (kp < nkp) step(kp++, S0{});
    if (kp < nkp) step(kp, S1{});

    // Epilogue: lane (i, hi), accumulator [ib][nb] register 4q + x holds
    // n = 32nb + 8q + 4hi + x. Each wave stages one 32-row block at a time in
    // LDS (the rings are free once every wave has left the K loop), signed so
    // that the result is base + staged, and stores it as whole 256-byte row
    // pieces: 16 lanes per row instead of 32-byte runs in 32 rows.
    constexpr int EP = CG_TN + 4;  // pitch (floats) of a staged row: 272 B
    static_assert(4 * 32 * EP * 4 <= CG_STAGES * STAGE, "the staging fits the rings");
    float* stg = reinterpret_cast<float*>(smem) + wave * 32 * EP;
    const float sgn = complement ? 1.f : -1.f;  // base - sum == base + (-sum) exactly
    const int rc = lane & 15;                   // the 16-byte piece of a row this lane stores
    const f32x4 base = complement ? f32x4{} : *(const f32x4*)(htot + bh * HS_ROW + n0 + 4 * rc);
    __syncthreads();
#pragma unroll
    for (int ib = 0; ib < CG_IB; ++ib) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x16& a = acc[ib][nb];
                *(f32x4*)(stg + l32 * EP + 32 * nb + 8 * q + 4 * hi) =
                    f32x4{sgn * a[4 * q], sgn * a[4 * q + 1], sgn * a[4 * q + 2], sgn * a[4 * q + 3]};
            }
        __syncthreads();
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const int r = 4 * rr + (lane >> 4);
            const int i = iw + 32 * ib + r;
            if (i >= nqb) continue;
            const f32x4 sum = *(const f32x4*)(stg + r * EP + 4 * rc);
            *(f32x4*)(hnon + (bh * nqb + i) * (int64_t)HS_ROW + n0 + 4 * rc) = base + sum;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------

hipError_t launch_linear_states(const uint16_t* k, const uint16_t* v, int64_t BH, int N,
                                uint16_t* vt, uint16_t* hs, uint16_t* hs_lo, float* hpart,
                                float* htot, float* kpart, float* kbarT, int ldk, hipStream_t st) {
    const int nkb = (N + KBLK - 1) / KBLK;
    const int ngroups = (nkb + LIN_GROUP - 1) / LIN_GROUP;
    if (kpart)
        hipLaunchKernelGGL((linear_states_kernel<true, true>), dim3(ngroups, BH), dim3(LS_THREADS),
                           0, st, k, v, N, nkb, ngroups, vt, hs, nullptr, hpart, kpart, kbarT, ldk);
    else if (hs_lo)
        hipLaunchKernelGGL((linear_states_kernel<true, false, true>), dim3(ngroups, BH),
                           dim3(LS_THREADS), 0, st, k, v, N, nkb, ngroups, vt, hs, hs_lo, hpart,
                           nullptr, nullptr, 0);
    else
        hipLaunchKernelGGL((linear_states_kernel<true, false>), dim3(ngroups, BH), dim3(LS_THREADS),
                           0, st, k, v, N, nkb, ngroups, vt, hs, nullptr, hpart, nullptr, nullptr, 0);
    hipLaunchKernelGGL(htot_kernel, dim3((HS_ROW / 4 + 255) / 256, BH), dim3(256), 0, st, hpart, ngroups,
                       htot);
    return hipGetLastError();
}

hipError_t launch_vt_only(const uint16_t* k, const uint16_t* v, int64_t BH, int N, uint16_t* vt,
                          float* kpart, float* kbarT, int ldk, hipStream_t st) {
    const int nkb = (N + KBLK - 1) / KBLK;
    if (kpart) {
        const int ngroups = (nkb + LIN_GROUP - 1) / LIN_GROUP;
        hipLaunchKernelGGL((linear_states_kernel<false, true>), dim3(ngroups, BH),
                           dim3(LS_THREADS), 0, st, k, v, N, nkb, ngroups, vt, nullptr, nullptr,
                           nullptr, kpart, kbarT, ldk);
    } else {
        hipLaunchKernelGGL((linear_states_kernel<false, false>), dim3(nkb, BH), dim3(LS_THREADS),
                           0, st, nullptr, v, N, nkb, nkb, vt, nullptr, nullptr, nullptr, nullptr,
                           nullptr, 0);
    }
    return hipGetLastError();
}

hipError_t launch_complement(const int32_t* kidx, int keep, const uint16_t* hs,
                             const uint16_t* hs_lo, const float* htot, int64_t BH, int N,
                             uint32_t* msel, float* hnon, hipStream_t st) {
    const int nqb = (N + QBLK - 1) / QBLK, nkb = (N + KBLK - 1) / KBLK;
    const int nkbp = (nkb + GEMM_KALIGN - 1) / GEMM_KALIGN * GEMM_KALIGN;
    // sum whichever of the kept and the non-kept sets is smaller
    const int complement = 2 * keep > nkb ? 1 : 0;
    hipLaunchKernelGGL(msel_kernel<false>, dim3((nqb + 1) & ~1, BH), dim3(256), 0, st, kidx, keep,
                       nullptr, nullptr, 0, nqb, nkb, nkbp / GEMM_KALIGN, complement, msel);
    const int64_t total = BH * complement_tiles_per_head(nqb);
    const int64_t grid = (total + 7) / 8 * 8;
    if (hs_lo)
        hipLaunchKernelGGL(complement_gemm_kernel<true>, dim3((unsigned)grid), dim3(256), 0, st,
                           msel, hs, hs_lo, htot, BH, nqb, nkb, nkbp, complement, hnon);
    else
        hipLaunchKernelGGL(complement_gemm_kernel<false>, dim3((unsigned)grid), dim3(256), 0, st,
                           msel, hs, nullptr, htot, BH, nqb, nkb, nkbp, complement, hnon);
    return hipGetLastError();
}

hipError_t launch_complement_lists(const uint16_t* lists, const int32_t* counts, int nrows,
                                   int nred, int complement, const uint16_t* stack,
                                   const uint16_t* stack_lo, const float* total, int64_t BH,
                                   uint32_t* msel, float* out, hipStream_t st) {
    const int nredp = (nred + GEMM_KALIGN - 1) / GEMM_KALIGN * GEMM_KALIGN;
    hipLaunchKernelGGL(msel_kernel<true>, dim3((nrows + 1) & ~1, BH), dim3(256), 0, st, nullptr, 0,
                       lists, counts, nred, nrows, nred, nredp / GEMM_KALIGN, complement, msel);
    const int64_t tiles = BH * complement_tiles_per_head(nrows);
    const int64_t grid = (tiles + 7) / 8 * 8;
    if (stack_lo)
        hipLaunchKernelGGL(complement_gemm_kernel<true>, dim3((unsigned)grid), dim3(256), 0, st,
                           msel, stack, stack_lo, total, BH, nrows, nred, nredp, complement, out);
    else
        hipLaunchKernelGGL(complement_gemm_kernel<false>, dim3((unsigned)grid), dim3(256), 0, st,
                           msel, stack, nullptr, total, BH, nrows, nred, nredp, complement, out);
    return hipGetLastError();
}

hipError_t launch_state_total(const float* part, int ngroups, int64_t BH, float* out,
                              hipStream_t st) {
    hipLaunchKernelGGL(htot_kernel, dim3((HS_ROW / 4 + 255) / 256, BH), dim3(256), 0, st, part,
                       ngroups, out);
    return hipGetLastError();
}

}  // namespace ssa
