// bwd.hip -- the SageSLA backward on gfx950.
//
// TurboDiffusion pages, page 5 "What is TurboDiffusion?" and the training
// guide: the sparse-linear attention is trainable (fine-tuned in training).
// Gradients pass the 8-bit quantizer straight through (its derivative is
// taken as the identity) and the block selection is held fixed. With the
// forward's row statistics m' = m + log2(l) and D = dO . o_s (handed over by
// the forward, D via dstat_kernel, or recomputed by the forward kernel's
// statistics mode), for a query t and a kept key u:
//   P = 2^(S*c - m'),  dP = dO_t . v_u,  dS = P (dP - D)
//   dq_t += sm sum_u dS sk k_i8_u      (query-block-major: dq_kernel)
//   dk_u += sm sum_t dS sq q_i8_t,  dv_u += sum_t P dO_t
//                                      (key-block-major over the query blocks
//                                       that kept the block: dkdv_kernel)
// S is the exact int32 product on the INT8 matrix cores; dP, dq, dk and dv
// run on the bf16 matrix cores with fp32 accumulation (P and dS rounded to
// bf16; the int8 operands are exact in bf16). The linear branch (phi = elu+1
// over the non-kept blocks) follows the same reading in fp32: per query block
// its gradient states G_i = sum_t phi(q_t) dnum_t^T, w_i = sum_t phi(q_t) dden_t,
// their sums over the query blocks that did NOT keep each key block (the
// forward's complement GEMM on the transposed selection), then per key block
// the key and value gradients.
#include <algorithm>
#include <type_traits>

#include "../../include/ssa.h"
#include "common.hpp"
#include "kernels.hpp"

namespace ssa {

// A value every lane reads at one address, from a buffer the kernel does not
// write, through the scalar cache: a load from the constant address space,
// which the compiler issues as s_load_dword and waits for on lgkmcnt. Loaded
// through the vector path instead, its use would get a vmcnt wait, and the
// compiler, which does not see the LDS DMAs, would make that vmcnt(0) and so
// drain every DMA in flight. p must be 4-byte aligned.
__device__ __forceinline__ uint32_t ld_uniform(const void* p) {
    return *(const __attribute__((address_space(4))) uint32_t*)p;
}
__device__ __forceinline__ float ld_uniform_f32(const float* p) {
    return __uint_as_float(ld_uniform(p));
}
// element e of a uint16 array whose base is 4-byte aligned (the aligned pair
// holding it is read, so the array must extend to an even element count)
__device__ __forceinline__ int ld_uniform_u16(const uint16_t* base, int64_t e) {
    return (int)((ld_uniform(base + (e & ~int64_t(1))) >> (16 * (int)(e & 1))) & 0xFFFFu);
}

// ---- the query blocks that kept each key block ----------------------------
// lists[bh][j][0..counts[bh][j]) = the query blocks i (ascending) whose kept
// list kidx[bh][i] holds j. Two passes over a bit matrix bits[bh][j][i / 32]:
// one workgroup per (head, 32 query blocks) sets the bits of its query blocks
// for every key block in LDS and writes its word of each key block's row
// (every word once, so nothing is cleared beforehand), then one thread per
// key block emits the set bits of its row in ascending i. Entries outside
// [0, nkb) are ignored.
__global__ __launch_bounds__(256) void keep_bits_kernel(const int32_t* __restrict__ kidx, int keep,
                                                        int nqb, int nkb,
                                                        uint32_t* __restrict__ bits) {
    extern __shared__ uint32_t wbits[];  // [nkb]: bit i - 32w of query block i
    const int w = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int words = (nqb + 31) >> 5;
    for (int j = threadIdx.x; j < nkb; j += 256) wbits[j] = 0;
    __syncthreads();
    const int i0 = 32 * w, ni = min(32, nqb - i0);
    const int32_t* src = kidx + (bh * nqb + i0) * (int64_t)keep;
    for (int e = threadIdx.x; e < ni * keep; e += 256) {
        const int j = src[e];
        if (j >= 0 && j < nkb) atomicOr(&wbits[j], 1u << (e / keep));
    }
    __syncthreads();
    for (int j = threadIdx.x; j < nkb; j += 256) bits[(bh * nkb + j) * words + w] = wbits[j];
}

__global__ __launch_bounds__(256) void inv_lists_kernel(const uint32_t* __restrict__ bits,
                                                        int nqb, int nkb,
                                                        uint16_t* __restrict__ lists,
                                                        int32_t* __restrict__ counts) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    const int64_t bh = blockIdx.y;
    if (j >= nkb) return;
    const int words = (nqb + 31) >> 5;
    const uint32_t* row = bits + (bh * nkb + j) * words;
    uint16_t* out = lists + (bh * nkb + j) * (int64_t)nqb;
    int cnt = 0;
    for (int w = 0; w < words; ++w) {
        uint32_t x = row[w];
        while (x) {
            out[cnt++] = (uint16_t)(32 * w + __builtin_ctz(x));
            x &= x - 1u;
        }
    }
    counts[bh * nkb + j] = cnt;
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ p, int64_t n) {
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256)
        p[x] = 0.f;
}

// ---- dq: one workgroup per (head, query block), 4 waves x 32 queries ------
// For each kept key block: its int8 K tile (8 KB, 64 rows of 128 channels)
// and raw bf16 V tile (16 KB, 64 rows of 256 B) arrive in a double-buffered
// LDS ring by LDS DMA; the workgroup widens the K tile to bf16 (exact) into a
// third tile [64 keys][128 channels] (row pitch 288 B) that the dQ product
// reads with transposing loads. Per wave (queries 32w + l32, lane pair hi):
//   S^T = K . Q^T         (int8; lane holds query l32, keys 8(r/4)+4hi+r%4 (+32))
//   dP^T = V . dO^T       (bf16; same layout)
//   dS^T = P (dP - D) sk  (registers, packed as the next product's B operand)
//   dQ^T += K^T . dS^T    (bf16, fp32 accumulation; lane l's A fragment is
//                          channel l%32 at 8 keys in dS's register order, two
//                          ds_read_b64_tr_b16 of 4 consecutive keys each)
// Each stage is refilled as soon as every wave has finished the step's S and
// dP (the barrier that also publishes the widened tile), so two barriers per
// step and about one and a half steps for each stage to land.
constexpr int DQ_KT = KBLK * HD;           // int8 K tile
constexpr int DQ_VT = KBLK * HD * 2;       // raw V tile
constexpr int DQ_STAGE = DQ_KT + DQ_VT;
constexpr int DQ_KB = 2 * DQ_STAGE;        // the widened K tile, after the two stages
constexpr int DQ_KBP = HD * 2 + 32;        // its row pitch: 288 B, so the 4 rows a transposing
                                           // read touches fall in disjoint bank groups
constexpr int DQ_LDS = DQ_KB + KBLK * DQ_KBP;
constexpr int DQ_DMAS = (DQ_STAGE / 1024) / 4;  // 1 KB LDS DMAs per wave per stage
static_assert(2 * DQ_LDS <= 160 * 1024, "two workgroups per CU");

__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// bf16 tiles [64 rows][256 B] keep 16-byte chunk c of row r at chunk c ^ qswz(r):
// 16 consecutive rows at one chunk (row reads) and 4 consecutive rows at 4
// chunks (transposing reads) both cover all banks
__device__ __forceinline__ int qswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <bool DENSE>
__global__ __launch_bounds__(256, 2) void dq_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[DQ_LDS];
    const int64_t item = blockIdx.x;
    if (item >= a.BH * a.nqb) return;
    const int64_t bh = item / a.nqb;
    const int i = (int)(item % a.nqb);
    const int N = a.N, nkb = a.nkb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31,
              hi = lane >> 5;
    const int tq = i * QBLK + 32 * wave + l32;
    const bool qok = tq < N;
    const int nsel = DENSE ? nkb : a.keep;
    const int32_t* krow = DENSE ? nullptr : a.kidx + (bh * a.nqb + i) * (int64_t)a.keep;
    // kept block indices and their K scales come through the scalar cache
    auto blk = [&](int jj) {
        return DENSE ? jj : min(max((int)ld_uniform(krow + jj), 0), nkb - 1);
    };
    const float sq = ld_uniform_f32(a.q_scale + bh * a.nqb + i);
    const float* ksc = a.k_scale + bh * nkb;

    // stage layout: K tile | V tile
    auto issue = [&](int j, int st) {
        uint8_t* base = smem + st * DQ_STAGE;
        const int nval = min(KBLK, N - j * KBLK);
        // K: 64 rows of 128 B, chunk c of row r at slot c ^ swz8(r); rows past
        // N re-read row N-1
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int row = 16 * wave + 8 * p + (lane >> 3);
            const int rr = min(row, nval - 1);
            dma16(a.k_i8 + (bh * N + (int64_t)j * KBLK) * HD,
                  rr * 128 + 16 * ((lane & 7) ^ swz8(row)),
                  lds_u32(base) + (16 * wave + 8 * p) * 128);
        }
        // V: 64 rows of 256 B, 16-byte chunk c of key row r at slot c ^ (r & 15)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = 16 * wave + 4 * p + (lane >> 4);
            const int rr = min(row, nval - 1);
            dma16(a.v + (bh * N + (int64_t)j * KBLK) * HD,
                  rr * 256 + 16 * ((lane & 15) ^ (row & 15)),
                  lds_u32(base + DQ_KT) + (16 * wave + 4 * p) * 256);
        }
    };

    // j0, sk0: the block of step jj and its scale; j1, j2: the blocks of steps
    // jj+1, jj+2. Each is loaded ahead of its use, so its latency stays off
    // the path.
    int j0 = blk(0), j1 = nsel > 1 ? blk(1) : 0, j2 = nsel > 2 ? blk(2) : 0;
    float sk0 = ld_uniform_f32(ksc + j0);
    issue(j0, 0);
    if (nsel > 1) issue(j1, 1);

    // per-lane operands: Q (int8 B operand of S^T), dO (bf16 B operand of dP^T)
    i32x4 qop[4];
    bf16x8 dop[8];
    {
        const int8_t* qp = a.q_i8 + (bh * N + (qok ? tq : 0)) * HD;
        const uint16_t* gp = a.dout + (bh * N + (qok ? tq : 0)) * HD;
#pragma unroll
        for (int c = 0; c < 4; ++c) qop[c] = qok ? *(const i32x4*)(qp + 32 * c + 16 * hi) : i32x4{};
#pragma unroll
        for (int s = 0; s < 8; ++s)
            dop[s] = qok ? __builtin_bit_cast(bf16x8, *(const u16x8*)(gp + 16 * s + 8 * hi)) : bf16x8{};
    }
    const float mq = qok ? a.mlog[bh * N + tq] : 0.f;
    const float Dq = qok ? a.dstat[bh * N + tq] : 0.f;
    // The compiler does not see the LDS DMAs: with these loads outstanding at
    // the loop, it would wait for them in every step with a vmcnt that also
    // covers the DMAs in flight. Waiting here (for them and the first two
    // stages) clears them once.
    wait_vm<0>();

    f32x16 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
    // transposing reads of the dQ product: lane l supplies key row
    // 16cc + 8t + 4hi + (l&15)/4 at channels 32dt + 16((l>>4)&1) + 4(l&3) .. +3,
    // one base address plus immediate offsets
    const uint8_t* kbl = smem + DQ_KB + (4 * hi + ((lane & 15) >> 2)) * DQ_KBP +
                         2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    for (int jj = 0; jj < nsel; ++jj) {
        const int st = jj & 1;
        // stage jj must land (stage jj+1 may stay in flight)
        if (jj + 1 < nsel) wait_vm<DQ_DMAS>(); else wait_vm<0>();
        __syncthreads();  // stage jj visible; every wave is done with the last widened tile
        const int j = j0;
        const int kval = min(KBLK, N - j * KBLK);
        const float sk = sk0;
        const float c = (sq * sk) * a.K32;
        const uint8_t* kt = smem + st * DQ_STAGE;
        const uint8_t* vt = kt + DQ_KT;
        // widen this step's K tile: 16 threads per row, each 8 channels (an
        // 8-byte read, a 16-byte store), so a 16-lane group reads and writes
        // one whole row without bank conflicts
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int x = tid + 256 * it, row = x >> 4, c8 = x & 15;
            const u32x2 kv =
                *(const u32x2*)(kt + row * 128 + 16 * ((c8 >> 1) ^ swz8(row)) + 8 * (c8 & 1));
            bf16x8 w;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int b = (int)((uint32_t)kv[e >> 2] << (24 - 8 * (e & 3))) >> 24;  // signed byte e
                w[e] = (__bf16)(float)b;
            }
            *(bf16x8*)(smem + DQ_KB + row * DQ_KBP + 16 * c8) = w;
        }
        i32x16 s[2];
        f32x16 dp[2];
        s[0] = s[1] = i32x16{};
        dp[0] = dp[1] = f32x16{};
#pragma unroll
        for (int cq = 0; cq < 4; ++cq) {
            const int slot = ((2 * cq + hi) ^ swz8(l32)) * 16;
            s[0] = mfma_i8_32x32x32(*(const i32x4*)(kt + l32 * 128 + slot), qop[cq], s[0]);
            s[1] = mfma_i8_32x32x32(*(const i32x4*)(kt + (32 + l32) * 128 + slot), qop[cq], s[1]);
        }
#pragma unroll
        for (int sd = 0; sd < 8; ++sd) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int key = 32 * h + l32;
                const bf16x8 va = *(const bf16x8*)(vt + key * 256 + 16 * ((2 * sd + hi) ^ (key & 15)));
                dp[h] = mfma_bf16_32x32x16(va, dop[sd], dp[h]);
            }
        }
        // the next scale and the block two steps on (stage jj+2), loaded here
        // and used after the barrier
        float sk1 = 0.f;
        int j3 = 0;
        if (jj + 1 < nsel) sk1 = ld_uniform_f32(ksc + j1);
        if (jj + 3 < nsel) j3 = blk(jj + 3);
        __syncthreads();  // the widened tile is visible; every wave is done with stage jj
        if (jj + 2 < nsel) issue(j2, st);
        // dS; in a ragged last key block the keys past N (copies of key N-1,
        // so p stays finite) are zeroed after the exp: one uniform branch per
        // block instead of a masked branch per score
        bf16x8 dsb[4];
        auto softmax = [&](auto ragged) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[h][r], c, -mq));
                    if constexpr (decltype(ragged)::value) p = 32 * h + mfma32_row(lane, r) < kval ? p : 0.f;
                    const float ds = p * (dp[h][r] - Dq) * sk;
                    dsb[2 * h + (r >> 3)][r & 7] = (__bf16)ds;
                }
        };
        if (kval == KBLK)
            softmax(std::false_type{});
        else
            softmax(std::true_type{});
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                i16x4 kp[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) kp[t] = lds_read_tr16(kbl + (16 * cc + 8 * t) * DQ_KBP + 64 * dt);
                const u32x2 k0 = __builtin_bit_cast(u32x2, kp[0]), k1 = __builtin_bit_cast(u32x2, kp[1]);
                const bf16x8 ka = __builtin_bit_cast(bf16x8, u32x4{k0[0], k0[1], k1[0], k1[1]});
                acc[dt] = mfma_bf16_32x32x16(ka, dsb[cc], acc[dt]);
            }
        j0 = j1;
        j1 = j2;
        j2 = j3;
        sk0 = sk1;
    }
    // accumulating: every value the row already holds is loaded before the
    // first store (rows past N read row N-1 and store nothing)
    float* row = a.dq + (bh * N + (qok ? tq : N - 1)) * HD;
    f32x4 prev[16];
    if (a.dq_accumulate) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) prev[4 * dt + q4] = *(const f32x4*)(row + 32 * dt + 8 * q4 + 4 * hi);
    }
    if (qok) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int dv = 32 * dt + 8 * q4 + 4 * hi;
                f32x4 g = f32x4{acc[dt][4 * q4] * a.sm, acc[dt][4 * q4 + 1] * a.sm,
                                acc[dt][4 * q4 + 2] * a.sm, acc[dt][4 * q4 + 3] * a.sm};
                if (a.dq_accumulate) g = g + prev[4 * dt + q4];
                *(f32x4*)(row + dv) = g;
            }
    }
}

// D[t] = dO_t . out_t - dol[t] per query row, from the forward's fp32 output
// (o_s + o_l) and the linear branch's dO . o_l (dol null: sparse branch only):
// the sparse branch's D = dO . o_s without re-running the forward. Sixteen
// lanes per row (each 8 channels: one 16-byte dO load, two 16-byte output
// loads), four rows per wave, the sum as a butterfly over the 16 lanes.
__global__ __launch_bounds__(256) void dstat_kernel(const uint16_t* __restrict__ dout,
                                                    const float* __restrict__ out32,
                                                    const float* __restrict__ dol, int64_t rows,
                                                    float* __restrict__ dstat) {
    const int c = threadIdx.x & 15;
    for (int64_t t = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4); t < rows;
         t += (int64_t)gridDim.x * 16) {
        const u16x8 g = *(const u16x8*)(dout + t * HD + 8 * c);
        const f32x4 o0 = *(const f32x4*)(out32 + t * HD + 8 * c);
        const f32x4 o1 = *(const f32x4*)(out32 + t * HD + 8 * c + 4);
        float s = bf2f(g[0]) * o0[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) s = __builtin_fmaf(bf2f(g[e]), e < 4 ? o0[e] : o1[e - 4], s);
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
        if (c == 0) dstat[t] = dol ? s - dol[t] : s;
    }
}

// ---- dk, dv: one workgroup per (head, key block), 4 waves, two per CU -----
// Over the query blocks that kept the block (every block when dense), each in
// two steps of 64 queries. The V tile of the block sits in LDS and each
// wave's K fragments in registers for the workgroup's whole life. Per step
// the workgroup stages q_i8 (as int8, and widened to bf16) and dO of the 64
// queries in LDS, and these tiles serve every product:
//   phase 1, wave w (queries 32(w&1) .. of the step, key tile h = w>>1):
//     S = Q . K^T  (int8; lane holds key 32h + l32, queries 8(r/4)+4hi+r%4)
//     dP = dO . V^T (bf16; same layout)
//     P = 2^(S c - m'), dS = P (dP - D) sq, stored in LDS as the B fragments
//     of phase 2 (k = 16 queries in the re-laid order, n = keys);
//   phase 2, wave w (channels 32w ..):
//     dV^T += dO^T . P, dK^T += Q^T . dS over the step's 64 queries, for both
//     key tiles, the A fragments read from the row-major tiles with
//     transposing LDS reads (ds_read_b64_tr_b16), which give a lane 4
//     consecutive queries of one channel; two reads make a fragment in the
//     order P's registers hold.
// Only q_i8 and dO cross the memory hierarchy per block pair (48 KB), loaded
// into registers a step ahead. The bf16 tiles [64 rows][256 B] keep 16-byte
// chunk c of row r at chunk c ^ qswz(r): 16 consecutive rows at one chunk
// (the row reads) and 4 consecutive rows at 4 chunks (the transposing reads)
// both cover all banks. 72.5 KB of LDS, so that two workgroups share a CU
// and each runs while the other waits at a barrier.
constexpr int DK_THREADS = 256;
constexpr int DK_Q = 64;                       // queries per step
constexpr int KV_F = 4 * 2 * 64 * 16;          // one fragment set: [4 query steps][2 key tiles][64 lanes] x 16 B
constexpr int DK_VT = 0;                       // bf16 V tile [64][256 B], chunk c at c ^ (r & 15)
constexpr int DK_QI = DK_VT + KBLK * HD * 2;   // int8 Q tile [64][128 B], chunk c at c ^ swz8(r)
constexpr int DK_QB = DK_QI + DK_Q * HD;       // bf16 Q tile [64][256 B], chunk c at c ^ qswz(r)
constexpr int DK_GO = DK_QB + DK_Q * HD * 2;   // bf16 dO tile, same layout
constexpr int DK_PF = DK_GO + DK_Q * HD * 2;   // P fragments
constexpr int DK_DF = DK_PF + KV_F;            // dS fragments
constexpr int DK_ST = DK_DF + KV_F;            // m' and -D sq of the step's 64 queries
constexpr int DK_LDS = DK_ST + 2 * DK_Q * 4;
static_assert(2 * DK_LDS <= 160 * 1024, "two workgroups per CU");

template <bool DENSE>
__global__ __launch_bounds__(DK_THREADS, 2) void dkdv_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[DK_LDS];
    float* stat = reinterpret_cast<float*>(smem + DK_ST);  // [m', -D sq][query of the step]
    const int64_t item = blockIdx.x;
    if (item >= a.BH * a.nkb) return;
    const int64_t bh = item / a.nkb;
    const int j = (int)(item % a.nkb);
    const int N = a.N, nqb = a.nqb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31,
              hi = lane >> 5;
    const int nval = min(KBLK, N - j * KBLK);
    // the block's V in LDS; rows past N re-read row N-1 (their P is zeroed)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int x = tid + DK_THREADS * it, r = x >> 4, c = x & 15, rr = min(r, nval - 1);
        *(u16x8*)(smem + DK_VT + r * 256 + 16 * (c ^ (r & 15))) =
            *(const u16x8*)(a.v + (bh * N + (int64_t)j * KBLK + rr) * HD + 8 * c);
    }
    // phase-1 roles; the wave's K fragments (key 32kh + l32, channels
    // 32cq + 16hi ..) stay in registers
    const int qw = wave & 1, kh = wave >> 1;
    const int key = 32 * kh + l32, trow = 32 * qw + l32;
    const bool kok = key < nval;
    i32x4 kfr[4];
    {
        const int8_t* kp = a.k_i8 + (bh * N + (int64_t)j * KBLK + min(key, nval - 1)) * HD;
#pragma unroll
        for (int cq = 0; cq < 4; ++cq) kfr[cq] = *(const i32x4*)(kp + 32 * cq + 16 * hi);
    }
    // the block's scale, list length and list entries come through the scalar cache
    const float sk = ld_uniform_f32(a.k_scale + bh * a.nkb + j);
    const int cnt = DENSE ? nqb : (int)ld_uniform(a.counts + bh * a.nkb + j);
    const int64_t lbase = (bh * a.nkb + j) * (int64_t)nqb;  // the block's list in a.lists
    // steps: (kept query block x, half f), halves entirely past N skipped
    auto qblock = [&](int x) { return DENSE ? x : ld_uniform_u16(a.lists, lbase + x); };
    auto has_half = [&](int i, int f) { return i * QBLK + DK_Q * f < N; };

    // one step's q_i8 and dO rows (rows past N re-read row N-1: their P and
    // dS are zeroed) and statistics, in registers until staged
    u16x8 gpre[4];
    i32x4 qpre[2];
    float spre = 0.f;
    auto prefetch = [&](int q0) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int x = tid + DK_THREADS * it, row = x >> 4, c = x & 15;
            const int t = min(q0 + row, N - 1);
            gpre[it] = *(const u16x8*)(a.dout + (bh * N + t) * HD + 8 * c);
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int x = tid + DK_THREADS * it, row = x >> 3, c = x & 7;
            const int t = min(q0 + row, N - 1);
            qpre[it] = *(const i32x4*)(a.q_i8 + (bh * N + t) * HD + 16 * c);
        }
        if (tid < 2 * DK_Q) {
            const int t = min(q0 + (tid & (DK_Q - 1)), N - 1);
            spre = (tid < DK_Q ? a.mlog : a.dstat)[bh * N + t];
        }
    };
    auto stage = [&](float sq) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int x = tid + DK_THREADS * it, row = x >> 4, c = x & 15;
            *(u16x8*)(smem + DK_GO + row * 256 + 16 * (c ^ qswz(row))) = gpre[it];
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int x = tid + DK_THREADS * it, row = x >> 3, c = x & 7;
            *(i32x4*)(smem + DK_QI + row * 128 + 16 * (c ^ swz8(row))) = qpre[it];
            bf16x8 w[2];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int b = (int)((uint32_t)qpre[it][e >> 2] << (24 - 8 * (e & 3))) >> 24;  // signed byte e
                w[e >> 3][e & 7] = (__bf16)(float)b;
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
                *(bf16x8*)(smem + DK_QB + row * 256 + 16 * ((2 * c + h) ^ qswz(row))) = w[h];
        }
        // m' as is; D as -D sq, so that dS = p (dP - D) sq is p (dP sq - D sq)
        if (tid < 2 * DK_Q) stat[tid] = tid < DK_Q ? spre : -(spre * sq);
    };

    f32x16 dva[2], dka[2];  // channels 32w + ..., key tiles 0, 1
    dva[0] = dva[1] = dka[0] = dka[1] = f32x16{};
    // phase-2 transposing-read addresses: lane l supplies row
    // 16qs + 8t + 4hi + (l&15)/4 at channels col .. col+3
    const int col = 32 * wave + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int rsub = 4 * hi + ((lane & 15) >> 2);
    // i, sq: the query block of this step and its scale; i1: the block after
    // it in the list. Each is loaded a step before its use.
    int x = 0, f = 0;
    int i = cnt > 0 ? qblock(0) : 0, i1 = cnt > 1 ? qblock(1) : 0;
    float sq = ld_uniform_f32(a.q_scale + bh * nqb + i);
    if (cnt > 0) prefetch(i * QBLK);
    while (x < cnt) {
        const int q0 = i * QBLK + DK_Q * f;
        // the step after this one
        int xn = x, fn = f + 1;
        if (fn == 2 || !has_half(i, fn)) {
            xn = x + 1;
            fn = 0;
        }
        const int in = xn == x ? i : i1;
        stage(sq);
        __syncthreads();  // tiles and statistics of the step visible
        int i1n = i1;
        float sqn = sq;
        if (xn < cnt) {
            prefetch(in * QBLK + DK_Q * fn);
            if (xn != x) {
                sqn = ld_uniform_f32(a.q_scale + bh * nqb + in);
                if (xn + 1 < cnt) i1n = qblock(xn + 1);
            }
        }
        const float c = (sq * sk) * a.K32;
        {
            i32x16 s = i32x16{};
            f32x16 dp = f32x16{};
#pragma unroll
            for (int cq = 0; cq < 4; ++cq)
                s = mfma_i8_32x32x32(
                    *(const i32x4*)(smem + DK_QI + trow * 128 + 16 * ((2 * cq + hi) ^ swz8(trow))),
                    kfr[cq], s);
#pragma unroll
            for (int sd = 0; sd < 8; ++sd)
                dp = mfma_bf16_32x32x16(
                    *(const bf16x8*)(smem + DK_GO + trow * 256 + 16 * ((2 * sd + hi) ^ qswz(trow))),
                    *(const bf16x8*)(smem + DK_VT + key * 256 + 16 * ((2 * sd + hi) ^ (key & 15))), dp);
            // P and dS; in a ragged last query or key block the rows and keys
            // past N (clamped copies of valid ones, so p stays finite) are
            // zeroed after the exp, under one uniform branch
            f32x16 pr;
            auto softmax = [&](auto ragged) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int r0 = 32 * qw + 8 * g + 4 * hi;  // queries of registers 4g .. 4g+3
                    const f32x4 mq = *(const f32x4*)(stat + r0);
                    const f32x4 nDsq = *(const f32x4*)(stat + DK_Q + r0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * g + e;
                        float p = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[r], c, -mq[e]));
                        if constexpr (decltype(ragged)::value) p = (kok && q0 + r0 + e < N) ? p : 0.f;
                        pr[r] = p;
                        dp[r] = p * __builtin_fmaf(dp[r], sq, nDsq[e]);
                    }
                }
            };
            if (nval == KBLK && q0 + DK_Q <= N)
                softmax(std::false_type{});
            else
                softmax(std::true_type{});
            // fragment [query step 2qw + ks][key tile kh][lane]
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 pb, db;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pb[e] = (__bf16)pr[8 * ks + e];
                    db[e] = (__bf16)dp[8 * ks + e];
                }
                const int slot = ((2 * qw + ks) * 2 + kh) * 64 + lane;
                *(bf16x8*)(smem + DK_PF + 16 * slot) = pb;
                *(bf16x8*)(smem + DK_DF + 16 * slot) = db;
            }
        }
        __syncthreads();  // fragments visible
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) {
            i16x4 gp[2], qp[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int row = 16 * qs + 8 * t + rsub;
                const int off = row * 256 + 16 * ((col >> 3) ^ qswz(row)) + 8 * ((col >> 2) & 1);
                gp[t] = lds_read_tr16(smem + DK_GO + off);
                qp[t] = lds_read_tr16(smem + DK_QB + off);
            }
            const u32x2 g0 = __builtin_bit_cast(u32x2, gp[0]), g1 = __builtin_bit_cast(u32x2, gp[1]);
            const u32x2 q0v = __builtin_bit_cast(u32x2, qp[0]), q1v = __builtin_bit_cast(u32x2, qp[1]);
            const bf16x8 gT = __builtin_bit_cast(bf16x8, u32x4{g0[0], g0[1], g1[0], g1[1]});
            const bf16x8 qT = __builtin_bit_cast(bf16x8, u32x4{q0v[0], q0v[1], q1v[0], q1v[1]});
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int slot = (qs * 2 + h) * 64 + lane;
                dva[h] = mfma_bf16_32x32x16(gT, *(const bf16x8*)(smem + DK_PF + 16 * slot), dva[h]);
                dka[h] = mfma_bf16_32x32x16(qT, *(const bf16x8*)(smem + DK_DF + 16 * slot), dka[h]);
            }
        }
        __syncthreads();  // the next step rewrites the tiles and fragments
        x = xn;
        f = fn;
        i = in;
        i1 = i1n;
        sq = sqn;
    }
    // lane (key column l32 of tile h, hi) holds channels 32w + 8(r/4) + 4hi + r%4
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int u = j * KBLK + 32 * h + l32;
        if (32 * h + l32 >= nval) continue;
        float* vrow = a.dv + (bh * N + u) * HD;
        float* krow = a.dk + (bh * N + u) * HD;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d = 32 * wave + 8 * q4 + 4 * hi;
            *(f32x4*)(vrow + d) = f32x4{dva[h][4 * q4], dva[h][4 * q4 + 1], dva[h][4 * q4 + 2],
                                        dva[h][4 * q4 + 3]};
            *(f32x4*)(krow + d) = f32x4{dka[h][4 * q4] * a.sm, dka[h][4 * q4 + 1] * a.sm,
                                        dka[h][4 * q4 + 2] * a.sm, dka[h][4 * q4 + 3] * a.sm};
        }
    }
}

// ---- the linear branch ------------------------------------------------------
// State rows (the forward's complement states and the gradient states alike):
// row e of the transposed 128 x 128 matrix, channel d at position
// pos(d) = 16(d/16) + 8((d>>2)&1) + 4(d>>3 & 1) + d%4, then the vector part at
// the same positions (the order one lane of the 32x32 MFMA output holds rows).
__device__ __forceinline__ int state_pos(int d) {
    return (d & ~15) | (((d >> 2) & 1) << 3) | (((d >> 3) & 1) << 2) | (d & 3);
}

// elu + 1 without branches: the exp of min(x, 0) is finite and is selected
// only for x <= 0
__device__ __forceinline__ float phi_f(float x) {
    const float ex = __expf(fminf(x, 0.f));
    return x > 0.f ? x + 1.f : ex;
}

// fp32 x fp32 -> fp32 on the matrix cores: lane l supplies A[l & 31][l >> 5]
// and B[l >> 5][l & 31]; the result has the 32x32 layout of mfma32_row.
__device__ __forceinline__ f32x16 mfma_f32_32x32x2(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

constexpr int LB_P = HD + 1;  // odd LDS pitch: row- and column-wise fragment reads hit distinct banks
constexpr int LB_T = 64;      // tokens staged at a time

// Stage a state row as M[d][e] (pitch LB_P) and its vector part as vec[d],
// in two halves so that a caller can put other loads in flight between them:
// load_state issues every load of the thread, store_state writes LDS.
struct StateRegs {
    f32x4 r[16];
    f32x4 z;
};
__device__ __forceinline__ void load_state(const float* __restrict__ row, StateRegs& s) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 16; ++it) s.r[it] = *(const f32x4*)(row + 4 * (tid + 256 * it));
    s.z = tid < 32 ? *(const f32x4*)(row + HD * HD + 4 * tid) : f32x4{};
}
__device__ __forceinline__ void store_state(const StateRegs& s, float* M, float* vec) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int x4 = tid + 256 * it, e = x4 >> 5;
        // positions 4c .. 4c+3 hold channels state_pos(4c) + 0 .. 3 (the map is
        // its own inverse and keeps the two low bits)
        const int d0 = state_pos(4 * (x4 & 31));
#pragma unroll
        for (int m = 0; m < 4; ++m) M[(d0 + m) * LB_P + e] = s.r[it][m];
    }
    if (tid < 32) {
        const int d0 = state_pos(4 * tid);
#pragma unroll
        for (int m = 0; m < 4; ++m) vec[d0 + m] = s.z[m];
    }
}

// Stage rows r0 .. r0+nrow-1 (64 of them, rows past nval zero) of a bf16
// [tokens x 128] tensor into X[row][channel] (pitch LB_P) in fp32, through fn;
// again as a load half and a store half.
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ src, int nval, u16x8 (&r)[4]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        // rows past nval re-read row nval-1 (finite values, scaled to 0 below)
        const int c = tid + 256 * it, tt = min(c >> 4, nval - 1);
        r[it] = *(const u16x8*)(src + (int64_t)tt * HD + 8 * (c & 15));
    }
}
template <typename F>
__device__ __forceinline__ void store_rows(const u16x8 (&r)[4], int nval, float* X, F fn) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int c = tid + 256 * it, tt = c >> 4, d0 = 8 * (c & 15);
#pragma unroll
        for (int m = 0; m < 8; ++m) X[tt * LB_P + d0 + m] = fn(bf2f(r[it][m])) * (tt < nval ? 1.f : 0.f);
    }
}

// Sum 16 per-lane values over the 32 lanes of a half-wave with 16 exchanges
// (each step keeps half of the values and adds the partner's copy of them).
// On return lane l holds the sum of value 8 b4 + 4 b3 + 2 b2 + b1, where
// b4 .. b1 are bits 4 .. 1 of l (bit 0 holds a duplicate).
__device__ __forceinline__ float halfwave_sum16(const float (&v)[16], int lane) {
    float a[8], b[4], c[2];
    const bool s4 = lane & 16, s3 = lane & 8, s2 = lane & 4, s1 = lane & 2;
#pragma unroll
    for (int x = 0; x < 8; ++x)
        a[x] = (s4 ? v[8 + x] : v[x]) + __shfl_xor(s4 ? v[x] : v[8 + x], 16, 64);
#pragma unroll
    for (int x = 0; x < 4; ++x) b[x] = (s3 ? a[4 + x] : a[x]) + __shfl_xor(s3 ? a[x] : a[4 + x], 8, 64);
#pragma unroll
    for (int x = 0; x < 2; ++x) c[x] = (s2 ? b[2 + x] : b[x]) + __shfl_xor(s2 ? b[x] : b[2 + x], 4, 64);
    const float d = (s1 ? c[1] : c[0]) + __shfl_xor(s1 ? c[0] : c[1], 2, 64);
    return d + __shfl_xor(d, 1, 64);
}

// Per (head, query block), with H, z its forward complement state (H[d][e],
// z[d]), a = phi(q_t), den = a . z, g = dO_t:
//   u = H g                  (so that g . o_l = a . u / den)
//   dden = -(a . u) / den^2
//   dq_t = (u / den + z dden) * phi'(q_t),   phi'(x) = min(phi(x), 1)
//   G^T[e][d] = sum_t (g[e] / den) a[d],  w[d] = sum_t a[d] dden
// The two products run on the fp32 matrix cores (exact fp32 products, fp32
// sums). G^T and w are written in fp32 (gf, for the total) and as bf16 plus
// its bf16 rest (gs, gs_lo: the GEMM's two stacks).
// Waves: u for row tile (w & 1) and channel tiles 2(w >> 1), +1; G^T for
// e-tile w and all four channel tiles.
__global__ __launch_bounds__(256, 1) void lin_bwd_q_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ dout,
                                                           const float* __restrict__ hnon, int N,
                                                           int nqb, float* __restrict__ dq,
                                                           float* __restrict__ gf,
                                                           uint16_t* __restrict__ gs,
                                                           uint16_t* __restrict__ gs_lo,
                                                           float* __restrict__ dol) {
    __shared__ float Hs[HD * LB_P];
    __shared__ float zv[HD];
    __shared__ float As[LB_T * LB_P], Gs[LB_T * LB_P];  // a and g, then g / den
    __shared__ float den_s[LB_T], dden_s[LB_T], gop[2][LB_T];
    const int i = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int nt = min(QBLK, N - i * QBLK);
    // rows of the half being staged (q and dO), loaded a half ahead: the
    // first half's together with the state, the second during the first's
    // products
    u16x8 qr[4], gr[4];
    {
        StateRegs sr;
        load_state(hnon + (bh * nqb + i) * (int64_t)HS_ROW, sr);
        load_rows(q + (bh * N + i * QBLK) * HD, nt, qr);
        load_rows(dout + (bh * N + i * QBLK) * HD, nt, gr);
        store_state(sr, Hs, zv);
    }
    f32x16 gacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) gacc[dt] = f32x16{};
    float wacc = 0.f;  // threads 0..127: w[tid]
    const int rt = wave & 1, ct0 = 2 * (wave >> 1);
    for (int h0 = 0; h0 < nt; h0 += LB_T) {
        __syncthreads();  // the state is staged / the previous half is done
        store_rows(qr, nt - h0, As, [](float x) { return phi_f(x); });
        store_rows(gr, nt - h0, Gs, [](float x) { return x; });
        __syncthreads();
        if (h0 + LB_T < nt) {
            const int64_t rn = bh * N + i * QBLK + h0 + LB_T;
            load_rows(q + rn * HD, nt - h0 - LB_T, qr);
            load_rows(dout + rn * HD, nt - h0 - LB_T, gr);
        }
        {  // den: four threads per token
            const int tt = tid >> 2, part = tid & 3;
            float dn = 0.f;
            for (int d = 32 * part; d < 32 * part + 32; ++d)
                dn = __builtin_fmaf(As[tt * LB_P + d], zv[d], dn);
            dn += __shfl_xor(dn, 1, 64);
            dn += __shfl_xor(dn, 2, 64);
            if (part == 0) den_s[tt] = h0 + tt < nt ? dn : 1.f;
        }
        // u[t][d] = sum_e g[t][e] H[d][e]
        f32x16 u[2] = {f32x16{}, f32x16{}};
        for (int k0 = 0; k0 < HD; k0 += 2) {
            const float ga = Gs[(32 * rt + l32) * LB_P + k0 + hi];
#pragma unroll
            for (int c = 0; c < 2; ++c)
                u[c] = mfma_f32_32x32x2(ga, Hs[(32 * (ct0 + c) + l32) * LB_P + k0 + hi], u[c]);
        }
        {  // partial a . u over this wave's 64 channels, one value per row
            float gp[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int t = 32 * rt + mfma32_row(lane, r);
                gp[r] = As[t * LB_P + 32 * ct0 + l32] * u[0][r] +
                        As[t * LB_P + 32 * (ct0 + 1) + l32] * u[1][r];
            }
            const float sum = halfwave_sum16(gp, lane);
            const int rr = (l32 >> 1) & 15;  // the value this lane holds the sum of
            if ((l32 & 1) == 0) gop[wave >> 1][32 * rt + mfma32_row(lane, rr)] = sum;
        }
        __syncthreads();
        if (tid < LB_T) {
            const float dn = den_s[tid];
            const float go = gop[0][tid] + gop[1][tid];  // g . o_l = go / den
            dden_s[tid] = h0 + tid < nt ? -go / (dn * dn) : 0.f;
            if (dol && h0 + tid < nt) dol[bh * N + i * QBLK + h0 + tid] = go / dn;
        }
        __syncthreads();
        // the row check only in a ragged last piece (one uniform branch)
        auto store_dq = [&](auto ragged) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int d = 32 * (ct0 + c) + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = 32 * rt + mfma32_row(lane, r);
                    if (decltype(ragged)::value && h0 + t >= nt) continue;
                    dq[(bh * N + i * QBLK + h0 + t) * HD + d] =
                        (u[c][r] / den_s[t] + zv[d] * dden_s[t]) * fminf(As[t * LB_P + d], 1.f);
                }
            }
        };
        if (h0 + LB_T <= nt)
            store_dq(std::false_type{});
        else
            store_dq(std::true_type{});
        for (int x = tid; x < LB_T * HD; x += 256) {
            const int tt = x >> 7, e = x & 127;
            Gs[tt * LB_P + e] = Gs[tt * LB_P + e] / den_s[tt];
        }
        if (tid < HD)
            for (int tt = 0; tt < LB_T; ++tt) wacc = __builtin_fmaf(As[tt * LB_P + tid], dden_s[tt], wacc);
        __syncthreads();
        // G^T[e][d] += sum_t (g / den)[t][e] a[t][d]
        for (int k0 = 0; k0 < LB_T; k0 += 2) {
            const float da = Gs[(k0 + hi) * LB_P + 32 * wave + l32];
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                gacc[dt] = mfma_f32_32x32x2(da, As[(k0 + hi) * LB_P + 32 * dt + l32], gacc[dt]);
        }
    }
    float* fr = gf + (bh * nqb + i) * (int64_t)HS_ROW;
    uint16_t* sr = gs + (bh * nqb + i) * (int64_t)HS_ROW;
    uint16_t* lr = gs_lo + (bh * nqb + i) * (int64_t)HS_ROW;
    auto put = [&](int64_t o, float x) {
        const uint16_t h = f2bf(x);
        fr[o] = x;
        sr[o] = h;
        lr[o] = f2bf(x - bf2f(h));
    };
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            put((int64_t)(32 * wave + mfma32_row(lane, r)) * HD + state_pos(32 * dt + l32), gacc[dt][r]);
    if (tid < HD) put(HD * HD + state_pos(tid), wacc);
}

// Per (head, key block): with Gc[d][e], wc the gradient-state sums over the
// query blocks that did not keep the block, for each key u: f = phi(k_u),
//   dk_u (+)= (Gc v_u + wc) * phi'(k_u),  dv_u (+)= Gc^T f
// on the fp32 matrix cores. Waves: row tile (w & 1), channel tiles
// 2(w >> 1), +1 of both products.
__global__ __launch_bounds__(256, 1) void lin_bwd_k_kernel(const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v,
                                                           const float* __restrict__ gc, int N,
                                                           int nkb, int accumulate,
                                                           float* __restrict__ dk,
                                                           float* __restrict__ dv) {
    __shared__ float Ms[HD * LB_P];
    __shared__ float wv[HD];
    __shared__ float Fs[KBLK * LB_P], Vs[KBLK * LB_P];
    const int j = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int nk = min(KBLK, N - j * KBLK);
    const int64_t r0 = bh * N + j * KBLK;
    {
        // every staging load (the state, K and V rows) in flight together
        StateRegs sr;
        u16x8 kr[4], vr[4];
        load_state(gc + (bh * nkb + j) * (int64_t)HS_ROW, sr);
        load_rows(k + r0 * HD, nk, kr);
        load_rows(v + r0 * HD, nk, vr);
        store_state(sr, Ms, wv);
        store_rows(kr, nk, Fs, [](float x) { return phi_f(x); });
        store_rows(vr, nk, Vs, [](float x) { return x; });
    }
    __syncthreads();
    const int rt = wave & 1, ct0 = 2 * (wave >> 1);
    // With accumulate, the sparse branch's dk and dv of this lane's outputs
    // are loaded before the products, so their latency hides behind them
    // (rows past nk re-read row nk-1; those outputs are not stored).
    float odk[2][16], odv[2][16];
    if (accumulate) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int uu = min(32 * rt + mfma32_row(lane, r), nk - 1);
                const int64_t o = (bh * N + j * KBLK + uu) * HD + 32 * (ct0 + c) + l32;
                odk[c][r] = dk[o];
                odv[c][r] = dv[o];
            }
    }
    f32x16 gk[2] = {f32x16{}, f32x16{}}, gv[2] = {f32x16{}, f32x16{}};
    for (int k0 = 0; k0 < HD; k0 += 2) {
        const float va = Vs[(32 * rt + l32) * LB_P + k0 + hi];  // v[u][e = k]
        const float fa = Fs[(32 * rt + l32) * LB_P + k0 + hi];  // f[u][d = k]
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int n = 32 * (ct0 + c) + l32;
            gk[c] = mfma_f32_32x32x2(va, Ms[n * LB_P + k0 + hi], gk[c]);    // Gc[d = n][e = k]
            gv[c] = mfma_f32_32x32x2(fa, Ms[(k0 + hi) * LB_P + n], gv[c]);  // Gc[d = k][e = n]
        }
    }
    // the key check only in the ragged last block (one uniform branch)
    auto store = [&](auto ragged, auto acc) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int n = 32 * (ct0 + c) + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int uu = 32 * rt + mfma32_row(lane, r);
                if (decltype(ragged)::value && uu >= nk) continue;
                const int64_t o = (bh * N + j * KBLK + uu) * HD + n;
                const float g = (gk[c][r] + wv[n]) * fminf(Fs[uu * LB_P + n], 1.f);
                dk[o] = decltype(acc)::value ? odk[c][r] + g : g;
                dv[o] = decltype(acc)::value ? odv[c][r] + gv[c][r] : gv[c][r];
            }
        }
    };
    if (nk == KBLK) {
        if (accumulate) store(std::false_type{}, std::true_type{});
        else store(std::false_type{}, std::false_type{});
    } else {
        if (accumulate) store(std::true_type{}, std::true_type{});
        else store(std::true_type{}, std::false_type{});
    }
}

// ---------------------------------------------------------------------------


size_t keep_bits_bytes(int64_t BH, int64_t nqb, int64_t nkb) {
    return (size_t)BH * nkb * ((nqb + 31) / 32) * 4;
}

hipError_t launch_inv_lists(const int32_t* kidx, int keep, int64_t BH, int nqb, int nkb,
                            uint32_t* bits, uint16_t* lists, int32_t* counts, hipStream_t st) {
    hipLaunchKernelGGL(keep_bits_kernel, dim3((nqb + 31) / 32, BH), dim3(256), (size_t)nkb * 4, st,
                       kidx, keep, nqb, nkb, bits);
    hipLaunchKernelGGL(inv_lists_kernel, dim3((nkb + 255) / 256, BH), dim3(256), 0, st, bits, nqb,
                       nkb, lists, counts);
    return hipGetLastError();
}

hipError_t launch_bwd_sparse(const BwdArgs& a, hipStream_t st) {
    const int64_t nq = a.BH * a.nqb, nk = a.BH * a.nkb;
    if (a.kidx) {
        hipLaunchKernelGGL(dq_kernel<false>, dim3((unsigned)nq), dim3(256), 0, st, a);
        hipLaunchKernelGGL(dkdv_kernel<false>, dim3((unsigned)nk), dim3(DK_THREADS), 0, st, a);
    } else {
        hipLaunchKernelGGL(dq_kernel<true>, dim3((unsigned)nq), dim3(256), 0, st, a);
        hipLaunchKernelGGL(dkdv_kernel<true>, dim3((unsigned)nk), dim3(DK_THREADS), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_lin_bwd_q(const uint16_t* q, const uint16_t* dout, const float* hnon, int64_t BH,
                            int N, float* dq, float* gf, uint16_t* gs, uint16_t* gs_lo, float* dol,
                            hipStream_t st) {
    const int nqb = (N + QBLK - 1) / QBLK;
    hipLaunchKernelGGL(lin_bwd_q_kernel, dim3(nqb, BH), dim3(256), 0, st, q, dout, hnon, N, nqb, dq,
                       gf, gs, gs_lo, dol);
    return hipGetLastError();
}

hipError_t launch_dstat(const uint16_t* dout, const float* out32, const float* dol, int64_t rows,
                        float* dstat, hipStream_t st) {
    const int64_t wg = std::min<int64_t>((rows + 15) / 16, 65536);
    hipLaunchKernelGGL(dstat_kernel, dim3((unsigned)wg), dim3(256), 0, st, dout, out32, dol, rows,
                       dstat);
    return hipGetLastError();
}

hipError_t launch_lin_bwd_k(const uint16_t* k, const uint16_t* v, const float* gc, int64_t BH,
                            int N, int accumulate, float* dk, float* dv, hipStream_t st) {
    const int nkb = (N + KBLK - 1) / KBLK;
    hipLaunchKernelGGL(lin_bwd_k_kernel, dim3(nkb, BH), dim3(256), 0, st, k, v, gc, N, nkb,
                       accumulate, dk, dv);
    return hipGetLastError();
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t st) {
    const int64_t wg = std::min<int64_t>((n + 255) / 256, 65536);
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)wg), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace ssa
