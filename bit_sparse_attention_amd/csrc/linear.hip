// linear.hip -- the linear-attention branch of SageSLA, and the V re-layout
// the sparse kernel reads.
//
// TurboDiffusion pages, page 5 "Four Technical Pillars", Pillar Two: the
// block interactions the sparse part skips are covered by a light global
// linear-attention term. With phi = elu + 1 on raw K, each 64-token key block
// j contributes the state h_j = sum_u phi(k_u) v_u^T (128 x 128) and
// z_j = sum_u phi(k_u). A query block needs the sums over the key blocks it did
// NOT keep. They are formed as H_i = H_total - sum_{j kept} h_j: H_total in
// fp32, the kept-block sum as a dense 0/1 x bf16 matrix-core GEMM, so the bf16
// rounding of h_j only touches the kept ~10% of the blocks.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ssa {

constexpr int TP = KBLK + 8;  // LDS pitch (bf16) of a [channel][token] tile: 144 B

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
// order, and each lane then stores 16-byte runs.
template <bool STATES>
__global__ __launch_bounds__(256) void linear_states_kernel(const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v, int N,
                                                            int nkb, int ngroups,
                                                            uint16_t* __restrict__ vt,
                                                            uint16_t* __restrict__ hs,
                                                            float* __restrict__ hpart) {
    __shared__ __attribute__((aligned(16))) uint16_t vtl[HD * TP];
    __shared__ __attribute__((aligned(16))) uint16_t fkh[STATES ? HD * TP : 8];
    __shared__ __attribute__((aligned(16))) uint16_t fkl[STATES ? HD * TP : 8];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31,
              hi = lane >> 5;
    const int64_t bh = blockIdx.y;
    const int g = blockIdx.x;
    const int G = STATES ? LIN_GROUP : 1;
    f32x16 tot[4], totz = f32x16{};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) tot[dt] = f32x16{};
    // raw K and V of one key block in registers: lane (tid) holds token
    // u = tid & 63, channels 8ch .. 8ch+7 for ch = (tid >> 6) + 4*it. Two sets,
    // so the loads of blocks j+1 and j+2 are in flight while block j is worked.
    u16x8 va[4], ka[4], vb[4], kb[4];
    auto load = [&](int j, u16x8 (&vv)[4], u16x8 (&kk)[4]) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int c = tid + 256 * it;
            const int u = c & 63, ch = c >> 6;
            const int tok = j * KBLK + u;
            const bool ok = tok < N;
            const int64_t off = (bh * N + (ok ? tok : 0)) * HD + 8 * ch;
            vv[it] = ok ? *(const u16x8*)(v + off) : u16x8{};
            if (STATES) kk[it] = ok ? *(const u16x8*)(k + off) : u16x8{};
        }
    };
    auto block = [&](int jb, u16x8 (&vv)[4], u16x8 (&kk)[4]) {
        const int j = g * G + jb;
        // channel-major LDS stores (u fastest: conflict free)
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int c = tid + 256 * it;
            const int u = c & 63, ch = c >> 6;
            const bool ok = j * KBLK + u < N;
#pragma unroll
            for (int e = 0; e < 8; ++e) vtl[(8 * ch + e) * TP + u] = vv[it][e];
            if (STATES) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float f = bf2f(kk[it][e]);
                    const float ph = ok ? (f > 0.f ? f + 1.f : __expf(f)) : 0.f;
                    __bf16 h, l;
                    split_bf16(ph, h, l);
                    fkh[(8 * ch + e) * TP + u] = __builtin_bit_cast(uint16_t, h);
                    fkl[(8 * ch + e) * TP + u] = __builtin_bit_cast(uint16_t, l);
                }
            }
        }
        __syncthreads();
        // the registers are free again: block j+2 goes in flight
        if (jb + 2 < G && j + 2 < nkb) load(j + 2, vv, kk);
        // V^T tile in the sparse kernel's key order: 128 rows x 8 chunks of 16 B
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int c = tid + 256 * it;
            const int dv = c >> 3, pc = c & 7, cc = pc >> 1, h2 = pc & 1;
            const u16x4 a = *(const u16x4*)(vtl + dv * TP + 16 * cc + 4 * h2);
            const u16x4 b = *(const u16x4*)(vtl + dv * TP + 16 * cc + 8 + 4 * h2);
            *(u16x8*)(vt + ((bh * nkb + j) * HD + dv) * KBLK + 8 * pc) =
                u16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        }
        if (STATES) {
            // (h_j^T)^T[d][e] = sum_u phi(K)[u][d] V[u][e]: A = phi(K)^T rows d (hi and
            // lo parts, two products, fp32 accumulation), B = V columns e. Wave w
            // takes columns e = 32w .. 32w+31; acc[dt] holds rows d = 32dt + ...
            f32x16 acc[4], accz = f32x16{};
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
            bf16x8 ones;
#pragma unroll
            for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
#pragma unroll
            for (int uc = 0; uc < 4; ++uc) {
                const bf16x8 b = *(const bf16x8*)(vtl + (32 * wave + l32) * TP + 16 * uc + 8 * hi);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const bf16x8 ah = *(const bf16x8*)(fkh + (32 * dt + l32) * TP + 16 * uc + 8 * hi);
                    const bf16x8 al = *(const bf16x8*)(fkl + (32 * dt + l32) * TP + 16 * uc + 8 * hi);
                    acc[dt] = mfma_bf16_32x32x16(ah, b, acc[dt]);
                    acc[dt] = mfma_bf16_32x32x16(al, b, acc[dt]);
                }
            }
            // z_j[d] for rows d = 32w + ...: the same product against ones
#pragma unroll
            for (int uc = 0; uc < 4; ++uc) {
                const int o = (32 * wave + l32) * TP + 16 * uc + 8 * hi;
                accz = mfma_bf16_32x32x16(*(const bf16x8*)(fkh + o), ones, accz);
                accz = mfma_bf16_32x32x16(*(const bf16x8*)(fkl + o), ones, accz);
            }
            // lane (column e = 32w + l32, hi) holds rows d = 32dt + 8(r/4) + 4hi + r%4:
            // registers 8rb .. 8rb+7 are positions 16(2dt + rb) + 8hi + 0..7 of row e
            uint16_t* hrow = hs + (bh * nkb + j) * (int64_t)HS_ROW;
            const int e = 32 * wave + l32;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    u16x8 o8;
#pragma unroll
                    for (int x = 0; x < 8; ++x) o8[x] = f2bf(acc[dt][8 * rb + x]);
                    *(u16x8*)(hrow + e * HD + 16 * (2 * dt + rb) + 8 * hi) = o8;
                }
                tot[dt] += acc[dt];
            }
            if (l32 == 0) {  // z rows d = 32w + ..., every column equal
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    u16x8 o8;
#pragma unroll
                    for (int x = 0; x < 8; ++x) o8[x] = f2bf(accz[8 * rb + x]);
                    *(u16x8*)(hrow + HD * HD + 16 * (2 * wave + rb) + 8 * hi) = o8;
                }
            }
            totz += accz;
        }
        __syncthreads();
    };
    const int nb = min(G, nkb - g * G);  // key blocks of this workgroup
    if (nb > 0) load(g * G, va, ka);
    if (nb > 1) load(g * G + 1, vb, kb);
    for (int jb = 0; jb < nb; jb += 2) {
        block(jb, va, ka);
        if (jb + 1 < nb) block(jb + 1, vb, kb);
    }
    if (STATES) {
        float* prow = hpart + (bh * ngroups + g) * (int64_t)HS_ROW;
        const int e = 32 * wave + l32;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                float* dst = prow + e * HD + 16 * (2 * dt + rb) + 8 * hi;
                *(f32x4*)dst = f32x4{tot[dt][8 * rb], tot[dt][8 * rb + 1], tot[dt][8 * rb + 2],
                                     tot[dt][8 * rb + 3]};
                *(f32x4*)(dst + 4) = f32x4{tot[dt][8 * rb + 4], tot[dt][8 * rb + 5],
                                           tot[dt][8 * rb + 6], tot[dt][8 * rb + 7]};
            }
        if (l32 == 0)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                float* dst = prow + HD * HD + 16 * (2 * wave + rb) + 8 * hi;
                *(f32x4*)dst = f32x4{totz[8 * rb], totz[8 * rb + 1], totz[8 * rb + 2], totz[8 * rb + 3]};
                *(f32x4*)(dst + 4) =
                    f32x4{totz[8 * rb + 4], totz[8 * rb + 5], totz[8 * rb + 6], totz[8 * rb + 7]};
            }
    }
}

// H_total[bh][n] = sum over groups, in group order, of the fp32 partials.
__global__ __launch_bounds__(256) void htot_kernel(const float* __restrict__ hpart, int ngroups,
                                                   float* __restrict__ htot) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    const int64_t bh = blockIdx.y;
    if (n >= HS_ROW) return;
    // loads in batches of 16 so they are in flight together; the adds stay in
    // group order
    const float* p = hpart + bh * ngroups * (int64_t)HS_ROW + n;
    float s = 0.f;
    for (int g0 = 0; g0 < ngroups; g0 += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = g0 + u < ngroups ? p[(int64_t)(g0 + u) * HS_ROW] : 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u)
            if (g0 + u < ngroups) s += v[u];
    }
    htot[bh * HS_ROW + n] = s;
}

// msel[bh][i][j] = 1 (bf16) if key block j is kept by query block i, else 0;
// j runs to nkbp (a multiple of GEMM_KALIGN) so the GEMM reads whole K steps.
__global__ __launch_bounds__(256) void msel_kernel(const int32_t* __restrict__ kidx, int keep,
                                                   int nqb, int nkbp, uint16_t* __restrict__ msel) {
    const int64_t bh = blockIdx.y;
    const int i = blockIdx.x;
    const int32_t* src = kidx + (bh * nqb + i) * (int64_t)keep;
    uint16_t* dst = msel + (bh * nqb + i) * (int64_t)nkbp;
    // zero the row, then set the kept blocks (indices clamped into the row)
    for (int j = threadIdx.x; j < nkbp; j += 256) dst[j] = 0;
    __syncthreads();
    for (int a = threadIdx.x; a < keep; a += 256) dst[min(max(src[a], 0), nkbp - 1)] = 0x3F80;
}

// Complement GEMM: hnon[bh][i][n] = htot[bh][n] - sum_j msel[bh][i][j] * hs[bh][j][n]
// (i < nqb query blocks, n < HS_ROW state entries, j < nkbp key blocks; msel
// is 0/1). bf16 operands, fp32 accumulation.
// Workgroup tile 128 (i) x 128 (n), K step GTK, 2 x 2 waves of 64 x 64, each a
// 2 x 2 grid of 32x32x16 bf16 MFMAs. Operand tiles arrive by LDS DMA into a
// GSTAGE-deep ring:
//   A [128 i][GTK j]: rows of GTK*2 bytes, 16-byte chunk c of row r at slot
//     c ^ aswz(r), so the 16 rows a 16-lane group reads hit 16 distinct
//     bank groups;
//   B [GTK j][128 n]: 256-byte rows kept j-major as in memory, 8-byte unit u of
//     row r at u ^ 8*(r & 3), read with transposing loads (lds_read_tr16) so
//     each lane gets 4 consecutive j of one column n; the 32 lanes of a half
//     wave then hit 32 distinct 8-byte bank groups.
#ifndef SSA_GEMM_TK
#define SSA_GEMM_TK 32
#endif
#ifndef SSA_GEMM_STAGES
#define SSA_GEMM_STAGES 3
#endif
constexpr int GTM = 128, GTN = 128, GTK = SSA_GEMM_TK, GSTAGE = SSA_GEMM_STAGES;
static_assert(GTK == 32 || GTK == 64, "K step");
static_assert(GEMM_KALIGN % GTK == 0, "padded key-block count must be whole K steps");
constexpr int GA_ROW = GTK * 2, GA_CH = GA_ROW / 16;   // A row bytes, 16-byte chunks per row
constexpr int GA_BYTES = GTM * GA_ROW, GB_BYTES = GTK * GTN * 2;
constexpr int NDA = 32 * GA_ROW / 1024;                // A DMAs per wave (32 rows each wave)
constexpr int NDB = GTK / 16;                          // B DMAs per wave (GTK/4 rows each wave)
constexpr int GPD = GSTAGE - 1;                        // prefetch distance (K steps)

__device__ __forceinline__ int aswz(int r) { return GA_CH == 4 ? (r >> 2) & 3 : (r >> 1) & 7; }

__global__ __launch_bounds__(256, 2) void complement_gemm_kernel(
    const uint16_t* __restrict__ msel, const uint16_t* __restrict__ hs, const float* __restrict__ htot,
    int64_t BH, int nqb, int nkb, int nkbp, float* __restrict__ hnon) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[GSTAGE * (GA_BYTES + GB_BYTES)];
    uint8_t(*As)[GA_BYTES] = reinterpret_cast<uint8_t(*)[GA_BYTES]>(smem);
    uint8_t(*Bs)[GB_BYTES] = reinterpret_cast<uint8_t(*)[GB_BYTES]>(smem + GSTAGE * GA_BYTES);
    const int nnt = HS_ROW / GTN, nmt = (nqb + GTM - 1) / GTM;
    const int64_t total = BH * nnt * nmt;
    const int64_t item = xcd_item(blockIdx.x, total);  // m fastest: B tiles shared in L2
    if (item >= total) return;
    const int mt = (int)(item % nmt);
    const int64_t rest = item / nmt;
    const int nt = (int)(rest % nnt);
    const int64_t bh = rest / nnt;
    const int i0 = mt * GTM, n0 = nt * GTN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31,
              h = lane >> 5, wm = wave >> 1, wn = wave & 1;

    // loop-invariant DMA lane offsets: wave w fills A rows 32w..32w+31 and
    // B rows (GTK/4)w .. +GTK/4, 1 KB per DMA
    constexpr int ARD = 1024 / GA_ROW;  // A rows per DMA
    uint32_t aoff[NDA], boff[NDB];
#pragma unroll
    for (int p = 0; p < NDA; ++p) {
        const int ra = 32 * wave + ARD * p + lane / GA_CH;
        const int ca = (lane % GA_CH) ^ aswz(ra);
        aoff[p] = (uint32_t)(min(i0 + ra, nqb - 1) * nkbp * 2 + ca * 16);
    }
#pragma unroll
    for (int p = 0; p < NDB; ++p) {
        const int rb = (GTK / 4) * wave + 4 * p + (lane >> 4);
        const int cb = (lane & 15) ^ (4 * (rb & 3));
        boff[p] = (uint32_t)(rb * HS_ROW * 2 + cb * 16);
    }
    const uint16_t* abase = msel + (bh * nqb) * (int64_t)nkbp;
    const uint16_t* bbase = hs + (bh * nkb) * (int64_t)HS_ROW + n0;
    // K step ks into ring stage st (a compile-time constant in the main loop)
    auto issue = [&](int ks, int st) {
        const int j0 = ks * GTK;
#pragma unroll
        for (int p = 0; p < NDA; ++p)
            dma16(abase + j0, aoff[p], lds_u32(As[st] + (32 * wave + ARD * p) * GA_ROW));
        // Rows past nkb (msel is 0 there) are fetched from row nkb-1. In such a
        // ragged step the offset is taken from the unshifted base with the
        // absolute row clamped: a K step may start at or past nkb (the
        // padded count is a multiple of GEMM_KALIGN), and a row relative to
        // j0 would then be negative, which the unsigned 32-bit lane offset of
        // the DMA cannot express.
        const bool ragged = j0 + GTK > nkb;
#pragma unroll
        for (int p = 0; p < NDB; ++p) {
            const uint32_t lds = lds_u32(Bs[st] + ((GTK / 4) * wave + 4 * p) * 256);
            if (ragged) {
                const int rb = (GTK / 4) * wave + 4 * p + (lane >> 4);
                const int cb = (lane & 15) ^ (4 * (rb & 3));
                const int r = min(j0 + rb, nkb - 1);
                dma16(bbase, (uint32_t)(r * HS_ROW * 2 + cb * 16), lds);
            } else {
                dma16(bbase + (int64_t)j0 * HS_ROW, boff[p], lds);
            }
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

    const int nks = nkbp / GTK;
    // prologue: steps 0 .. GPD-1 in flight, step 0 landed
    for (int ks = 0; ks < GPD && ks < nks; ++ks) issue(ks, ks);
    if (GPD > 1 && nks > 1) wait_vm<(GPD - 1) * (NDA + NDB)>(); else wait_vm<0>();
    __syncthreads();
    // one K step from ring stage R (compile-time: LDS addresses are immediates)
    auto kstep = [&](int ks, auto stage) {
        constexpr int R = decltype(stage)::value;
        if (ks + GPD < nks) issue(ks + GPD, (R + GPD) % GSTAGE);
        const uint8_t* A = As[R];
        const uint8_t* B = Bs[R];
#pragma unroll
        for (int kc = 0; kc < GTK / 16; ++kc) {
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const int row = 64 * wm + 32 * a + l32;
                const int slot = (2 * kc + h) ^ aswz(row);
                af[a] = *(const bf16x8*)(A + row * GA_ROW + slot * 16);
            }
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int col = 64 * wn + 32 * b + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
                i16x4 part[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int row = 16 * kc + 8 * h + 4 * t + ((lane & 15) >> 2);
                    const int unit = (col >> 2) ^ (8 * (row & 3));
                    part[t] = lds_read_tr16(B + row * 256 + unit * 8);
                }
                // k-slots 0-3 from the first read, 4-7 from the second (whole dwords)
                const u32x2 w0 = __builtin_bit_cast(u32x2, part[0]);
                const u32x2 w1 = __builtin_bit_cast(u32x2, part[1]);
                bfr[b] = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[a][b] = mfma_bf16_32x32x16(af[a], bfr[b], acc[a][b]);
        }
        // step ks+1 must land; later steps may stay in flight
        if (GPD > 1 && ks + GPD < nks) wait_vm<(GPD - 1) * (NDA + NDB)>(); else wait_vm<0>();
        __syncthreads();
    };
    static_assert(GSTAGE >= 2 && GSTAGE <= 4, "the K loop is unrolled by the ring depth");
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, (GSTAGE > 2 ? 2 : 0)>;
    using S3 = std::integral_constant<int, (GSTAGE > 3 ? 3 : 0)>;
    int ks = 0;
    for (; ks + GSTAGE <= nks; ks += GSTAGE) {
        kstep(ks, S0{});
        kstep(ks + 1, S1{});
        if (GSTAGE > 2) kstep(ks + 2, S2{});
        if (GSTAGE > 3) kstep(ks + 3, S3{});
    }
    if (ks < nks) kstep(ks++, S0{});
    if (ks < nks) kstep(ks++, S1{});
    if (GSTAGE > 3 && ks < nks) kstep(ks, S2{});
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = i0 + 64 * wm + 32 * a + mfma32_row(lane, r);
                const int n = n0 + 64 * wn + 32 * b + l32;
                if (i < nqb) hnon[(bh * nqb + i) * HS_ROW + n] = htot[bh * HS_ROW + n] - acc[a][b][r];
            }
}

// ---------------------------------------------------------------------------

hipError_t launch_linear_states(const uint16_t* k, const uint16_t* v, int64_t BH, int N,
                                uint16_t* vt, uint16_t* hs, float* hpart, float* htot,
                                hipStream_t st) {
    const int nkb = (N + KBLK - 1) / KBLK;
    const int ngroups = (nkb + LIN_GROUP - 1) / LIN_GROUP;
    hipLaunchKernelGGL((linear_states_kernel<true>), dim3(ngroups, BH), dim3(256), 0, st, k, v, N,
                       nkb, ngroups, vt, hs, hpart);
    hipLaunchKernelGGL(htot_kernel, dim3((HS_ROW + 255) / 256, BH), dim3(256), 0, st, hpart, ngroups,
                       htot);
    return hipGetLastError();
}

hipError_t launch_vt_only(const uint16_t* v, int64_t BH, int N, uint16_t* vt, hipStream_t st) {
    const int nkb = (N + KBLK - 1) / KBLK;
    hipLaunchKernelGGL((linear_states_kernel<false>), dim3(nkb, BH), dim3(256), 0, st, nullptr, v, N,
                       nkb, nkb, vt, nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_complement(const int32_t* kidx, int keep, const uint16_t* hs, const float* htot,
                             int64_t BH, int N, uint16_t* msel, float* hnon, hipStream_t st) {
    const int nqb = (N + QBLK - 1) / QBLK, nkb = (N + KBLK - 1) / KBLK;
    const int nkbp = (nkb + GEMM_KALIGN - 1) / GEMM_KALIGN * GEMM_KALIGN;
    hipLaunchKernelGGL(msel_kernel, dim3(nqb, BH), dim3(256), 0, st, kidx, keep, nqb,
                       nkbp, msel);
    const int64_t total = BH * (HS_ROW / 128) * ((nqb + 127) / 128);
    const int64_t grid = (total + 7) / 8 * 8;
    hipLaunchKernelGGL(complement_gemm_kernel, dim3((unsigned)grid), dim3(256), 0, st, msel, hs, htot,
                       BH, nqb, nkb, nkbp, hnon);
    return hipGetLastError();
}

}  // namespace ssa
