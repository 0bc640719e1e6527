// w8a8.hip -- the W8A8 linear layer: 128x128 block INT8 quantization and the
// block-dequantized INT8 matrix-core product.
//
// TurboDiffusion pages, page 5 "Four Technical Pillars", Pillar Three: the
// linear layers run with INT8 weights and activations, quantized with a
// block-wise granularity of 128x128. y = x . w^T for activations x [M][K]
// and weights w [N][K] (a linear layer's [out][in] layout); each operand is
// quantized per 128 x 128 block with the Pillar One rule (scale = max|v|/127,
// round half to even). The product is exact in int32 within each 128-wide
// block of K and is dequantized block by block:
//   y = fmaf((float)I_kb, fl32(sx[m/128][kb] * sw[n/128][kb]), y), kb ascending.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ssa {

constexpr int W8 = 128;  // block edge

// One 128 x 128 block of a row-major [rows][cols] bf16 matrix per workgroup:
// thread (row r = tid/16 + 16it, 16-byte chunk g = tid%16) holds 8 values of
// each of its 8 rows. Rows past the end re-read the last row and are dropped.
__global__ __launch_bounds__(256) void w8a8_quant_kernel(const uint16_t* __restrict__ x,
                                                         int rows, int cols,
                                                         int8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
    __shared__ float wmax[4];
    const int tid = threadIdx.x, g = tid & 15;
    const int cb = blockIdx.x, rb = blockIdx.y, ncb = gridDim.x;
    const int r0 = rb * W8;
    const int valid = min(W8, rows - r0);
    const uint16_t* base = x + (int64_t)r0 * cols + cb * W8 + 8 * g;
    u16x8 r8[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int row = min((tid >> 4) + 16 * it, valid - 1);
        r8[it] = *(const u16x8*)(base + (int64_t)row * cols);
    }
    float v[8][8];
    float amax = 0.f;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const bool ok = (tid >> 4) + 16 * it < valid;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v[it][e] = ok ? bf2f(r8[it][e]) : 0.f;
            amax = fmaxf(amax, fabsf(v[it][e]));
        }
    }
    amax = wave_max_f32(amax);
    if ((tid & 63) == 0) wmax[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float s = amax / 127.0f;
    if (tid == 0) scale[rb * ncb + cb] = s;
    int8_t* qbase = q + (int64_t)r0 * cols + cb * W8 + 8 * g;
    // q = clamp(rint(v / s)); the quotient through div_by_scale when the
    // (block-uniform) scale allows, which gives the same bytes
    auto store = [&](auto fast) {
        const float rs = decltype(fast)::value ? 1.0f / s : 0.f;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int row = (tid >> 4) + 16 * it;
            if (row < valid) {
                uint32_t w[2] = {0u, 0u};
                if (s > 0.f) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float qt = decltype(fast)::value ? div_by_scale(v[it][e], s, rs)
                                                               : v[it][e] / s;
                        const float r = fminf(fmaxf(__builtin_rintf(qt), -127.f), 127.f);
                        w[e >> 2] |= (uint32_t)(uint8_t)(int8_t)(int)r << (8 * (e & 3));
                    }
                }
                *(u32x2*)(qbase + (int64_t)row * cols) = u32x2{w[0], w[1]};
            }
        }
    };
    if (s >= FAST_DIV_MIN_SCALE && s <= FAST_DIV_MAX_SCALE)
        store(std::true_type{});
    else
        store(std::false_type{});
}

// ---- the product -------------------------------------------------------------
// Computed transposed, C^T = W . X^T, on v_mfma_i32_32x32x32_i8: the A operand
// is a weight fragment (rows n), the B operand an activation fragment (columns
// m), so each lane of a result holds four consecutive n of one m and stores
// them as one run.
//
// Workgroup: 16 waves (four per SIMD), tile 256 m x 128 n. Wave w owns
// m 64*(w/4) .. +63 and n 32*(w%4) .. +31: two 32x32 tiles, each with an int32
// accumulator for the current 128-wide K block and an fp32 one for the
// dequantized sum (about 120 VGPRs: four waves per SIMD hide each other's
// LDS-read and dequantization latencies). A stage is one K block: the X tile
// [256 m][128 k] (32 KB) and the W tile [128 n][128 k] (16 KB), 128-byte rows
// with 16-byte chunk c of row r at slot c ^ swz(r) (a 16-lane group reading 16
// consecutive rows at one chunk hits 16 distinct bank groups), fetched by LDS
// DMA into a 3-deep ring two stages ahead: 3 DMAs of 1 KB per wave per stage.
constexpr int WG_TM = 256, WG_TN = 128, WG_STAGES = 3;
constexpr int WG_WAVES = 16, WG_THREADS = 64 * WG_WAVES;
constexpr int WG_XT = WG_TM * W8, WG_WT = WG_TN * W8;  // bytes of the stage's tiles
constexpr int WG_STAGE = WG_XT + WG_WT;
constexpr int XD = WG_TM / 8 / WG_WAVES, WD = WG_TN / 8 / WG_WAVES;  // DMAs per wave per stage
constexpr int WG_GROUP_M = 4;  // m tiles per group of the tile order
static_assert(XD == 2 && WD == 1, "the stage is 48 DMAs of 1 KB over 16 waves");

__device__ __forceinline__ int w8swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__global__ __launch_bounds__(WG_THREADS, 1) void w8a8_gemm_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ sx, const int8_t* __restrict__ wq,
    const float* __restrict__ sw, const float* __restrict__ bias, int M, int N, int K,
    uint16_t* __restrict__ y, float* __restrict__ y32) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[WG_STAGES * WG_STAGE];
    const int nmt = (M + WG_TM - 1) / WG_TM, nnt = N / WG_TN, nkb = K / W8;
    const int64_t total = (int64_t)nmt * nnt;
    const int64_t item = xcd_item(blockIdx.x, total);
    if (item >= total) return;
    // grouped order: WG_GROUP_M m tiles share each n tile in turn, so the
    // workgroups running together on one XCD share X and W K-slices in L2
    const int64_t per_group = (int64_t)WG_GROUP_M * nnt;
    const int grp = (int)(item / per_group);
    const int gm = min(WG_GROUP_M, nmt - grp * WG_GROUP_M);
    const int rem = (int)(item - grp * per_group);
    const int mt = grp * WG_GROUP_M + rem % gm, nt = rem / gm;
    const int m0 = mt * WG_TM, n0 = nt * WG_TN;
    // (the wave index through readfirstlane: the compiler then keeps everything
    // derived from it in scalar registers and loads the scales through the
    // scalar cache)
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63,
              l32 = lane & 31, hi = lane >> 5, wm = wave >> 2, wn = wave & 3;

    // DMA lane offsets: DMA p of wave w fills 8 rows at 8*(2w + p) (X) or 8w
    // (W); lane l fetches row + l/8, chunk (l%8) ^ swz(row). X rows past M
    // re-read row M-1 (never stored).
    uint32_t xoff[XD], woff[WD];
#pragma unroll
    for (int p = 0; p < XD; ++p) {
        const int row = 8 * (XD * wave + p) + (lane >> 3);
        xoff[p] = (uint32_t)(min(m0 + row, M - 1) - m0) * (uint32_t)K + 16 * ((lane & 7) ^ w8swz(row));
    }
#pragma unroll
    for (int p = 0; p < WD; ++p) {
        const int row = 8 * (WD * wave + p) + (lane >> 3);
        woff[p] = (uint32_t)row * (uint32_t)K + 16 * ((lane & 7) ^ w8swz(row));
    }
    const int8_t* xbase = xq + (int64_t)m0 * K;
    const int8_t* wbase = wq + (int64_t)n0 * K;
    auto issue = [&](int kb, int st) {
        uint8_t* X = smem + st * WG_STAGE;
        uint8_t* W = X + WG_XT;
#pragma unroll
        for (int p = 0; p < XD; ++p)
            dma16(xbase + kb * W8, xoff[p], lds_u32(X + 8 * (XD * wave + p) * W8));
#pragma unroll
        for (int p = 0; p < WD; ++p)
            dma16(wbase + kb * W8, woff[p], lds_u32(W + 8 * (WD * wave + p) * W8));
    };

    f32x16 acc[2] = {f32x16{}, f32x16{}};  // [m tile], dequantized
    // this wave's 128-blocks (rows past M, never stored, use the last m block)
    const int mb = min((m0 + 64 * wm) / W8, (M - 1) / W8), nb = n0 / W8;
    const float* sxr = sx + (int64_t)mb * nkb;
    const float* swr = sw + (int64_t)nb * nkb;

    // Fragment addresses: the rows a lane reads are 32wn + l32 (W) and
    // 64wm + 32t + l32 (X), whose swizzle depends on l32 only, so a lane needs
    // one chunk offset per K step; t and the ring stage are immediate offsets.
    const int sl = w8swz(l32);
    uint32_t coff[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) coff[ks] = (uint32_t)(((2 * ks + hi) ^ sl) * 16);
    const uint32_t wrow = (uint32_t)(WG_XT + (32 * wn + l32) * W8), xrow = (uint32_t)((64 * wm + l32) * W8);

    // K block kb from ring stage R: 4 K steps of 2 MFMAs, the fragments of
    // step ks+1 read while those of step ks are in use; then the block's
    // int32 sums are scaled into the fp32 sums (y = fmaf(I, sx*sw, y)).
    auto kblock = [&](int kb, auto stage) {
        constexpr int R = decltype(stage)::value;
        const uint8_t* S = smem + R * WG_STAGE;
        auto frag = [&](int ks, i32x4& w, i32x4 (&x)[2]) {
            w = *(const i32x4*)(S + wrow + coff[ks]);
#pragma unroll
            for (int t = 0; t < 2; ++t) x[t] = *(const i32x4*)(S + xrow + coff[ks] + 32 * t * W8);
        };
        i32x4 nwf, nxf[2];
        frag(0, nwf, nxf);
        i32x16 ia[2];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const i32x4 wf = nwf, xf[2] = {nxf[0], nxf[1]};
            if (ks < 3) frag(ks + 1, nwf, nxf);
#pragma unroll
            for (int b = 0; b < 2; ++b) ia[b] = mfma_i8_32x32x32(wf, xf[b], ks ? ia[b] : i32x16{});
        }
        const float s = sxr[kb] * swr[kb];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[b][r] = __builtin_fmaf((float)ia[b][r], s, acc[b][r]);
        // pin the dequantization here: left free, the compiler sinks it past
        // the following blocks and keeps their int32 sums all live
#pragma unroll
        for (int b = 0; b < 2; ++b) asm volatile("" : "+v"(acc[b]));
    };

    // Pipeline: stage kb % 3, two stages ahead; at the end of step kb only the
    // DMAs of stage kb+2 may still be in flight.
    issue(0, 0);
    if (nkb > 1) issue(1, 1);
    if (nkb > 1) wait_vm<XD + WD>(); else wait_vm<0>();
    __syncthreads();
    auto step = [&](int kb, auto stage) {
        constexpr int R = decltype(stage)::value;
        if (kb + 2 < nkb) issue(kb + 2, (R + 2) % WG_STAGES);
        kblock(kb, stage);
        if (kb + 1 < nkb) {
            if (kb + 2 < nkb) wait_vm<XD + WD>(); else wait_vm<0>();
            __syncthreads();
        }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    static_assert(WG_STAGES == 3, "the K loop is unrolled by the ring depth");
    int kb = 0;
    for (; kb + 3 <= nkb; kb += 3) {
        step(kb, S0{});
        step(kb + 1, S1{});
        step(kb + 2, S2{});
    }
    if (kb < nkb) step(kb++, S0{});
    if (kb < nkb) step(kb++, S1{});

    // lane (m = l32, hi), tile [b] register 4q + x holds n = 8q + 4hi + x; the
    // bias (one fp32 add after the whole chain) is the same for both m tiles
    f32x4 bq[4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
        bq[qd] = bias ? *(const f32x4*)(bias + n0 + 32 * wn + 8 * qd + 4 * hi) : f32x4{};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int m = m0 + 64 * wm + 32 * b + l32;
        if (m >= M) continue;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int n = n0 + 32 * wn + 8 * qd + 4 * hi;
            f32x4 c = f32x4{acc[b][4 * qd], acc[b][4 * qd + 1], acc[b][4 * qd + 2], acc[b][4 * qd + 3]};
            if (bias) c = c + bq[qd];
            *(u16x4*)(y + (int64_t)m * N + n) = u16x4{f2bf(c[0]), f2bf(c[1]), f2bf(c[2]), f2bf(c[3])};
            if (y32) *(f32x4*)(y32 + (int64_t)m * N + n) = c;
        }
    }
}

hipError_t launch_w8a8_quant(const uint16_t* x, int rows, int cols, int8_t* q, float* scale,
                             hipStream_t st) {
    hipLaunchKernelGGL(w8a8_quant_kernel, dim3(cols / W8, (rows + W8 - 1) / W8), dim3(256), 0, st,
                       x, rows, cols, q, scale);
    return hipGetLastError();
}

int64_t w8a8_gemm_workgroups(int64_t M, int64_t N) {
    const int64_t total = ((M + WG_TM - 1) / WG_TM) * (N / WG_TN);
    return (total + 7) / 8 * 8;
}

hipError_t launch_w8a8_gemm(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                            const float* bias, int M, int N, int K, uint16_t* y, float* y32,
                            hipStream_t st) {
    const int64_t grid = w8a8_gemm_workgroups(M, N);
    hipLaunchKernelGGL(w8a8_gemm_kernel, dim3((unsigned)grid), dim3(WG_THREADS), 0, st, xq, sx, wq, sw,
                       bias, M, N, K, y, y32);
    return hipGetLastError();
}

}  // namespace ssa
