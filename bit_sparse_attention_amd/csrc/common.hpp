// common.hpp -- shared device helpers for the gfx950 SageSLA kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

constexpr int HD = 128;    // head dimension
constexpr int QBLK = 128;  // query block (tokens)
constexpr int KBLK = 64;   // key block (tokens)
constexpr int HS_ROW = HD * HD + HD;  // one linear state: h^T [e][d] then z [d]

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 honours the RNE mode).
__device__ __forceinline__ uint16_t f2bf(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ i32x16 mfma_i8_32x32x32(i32x4 a, i32x4 b, i32x16 c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Output layout of the 32x32 MFMA families: lane l, accumulator r holds
// column (l & 31) and row 8*(r/4) + 4*(l/32) + (r%4).
__device__ __forceinline__ int mfma32_row(int lane, int r) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Split an fp32 value into bf16 hi + bf16 lo (hi + lo carries ~16 bits).
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

__device__ __forceinline__ int wave_max_i32(int v) {
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Workgroup id -> logical work item so that consecutive items run on the same
// XCD. Workgroups are dispatched round-robin over the 8 XCDs; each XCD gets a
// contiguous range of items, processed in order, so neighbouring items (which
// share K/V or GEMM operand tiles) meet in that XCD's L2.
__device__ __forceinline__ int64_t xcd_item(int64_t wg, int64_t total) {
    const int64_t per = (total + 7) / 8;
    return (wg & 7) * per + (wg >> 3);
}

// ---- asynchronous global -> LDS copies (gfx950 LDS DMA) -------------------
// global_load_lds_dwordx4 writes lane l's 16 bytes at M0 + 16*l. It is issued
// from inline asm so the compiler neither tracks it nor inserts vmcnt waits
// before LDS reads; callers wait with wait_vm<N>() and a barrier. No "memory"
// clobber: callers only target LDS buffers nobody reads in the same pipeline
// step (a clobber would also demote read-only scalar loads to vector loads,
// whose vmcnt(0) waits would drain the pipeline).
// The compiler's hazard recognizer does not look inside the asm, so the block
// keeps the GFX9-family wait states itself: a vector memory instruction must
// not read an SGPR within 5 wait states of a VALU write of it (the base may
// come straight from v_readfirstlane), and an LDS DMA must not read M0 in the
// wait state right after an SALU write of it. The s_mov and s_nop 3 give 5.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
    const uint64_t b = (uint64_t)base;
    const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const void* sbase = (const void*)sb;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 3\n\tglobal_load_lds_dwordx4 %0, %1\n\ts_nop 0" ::"v"(voff),
                 "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_addr)));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    // s_waitcnt vmcnt(N); expcnt and lgkmcnt left unconstrained (gfx9 encoding)
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane g
// points at 4 contiguous 16-bit elements (row g of a 16 x 4 block) and lane i
// receives, as element k, row 4k + i/4 at column i%4.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(uintptr_t)lds_u32(p));
}

}  // namespace ssa
