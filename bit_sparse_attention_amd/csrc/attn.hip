// attn.hip -- the SageSLA sparse attention kernel for gfx950.
//
// TurboDiffusion pages, page 5 "Four Technical Pillars": Pillar One
// (attention in 8-bit integers on the integer matrix units) and Pillar Two
// (only the kept block interactions are computed exactly; a linear-attention
// term covers the rest), stacked as SageSLA.
//
// One workgroup = one 128-token query block of one head: 4 waves of 32 query
// rows, two workgroups per CU (two waves per SIMD). For each kept 64-token
// key block j (ascending):
//   S^T = K_j . Q^T        v_mfma_i32_32x32x32_i8, exact int32
//   x = S * c_ij           c_ij = fl32(fl32(sq*sk) * fl32(sm*log2 e))
//   m = integer normalizer (raised only when a tile's max exceeds it by more
//       than HEADROOM); rescaling by 2^k is exact and bf16 rounding commutes
//       with it, so p and the output do not depend on the tile order except
//       through the fp32 rounding of the exponent S*c - m, which depends on
//       the m in use: a p within that error of a bf16 rounding midpoint may
//       round either way (the flip window its tests allow for)
//   p = bf16(2^(S*c - m)), l += p (v_dot2 on packed pairs)
//   O^T += V_j^T . P^T     v_mfma_f32_32x32x16_bf16, fp32 accumulation
// S^T puts one query per lane column: row max and row sum stay in a lane
// pair, and the int32 accumulator order is the bf16 B-operand order of the
// PV product, so P never leaves registers. V arrives pre-transposed in that
// key order (linear.hip).
//
// Software pipeline: K and V tiles stream through 3-deep LDS rings by LDS
// DMA, K three blocks ahead and V two ahead, with one workgroup barrier per
// block. Each step issues QK(j+1) and PV(j) to the matrix cores in a fixed
// order, reading every LDS fragment ~8 MFMAs before its use, and runs the
// softmax of tile j+1 in slices between the PV MFMAs.
//
// The linear branch is applied in the epilogue from the complement states
// (phi(Q) . H_i / phi(Q) . z_i, split-bf16 MFMA) and added to the output.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ssa {

constexpr int WAVES = 4;               // 32 query rows each
constexpr int ATTN_THREADS = 64 * WAVES;
constexpr int NSTAGE = 3;            // LDS buffers per operand
constexpr int KTILE = KBLK * HD;     // bytes of an int8 K tile
constexpr int VTILE = HD * KBLK * 2; // bytes of a bf16 V^T tile

// Headroom of the integer normalizer: m is raised only when a tile's max
// exceeds it by more than this (log2 units). Any integer m gives the same
// result (rescaling by 2^k is exact and rounding commutes with it), so this
// only bounds p <= 2^HEADROOM (far from the fp32 / bf16 range limit of
// 2^127 even after summing 2^20 keys) and keeps rescales rare.
constexpr float HEADROOM = 64.0f;

// ---- tile staging: global -> LDS DMA, 128 threads ---------------------------
// Both tiles are 128-byte rows (K: 64 rows of int8 channels; V^T: 128 rows of
// 64 bf16 keys) stored with the 16-byte chunk c of row r at slot
// c ^ swz(r): reads of 8 or 16 consecutive rows at one chunk then hit
// distinct banks. Tiles arrive by LDS DMA (dma16): each lane fetches the
// chunk its slot must hold; the pipeline waits explicitly (wait_vm).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Two wave-uniform 32-bit loads through the scalar cache, completed inside
// the asm block. They stay off the vector-memory counter, so fetching the
// next kept-block index and scale never waits for the tile DMAs in flight.
// The outputs are early-clobber: the first load's destination is written
// while the second load's address may still be needed, so no output may
// share a register with either address.
__device__ __forceinline__ void sload2(const void* p1, const void* p2, int& v1, int& v2) {
    const uint64_t a = (uint64_t)p1, b = (uint64_t)p2;
    const uint64_t sa = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    asm volatile(
        "s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
        : "=&s"(v1), "=&s"(v2)
        : "s"((const void*)sa), "s"((const void*)sb));
}

// Per-lane byte offset inside a tile: DMA p of wave w fills rows
// r0 = rows_per_wave*w + 8p .. +7; lane l fetches the chunk its slot holds.
__device__ __forceinline__ uint32_t tile_voff(int rows_per_wave, int wave, int p, int lane) {
    const int row = rows_per_wave * wave + 8 * p + (lane >> 3);
    return row * 128 + 16 * ((lane & 7) ^ swz(row));
}

// K tile of key block j into LDS at lds_base (8/WAVES DMAs per wave). koff
// holds the loop-invariant lane offsets, krag those of the ragged last block,
// whose rows past N are fetched from row N-1 (those keys are masked out of
// every use).
__device__ __forceinline__ void dma_k_tile(const int8_t* __restrict__ k_i8, int64_t bh, int N, int j,
                                           uint32_t lds_base, int wave,
                                           const uint32_t (&koff)[8 / WAVES],
                                           const uint32_t (&krag)[8 / WAVES]) {
    const int8_t* base = k_i8 + (bh * N + (int64_t)j * KBLK) * HD;
    const bool ragged = (j + 1) * KBLK > N;
#pragma unroll
    for (int p = 0; p < 8 / WAVES; ++p)
        dma16(base, ragged ? krag[p] : koff[p],
              __builtin_amdgcn_readfirstlane(lds_base + ((64 / WAVES) * wave + 8 * p) * 128));
}

// Lane offsets of the ragged last key block (valid rows = nval < 64): row r
// is fetched from row min(r, nval - 1), into the slot that row r occupies.
__device__ __forceinline__ uint32_t tile_voff_ragged(int wave, int p, int lane, int nval) {
    const int row = (64 / WAVES) * wave + 8 * p + (lane >> 3);
    const int rr = min(row, nval - 1);
    return rr * 128 + 16 * ((lane & 7) ^ swz(row));
}

// V^T tile (128 rows of 64 keys, zero past N) into LDS (16/WAVES DMAs per wave).
__device__ __forceinline__ void dma_v_tile(const uint16_t* __restrict__ vtile, uint32_t lds_base,
                                           int wave, const uint32_t (&voff)[16 / WAVES]) {
#pragma unroll
    for (int p = 0; p < 16 / WAVES; ++p)
        dma16(vtile, voff[p], __builtin_amdgcn_readfirstlane(lds_base + ((128 / WAVES) * wave + 8 * p) * 128));
}

// Q operand of one 32-row group: lane supplies query (lane & 31), channels
// 32c + 16*(lane>>5) .. +15 for c = 0..3 (zero past N).
__device__ __forceinline__ void load_q_operand(const int8_t* __restrict__ q_i8, int64_t bh, int N,
                                               int t, int hi, i32x4 (&qop)[4]) {
    const bool ok = t < N;
    const int8_t* qp = q_i8 + (bh * N + (ok ? t : 0)) * HD;
#pragma unroll
    for (int c = 0; c < 4; ++c) qop[c] = ok ? *(const i32x4*)(qp + 32 * c + 16 * hi) : i32x4{};
}

// The shared QK^T routine: S^T of the LDS K tile against the wave's 32
// queries. Lane (l32, hi), register r of s[0] holds key 8*(r/4) + 4*hi + r%4
// for query l32 (s[1]: that key + 32).
__device__ __forceinline__ void qk_tile_mfma(const uint8_t* ks, const i32x4 (&qop)[4], int l32,
                                             int hi, i32x16 (&s)[2]) {
    s[0] = s[1] = i32x16{};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int slot = ((2 * c + hi) ^ swz(l32)) * 16;
        const i32x4 a0 = *(const i32x4*)(ks + l32 * 128 + slot);
        const i32x4 a1 = *(const i32x4*)(ks + (32 + l32) * 128 + slot);
        s[0] = mfma_i8_32x32x32(a0, qop[c], s[0]);
        s[1] = mfma_i8_32x32x32(a1, qop[c], s[1]);
    }
}

// Row max of an S^T tile (the lane pair holds a query's 64 keys). In the
// ragged last key block the rows past N hold copies of row N-1, a key of the
// same block, so the max over all 64 columns is the max over the valid ones.
__device__ __forceinline__ int tile_rowmax(const i32x16 (&s)[2]) {
    int smax = max(s[0][0], s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) smax = max(smax, max(s[0][r], s[1][r]));
    return max(smax, __shfl_xor(smax, 32, 64));
}

// Adds the two rounded p of a packed bf16 pair to a running sum (one v_dot2
// with ones: fewer VALU cycles than widening both halves and adding).
__device__ __forceinline__ void add_pair(bf16x2 pr, float& acc) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, acc, false);
}

// One slice of the softmax of a tile: keys 2p and 2p+1 of this lane's 32
// (convert, scale, exp2, round the pair to bf16, add the pair to the sum),
// written into the PV B operand (chunk cc holds keys 16cc + 8*(s/4) + 4*hi
// + s%4).
__device__ __forceinline__ void softmax_slice(int p, const i32x16 (&s)[2], float c, float nm,
                                              bf16x8 (&pn)[4], float& acc) {
    const int cc = p >> 2, e = 2 * (p & 3), r = 8 * (cc & 1) + e;
    const int sa = s[cc >> 1][r], sb = s[cc >> 1][r + 1];
    const float pa = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sa, c, nm));
    const float pz = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sb, c, nm));
    const bf16x2 pr = __builtin_convertvector(f32x2{pa, pz}, bf16x2);
    add_pair(pr, acc);
    pn[cc][e] = pr[0];
    pn[cc][e + 1] = pr[1];
}

// p = bf16(2^(S*c + nm)) of a whole tile; returns the sum of the rounded p.
__device__ __forceinline__ float tile_p(const i32x16 (&s)[2], float c, float nm, bf16x8 (&pb)[4]) {
    float acc = 0.f;
#pragma unroll
    for (int p = 0; p < 16; ++p) softmax_slice(p, s, c, nm, pb, acc);
    return acc;
}

// Ragged last key block: zero p of the keys >= kval and return the new sum.
__device__ __forceinline__ float mask_p(int kval, int hi, bf16x8 (&pb)[4]) {
    float acc = 0.f;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
        for (int s = 0; s < 8; s += 2) {
            const int key = 16 * cc + 8 * (s >> 2) + 4 * hi + (s & 3);
            if (key >= kval) pb[cc][s] = (__bf16)0.0f;
            if (key + 1 >= kval) pb[cc][s + 1] = (__bf16)0.0f;
            add_pair(bf16x2{pb[cc][s], pb[cc][s + 1]}, acc);
        }
    }
    return acc;
}

// Softmax of a tile, in two parts. The fast part (softmax_slice / tile_p)
// computes P with the current normalizer and its sum. The tile's row max is
// not needed there: if some query's max exceeds the normalizer by more than
// HEADROOM, one of its p is >= 2^HEADROOM, so the lane holding it sees a sum
// above 2^(HEADROOM-1) (the first tile, with m = -inf, always does). Only then
// does the rare part compute the exact max, rescale O and l by exact powers of
// two where it is exceeded and recompute P. The rare part also zeroes the keys
// past N of the ragged last key block (kval < 64).
constexpr float RESCALE_TRIGGER = 0x1p63f;  // 2^(HEADROOM - 1)

__device__ __forceinline__ void softmax_rare(bool trig, const i32x16 (&s)[2], float c, int kval,
                                             int hi, float& m_run, float& l_run, f32x16 (&o)[4],
                                             bf16x8 (&pb)[4], float& lsum) {
    if (__builtin_amdgcn_ballot_w64(trig)) {
        const float mt = ceilf((float)tile_rowmax(s) * c);  // c > 0
        const bool need = mt > m_run + HEADROOM;
        const float alpha =
            need ? ((m_run == -INFINITY) ? 0.f : __builtin_amdgcn_ldexpf(1.0f, (int)(m_run - mt)))
                 : 1.0f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
        l_run *= alpha;
        m_run = need ? mt : m_run;
        lsum = tile_p(s, c, -m_run, pb);
    }
    if (kval < KBLK) lsum = mask_p(kval, hi, pb);
    l_run += lsum;
}

// O^T += V^T . P^T for one tile.
__device__ __forceinline__ void tile_pv(const uint8_t* vs, const bf16x8 (&pb)[4], int l32, int hi,
                                        f32x16 (&o)[4]) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const bf16x8 va =
                *(const bf16x8*)(vs + (32 * dt + l32) * 128 + ((2 * cc + hi) ^ swz(l32)) * 16);
            o[dt] = mfma_bf16_32x32x16(va, pb[cc], o[dt]);
        }
}

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// One step of the three-tile pipeline, written in issue order with
// scheduling fences between the pieces. For kept blocks j, j+1, j+2:
//   PV(j)   16 bf16 MFMAs with P(j) (pb) and the LDS V^T tile vs;
//   QK(j+2)  8 int8 MFMAs against the LDS K tile ks, into sn (only with QK);
//   softmax(j+1) of sc, already in registers, into pn: 16 slices of 2 keys.
// The MFMAs run as QK, PV, PV, QK, PV, PV, ... so the VALU slices (one after
// each PV) sit beside every kind of MFMA, and each LDS fragment is read three
// MFMAs before its use. The softmax of a tile never waits for its own QK.
template <bool QK>
__device__ __forceinline__ void pipeline_step(const uint8_t* ks, const uint8_t* vs,
                                              const i32x4 (&qop)[4], int l32, int hi,
                                              const bf16x8 (&pb)[4], f32x16 (&o)[4],
                                              const i32x16 (&sc)[2], float c, float nm,
                                              i32x16 (&sn)[2], bf16x8 (&pn)[4], float& lsum) {
    constexpr int NT = QK ? 24 : 16;  // MFMAs in the step
    constexpr int AHEAD = 3;          // fragment read distance, in MFMAs
    const int sl = swz(l32);
    // MFMA t: with QK, t = 3g is QK(g) (K fragment g = 2*c4 + h), t = 3g+1,
    // 3g+2 are PV(2g), PV(2g+1); without, t is PV(t). PV i uses the V^T
    // fragment i = 4*cc + dt.
    auto is_qk = [](int t) { return QK && (t % 3 == 0); };
    auto pv_of = [](int t) { return QK ? 2 * (t / 3) + (t % 3) - 1 : t; };
    i32x4 ka[8];
    bf16x8 va[16];
    auto fetch = [&](int t) {
        if (is_qk(t)) {
            const int g = t / 3, c4 = g >> 1, h = g & 1;
            ka[g] = *(const i32x4*)(ks + (32 * h + l32) * 128 + ((2 * c4 + hi) ^ sl) * 16);
        } else {
            const int i = pv_of(t), cc = i >> 2, dt = i & 3;
            va[i] = *(const bf16x8*)(vs + (32 * dt + l32) * 128 + ((2 * cc + hi) ^ sl) * 16);
        }
    };
#pragma unroll
    for (int t = 0; t < AHEAD; ++t) fetch(t);
    fence();
    if (QK) sn[0] = sn[1] = i32x16{};
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t + AHEAD < NT) fetch(t + AHEAD);
        if (is_qk(t)) {
            const int g = t / 3, c4 = g >> 1, h = g & 1;
            sn[h] = mfma_i8_32x32x32(ka[g], qop[c4], sn[h]);
        } else {
            const int i = pv_of(t);
            o[i & 3] = mfma_bf16_32x32x16(va[i], pb[i >> 2], o[i & 3]);
            softmax_slice(i, sc, c, nm, pn, acc);
        }
        fence();
    }
    lsum = acc;
}

// Complement state staged in LDS for the linear epilogue: row r (0..127: h^T
// row e; 128: z) of 128 floats, 16-byte unit u at unit u ^ (r & 31). The h^T
// rows are then split in place: each unit holds its four values as bf16 high
// parts followed by the bf16 rests.
constexpr int HSTAGE_DMAS = (HD + 2) / 2;                   // 1 KB DMAs: rows 0..129
constexpr int HSTAGE_BYTES = HSTAGE_DMAS * 1024;
__device__ __forceinline__ f32x4 hstage_read(const uint8_t* smem, int row, int pos) {
    const int unit = pos >> 2;
    return *(const f32x4*)(smem + row * 512 + ((unit ^ (row & 31)) * 16));
}

// One query block i of head bh. smem holds the K and V rings; after the main
// loop the same bytes hold the block's complement state for the linear
// epilogue.
constexpr int ATTN_LDS = NSTAGE * (KTILE + VTILE);
static_assert(ATTN_LDS >= HSTAGE_BYTES, "state staging fits the rings");

// MODE: ATTN_SPARSE (sparse branch only), ATTN_LINEAR (plus the linear
// epilogue), ATTN_STATS (the backward's row statistics: instead of the
// output, the normalizer m + log2(l) and D = dO . o_s of every query row).
enum { ATTN_SPARSE = 0, ATTN_LINEAR = 1, ATTN_STATS = 2 };

template <int MODE>
__device__ __forceinline__ void attn_block(const AttnArgs& a, uint8_t* smem, int64_t bh, int i) {
    constexpr bool LIN = MODE == ATTN_LINEAR;
    uint8_t(*ks)[KTILE] = reinterpret_cast<uint8_t(*)[KTILE]>(smem);
    uint8_t(*vs)[VTILE] = reinterpret_cast<uint8_t(*)[VTILE]>(smem + NSTAGE * KTILE);
    const int N = a.N, nkb = a.nkb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31,
              hi = lane >> 5;
    const int tq = i * QBLK + 32 * wave + l32;  // this lane's query token

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    if (a.do_sparse) {
        const float sq = a.q_scale[bh * a.nqb + i];
        const float* ksc = a.k_scale + bh * nkb;
        const int nsel = a.kidx ? a.keep : nkb;
        const int32_t* krow = a.kidx ? a.kidx + (bh * a.nqb + i) * (int64_t)a.keep : nullptr;
        const uint16_t* vtb = a.vt + bh * (int64_t)nkb * HD * KBLK;
        // kept block indices are clamped into [0, nkb): a malformed kidx can
        // give wrong values but never an access outside K or V
        auto blk = [&](int jj) { return krow ? min(max(krow[jj], 0), nkb - 1) : jj; };
        auto kval_of = [&](int j) { return min(KBLK, N - j * KBLK); };
        uint32_t koff[8 / WAVES], krag[8 / WAVES], voff[16 / WAVES];
        const int nlast = N - (nkb - 1) * KBLK;  // valid keys of the last key block
#pragma unroll
        for (int p = 0; p < 8 / WAVES; ++p) {
            koff[p] = tile_voff(64 / WAVES, wave, p, lane);
            krag[p] = tile_voff_ragged(wave, p, lane, nlast);
        }
#pragma unroll
        for (int p = 0; p < 16 / WAVES; ++p) voff[p] = tile_voff(128 / WAVES, wave, p, lane);
        auto kdma = [&](int j, int stage) {
            dma_k_tile(a.k_i8, bh, N, j, lds_u32(ks[stage]), wave, koff, krag);
        };
        auto vdma = [&](int j, int stage) {
            dma_v_tile(vtb + (int64_t)j * HD * KBLK, lds_u32(vs[stage]), wave, voff);
        };
        constexpr int KD = 8 / WAVES, VD = 16 / WAVES;  // DMAs per wave per tile

        // Prologue: K(0), V(0), K(1), K(2) resident; P(0) and S(1) in
        // registers; V(1) and K(3) in flight. jn1..jn4 hold kept blocks 1..4,
        // ksc1 the k_scale of block 1.
        const int j0 = blk(0);
        int jn1 = nsel > 1 ? blk(1) : 0, jn2 = nsel > 2 ? blk(2) : 0, jn3 = nsel > 3 ? blk(3) : 0,
            jn4 = nsel > 4 ? blk(4) : 0;
        float ksc1 = ksc[jn1];
        kdma(j0, 0);
        vdma(j0, 0);
        if (nsel > 1) kdma(jn1, 1);
        if (nsel > 2) kdma(jn2, 2);
        i32x4 qop[4];
        load_q_operand(a.q_i8, bh, N, tq, hi, qop);
        const float c0 = (sq * ksc[j0]) * a.K32;
        wait_vm<0>();
        __syncthreads();
        if (nsel > 1) vdma(jn1, 1);

        bf16x8 pb[4];
        i32x16 sc[2];
        {
            i32x16 s0[2];
            qk_tile_mfma(ks[0], qop, l32, hi, s0);
            float lsum = tile_p(s0, c0, -m_run, pb);
            softmax_rare(!(lsum <= RESCALE_TRIGGER), s0, c0, kval_of(j0), hi, m_run, l_run, o, pb,
                         lsum);
        }
        if (nsel > 1) qk_tile_mfma(ks[1], qop, l32, hi, sc);
        // K(3) refills stage 0: every wave must be done reading K(0) and K(1)
        // first (step 0 refills stage 1). Later steps reuse a stage only after
        // the barrier that ends the step which read it.
        __syncthreads();
        if (nsel > 3) kdma(jn3, 0);

        // Full step jj (ring stage R = jj % NSTAGE, a compile-time constant so
        // every LDS address is an immediate offset), for jj + 2 < nsel:
        // resident K(jj+2), V(jj); in flight K(jj+3), V(jj+1); registers
        // P(jj) (pb) and S(jj+1) (sc). Issues K(jj+4), V(jj+2).
        auto step = [&](int jj, auto stage) {
            constexpr int R = decltype(stage)::value;
            const bool k4 = jj + 4 < nsel;
            if (k4) kdma(jn4, (R + 1) % NSTAGE);
            vdma(jn2, (R + 2) % NSTAGE);
            const float c = (sq * ksc1) * a.K32;  // of tile jj+1
            i32x16 sn[2];
            bf16x8 pn[4];
            float lsum;
            pipeline_step<true>(ks[(R + 2) % NSTAGE], vs[R], qop, l32, hi, pb, o, sc, c, -m_run,
                                sn, pn, lsum);
            const bool trig = !(lsum <= RESCALE_TRIGGER);
            // keep the common-case P in this block, above the rare branch
            asm volatile("" ::"v"(pn[0]), "v"(pn[1]), "v"(pn[2]), "v"(pn[3]), "v"(lsum));
            softmax_rare(trig, sc, c, kval_of(jn1), hi, m_run, l_run, o, pn, lsum);
            // next kept block (jj+5) and the scale of jn2 via the scalar cache
            int nxt = 0, kscb = 0;
            const int32_t* kp = krow ? krow + min(jj + 5, nsel - 1) : (const int32_t*)ksc;
            sload2(kp, ksc + jn2, nxt, kscb);
            // K(jj+3) and V(jj+1) must land; this step's DMAs may stay in flight
            if (k4)
                wait_vm<KD + VD>();
            else
                wait_vm<VD>();
            __syncthreads();
            jn1 = jn2;
            jn2 = jn3;
            jn3 = jn4;
            jn4 = krow ? min(max(nxt, 0), nkb - 1) : min(jj + 5, nkb - 1);
            ksc1 = __int_as_float(kscb);
#pragma unroll
            for (int h = 0; h < 2; ++h) sc[h] = sn[h];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) pb[cc] = pn[cc];
        };
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        using S2 = std::integral_constant<int, 2>;
        static_assert(NSTAGE == 3, "the step loop is unrolled by the ring depth");
        const int full = nsel - 2;  // full steps: jj = 0 .. nsel-3
        int jj = 0;
        for (; jj + 3 <= full; jj += 3) {
            step(jj, S0{});
            step(jj + 1, S1{});
            step(jj + 2, S2{});
        }
        if (jj < full) step(jj++, S0{});
        if (jj < full) step(jj++, S1{});
        // Last two tiles: PV(nsel-2) with the softmax of tile nsel-1, then
        // PV(nsel-1).
        if (nsel > 1) {
            const float c = (sq * ksc1) * a.K32;
            i32x16 sn[2];
            bf16x8 pn[4];
            float lsum;
            pipeline_step<false>(nullptr, vs[(nsel - 2) % NSTAGE], qop, l32, hi, pb, o, sc, c,
                                 -m_run, sn, pn, lsum);
            softmax_rare(!(lsum <= RESCALE_TRIGGER), sc, c, kval_of(jn1), hi, m_run, l_run, o, pn,
                         lsum);
            wait_vm<0>();
            __syncthreads();
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) pb[cc] = pn[cc];
        }
        tile_pv(vs[(nsel - 1) % NSTAGE], pb, l32, hi, o);
    }

    const float lt = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = a.do_sparse ? 1.0f / lt : 0.f;
    // the row's m + log2(l) for a backward pass (the statistics mode writes the
    // same expression)
    if (MODE != ATTN_STATS && a.lse && a.do_sparse && tq < N && hi == 0)
        a.lse[bh * N + tq] = m_run + __log2f(lt);
    if (MODE == ATTN_STATS) {
        // P of the backward is 2^(S*c - (m + log2 l)); D = dO . (o / l), the
        // lane pair holding the query's 128 channels
        float dsum = 0.f;
        const bool ok = tq < N;
        const uint16_t* grow = a.dout + (bh * N + (ok ? tq : 0)) * HD;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const u16x4 g4 = ok ? *(const u16x4*)(grow + 32 * dt + 8 * q4 + 4 * hi) : u16x4{};
#pragma unroll
                for (int u = 0; u < 4; ++u) dsum = __builtin_fmaf(bf2f(g4[u]), o[dt][4 * q4 + u] * inv, dsum);
            }
        dsum += __shfl_xor(dsum, 32, 64);
        if (ok && hi == 0) {
            a.mlog[bh * N + tq] = m_run + __log2f(lt);
            a.dstat[bh * N + tq] = dsum;
        }
        return;
    }
    if (LIN) {
        // Stage Hnon_i (128 rows of h^T, then z: 129 rows of 512 bytes) in LDS
        // with one batch of DMAs. The 16-byte unit u of row r sits at unit
        // u ^ (r & 31), so the 16 rows a 16-lane group reads land in distinct
        // banks. DMA p fills rows 2p, 2p+1; the last one's second half
        // re-fetches the z row into the spare bytes past the state.
        __syncthreads();  // every wave is done with the rings
        const float* hp = a.hnon + (bh * a.nqb + i) * (int64_t)HS_ROW;
        for (int p = wave; p < HSTAGE_DMAS; p += WAVES) {
            const int row = min(2 * p + (lane >> 5), HD);
            const uint32_t goff = row * 512 + ((lane & 31) ^ (row & 31)) * 16;
            dma16(hp, goff, __builtin_amdgcn_readfirstlane(lds_u32(smem) + 1024 * p));
        }
        wait_vm<0>();
        __syncthreads();
        // split the h^T rows once for all waves: each 16-byte unit of four fp32
        // becomes their bf16 high parts, then the bf16 rests (the z row stays)
        for (int u = tid; u < HD * 32; u += ATTN_THREADS) {
            const f32x4 x = *(const f32x4*)(smem + u * 16);
            __bf16 h[4], l[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) split_bf16(x[e], h[e], l[e]);
            *(bf16x8*)(smem + u * 16) = bf16x8{h[0], h[1], h[2], h[3], l[0], l[1], l[2], l[3]};
        }
        __syncthreads();
    }

    const int t = tq;
    f32x16 ol[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) ol[dt] = f32x16{};
    float linv = 0.f;
    if (LIN) {
        const bool ok = t < N;
        const uint16_t* qr = a.q + (bh * N + (ok ? t : 0)) * HD;
        float den = 0.f;
#pragma unroll 2
        for (int cd = 0; cd < 8; ++cd) {
            // k-slots of this lane: d = 16cd + 8(s/4) + 4hi + s%4, stored at
            // positions d0 .. d0+7 of the state rows
            const int d0 = 16 * cd + 8 * hi;
            const u16x4 q0 = ok ? *(const u16x4*)(qr + 16 * cd + 4 * hi) : u16x4{};
            const u16x4 q1 = ok ? *(const u16x4*)(qr + 16 * cd + 8 + 4 * hi) : u16x4{};
            const u16x8 qv = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
            const f32x4 z0 = hstage_read(smem, HD, d0);
            const f32x4 z1 = hstage_read(smem, HD, d0 + 4);
            bf16x8 bqh, bql;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = bf2f(qv[e]);
                const float ex = __expf(fminf(f, 0.f));  // selected for f <= 0 only: no branch
                const float ph = f > 0.f ? f + 1.f : ex;
                __bf16 x, y;
                split_bf16(ph, x, y);
                bqh[e] = x;
                bql[e] = y;
                den = __builtin_fmaf(ph, e < 4 ? z0[e] : z1[e - 4], den);
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                // two split units: high parts in dwords 0-1, rests in 2-3
                const u32x4 w0 = __builtin_bit_cast(u32x4, hstage_read(smem, 32 * dt + l32, d0));
                const u32x4 w1 = __builtin_bit_cast(u32x4, hstage_read(smem, 32 * dt + l32, d0 + 4));
                const bf16x8 ah = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
                const bf16x8 al = __builtin_bit_cast(bf16x8, u32x4{w0[2], w0[3], w1[2], w1[3]});
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
            for (int q4 = 0; q4 < 4; ++q4) {
                const int dv = 32 * dt + 8 * q4 + 4 * hi;
                float r4[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float val = o[dt][4 * q4 + u] * inv;
                    if (LIN) val += ol[dt][4 * q4 + u] * linv;
                    r4[u] = val;
                }
                *(u16x4*)(orow + dv) = u16x4{f2bf(r4[0]), f2bf(r4[1]), f2bf(r4[2]), f2bf(r4[3])};
                if (orow32) *(f32x4*)(orow32 + dv) = f32x4{r4[0], r4[1], r4[2], r4[3]};
            }
    }
}

template <int MODE>
__global__ __launch_bounds__(ATTN_THREADS, 2) void sagesla_attn_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[ATTN_LDS];
    const int64_t item = blockIdx.x;
    if (item >= a.BH * a.nqb) return;
    attn_block<MODE>(a, smem, item / a.nqb, (int)(item % a.nqb));
}

// Raw int32 tiles through the same LDS staging and qk_tile_mfma routine as
// the attention kernel (4 waves x 32 query rows).
__global__ __launch_bounds__(ATTN_THREADS) void qk_tiles_kernel(const int8_t* __restrict__ q_i8,
                                                                const int8_t* __restrict__ k_i8,
                                                                int64_t BH, int N,
                                                                const int32_t* __restrict__ tiles,
                                                                int32_t* __restrict__ out) {
    __shared__ __attribute__((aligned(1024))) uint8_t ks[KTILE];
    const int64_t tix = blockIdx.x;
    const int nqb = (N + QBLK - 1) / QBLK, nkb = (N + KBLK - 1) / KBLK;
    const int64_t bh = tiles[3 * tix];
    const int i = tiles[3 * tix + 1], j = tiles[3 * tix + 2];
    const bool valid = bh >= 0 && bh < BH && i >= 0 && i < nqb && j >= 0 && j < nkb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31,
              hi = lane >> 5;
    int32_t* ot = out + tix * QBLK * KBLK;
    if (!valid) {
        for (int x = tid; x < QBLK * KBLK; x += ATTN_THREADS) ot[x] = 0;
        return;
    }
    uint32_t koff[8 / WAVES], krag[8 / WAVES];
#pragma unroll
    for (int p = 0; p < 8 / WAVES; ++p) {
        koff[p] = tile_voff(64 / WAVES, wave, p, lane);
        krag[p] = tile_voff_ragged(wave, p, lane, min(KBLK, N - j * KBLK));
    }
    dma_k_tile(k_i8, bh, N, j, lds_u32(ks), wave, koff, krag);
    wait_vm<0>();
    __syncthreads();
    i32x4 qop[4];
    load_q_operand(q_i8, bh, N, i * QBLK + 32 * wave + l32, hi, qop);
    i32x16 s[2];
    qk_tile_mfma(ks, qop, l32, hi, s);
    const int kval = min(KBLK, N - j * KBLK);
    const int row = 32 * wave + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int key = mfma32_row(lane, r);
        // keys past N were staged from row N-1; the export reports them as 0
        ot[row * KBLK + key] = key < kval ? s[0][r] : 0;
        ot[row * KBLK + key + 32] = key + 32 < kval ? s[1][r] : 0;
    }
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
    const int64_t total = a.BH * a.nqb;
    if (a.mlog)
        hipLaunchKernelGGL((sagesla_attn_kernel<ATTN_STATS>), dim3((unsigned)total),
                           dim3(ATTN_THREADS), 0, st, a);
    else if (a.hnon)
        hipLaunchKernelGGL((sagesla_attn_kernel<ATTN_LINEAR>), dim3((unsigned)total),
                           dim3(ATTN_THREADS), 0, st, a);
    else
        hipLaunchKernelGGL((sagesla_attn_kernel<ATTN_SPARSE>), dim3((unsigned)total),
                           dim3(ATTN_THREADS), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_qk_tiles(const int8_t* q_i8, const int8_t* k_i8, int64_t BH, int N,
                           const int32_t* tiles, int64_t T, int32_t* out, hipStream_t st) {
    hipLaunchKernelGGL(qk_tiles_kernel, dim3((unsigned)T), dim3(ATTN_THREADS), 0, st, q_i8, k_i8, BH,
                       N, tiles, out);
    return hipGetLastError();
}

}  // namespace ssa
