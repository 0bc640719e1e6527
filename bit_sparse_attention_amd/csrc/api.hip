// api.hip -- the C ABI (include/ssa.h): argument validation, workspace layout
// and kernel launches. Validation runs before any HIP call, so every argument
// error (shapes whose launch grids the device cannot take included) returns
// with nothing enqueued. A call that enqueues several kernels and then sees a
// launch fail returns SSA_ERR_HIP with the earlier launches still enqueued.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/ssa.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace ssa;

// Fixed device scratch of the allocation-free quantization call: the K-mean
// block partials (B*H*Nkb*128 fp32) that sage_quant_qk keeps in the caller's
// workspace. Every GPU the library runs on holds its own copy until the
// process ends. Host code never uses this name as an address: the per-device
// address comes from hipGetSymbolAddress (scratch_address below).
constexpr size_t SCRATCH_BYTES = (size_t)32 << 20;  // 32 MiB: B*H*Nkb <= 65536
static __device__ __align__(256) float scratch[SCRATCH_BYTES / sizeof(float)];

namespace {

thread_local char g_err[512] = "";

ssa_status fail(ssa_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

ssa_status hip_fail(hipError_t e, const char* what) {
    return fail(SSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Dims {
    int64_t BH, N, nqb, nkb, nkbp, ngroups;
};

// Largest launch grids, in workgroups: a dispatch covers fewer than 2^32
// work-items per dimension, and B*H rides on the grid's y dimension.
constexpr int64_t MAX_GRID_Y = 65535;
constexpr int64_t MAX_WG_256 = ((int64_t)1 << 24) - 1;  // 256-thread workgroups in x

ssa_status check_shape(const ssa_shape& s, Dims* d) {
    if (s.B < 1 || s.H < 1 || s.N < 1 || s.D < 1)
        return fail(SSA_ERR_INVALID, "shape must be positive (B=%lld H=%lld N=%lld D=%lld)",
                    (long long)s.B, (long long)s.H, (long long)s.N, (long long)s.D);
    if (s.D != SSA_HEAD_DIM) return fail(SSA_ERR_UNSUPPORTED, "head dim %lld != 128", (long long)s.D);
    if (s.N > SSA_MAX_N)
        return fail(SSA_ERR_UNSUPPORTED, "N=%lld exceeds %d", (long long)s.N, SSA_MAX_N);
    if (s.B > MAX_GRID_Y || s.H > MAX_GRID_Y || s.B * s.H > MAX_GRID_Y)
        return fail(SSA_ERR_UNSUPPORTED, "B*H=%lld exceeds %lld", (long long)(s.B * s.H),
                    (long long)MAX_GRID_Y);
    d->BH = s.B * s.H;
    d->N = s.N;
    d->nqb = (s.N + QBLK - 1) / QBLK;
    d->nkb = (s.N + KBLK - 1) / KBLK;
    d->nkbp = (d->nkb + GEMM_KALIGN - 1) / GEMM_KALIGN * GEMM_KALIGN;
    d->ngroups = (d->nkb + LIN_GROUP - 1) / LIN_GROUP;
    // the attention grid (one workgroup per head and query block) and the
    // complement GEMM grid (every 64-entry state tile of every 640 query
    // blocks of every head)
    if (d->BH * d->nqb > MAX_WG_256)
        return fail(SSA_ERR_UNSUPPORTED, "B*H*Nqb=%lld exceeds %lld (attention grid)",
                    (long long)(d->BH * d->nqb), (long long)MAX_WG_256);
    if (d->BH * complement_tiles_per_head(d->nqb) > MAX_WG_256)
        return fail(SSA_ERR_UNSUPPORTED, "B*H=%lld too large for N=%lld (linear-branch grid)",
                    (long long)d->BH, (long long)s.N);
    return SSA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

ssa_status need_ptr(const void* p, size_t align, const char* name) {
    if (!p) return fail(SSA_ERR_INVALID, "%s is NULL", name);
    if (!aligned(p, align)) return fail(SSA_ERR_INVALID, "%s is not %zu-byte aligned", name, align);
    return SSA_OK;
}

struct Range {
    const void* p;
    size_t n;
    const char* name;
};

bool overlap(const Range& a, const Range& b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// every output against every input and every other output
ssa_status check_alias(const Range* outs, int no, const Range* ins, int ni) {
    for (int x = 0; x < no; ++x) {
        for (int y = 0; y < ni; ++y)
            if (overlap(outs[x], ins[y]))
                return fail(SSA_ERR_INVALID, "output %s overlaps input %s", outs[x].name, ins[y].name);
        for (int y = x + 1; y < no; ++y)
            if (overlap(outs[x], outs[y]))
                return fail(SSA_ERR_INVALID, "output %s overlaps output %s", outs[x].name,
                            outs[y].name);
    }
    return SSA_OK;
}

// gfx950 check, once per device
std::atomic<int> g_dev_ok[64];

ssa_status check_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(SSA_ERR_UNSUPPORTED, "device index %d", dev);
    int st = g_dev_ok[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
        st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_dev_ok[dev].store(st, std::memory_order_release);
    }
    if (st != 1) return fail(SSA_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    return SSA_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
std::mutex g_scratch_mu;
void* g_scratch_addr[64];

ssa_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(SSA_ERR_UNSUPPORTED, "device index %d", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(SSA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return SSA_OK;
}

// workspace layouts ----------------------------------------------------------

size_t ws_quant(const Dims& d) { return align256((size_t)d.BH * d.nkb * HD * 4); }

struct MaskWs {
    size_t qbar, kbarT, total;
    int64_t ldk;
};
MaskWs ws_mask(const Dims& d) {
    MaskWs w;
    w.ldk = (d.nkb + 15) / 16 * 16;
    w.qbar = 0;
    w.kbarT = align256((size_t)d.BH * d.nqb * HD * 4);
    w.total = w.kbarT + align256((size_t)d.BH * HD * w.ldk * 4);
    return w;
}

struct AttnWs {
    size_t vt, hs, hs_lo, hpart, htot, msel, hnon, total;
    bool lo;
};
// lo: also the states' bf16 rests (the backward's complement states)
AttnWs ws_attn(const Dims& d, bool linear, bool lo = false) {
    AttnWs w{};
    w.lo = linear && lo;
    size_t off = 0;
    w.vt = off;
    off += align256((size_t)d.BH * d.nkb * HD * KBLK * 2);
    if (linear) {
        w.hs = off;
        off += align256((size_t)d.BH * d.nkb * HS_ROW * 2);
        if (w.lo) {
            w.hs_lo = off;
            off += align256((size_t)d.BH * d.nkb * HS_ROW * 2);
        }
        w.hpart = off;
        off += align256((size_t)d.BH * d.ngroups * HS_ROW * 4);
        w.htot = off;
        off += align256((size_t)d.BH * HS_ROW * 4);
        w.msel = off;
        off += align256(msel_bytes(d.BH, d.nqb, d.nkbp));
        w.hnon = off;
        off += align256((size_t)d.BH * d.nqb * HS_ROW * 4);
    }
    w.total = off;
    return w;
}

// the whole step: the attention's workspace, then the pooled means, then the
// K-mean block partials
struct StepWs {
    AttnWs attn;
    size_t pool, part, total;
};
StepWs ws_step(const Dims& d, bool linear) {
    StepWs w;
    w.attn = ws_attn(d, linear);
    w.pool = w.attn.total;
    w.part = w.pool + ws_mask(d).total;
    w.total = w.part + ws_quant(d);
    return w;
}

// the backward: the forward attention's workspace (V layout, and the linear
// branch's complement states), the row statistics, the inverse selection
// lists and the linear branch's gradient states
struct BwdWs {
    AttnWs attn;
    size_t mlog, dstat, dol, counts, lists, bits, gf, gs, gs_lo, gtot, msel, gc, total;
};
BwdWs ws_bwd(const Dims& d, bool sel, bool linear) {
    BwdWs w{};
    w.attn = ws_attn(d, linear, true);
    size_t off = w.attn.total;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    w.mlog = take((size_t)d.BH * d.N * 4);
    w.dstat = take((size_t)d.BH * d.N * 4);
    w.dol = linear ? take((size_t)d.BH * d.N * 4) : 0;
    if (sel) {
        w.counts = take((size_t)d.BH * d.nkb * 4);
        w.lists = take((size_t)d.BH * d.nkb * d.nqb * 2);
        w.bits = take(keep_bits_bytes(d.BH, d.nqb, d.nkb));
    }
    if (linear) {
        const int64_t nqbp = (d.nqb + GEMM_KALIGN - 1) / GEMM_KALIGN * GEMM_KALIGN;
        w.gf = take((size_t)d.BH * d.nqb * HS_ROW * 4);
        w.gs = take((size_t)d.BH * d.nqb * HS_ROW * 2);
        w.gs_lo = take((size_t)d.BH * d.nqb * HS_ROW * 2);
        w.gtot = take((size_t)d.BH * HS_ROW * 4);
        w.msel = take(msel_bytes(d.BH, d.nkb, nqbp));
        w.gc = take((size_t)d.BH * d.nkb * HS_ROW * 4);
    }
    w.total = off;
    return w;
}

ssa_status check_ws(void* ws, size_t have, size_t need) {
    if (need == 0) return SSA_OK;
    if (!ws) return fail(SSA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned(ws, 256)) return fail(SSA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (have < need) return fail(SSA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
    return SSA_OK;
}

// kernel timer (benchmark hook): event pairs around the sparse-attention launch
std::mutex g_tm;
std::vector<hipEvent_t> g_ev0, g_ev1;
int g_tcount = 0;

void timer_destroy_locked() {
    for (auto e : g_ev0) (void)hipEventDestroy(e);
    for (auto e : g_ev1) (void)hipEventDestroy(e);
    g_ev0.clear();
    g_ev1.clear();
    g_tcount = 0;
}

// index of the event pair for the next launch, or -1 when the timer is off/full
int timer_slot() {
    std::lock_guard<std::mutex> lk(g_tm);
    if (g_tcount >= (int)g_ev0.size()) return -1;
    return g_tcount++;
}

#define TRY(x)                          \
    do {                                \
        ssa_status _st = (x);           \
        if (_st != SSA_OK) return _st;  \
    } while (0)

// The attention call's launches after validation, shared by the staged and
// the one-call step. kpart non-null: the V-layout pass also writes the K-mean
// block partials (and, with kbarT, the pooled key means).
hipError_t enqueue_states(const Dims& d, bool linear, const uint16_t* k, const uint16_t* v,
                          char* base, const AttnWs& w, float* kpart, float* kbarT, int ldk,
                          hipStream_t st) {
    uint16_t* vt = (uint16_t*)(base + w.vt);
    if (linear)
        return launch_linear_states(k, v, d.BH, (int)d.N, vt, (uint16_t*)(base + w.hs),
                                    w.lo ? (uint16_t*)(base + w.hs_lo) : nullptr,
                                    (float*)(base + w.hpart), (float*)(base + w.htot), kpart,
                                    kbarT, ldk, st);
    return launch_vt_only(k, v, d.BH, (int)d.N, vt, kpart, kbarT, ldk, st);
}

hipError_t enqueue_complement(const Dims& d, const int32_t* kidx, int64_t keep, char* base,
                              const AttnWs& w, hipStream_t st) {
    return launch_complement(kidx, (int)keep, (const uint16_t*)(base + w.hs),
                             w.lo ? (const uint16_t*)(base + w.hs_lo) : nullptr,
                             (const float*)(base + w.htot), d.BH, (int)d.N,
                             (uint32_t*)(base + w.msel), (float*)(base + w.hnon), st);
}

hipError_t enqueue_attn(const Dims& d, bool sparse, bool linear, const uint16_t* q,
                        const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                        const float* k_scale, const int32_t* kidx, int64_t keep, float sm_scale,
                        uint16_t* out, float* out_f32, float* lse, char* base,
                        const AttnWs& w, hipStream_t st) {
    const float sm = sm_scale > 0.f ? sm_scale : (float)(1.0 / std::sqrt((double)HD));
    AttnArgs a;
    a.q_i8 = q_i8;
    a.q_scale = q_scale;
    a.k_i8 = k_i8;
    a.k_scale = k_scale;
    a.vt = (const uint16_t*)(base + w.vt);
    a.kidx = kidx;
    a.keep = (int)keep;
    a.N = (int)d.N;
    a.nqb = (int)d.nqb;
    a.nkb = (int)d.nkb;
    a.BH = d.BH;
    a.K32 = (float)((double)sm * 1.4426950408889634074);
    a.do_sparse = sparse ? 1 : 0;
    a.q = q;
    a.hnon = linear ? (const float*)(base + w.hnon) : nullptr;
    a.out = out;
    a.out32 = out_f32;
    a.dout = nullptr;
    a.mlog = nullptr;
    a.dstat = nullptr;
    a.lse = lse;
    const int slot = timer_slot();
    if (slot >= 0) (void)hipEventRecord(g_ev0[slot], st);
    const hipError_t e = launch_attn(a, st);
    if (slot >= 0) (void)hipEventRecord(g_ev1[slot], st);
    return e;
}

}  // namespace

extern "C" {

int64_t ssa_num_q_blocks(int64_t N) { return N < 1 ? 0 : (N + QBLK - 1) / QBLK; }
int64_t ssa_num_k_blocks(int64_t N) { return N < 1 ? 0 : (N + KBLK - 1) / KBLK; }

int64_t ssa_keep_blocks(int64_t N, double topk) {
    const int64_t nkb = ssa_num_k_blocks(N);
    if (nkb < 1) return 0;
    if (!(topk == topk)) return 1;  // NaN
    double x = std::floor(topk * (double)nkb + 0.5);
    if (x < 1.0) return 1;
    if (x > (double)nkb) return nkb;
    return (int64_t)x;
}

size_t ssa_pool_bytes(ssa_shape s) {
    Dims d;
    if (check_shape(s, &d) != SSA_OK) return 0;
    return ws_mask(d).total;
}

size_t ssa_workspace_bytes(int op, ssa_shape s, int64_t keep, int branches) {
    Dims d;
    if (check_shape(s, &d) != SSA_OK) return 0;
    switch (op) {
        case SSA_OP_QUANT: return ws_quant(d);
        case SSA_OP_MASK: return ws_mask(d).total;
        case SSA_OP_ATTN:
        case SSA_OP_STEP: {
            const bool linear = (branches & SSA_BRANCH_LINEAR) && keep >= 1 && keep < d.nkb;
            return op == SSA_OP_ATTN ? ws_attn(d, linear).total : ws_step(d, linear).total;
        }
        case SSA_OP_BWD: {
            const bool sel = keep >= 1 && keep < d.nkb;
            const bool linear = (branches & SSA_BRANCH_LINEAR) && sel;
            return ws_bwd(d, sel, linear).total;
        }
        default: return 0;
    }
}

const char* ssa_status_str(ssa_status st) {
    switch (st) {
        case SSA_OK: return "ok";
        case SSA_ERR_INVALID: return "invalid argument";
        case SSA_ERR_UNSUPPORTED: return "unsupported";
        case SSA_ERR_WORKSPACE: return "workspace too small";
        case SSA_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* ssa_last_error(void) { return g_err; }

ssa_status sage_quant_qk(const uint16_t* q, const uint16_t* k, ssa_shape s, int8_t* q_i8,
                         float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean, void* pool,
                         void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    Dims d;
    TRY(check_shape(s, &d));
    TRY(need_ptr(q, 16, "q"));
    TRY(need_ptr(k, 16, "k"));
    TRY(need_ptr(q_i8, 16, "q_i8"));
    TRY(need_ptr(k_i8, 16, "k_i8"));
    TRY(need_ptr(q_scale, 4, "q_scale"));
    TRY(need_ptr(k_scale, 4, "k_scale"));
    TRY(need_ptr(k_mean, 4, "k_mean"));
    const size_t nel = (size_t)d.BH * d.N * HD;
    const Range ins[] = {{q, nel * 2, "q"}, {k, nel * 2, "k"}};
    if (pool && !aligned(pool, 256)) return fail(SSA_ERR_INVALID, "pool is not 256-byte aligned");
    const MaskWs pw = ws_mask(d);  // the pool holds the block mask's pooled means
    const Range outs[] = {{q_i8, nel, "q_i8"},
                          {k_i8, nel, "k_i8"},
                          {q_scale, (size_t)d.BH * d.nqb * 4, "q_scale"},
                          {k_scale, (size_t)d.BH * d.nkb * 4, "k_scale"},
                          {k_mean, (size_t)d.BH * HD * 4, "k_mean"},
                          {pool, pool ? pw.total : 0, "pool"},
                          {ws, ws_bytes, "workspace"}};
    TRY(check_alias(outs, 7, ins, 2));
    TRY(check_ws(ws, ws_bytes, ws_quant(d)));
    TRY(check_device());
    float* qbar = pool ? (float*)((char*)pool + pw.qbar) : nullptr;
    float* kbarT = pool ? (float*)((char*)pool + pw.kbarT) : nullptr;
    hipError_t e = launch_quant_qk(q, k, d.BH, (int)d.N, q_i8, q_scale, k_i8, k_scale, k_mean,
                                   (float*)ws, qbar, kbarT, (int)pw.ldk, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "sage_quant_qk launch");
    return SSA_OK;
}

ssa_status sage_quant_qk_noalloc(const uint16_t* q, const uint16_t* k, ssa_shape s, int8_t* q_i8,
                                 float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                                 void* pool, void* stream) {
    g_err[0] = 0;
    Dims d;
    TRY(check_shape(s, &d));
    const size_t need = ws_quant(d);
    if (need > SCRATCH_BYTES)
        return fail(SSA_ERR_UNSUPPORTED,
                    "sage_quant_qk_noalloc: B*H*Nkb=%lld needs %zu bytes of scratch; the library "
                    "holds %zu (B*H*Nkb <= 65536); use sage_quant_qk with a workspace",
                    (long long)(d.BH * d.nkb), need, SCRATCH_BYTES);
    TRY(need_ptr(q, 16, "q"));
    TRY(need_ptr(k, 16, "k"));
    TRY(need_ptr(q_i8, 16, "q_i8"));
    TRY(need_ptr(k_i8, 16, "k_i8"));
    TRY(need_ptr(q_scale, 4, "q_scale"));
    TRY(need_ptr(k_scale, 4, "k_scale"));
    TRY(need_ptr(k_mean, 4, "k_mean"));
    const size_t nel = (size_t)d.BH * d.N * HD;
    const Range ins[] = {{q, nel * 2, "q"}, {k, nel * 2, "k"}};
    if (pool && !aligned(pool, 256)) return fail(SSA_ERR_INVALID, "pool is not 256-byte aligned");
    const MaskWs pw = ws_mask(d);
    const Range outs[] = {{q_i8, nel, "q_i8"},
                          {k_i8, nel, "k_i8"},
                          {q_scale, (size_t)d.BH * d.nqb * 4, "q_scale"},
                          {k_scale, (size_t)d.BH * d.nkb * 4, "k_scale"},
                          {k_mean, (size_t)d.BH * HD * 4, "k_mean"},
                          {pool, pool ? pw.total : 0, "pool"}};
    TRY(check_alias(outs, 6, ins, 2));
    TRY(check_device());
    void* part = nullptr;
    TRY(scratch_address(&part));
    float* qbar = pool ? (float*)((char*)pool + pw.qbar) : nullptr;
    float* kbarT = pool ? (float*)((char*)pool + pw.kbarT) : nullptr;
    // every block partial the mean reads is written first by the same call,
    // so the scratch needs no clearing
    hipError_t e = launch_quant_qk(q, k, d.BH, (int)d.N, q_i8, q_scale, k_i8, k_scale, k_mean,
                                   (float*)part, qbar, kbarT, (int)pw.ldk, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "sage_quant_qk_noalloc launch");
    return SSA_OK;
}

ssa_status sla_block_mask(const uint16_t* q, const uint16_t* k, ssa_shape s, int64_t keep,
                          const void* pool, int32_t* kidx, uint8_t* mask, void* ws, size_t ws_bytes,
                          void* stream) {
    g_err[0] = 0;
    Dims d;
    TRY(check_shape(s, &d));
    if (keep < 1 || keep > d.nkb)
        return fail(SSA_ERR_INVALID, "keep=%lld outside [1, %lld]", (long long)keep,
                    (long long)d.nkb);
    if (pool) {
        if (!aligned(pool, 256)) return fail(SSA_ERR_INVALID, "pool is not 256-byte aligned");
    } else {
        TRY(need_ptr(q, 16, "q"));
        TRY(need_ptr(k, 16, "k"));
    }
    TRY(need_ptr(kidx, 4, "kidx"));
    if (mask && !aligned(mask, 1)) return fail(SSA_ERR_INVALID, "mask misaligned");
    const size_t nel = (size_t)d.BH * d.N * HD;
    const MaskWs w = ws_mask(d);
    const Range ins[] = {{pool ? nullptr : q, nel * 2, "q"},
                         {pool ? nullptr : k, nel * 2, "k"},
                         {pool, pool ? w.total : 0, "pool"}};
    const Range outs[] = {{kidx, (size_t)d.BH * d.nqb * keep * 4, "kidx"},
                          {mask, mask ? (size_t)d.BH * d.nqb * d.nkb : 0, "mask"},
                          {pool ? nullptr : ws, ws_bytes, "workspace"}};
    TRY(check_alias(outs, 3, ins, 3));
    if (!pool) TRY(check_ws(ws, ws_bytes, w.total));
    TRY(check_device());
    const char* base = pool ? (const char*)pool : (const char*)ws;
    float* qbar = (float*)(base + w.qbar);
    float* kbarT = (float*)(base + w.kbarT);
    hipError_t e = hipSuccess;
    if (!pool)
        e = launch_pool(q, k, d.BH, (int)d.N, qbar, kbarT, (int)w.ldk, (hipStream_t)stream);
    if (e == hipSuccess)
        e = launch_score_topk(qbar, kbarT, (int)w.ldk, d.BH, (int)d.nqb, (int)d.nkb, (int)keep, kidx,
                              mask, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "sla_block_mask launch");
    return SSA_OK;
}

ssa_status sage_sla_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, ssa_shape s,
                             const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                             const float* k_scale, const int32_t* kidx, int64_t keep, int branches,
                             float sm_scale, uint16_t* out, float* out_f32, float* lse, void* ws,
                             size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    Dims d;
    TRY(check_shape(s, &d));
    if (branches < 1 || branches > 3)
        return fail(SSA_ERR_INVALID, "branches=%d must be SPARSE, LINEAR or both", branches);
    if (keep < 1 || keep > d.nkb)
        return fail(SSA_ERR_INVALID, "keep=%lld outside [1, %lld]", (long long)keep,
                    (long long)d.nkb);
    if (!kidx && keep != d.nkb)
        return fail(SSA_ERR_INVALID, "dense call (kidx NULL) needs keep == Nkb (%lld)",
                    (long long)d.nkb);
    if (!(sm_scale == sm_scale) || std::isinf(sm_scale))
        return fail(SSA_ERR_INVALID, "sm_scale is not finite");
    const bool sparse = branches & SSA_BRANCH_SPARSE;
    const bool linear = (branches & SSA_BRANCH_LINEAR) && kidx && keep < d.nkb;
    TRY(need_ptr(v, 16, "v"));
    TRY(need_ptr(q_i8, 16, "q_i8"));
    TRY(need_ptr(k_i8, 16, "k_i8"));
    TRY(need_ptr(q_scale, 4, "q_scale"));
    TRY(need_ptr(k_scale, 4, "k_scale"));
    TRY(need_ptr(out, 16, "out"));
    if (out_f32) TRY(need_ptr(out_f32, 16, "out_f32"));
    if (lse) TRY(need_ptr(lse, 4, "lse"));
    if (kidx) TRY(need_ptr(kidx, 4, "kidx"));
    if (linear) {
        TRY(need_ptr(q, 16, "q"));
        TRY(need_ptr(k, 16, "k"));
    }
    const size_t nel = (size_t)d.BH * d.N * HD;
    const Range ins[] = {{q, nel * 2, "q"},
                         {k, nel * 2, "k"},
                         {v, nel * 2, "v"},
                         {q_i8, nel, "q_i8"},
                         {k_i8, nel, "k_i8"},
                         {q_scale, (size_t)d.BH * d.nqb * 4, "q_scale"},
                         {k_scale, (size_t)d.BH * d.nkb * 4, "k_scale"},
                         {kidx, kidx ? (size_t)d.BH * d.nqb * keep * 4 : 0, "kidx"}};
    const Range outs[] = {{out, nel * 2, "out"},
                          {out_f32, out_f32 ? nel * 4 : 0, "out_f32"},
                          {lse, lse ? (size_t)d.BH * d.N * 4 : 0, "lse"},
                          {ws, ws_bytes, "workspace"}};
    TRY(check_alias(outs, 4, ins, 8));
    const AttnWs w = ws_attn(d, linear);
    TRY(check_ws(ws, ws_bytes, w.total));
    TRY(check_device());

    hipStream_t st = (hipStream_t)stream;
    hipError_t e = enqueue_states(d, linear, k, v, (char*)ws, w, nullptr, nullptr, 0, st);
    if (e == hipSuccess && linear) e = enqueue_complement(d, kidx, keep, (char*)ws, w, st);
    if (e != hipSuccess) return hip_fail(e, "sage_sla_attn_fwd launch (linear / V layout)");
    e = enqueue_attn(d, sparse, linear, q, q_i8, q_scale, k_i8, k_scale, kidx, keep, sm_scale,
                     out, out_f32, lse, (char*)ws, w, st);
    if (e != hipSuccess) return hip_fail(e, "sage_sla_attn_fwd launch");
    return SSA_OK;
}

ssa_status sage_sla_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, ssa_shape s,
                        int64_t keep, int branches, float sm_scale, int8_t* q_i8, float* q_scale,
                        int8_t* k_i8, float* k_scale, float* k_mean, int32_t* kidx,
                        uint8_t* mask, uint16_t* out, float* out_f32, float* lse, void* ws,
                        size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    Dims d;
    TRY(check_shape(s, &d));
    if (branches < 1 || branches > 3)
        return fail(SSA_ERR_INVALID, "branches=%d must be SPARSE, LINEAR or both", branches);
    if (keep < 1 || keep > d.nkb)
        return fail(SSA_ERR_INVALID, "keep=%lld outside [1, %lld]", (long long)keep,
                    (long long)d.nkb);
    if (!kidx && keep != d.nkb)
        return fail(SSA_ERR_INVALID, "dense call (kidx NULL) needs keep == Nkb (%lld)",
                    (long long)d.nkb);
    if (mask && !kidx) return fail(SSA_ERR_INVALID, "mask needs kidx (a dense call selects nothing)");
    if (!(sm_scale == sm_scale) || std::isinf(sm_scale))
        return fail(SSA_ERR_INVALID, "sm_scale is not finite");
    const bool sparse = branches & SSA_BRANCH_SPARSE;
    const bool linear = (branches & SSA_BRANCH_LINEAR) && kidx && keep < d.nkb;
    TRY(need_ptr(q, 16, "q"));
    TRY(need_ptr(k, 16, "k"));
    TRY(need_ptr(v, 16, "v"));
    TRY(need_ptr(q_i8, 16, "q_i8"));
    TRY(need_ptr(k_i8, 16, "k_i8"));
    TRY(need_ptr(q_scale, 4, "q_scale"));
    TRY(need_ptr(k_scale, 4, "k_scale"));
    TRY(need_ptr(k_mean, 4, "k_mean"));
    TRY(need_ptr(out, 16, "out"));
    if (out_f32) TRY(need_ptr(out_f32, 16, "out_f32"));
    if (lse) TRY(need_ptr(lse, 4, "lse"));
    if (kidx) TRY(need_ptr(kidx, 4, "kidx"));
    const size_t nel = (size_t)d.BH * d.N * HD;
    const Range ins[] = {{q, nel * 2, "q"}, {k, nel * 2, "k"}, {v, nel * 2, "v"}};
    const Range outs[] = {{q_i8, nel, "q_i8"},
                          {k_i8, nel, "k_i8"},
                          {q_scale, (size_t)d.BH * d.nqb * 4, "q_scale"},
                          {k_scale, (size_t)d.BH * d.nkb * 4, "k_scale"},
                          {k_mean, (size_t)d.BH * HD * 4, "k_mean"},
                          {kidx, kidx ? (size_t)d.BH * d.nqb * keep * 4 : 0, "kidx"},
                          {mask, mask ? (size_t)d.BH * d.nqb * d.nkb : 0, "mask"},
                          {out, nel * 2, "out"},
                          {out_f32, out_f32 ? nel * 4 : 0, "out_f32"},
                          {lse, lse ? (size_t)d.BH * d.N * 4 : 0, "lse"},
                          {ws, ws_bytes, "workspace"}};
    TRY(check_alias(outs, 11, ins, 3));
    const StepWs w = ws_step(d, linear);
    TRY(check_ws(ws, ws_bytes, w.total));
    TRY(check_device());

    hipStream_t st = (hipStream_t)stream;
    char* base = (char*)ws;
    const MaskWs pw = ws_mask(d);
    float* qbar = (float*)(base + w.pool + pw.qbar);
    float* kbarT = (float*)(base + w.pool + pw.kbarT);
    float* part = (float*)(base + w.part);
    // one pass over K and V: V layout (and linear states), K-mean partials and
    // pooled key means; then mean, quantization and pooled query means
    hipError_t e = enqueue_states(d, linear, k, v, base, w.attn, part, kidx ? kbarT : nullptr,
                                  (int)pw.ldk, st);
    if (e == hipSuccess)
        e = launch_quant_from_sums(q, k, d.BH, (int)d.N, q_i8, q_scale, k_i8, k_scale, k_mean,
                                   part, kidx ? qbar : nullptr, st);
    if (e == hipSuccess && kidx)
        e = launch_score_topk(qbar, kbarT, (int)pw.ldk, d.BH, (int)d.nqb, (int)d.nkb, (int)keep,
                              kidx, mask, st);
    if (e == hipSuccess && linear) e = enqueue_complement(d, kidx, keep, base, w.attn, st);
    if (e != hipSuccess) return hip_fail(e, "sage_sla_fwd launch (quantization / selection)");
    e = enqueue_attn(d, sparse, linear, q, q_i8, q_scale, k_i8, k_scale, kidx, keep, sm_scale,
                     out, out_f32, lse, base, w.attn, st);
    if (e != hipSuccess) return hip_fail(e, "sage_sla_fwd launch");
    return SSA_OK;
}

ssa_status sage_sla_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, ssa_shape s,
                             const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                             const float* k_scale, const int32_t* kidx, int64_t keep, int branches,
                             float sm_scale, const uint16_t* dout, const float* out_f32,
                             const float* lse, float* dq, float* dk, float* dv, void* ws,
                             size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    Dims d;
    TRY(check_shape(s, &d));
    if (branches < 1 || branches > 3)
        return fail(SSA_ERR_INVALID, "branches=%d must be SPARSE, LINEAR or both", branches);
    if (keep < 1 || keep > d.nkb)
        return fail(SSA_ERR_INVALID, "keep=%lld outside [1, %lld]", (long long)keep,
                    (long long)d.nkb);
    if (!kidx && keep != d.nkb)
        return fail(SSA_ERR_INVALID, "dense call (kidx NULL) needs keep == Nkb (%lld)",
                    (long long)d.nkb);
    if (!(sm_scale == sm_scale) || std::isinf(sm_scale))
        return fail(SSA_ERR_INVALID, "sm_scale is not finite");
    const bool sparse = branches & SSA_BRANCH_SPARSE;
    const bool sel = kidx && keep < d.nkb;
    const bool linear = (branches & SSA_BRANCH_LINEAR) && sel;
    // the linear branch's transposed state GEMM has a row per key block
    if (linear && d.BH * complement_tiles_per_head(d.nkb) > MAX_WG_256)
        return fail(SSA_ERR_UNSUPPORTED, "B*H=%lld too large for N=%lld (linear-branch grid)",
                    (long long)d.BH, (long long)s.N);
    TRY(need_ptr(q, 16, "q"));
    TRY(need_ptr(k, 16, "k"));
    TRY(need_ptr(v, 16, "v"));
    TRY(need_ptr(q_i8, 16, "q_i8"));
    TRY(need_ptr(k_i8, 16, "k_i8"));
    TRY(need_ptr(q_scale, 4, "q_scale"));
    TRY(need_ptr(k_scale, 4, "k_scale"));
    TRY(need_ptr(dout, 16, "dout"));
    TRY(need_ptr(dq, 16, "dq"));
    TRY(need_ptr(dk, 16, "dk"));
    TRY(need_ptr(dv, 16, "dv"));
    if (kidx) TRY(need_ptr(kidx, 4, "kidx"));
    if (!out_f32 != !lse)
        return fail(SSA_ERR_INVALID, "out_f32 and lse are given together or not at all");
    const bool saved = sparse && out_f32;  // the forward's output and row statistics
    if (out_f32) TRY(need_ptr(out_f32, 16, "out_f32"));
    if (lse) TRY(need_ptr(lse, 4, "lse"));
    const size_t nel = (size_t)d.BH * d.N * HD;
    const Range ins[] = {{q, nel * 2, "q"},
                         {k, nel * 2, "k"},
                         {v, nel * 2, "v"},
                         {q_i8, nel, "q_i8"},
                         {k_i8, nel, "k_i8"},
                         {q_scale, (size_t)d.BH * d.nqb * 4, "q_scale"},
                         {k_scale, (size_t)d.BH * d.nkb * 4, "k_scale"},
                         {kidx, kidx ? (size_t)d.BH * d.nqb * keep * 4 : 0, "kidx"},
                         {dout, nel * 2, "dout"},
                         {out_f32, out_f32 ? nel * 4 : 0, "out_f32"},
                         {lse, lse ? (size_t)d.BH * d.N * 4 : 0, "lse"}};
    const Range outs[] = {{dq, nel * 4, "dq"},
                          {dk, nel * 4, "dk"},
                          {dv, nel * 4, "dv"},
                          {ws, ws_bytes, "workspace"}};
    TRY(check_alias(outs, 4, ins, 11));
    const BwdWs w = ws_bwd(d, sel, linear);
    TRY(check_ws(ws, ws_bytes, w.total));
    TRY(check_device());

    hipStream_t st = (hipStream_t)stream;
    char* base = (char*)ws;
    const float sm = sm_scale > 0.f ? sm_scale : (float)(1.0 / std::sqrt((double)HD));
    hipError_t e = hipSuccess;
    if (!sparse && !linear) {
        // only the linear branch was asked for and it is empty: zero gradients
        e = launch_zero(dq, (int64_t)nel, st);
        if (e == hipSuccess) e = launch_zero(dk, (int64_t)nel, st);
        if (e == hipSuccess) e = launch_zero(dv, (int64_t)nel, st);
        if (e != hipSuccess) return hip_fail(e, "sage_sla_attn_bwd launch");
        return SSA_OK;
    }
    // the forward's V layout and, for the linear branch, its complement states
    e = enqueue_states(d, linear, k, v, base, w.attn, nullptr, nullptr, 0, st);
    if (e == hipSuccess && linear) e = enqueue_complement(d, kidx, keep, base, w.attn, st);
    if (e == hipSuccess && sel)
        e = launch_inv_lists(kidx, (int)keep, d.BH, (int)d.nqb, (int)d.nkb,
                             (uint32_t*)(base + w.bits), (uint16_t*)(base + w.lists),
                             (int32_t*)(base + w.counts), st);
    if (e != hipSuccess) return hip_fail(e, "sage_sla_attn_bwd launch (states)");
    // the linear branch's dq first (the sparse branch adds to it), with dO . o_l
    // per row when D comes from the forward's output
    float* gf = linear ? (float*)(base + w.gf) : nullptr;
    uint16_t* gs = linear ? (uint16_t*)(base + w.gs) : nullptr;
    uint16_t* gs_lo = linear ? (uint16_t*)(base + w.gs_lo) : nullptr;
    float* dol = (linear && saved) ? (float*)(base + w.dol) : nullptr;
    if (linear) {
        e = launch_lin_bwd_q(q, dout, (const float*)(base + w.attn.hnon), d.BH, (int)d.N, dq, gf, gs,
                             gs_lo, dol, st);
        if (e != hipSuccess) return hip_fail(e, "sage_sla_attn_bwd launch (linear branch)");
    }
    if (sparse) {
        const float K32 = (float)((double)sm * 1.4426950408889634074);
        float* dstat = (float*)(base + w.dstat);
        const float* mlog = saved ? lse : (const float*)(base + w.mlog);
        if (saved) {
            // D = dO . o_s = dO . out - dO . o_l from the forward's output
            e = launch_dstat(dout, out_f32, dol, d.BH * d.N, dstat, st);
        } else {
            // the forward's row statistics, recomputed
            AttnArgs f;
            f.q_i8 = q_i8;
            f.q_scale = q_scale;
            f.k_i8 = k_i8;
            f.k_scale = k_scale;
            f.vt = (const uint16_t*)(base + w.attn.vt);
            f.kidx = kidx;
            f.keep = (int)keep;
            f.N = (int)d.N;
            f.nqb = (int)d.nqb;
            f.nkb = (int)d.nkb;
            f.BH = d.BH;
            f.K32 = K32;
            f.do_sparse = 1;
            f.q = q;
            f.hnon = nullptr;
            f.out = nullptr;
            f.out32 = nullptr;
            f.dout = dout;
            f.mlog = (float*)(base + w.mlog);
            f.dstat = dstat;
            f.lse = nullptr;
            e = launch_attn(f, st);
        }
        BwdArgs b;
        b.q_i8 = q_i8;
        b.q_scale = q_scale;
        b.k_i8 = k_i8;
        b.k_scale = k_scale;
        b.v = v;
        b.dout = dout;
        b.kidx = kidx;
        b.keep = (int)keep;
        b.lists = sel ? (const uint16_t*)(base + w.lists) : nullptr;
        b.counts = sel ? (const int32_t*)(base + w.counts) : nullptr;
        b.dq_accumulate = linear ? 1 : 0;
        b.N = (int)d.N;
        b.nqb = (int)d.nqb;
        b.nkb = (int)d.nkb;
        b.BH = d.BH;
        b.K32 = K32;
        b.sm = sm;
        b.mlog = mlog;
        b.dstat = dstat;
        b.dq = dq;
        b.dk = dk;
        b.dv = dv;
        if (e == hipSuccess) e = launch_bwd_sparse(b, st);
        if (e != hipSuccess) return hip_fail(e, "sage_sla_attn_bwd launch (sparse branch)");
    }
    if (linear) {
        float* gtot = (float*)(base + w.gtot);
        float* gc = (float*)(base + w.gc);
        e = launch_state_total(gf, (int)d.nqb, d.BH, gtot, st);
        // the gradient states summed over the query blocks that did not keep
        // each key block: the complement GEMM on the transposed selection
        if (e == hipSuccess)
            e = launch_complement_lists((const uint16_t*)(base + w.lists),
                                        (const int32_t*)(base + w.counts), (int)d.nkb, (int)d.nqb,
                                        2 * keep > d.nkb ? 1 : 0, gs, gs_lo, gtot, d.BH,
                                        (uint32_t*)(base + w.msel), gc, st);
        if (e == hipSuccess)
            e = launch_lin_bwd_k(k, v, gc, d.BH, (int)d.N, sparse ? 1 : 0, dk, dv, st);
        if (e != hipSuccess) return hip_fail(e, "sage_sla_attn_bwd launch (linear branch)");
    }
    return SSA_OK;
}

ssa_status sage_qk_int32_tiles(const int8_t* q_i8, const int8_t* k_i8, ssa_shape s,
                               const int32_t* tiles, int64_t T, int32_t* out, void* stream) {
    g_err[0] = 0;
    Dims d;
    TRY(check_shape(s, &d));
    if (T < 1 || T > (1 << 24)) return fail(SSA_ERR_INVALID, "T=%lld out of range", (long long)T);
    TRY(need_ptr(q_i8, 16, "q_i8"));
    TRY(need_ptr(k_i8, 16, "k_i8"));
    TRY(need_ptr(tiles, 4, "tiles"));
    TRY(need_ptr(out, 16, "out"));
    const size_t nel = (size_t)d.BH * d.N * HD;
    const Range ins[] = {{q_i8, nel, "q_i8"}, {k_i8, nel, "k_i8"}, {tiles, (size_t)T * 12, "tiles"}};
    const Range outs[] = {{out, (size_t)T * QBLK * KBLK * 4, "out"}};
    TRY(check_alias(outs, 1, ins, 3));
    TRY(check_device());
    hipError_t e = launch_qk_tiles(q_i8, k_i8, d.BH, (int)d.N, tiles, T, out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "sage_qk_int32_tiles launch");
    return SSA_OK;
}

// ---- W8A8 linear layer --------------------------------------------------------

static const int64_t W8_MAX = 1 << 20;  // rows, columns and K at most 2^20

ssa_status w8a8_quant(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                      void* stream) {
    g_err[0] = 0;
    if (rows < 1 || rows > W8_MAX || cols < 128 || cols > W8_MAX || cols % 128)
        return fail(SSA_ERR_INVALID, "w8a8_quant: rows=%lld cols=%lld (cols a multiple of 128, "
                    "both in [1, 2^20])", (long long)rows, (long long)cols);
    TRY(need_ptr(x, 16, "x"));
    TRY(need_ptr(q, 16, "q"));
    TRY(need_ptr(scale, 4, "scale"));
    const size_t nel = (size_t)rows * cols;
    const size_t nsc = (size_t)((rows + 127) / 128) * (cols / 128);
    const Range ins[] = {{x, nel * 2, "x"}};
    const Range outs[] = {{q, nel, "q"}, {scale, nsc * 4, "scale"}};
    TRY(check_alias(outs, 2, ins, 1));
    TRY(check_device());
    hipError_t e = launch_w8a8_quant(x, (int)rows, (int)cols, q, scale, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "w8a8_quant launch");
    return SSA_OK;
}

ssa_status w8a8_gemm(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                     const float* bias, int64_t M, int64_t N, int64_t K, uint16_t* y, float* y32,
                     void* stream) {
    g_err[0] = 0;
    if (M < 1 || M > W8_MAX || N < 128 || N > W8_MAX || N % 128 || K < 128 || K > W8_MAX ||
        K % 128)
        return fail(SSA_ERR_INVALID, "w8a8_gemm: M=%lld N=%lld K=%lld (N, K multiples of 128, "
                    "all in [1, 2^20])", (long long)M, (long long)N, (long long)K);
    if (w8a8_gemm_workgroups(M, N) > ((int64_t)1 << 22) - 8)
        return fail(SSA_ERR_UNSUPPORTED, "w8a8_gemm: M=%lld N=%lld give more workgroups than one "
                    "launch takes", (long long)M, (long long)N);
    TRY(need_ptr(xq, 16, "xq"));
    TRY(need_ptr(wq, 16, "wq"));
    TRY(need_ptr(sx, 4, "sx"));
    TRY(need_ptr(sw, 4, "sw"));
    TRY(need_ptr(y, 16, "y"));
    if (y32 && !aligned(y32, 16)) return fail(SSA_ERR_INVALID, "y32 is not 16-byte aligned");
    if (bias && !aligned(bias, 16)) return fail(SSA_ERR_INVALID, "bias is not 16-byte aligned");
    const size_t nkb = (size_t)K / 128;
    const Range ins[] = {{xq, (size_t)M * K, "xq"},
                         {wq, (size_t)N * K, "wq"},
                         {sx, (size_t)((M + 127) / 128) * nkb * 4, "sx"},
                         {sw, (size_t)(N / 128) * nkb * 4, "sw"},
                         {bias, bias ? (size_t)N * 4 : 0, "bias"}};
    const Range outs[] = {{y, (size_t)M * N * 2, "y"}, {y32, y32 ? (size_t)M * N * 4 : 0, "y32"}};
    TRY(check_alias(outs, 2, ins, 5));
    TRY(check_device());
    hipError_t e = launch_w8a8_gemm(xq, sx, wq, sw, bias, (int)M, (int)N, (int)K, y, y32,
                                    (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "w8a8_gemm launch");
    return SSA_OK;
}

ssa_status ssa_kernel_timer_start(int max_launches) {
    g_err[0] = 0;
    if (max_launches < 1 || max_launches > (1 << 16))
        return fail(SSA_ERR_INVALID, "max_launches=%d outside [1, 65536]", max_launches);
    std::lock_guard<std::mutex> lk(g_tm);
    timer_destroy_locked();
    for (int x = 0; x < max_launches; ++x) {
        hipEvent_t a, b;
        hipError_t e = hipEventCreate(&a);
        if (e == hipSuccess) e = hipEventCreate(&b);
        if (e != hipSuccess) {
            timer_destroy_locked();
            return hip_fail(e, "hipEventCreate");
        }
        g_ev0.push_back(a);
        g_ev1.push_back(b);
    }
    return SSA_OK;
}

int ssa_kernel_timer_read(float* ms, int cap) {
    std::lock_guard<std::mutex> lk(g_tm);
    const int n = g_tcount < cap ? g_tcount : cap;
    for (int x = 0; x < n; ++x) {
        if (hipEventSynchronize(g_ev1[x]) != hipSuccess ||
            hipEventElapsedTime(&ms[x], g_ev0[x], g_ev1[x]) != hipSuccess)
            ms[x] = -1.f;
    }
    return n;
}

void ssa_kernel_timer_stop(void) {
    std::lock_guard<std::mutex> lk(g_tm);
    timer_destroy_locked();
}

}  // extern "C"
