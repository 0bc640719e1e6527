"""SageSLA attention for AMD MI355X (gfx950): thin Python binding of libssa.so.

The C ABI (include/ssa.h) does all the work in HIP kernels; this module only
checks tensors, allocates outputs and workspaces with torch, and passes raw
device pointers and the current HIP stream. There is no CPU fallback: every
entry point raises if the library is missing or a tensor is not on a GPU.

Entry points keep the ABI's names:
    sage_quant_qk, sla_block_mask, sage_sla_attn_fwd, sage_qk_int32_tiles
plus ``sagesla`` (all three in order) and ``SageSLAPlan`` (preallocated
buffers, for repeated calls on one shape).
"""
from __future__ import annotations

import ctypes as C
import os

import torch

__all__ = [
    "sage_quant_qk", "sla_block_mask", "sage_sla_attn_fwd", "sage_sla_fwd", "sage_qk_int32_tiles",
    "sagesla",
    "SageSLAPlan", "KernelTimer", "keep_blocks", "num_q_blocks", "num_k_blocks", "workspace_bytes",
    "pool_bytes", "new_pool", "lib_path", "w8a8_quant", "w8a8_gemm", "w8a8_linear",
    "SPARSE", "LINEAR", "OP_QUANT", "OP_MASK", "OP_ATTN", "OP_STEP",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssa.so")

SPARSE, LINEAR = 1, 2
OP_QUANT, OP_MASK, OP_ATTN, OP_STEP, OP_BWD = 0, 1, 2, 3, 4
HEAD_DIM = 128

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small",
           4: "HIP error"}


class SSAError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


class Shape(C.Structure):
    _fields_ = [("B", C.c_int64), ("H", C.c_int64), ("N", C.c_int64), ("D", C.c_int64)]


_lib = None
_p = C.c_void_p


def lib_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"libssa.so not found at {_LIB_PATH}: build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` (no CPU fallback exists)")
    L = C.CDLL(_LIB_PATH)
    i32, i64, sz = C.c_int, C.c_int64, C.c_size_t
    sig = {
        "ssa_num_q_blocks": (i64, [i64]),
        "ssa_num_k_blocks": (i64, [i64]),
        "ssa_keep_blocks": (i64, [i64, C.c_double]),
        "ssa_workspace_bytes": (sz, [i32, Shape, i64, i32]),
        "ssa_status_str": (C.c_char_p, [i32]),
        "ssa_last_error": (C.c_char_p, []),
        "sage_quant_qk": (i32, [_p, _p, Shape, _p, _p, _p, _p, _p, _p, _p, sz, _p]),
        "sage_quant_qk_noalloc": (i32, [_p, _p, Shape, _p, _p, _p, _p, _p, _p, _p]),
        "sla_block_mask": (i32, [_p, _p, Shape, i64, _p, _p, _p, _p, sz, _p]),
        "ssa_pool_bytes": (sz, [Shape]),
        "w8a8_quant": (i32, [_p, i64, i64, _p, _p, _p]),
        "w8a8_gemm": (i32, [_p, _p, _p, _p, _p, i64, i64, i64, _p, _p, _p]),
        "sage_sla_attn_fwd": (i32, [_p, _p, _p, Shape, _p, _p, _p, _p, _p, i64, i32, C.c_float,
                                    _p, _p, _p, _p, sz, _p]),
        "sage_sla_fwd": (i32, [_p, _p, _p, Shape, i64, i32, C.c_float, _p, _p, _p, _p, _p, _p,
                               _p, _p, _p, _p, _p, sz, _p]),
        "sage_qk_int32_tiles": (i32, [_p, _p, Shape, _p, i64, _p, _p]),
        "sage_sla_attn_bwd": (i32, [_p, _p, _p, Shape, _p, _p, _p, _p, _p, i64, i32, C.c_float,
                                    _p, _p, _p, _p, _p, _p, _p, sz, _p]),
        "ssa_kernel_timer_start": (i32, [i32]),
        "ssa_kernel_timer_read": (i32, [C.POINTER(C.c_float), i32]),
        "ssa_kernel_timer_stop": (None, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(fn, st):
    if st != 0:
        raise SSAError(fn, st, _load().ssa_last_error().decode())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(dev):
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _shape_of(q) -> Shape:
    B, H, N, D = q.shape
    return Shape(B, H, N, D)


def _need_gpu(name, t, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (no CPU path exists), got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def num_q_blocks(N: int) -> int:
    return int(_load().ssa_num_q_blocks(N))


def num_k_blocks(N: int) -> int:
    return int(_load().ssa_num_k_blocks(N))


def keep_blocks(N: int, topk: float) -> int:
    return int(_load().ssa_keep_blocks(N, float(topk)))


def workspace_bytes(op: int, shape, keep: int = 0, branches: int = 0) -> int:
    s = shape if isinstance(shape, Shape) else Shape(*shape)
    return int(_load().ssa_workspace_bytes(op, s, int(keep), int(branches)))


def _ws(op, s, dev, keep=0, branches=0):
    n = workspace_bytes(op, s, keep, branches)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=dev), n


def _qkv_shape(q, k, v=None):
    _need_gpu("q", q, torch.bfloat16)
    if q.dim() != 4 or q.shape[-1] != HEAD_DIM:
        raise ValueError(f"q must be [B,H,N,{HEAD_DIM}], got {tuple(q.shape)}")
    _need_gpu("k", k, torch.bfloat16, q.shape)
    if v is not None:
        _need_gpu("v", v, torch.bfloat16, q.shape)
    return _shape_of(q)


def pool_bytes(shape) -> int:
    """Bytes of the pooled-means buffer that sage_quant_qk can fill for sla_block_mask."""
    return int(_load().ssa_pool_bytes(Shape(*shape)))


def new_pool(q):
    """A pooled-means buffer for tensors shaped like q."""
    return torch.empty(pool_bytes(tuple(q.shape)), dtype=torch.uint8, device=q.device)


def sage_quant_qk(q, k, pool=None):
    """K smoothing + per-block INT8 quantization.
    Returns (q_i8, q_scale [B,H,Nqb], k_i8, k_scale [B,H,Nkb], k_mean [B,H,D]).
    pool (from new_pool) also receives the block mask's pooled means."""
    s = _qkv_shape(q, k)
    B, H, N, D = q.shape
    dev = q.device
    q_i8 = torch.empty((B, H, N, D), dtype=torch.int8, device=dev)
    k_i8 = torch.empty_like(q_i8)
    q_scale = torch.empty((B, H, num_q_blocks(N)), dtype=torch.float32, device=dev)
    k_scale = torch.empty((B, H, num_k_blocks(N)), dtype=torch.float32, device=dev)
    k_mean = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    ws, n = _ws(OP_QUANT, s, dev)
    if pool is not None:
        _need_gpu("pool", pool, torch.uint8, (pool_bytes(tuple(q.shape)),))
    _check("sage_quant_qk", _load().sage_quant_qk(
        _ptr(q), _ptr(k), s, _ptr(q_i8), _ptr(q_scale), _ptr(k_i8), _ptr(k_scale), _ptr(k_mean),
        _ptr(pool), _ptr(ws), n, _stream(dev)))
    return q_i8, q_scale, k_i8, k_scale, k_mean


def sla_block_mask(q, k, keep: int, return_mask: bool = False, pool=None):
    """kidx [B,H,Nqb,keep] (ascending key blocks), and the uint8 mask
    [B,H,Nqb,Nkb] when return_mask. pool: a buffer sage_quant_qk filled for the
    same q, k (then q and k are not read)."""
    s = _qkv_shape(q, k)
    B, H, N, D = q.shape
    dev = q.device
    kidx = torch.empty((B, H, num_q_blocks(N), int(keep)), dtype=torch.int32, device=dev)
    mask = (torch.empty((B, H, num_q_blocks(N), num_k_blocks(N)), dtype=torch.uint8, device=dev)
            if return_mask else None)
    if pool is not None:
        _need_gpu("pool", pool, torch.uint8, (pool_bytes(tuple(q.shape)),))
        ws, n = None, 0
    else:
        ws, n = _ws(OP_MASK, s, dev, keep)
    _check("sla_block_mask", _load().sla_block_mask(
        _ptr(q), _ptr(k), s, int(keep), _ptr(pool), _ptr(kidx), _ptr(mask), _ptr(ws), n,
        _stream(dev)))
    return (kidx, mask) if return_mask else kidx


def sage_sla_attn_fwd(q, k, v, q_i8, q_scale, k_i8, k_scale, kidx=None, keep=None,
                      branches: int = SPARSE | LINEAR, sm_scale: float = 0.0,
                      return_f32: bool = False, return_lse: bool = False):
    """SageSLA forward. kidx=None runs dense (every key block kept). Returns
    out, then out32 if return_f32, then lse [B,H,N] (m + log2 l per row, for
    the backward) if return_lse."""
    s = _qkv_shape(q, k, v)
    B, H, N, D = q.shape
    dev = q.device
    nqb, nkb = num_q_blocks(N), num_k_blocks(N)
    _need_gpu("q_i8", q_i8, torch.int8, q.shape)
    _need_gpu("k_i8", k_i8, torch.int8, q.shape)
    _need_gpu("q_scale", q_scale, torch.float32, (B, H, nqb))
    _need_gpu("k_scale", k_scale, torch.float32, (B, H, nkb))
    if kidx is None:
        keep = nkb
    else:
        keep = kidx.shape[-1] if keep is None else int(keep)
        _need_gpu("kidx", kidx, torch.int32, (B, H, nqb, keep))
    out = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
    out32 = torch.empty((B, H, N, D), dtype=torch.float32, device=dev) if return_f32 else None
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if return_lse else None
    ws, n = _ws(OP_ATTN, s, dev, keep, branches)
    _check("sage_sla_attn_fwd", _load().sage_sla_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), s, _ptr(q_i8), _ptr(q_scale), _ptr(k_i8), _ptr(k_scale),
        _ptr(kidx), int(keep), int(branches), float(sm_scale), _ptr(out), _ptr(out32), _ptr(lse),
        _ptr(ws), n, _stream(dev)))
    res = (out,) + ((out32,) if return_f32 else ()) + ((lse,) if return_lse else ())
    return res if len(res) > 1 else out


def sage_sla_attn_bwd(q, k, v, q_i8, q_scale, k_i8, k_scale, dout, kidx=None, keep=None,
                      branches: int = SPARSE | LINEAR, sm_scale: float = 0.0, out32=None,
                      lse=None):
    """SageSLA backward: (dq, dk, dv) fp32 [B,H,N,D] for dL/dO = dout (bf16),
    with the same quantized tensors, selection and branches as the forward.
    out32 and lse (the forward's fp32 output and row statistics, given
    together) spare the backward its recomputation of the forward."""
    s = _qkv_shape(q, k, v)
    B, H, N, D = q.shape
    dev = q.device
    nqb, nkb = num_q_blocks(N), num_k_blocks(N)
    _need_gpu("q_i8", q_i8, torch.int8, q.shape)
    _need_gpu("k_i8", k_i8, torch.int8, q.shape)
    _need_gpu("q_scale", q_scale, torch.float32, (B, H, nqb))
    _need_gpu("k_scale", k_scale, torch.float32, (B, H, nkb))
    _need_gpu("dout", dout, torch.bfloat16, q.shape)
    if kidx is None:
        keep = nkb
    else:
        keep = kidx.shape[-1] if keep is None else int(keep)
        _need_gpu("kidx", kidx, torch.int32, (B, H, nqb, keep))
    if (out32 is None) != (lse is None):
        raise ValueError("out32 and lse are given together or not at all")
    if out32 is not None:
        _need_gpu("out32", out32, torch.float32, q.shape)
        _need_gpu("lse", lse, torch.float32, (B, H, N))
    grads = [torch.empty((B, H, N, D), dtype=torch.float32, device=dev) for _ in range(3)]
    ws, n = _ws(OP_BWD, s, dev, keep, branches)
    _check("sage_sla_attn_bwd", _load().sage_sla_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), s, _ptr(q_i8), _ptr(q_scale), _ptr(k_i8), _ptr(k_scale),
        _ptr(kidx), int(keep), int(branches), float(sm_scale), _ptr(dout), _ptr(out32),
        _ptr(lse), *map(_ptr, grads), _ptr(ws), n, _stream(dev)))
    return tuple(grads)


def sage_qk_int32_tiles(q_i8, k_i8, tiles):
    """Raw int32 score tiles [T,128,64] for (b*H+h, i, j) triples (int32 [T,3])."""
    _need_gpu("q_i8", q_i8, torch.int8)
    _need_gpu("k_i8", k_i8, torch.int8, q_i8.shape)
    _need_gpu("tiles", tiles, torch.int32)
    if tiles.dim() != 2 or tiles.shape[1] != 3:
        raise ValueError("tiles must be [T,3]")
    T = tiles.shape[0]
    out = torch.empty((T, 128, 64), dtype=torch.int32, device=q_i8.device)
    _check("sage_qk_int32_tiles", _load().sage_qk_int32_tiles(
        _ptr(q_i8), _ptr(k_i8), _shape_of(q_i8), _ptr(tiles), T, _ptr(out),
        _stream(q_i8.device)))
    return out


def sage_sla_fwd(q, k, v, topk: float | None = 0.1, linear: bool = True, sm_scale: float = 0.0,
                 return_f32: bool = False, return_mask: bool = False, return_all: bool = False,
                 return_lse: bool = False):
    """The whole step in one library call (quantize, select unless topk is
    None, attend), bit-identical to the three staged calls. Returns out, then
    out32 if return_f32, then the u8 block mask if return_mask (None when
    dense), then lse if return_lse, then, if return_all, a dict of the
    intermediates (q_i8, q_scale, k_i8, k_scale, k_mean, kidx)."""
    s = _qkv_shape(q, k, v)
    B, H, N, D = q.shape
    dev = q.device
    nqb, nkb = num_q_blocks(N), num_k_blocks(N)
    dense = topk is None
    keep = nkb if dense else keep_blocks(N, topk)
    branches = SPARSE | (LINEAR if (linear and not dense) else 0)
    e = dict(device=dev)
    q_i8 = torch.empty((B, H, N, D), dtype=torch.int8, **e)
    k_i8 = torch.empty_like(q_i8)
    q_scale = torch.empty((B, H, nqb), dtype=torch.float32, **e)
    k_scale = torch.empty((B, H, nkb), dtype=torch.float32, **e)
    k_mean = torch.empty((B, H, D), dtype=torch.float32, **e)
    kidx = None if dense else torch.empty((B, H, nqb, keep), dtype=torch.int32, **e)
    mask = (torch.empty((B, H, nqb, nkb), dtype=torch.uint8, **e)
            if (return_mask and not dense) else None)
    out = torch.empty((B, H, N, D), dtype=torch.bfloat16, **e)
    out32 = torch.empty((B, H, N, D), dtype=torch.float32, **e) if return_f32 else None
    lse = torch.empty((B, H, N), dtype=torch.float32, **e) if return_lse else None
    ws, n = _ws(OP_STEP, s, dev, keep, branches)
    _check("sage_sla_fwd", _load().sage_sla_fwd(
        _ptr(q), _ptr(k), _ptr(v), s, int(keep), int(branches), float(sm_scale), _ptr(q_i8),
        _ptr(q_scale), _ptr(k_i8), _ptr(k_scale), _ptr(k_mean), _ptr(kidx), _ptr(mask),
        _ptr(out), _ptr(out32), _ptr(lse), _ptr(ws), n, _stream(dev)))
    res = (out, out32) if return_f32 else (out,)
    if return_mask:
        res = res + (mask,)
    if return_lse:
        res = res + (lse,)
    if return_all:
        res = res + (dict(q_i8=q_i8, q_scale=q_scale, k_i8=k_i8, k_scale=k_scale, k_mean=k_mean,
                          kidx=kidx),)
    return res if len(res) > 1 else res[0]


def sagesla(q, k, v, topk: float | None = 0.1, linear: bool = True, sm_scale: float = 0.0,
            return_f32: bool = False):
    """The whole path as the three staged calls: quantize, select blocks
    (unless topk is None: dense), attend. The meaning of topk is --sla_topk's:
    the fraction of key blocks kept per query block. sage_sla_fwd gives the
    same result from one call."""
    pool = None if topk is None else new_pool(q)
    q_i8, q_scale, k_i8, k_scale, _ = sage_quant_qk(q, k, pool)
    if topk is None:
        return sage_sla_attn_fwd(q, k, v, q_i8, q_scale, k_i8, k_scale, None, None, SPARSE,
                                 sm_scale, return_f32)
    keep = keep_blocks(q.shape[2], topk)
    kidx = sla_block_mask(q, k, keep, pool=pool)
    br = SPARSE | (LINEAR if linear else 0)
    return sage_sla_attn_fwd(q, k, v, q_i8, q_scale, k_i8, k_scale, kidx, keep, br, sm_scale,
                             return_f32)


W8_BLK = 128


def w8a8_quant(x):
    """128x128 block INT8 quantization of a bf16 [rows][cols] matrix (page 5,
    Pillar Three). Returns (q int8 [rows][cols], scale fp32 [ceil(rows/128)][cols/128])."""
    _need_gpu("x", x, torch.bfloat16)
    if x.dim() != 2 or x.shape[1] % W8_BLK:
        raise ValueError(f"x must be [rows][cols] with cols a multiple of 128, got {tuple(x.shape)}")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    sc = torch.empty(((rows + W8_BLK - 1) // W8_BLK, cols // W8_BLK), dtype=torch.float32,
                     device=x.device)
    _check("w8a8_quant", _load().w8a8_quant(_ptr(x), rows, cols, _ptr(q), _ptr(sc),
                                            _stream(x.device)))
    return q, sc


def w8a8_gemm(xq, sx, wq, sw, return_f32: bool = False, bias=None):
    """y = x . w^T (+ bias) from the block-quantized operands (w in the
    [out][in] layout; bias fp32 [N] or None)."""
    _need_gpu("xq", xq, torch.int8)
    M, K = xq.shape
    _need_gpu("wq", wq, torch.int8)
    N = wq.shape[0]
    if wq.shape[1] != K or K % W8_BLK or N % W8_BLK:
        raise ValueError("wq must be [N][K] with N and K multiples of 128")
    _need_gpu("sx", sx, torch.float32, ((M + W8_BLK - 1) // W8_BLK, K // W8_BLK))
    _need_gpu("sw", sw, torch.float32, (N // W8_BLK, K // W8_BLK))
    if bias is not None:
        _need_gpu("bias", bias, torch.float32, (N,))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    y32 = torch.empty((M, N), dtype=torch.float32, device=xq.device) if return_f32 else None
    _check("w8a8_gemm", _load().w8a8_gemm(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(bias), M,
                                          N, K, _ptr(y), _ptr(y32), _stream(xq.device)))
    return (y, y32) if return_f32 else y


def w8a8_linear(x, wq, sw, bias=None, return_f32: bool = False):
    """The W8A8 linear layer on bf16 activations x [M][K] with pre-quantized
    weights (w8a8_quant of w [N][K]) and an optional fp32 bias [N]: quantize
    x, then the INT8 product."""
    xq, sx = w8a8_quant(x)
    return w8a8_gemm(xq, sx, wq, sw, return_f32, bias)


class KernelTimer:
    """HIP-event durations of the sparse-attention kernel launches made while
    the timer is active (see ssa_kernel_timer_start in include/ssa.h)."""

    def __init__(self, max_launches: int):
        self.n = int(max_launches)

    def __enter__(self):
        _check("ssa_kernel_timer_start", _load().ssa_kernel_timer_start(self.n))
        return self

    def read(self):
        buf = (C.c_float * self.n)()
        got = _load().ssa_kernel_timer_read(buf, self.n)
        return [float(buf[x]) for x in range(got)]

    def __exit__(self, *exc):
        _load().ssa_kernel_timer_stop()
        return False


class SageSLAPlan:
    """Preallocated buffers for repeated SageSLA calls on one shape.

    run() enqueues the step on the current stream: one sage_sla_fwd call, or
    with fused=False the staged calls sage_quant_qk, sla_block_mask (unless
    dense) and sage_sla_attn_fwd (run_staged()); each stage can also be
    enqueued on its own (quant(), mask(), attn()). Both forms write the same
    buffers with bit-identical contents."""

    def __init__(self, B, H, N, topk: float | None, linear: bool = True, device="cuda",
                 sm_scale: float = 0.0, want_f32: bool = False, fused: bool = True,
                 want_lse: bool = False):
        L = _load()
        dev = torch.device(device)
        self.shape = Shape(B, H, N, HEAD_DIM)
        self.B, self.H, self.N = B, H, N
        self.nqb, self.nkb = num_q_blocks(N), num_k_blocks(N)
        self.dense = topk is None
        self.keep = self.nkb if self.dense else keep_blocks(N, topk)
        self.branches = SPARSE | (LINEAR if (linear and not self.dense) else 0)
        self.sm_scale = float(sm_scale)
        e = dict(device=dev)
        self.q_i8 = torch.empty((B, H, N, HEAD_DIM), dtype=torch.int8, **e)
        self.k_i8 = torch.empty_like(self.q_i8)
        self.q_scale = torch.empty((B, H, self.nqb), dtype=torch.float32, **e)
        self.k_scale = torch.empty((B, H, self.nkb), dtype=torch.float32, **e)
        self.k_mean = torch.empty((B, H, HEAD_DIM), dtype=torch.float32, **e)
        self.kidx = None if self.dense else torch.empty((B, H, self.nqb, self.keep),
                                                        dtype=torch.int32, **e)
        # pooled means: sage_quant_qk hands them to sla_block_mask
        self.pool = None if self.dense else torch.empty(
            int(L.ssa_pool_bytes(self.shape)), dtype=torch.uint8, **e)
        self.out = torch.empty((B, H, N, HEAD_DIM), dtype=torch.bfloat16, **e)
        self.out32 = torch.empty((B, H, N, HEAD_DIM), dtype=torch.float32, **e) if want_f32 else None
        # each row's m + log2 l, kept with out32 for a backward pass
        self.lse = torch.empty((B, H, N), dtype=torch.float32, **e) if want_lse else None
        self.ws_n = {
            OP_QUANT: workspace_bytes(OP_QUANT, self.shape),
            OP_ATTN: workspace_bytes(OP_ATTN, self.shape, self.keep, self.branches),
            OP_STEP: workspace_bytes(OP_STEP, self.shape, self.keep, self.branches),
        }
        self.fused = bool(fused)
        # one workspace serves every call (they run in order on one stream)
        self.ws = torch.empty(max(self.ws_n.values()), dtype=torch.uint8, **e)
        self.device = dev
        self._L = L

    def bind(self, q, k, v):
        _qkv_shape(q, k, v)
        if tuple(q.shape) != (self.B, self.H, self.N, HEAD_DIM):
            raise ValueError("tensor shape differs from the plan")
        self.q, self.k, self.v = q, k, v
        return self

    def quant(self):
        _check("sage_quant_qk", self._L.sage_quant_qk(
            _ptr(self.q), _ptr(self.k), self.shape, _ptr(self.q_i8), _ptr(self.q_scale),
            _ptr(self.k_i8), _ptr(self.k_scale), _ptr(self.k_mean), _ptr(self.pool),
            _ptr(self.ws), self.ws_n[OP_QUANT], _stream(self.device)))

    def mask(self):
        if self.dense:
            return
        _check("sla_block_mask", self._L.sla_block_mask(
            _ptr(self.q), _ptr(self.k), self.shape, self.keep, _ptr(self.pool), _ptr(self.kidx),
            None, None, 0, _stream(self.device)))

    def attn(self):
        _check("sage_sla_attn_fwd", self._L.sage_sla_attn_fwd(
            _ptr(self.q), _ptr(self.k), _ptr(self.v), self.shape, _ptr(self.q_i8),
            _ptr(self.q_scale), _ptr(self.k_i8), _ptr(self.k_scale), _ptr(self.kidx), self.keep,
            self.branches, self.sm_scale, _ptr(self.out), _ptr(self.out32), _ptr(self.lse),
            _ptr(self.ws), self.ws_n[OP_ATTN], _stream(self.device)))

    def step(self):
        _check("sage_sla_fwd", self._L.sage_sla_fwd(
            _ptr(self.q), _ptr(self.k), _ptr(self.v), self.shape, self.keep, self.branches,
            self.sm_scale, _ptr(self.q_i8), _ptr(self.q_scale), _ptr(self.k_i8),
            _ptr(self.k_scale), _ptr(self.k_mean), _ptr(self.kidx), None, _ptr(self.out),
            _ptr(self.out32), _ptr(self.lse), _ptr(self.ws), self.ws_n[OP_STEP],
            _stream(self.device)))

    def run_staged(self):
        self.quant()
        self.mask()
        self.attn()
        return self.out

    def run(self):
        if not self.fused:
            return self.run_staged()
        self.step()
        return self.out

    def capture(self):
        """Record one run() into a HIP graph (torch.cuda.CUDAGraph). The calls
        allocate nothing, set no memory with hipMemset and synchronize nothing,
        so the whole step is capturable; replay() then re-executes it on the
        bound tensors (rebinding other tensors needs a new capture). An eager
        run() first checks the device and loads the code objects."""
        self.run()
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        self._graph = g
        return g

    def replay(self):
        if getattr(self, "_graph", None) is None:
            raise RuntimeError("capture() the plan before replay()")
        self._graph.replay()
        return self.out
