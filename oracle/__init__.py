"""ctypes wrapper of the CPU oracle (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path under
``bit_sparse_attention_amd`` never does.

All arrays are numpy. bf16 tensors are passed as uint16 bit patterns with
shape [BH, N, D] (B and H flattened).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

QBLK, KBLK = 128, 64

_p = C.c_void_p
_i64 = C.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(
                os.path.join(_HERE, "oracle.c")):
            _build.build()
        L = C.CDLL(_LIB_PATH)
        sig = {
            "orc_nqb": (_i64, [_i64]),
            "orc_nkb": (_i64, [_i64]),
            "orc_keep": (_i64, [_i64, C.c_double]),
            "orc_bf16_to_f32": (C.c_float, [C.c_uint16]),
            "orc_f32_to_bf16": (C.c_uint16, [C.c_float]),
            "orc_round_bf16": (C.c_double, [C.c_double]),
            "orc_p_ambiguous": (C.c_double, [C.c_double, C.c_double, C.c_double, C.c_double]),
            "orc_k_mean": (None, [_p, _i64, _i64, _i64, _p]),
            "orc_quant": (None, [_p, _p, _i64, _i64, _i64, _i64, _p, _p, C.c_int]),
            "orc_qk_tile": (None, [_p, _p, _i64, _i64, _i64, _i64, _i64, _p]),
            "orc_pool": (None, [_p, _i64, _i64, _i64, _i64, _p]),
            "orc_block_scores": (None, [_p, _p, _i64, _i64, _p, _i64, _p]),
            "orc_topk": (None, [_p, _i64, _i64, _i64, _p, _p]),
            "orc_sparse_rows": (None, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, C.c_float,
                                       _p, _i64, _p, _p, _p, C.c_int]),
            "orc_linear_states": (None, [_p, _p, _i64, _i64, _i64, _p, _p, C.c_int]),
            "orc_linear_rows": (None, [_p, _i64, _i64, _i64, _p, _p, _p, _i64, _p, _i64, _p,
                                       C.c_int]),
            "orc_dense_rows": (None, [_p, _p, _p, _i64, _i64, _i64, C.c_float, _p, _i64, _p,
                                      C.c_int]),
            "orc_sagesla_bwd": (None, [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64,
                                       C.c_int, C.c_float, _p, _p, _p, _p, C.c_int]),
            "orc_sagesla_bwd_sel": (None, [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p,
                                           _i64, C.c_int, C.c_float, _p, _p, _p, _p, _p, _p,
                                           C.c_int]),
            "orc_sagesla_loss": (C.c_double, [_p, _p, _p, _p, _p, _i64, _i64, _p, _i64, C.c_int,
                                              C.c_double, _p]),
            "orc_w8a8_quant": (None, [_p, _i64, _i64, _p, _p, C.c_int]),
            "orc_w8a8_gemm": (None, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _p, C.c_int]),
            "orc_w8a8_gemm_f64": (None, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _p, _p,
                                         C.c_int]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def threads() -> int:
    """Worker threads: the CPUs this process may run on (its affinity set,
    which a batch job's CPU share restricts), capped by OMP_NUM_THREADS when
    that is set."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def nqb(N):
    return int(lib().orc_nqb(N))


def nkb(N):
    return int(lib().orc_nkb(N))


def keep_blocks(N, topk):
    return int(lib().orc_keep(N, float(topk)))


def round_bf16(x: float) -> float:
    return float(lib().orc_round_bf16(float(x)))


def p_ambiguous(p, xa, xabs_max, m) -> float:
    """bf16 ulp at p if a GPU may round p = 2^(x - m) the other way (the flip
    window of the declared numerics), else 0."""
    return float(lib().orc_p_ambiguous(float(p), float(xa), float(xabs_max), float(m)))


NORM_LAG = 64.0  # the normalizer lag the flip window allows (oracle.h ORC_NORM_LAG)


def f32_to_bf16_bits(x: float) -> int:
    return int(lib().orc_f32_to_bf16(float(x)))


def _u16(x):
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16, x.dtype
    return x


def k_mean(k):
    k = _u16(k)
    BH, N, D = k.shape
    mu = np.empty((BH, D), np.float32)
    lib().orc_k_mean(_ptr(k), BH, N, D, _ptr(mu))
    return mu


def quant(x, mu, blk, nthreads=None):
    x = _u16(x)
    BH, N, D = x.shape
    nb = (N + blk - 1) // blk
    xq = np.empty((BH, N, D), np.int8)
    sc = np.empty((BH, nb), np.float32)
    mu = None if mu is None else np.ascontiguousarray(mu, dtype=np.float32)
    lib().orc_quant(_ptr(x), _ptr(mu), BH, N, D, blk, _ptr(xq), _ptr(sc),
                    nthreads or threads())
    return xq, sc


def quant_qk(q, k, nthreads=None):
    """(q_i8, q_scale, k_i8, k_scale, k_mean) as the method defines them."""
    mu = k_mean(k)
    qi, qs = quant(q, None, QBLK, nthreads)
    ki, ks = quant(k, mu, KBLK, nthreads)
    return qi, qs, ki, ks, mu


def qk_tile(q_i8, k_i8, bh, i, j):
    q_i8 = np.ascontiguousarray(q_i8)
    k_i8 = np.ascontiguousarray(k_i8)
    BH, N, D = q_i8.shape
    out = np.empty((QBLK, KBLK), np.int32)
    lib().orc_qk_tile(_ptr(q_i8), _ptr(k_i8), N, D, bh, i, j, _ptr(out))
    return out


def pool(x, bh, blk):
    x = _u16(x)
    BH, N, D = x.shape
    nb = (N + blk - 1) // blk
    out = np.empty((nb, D), np.float32)
    lib().orc_pool(_ptr(x), N, D, bh, blk, _ptr(out))
    return out


def block_scores(qbar, kbar, qblocks):
    qbar = np.ascontiguousarray(qbar, np.float32)
    kbar = np.ascontiguousarray(kbar, np.float32)
    qb = np.ascontiguousarray(qblocks, np.int64)
    Nkb, D = kbar.shape
    out = np.empty((len(qb), Nkb), np.float32)
    lib().orc_block_scores(_ptr(qbar), _ptr(kbar), Nkb, D, _ptr(qb), len(qb), _ptr(out))
    return out


def topk(scores, keep):
    scores = np.ascontiguousarray(scores, np.float32)
    R, Nkb = scores.shape
    kidx = np.empty((R, keep), np.int32)
    mask = np.empty((R, Nkb), np.uint8)
    lib().orc_topk(_ptr(scores), R, Nkb, keep, _ptr(kidx), _ptr(mask))
    return kidx, mask


def block_mask_head(q, k, bh, keep, qblocks=None):
    """kidx [R, keep] and mask [R, Nkb] for the listed query blocks of head bh
    (all query blocks when qblocks is None)."""
    q = _u16(q)
    k = _u16(k)
    N = q.shape[1]
    qbar = pool(q, bh, QBLK)
    kbar = pool(k, bh, KBLK)
    if qblocks is None:
        qblocks = np.arange(qbar.shape[0], dtype=np.int64)
    sc = block_scores(qbar, kbar, qblocks)
    return topk(sc, keep)


def block_mask(q, k, keep):
    q = _u16(q)
    BH, N, D = q.shape
    ks, ms = [], []
    for bh in range(BH):
        a, b = block_mask_head(q, k, bh, keep)
        ks.append(a)
        ms.append(b)
    return np.stack(ks), np.stack(ms)


def sparse_rows(q_i8, q_scale, k_i8, k_scale, v, bh, tokens, kidx_head=None, keep=None,
                sm_scale=0.0, want=("decl", "exact", "amb"), nthreads=None):
    """Sparse softmax branch for tokens of head bh.

    Returns dict with 'decl', 'exact' ([R, D] float64) and 'amb' ([R])."""
    q_i8 = np.ascontiguousarray(q_i8)
    k_i8 = np.ascontiguousarray(k_i8)
    v = _u16(v)
    BH, N, D = q_i8.shape
    tok = np.ascontiguousarray(tokens, np.int64)
    R = len(tok)
    if kidx_head is None:
        keep = nkb(N)
    else:
        kidx_head = np.ascontiguousarray(kidx_head, np.int32)
        keep = kidx_head.shape[-1]
    out = {}
    od = np.empty((R, D)) if "decl" in want else None
    oe = np.empty((R, D)) if "exact" in want else None
    am = np.empty((R,)) if "amb" in want else None
    lib().orc_sparse_rows(_ptr(q_i8), _ptr(np.ascontiguousarray(q_scale, np.float32)),
                          _ptr(k_i8), _ptr(np.ascontiguousarray(k_scale, np.float32)), _ptr(v),
                          N, D, bh, _ptr(kidx_head), keep, float(sm_scale), _ptr(tok), R,
                          _ptr(od), _ptr(oe), _ptr(am), nthreads or threads())
    if od is not None:
        out["decl"] = od
    if oe is not None:
        out["exact"] = oe
    if am is not None:
        out["amb"] = am
    return out


def linear_states(k, v, bh, nthreads=None):
    k = _u16(k)
    v = _u16(v)
    BH, N, D = k.shape
    nb = nkb(N)
    h = np.empty((nb, D, D))
    z = np.empty((nb, D))
    lib().orc_linear_states(_ptr(k), _ptr(v), N, D, bh, _ptr(h), _ptr(z), nthreads or threads())
    return h, z


def linear_rows(q, h, z, bh, tokens, kidx_head=None, nthreads=None):
    q = _u16(q)
    BH, N, D = q.shape
    tok = np.ascontiguousarray(tokens, np.int64)
    out = np.empty((len(tok), D))
    keep = 0 if kidx_head is None else kidx_head.shape[-1]
    kh = None if kidx_head is None else np.ascontiguousarray(kidx_head, np.int32)
    lib().orc_linear_rows(_ptr(q), N, D, bh, _ptr(np.ascontiguousarray(h)),
                          _ptr(np.ascontiguousarray(z)), _ptr(kh), keep, _ptr(tok), len(tok),
                          _ptr(out), nthreads or threads())
    return out


def dense_rows(q, k, v, bh, tokens, sm_scale=0.0, nthreads=None):
    q, k, v = _u16(q), _u16(k), _u16(v)
    BH, N, D = q.shape
    tok = np.ascontiguousarray(tokens, np.int64)
    out = np.empty((len(tok), D))
    lib().orc_dense_rows(_ptr(q), _ptr(k), _ptr(v), N, D, bh, float(sm_scale), _ptr(tok),
                         len(tok), _ptr(out), nthreads or threads())
    return out


def sagesla_rows(q, k, v, quantized, bh, tokens, kidx_head=None, branches=3, sm_scale=0.0,
                 nthreads=None):
    """Full output (sparse + linear branch) for tokens of head bh.

    quantized = (q_i8, q_scale, k_i8, k_scale). branches: 1 sparse, 2 linear,
    3 both. Returns dict: 'decl', 'exact' (with the linear term added when
    enabled) and 'amb' (zero when the sparse branch is off)."""
    q_i8, q_scale, k_i8, k_scale = quantized
    tok = np.ascontiguousarray(tokens, np.int64)
    D = q.shape[-1]
    res = {"decl": np.zeros((len(tok), D)), "exact": np.zeros((len(tok), D)),
           "amb": np.zeros((len(tok),))}
    if branches & 1:
        s = sparse_rows(q_i8, q_scale, k_i8, k_scale, v, bh, tok, kidx_head,
                        sm_scale=sm_scale, nthreads=nthreads)
        res = s
    if branches & 2 and kidx_head is not None:
        h, z = linear_states(k, v, bh, nthreads)
        ol = linear_rows(q, h, z, bh, tok, kidx_head, nthreads)
        res["decl"] = res["decl"] + ol
        res["exact"] = res["exact"] + ol
        res["linear"] = ol
    return res


def sagesla_bwd(q, k, v, quantized, bh, dout, kidx_head=None, branches=3, sm_scale=0.0,
                nthreads=None, qrows=None, kcols=None):
    """fp64 (dq, dk, dv) [N, D] of head bh: the SageSLA backward with the
    quantizer passed straight through and the selection held fixed.
    q, k, v, dout: uint16 bf16 bits [BH, N, D]; quantized = (q_i8, q_scale,
    k_i8, k_scale) as quant_qk returns them. qrows / kcols (token indices)
    restrict the work to those rows of dq / of dk and dv; the other rows of
    the results are then unspecified."""
    q, k, v, dout = _u16(q), _u16(k), _u16(v), _u16(dout)
    q_i8, q_scale, k_i8, k_scale = (np.ascontiguousarray(x) for x in quantized)
    BH, N, D = q.shape
    keep = 0
    if kidx_head is not None:
        kidx_head = np.ascontiguousarray(kidx_head, np.int32)
        keep = kidx_head.shape[-1]
    dq = np.empty((N, D))
    dk = np.empty((N, D))
    dv = np.empty((N, D))

    def sel(rows):
        if rows is None:
            return None
        m = np.zeros(N, np.uint8)
        m[np.asarray(rows, np.int64)] = 1
        return m

    qsel, ksel = sel(qrows), sel(kcols)
    lib().orc_sagesla_bwd_sel(_ptr(q), _ptr(k), _ptr(v), _ptr(q_i8),
                              _ptr(np.ascontiguousarray(q_scale, np.float32)), _ptr(k_i8),
                              _ptr(np.ascontiguousarray(k_scale, np.float32)), N, D, bh,
                              _ptr(kidx_head), keep, int(branches), float(sm_scale), _ptr(dout),
                              _ptr(qsel), _ptr(ksel), _ptr(dq), _ptr(dk), _ptr(dv),
                              nthreads or threads())
    return dq, dk, dv


def sagesla_loss(qh, kh, vv, ql, kl, dout, kidx_head=None, branches=3, sm=None):
    """sum(dout * O) of the forward on continuous fp64 inputs [N, D] (one head)."""
    arrs = [np.ascontiguousarray(x, np.float64) for x in (qh, kh, vv, ql, kl, dout)]
    N, D = arrs[0].shape
    keep = 0
    if kidx_head is not None:
        kidx_head = np.ascontiguousarray(kidx_head, np.int32)
        keep = kidx_head.shape[-1]
    if sm is None:
        sm = float(np.float32(1.0 / np.sqrt(D)))
    return float(lib().orc_sagesla_loss(_ptr(arrs[0]), _ptr(arrs[1]), _ptr(arrs[2]),
                                        _ptr(arrs[3]), _ptr(arrs[4]), N, D, _ptr(kidx_head),
                                        keep, int(branches), float(sm), _ptr(arrs[5])))


# ---------------------------------------------------------------------------
# W8A8 linear layer (page 5, Pillar Three): 128 x 128 block INT8 quantization
# of activations x [M][K] and weights w [N][K]; y = x . w^T.

W8_BLK = 128


def w8a8_quant(x, nthreads=None):
    """(q int8 [rows][cols], scale fp32 [ceil(rows/128)][cols/128]) of a bf16 matrix."""
    x = _u16(x)
    rows, cols = x.shape
    assert cols % W8_BLK == 0
    q = np.empty((rows, cols), np.int8)
    sc = np.empty(((rows + W8_BLK - 1) // W8_BLK, cols // W8_BLK), np.float32)
    lib().orc_w8a8_quant(_ptr(x), rows, cols, _ptr(q), _ptr(sc), nthreads or threads())
    return q, sc


def w8a8_gemm(xq, sx, wq, sw, rows=None, nthreads=None, bias=None):
    """fp32 y [len(rows)][N] (all rows when rows is None) of the quantized
    product, plus the fp32 bias [N] when given."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    sx = np.ascontiguousarray(sx, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and K % W8_BLK == 0 and N % W8_BLK == 0
    rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    y = np.empty((len(rows), N), np.float32)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.shape == (N,)
    lib().orc_w8a8_gemm(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(bias), M, N, K, _ptr(rows),
                        len(rows), _ptr(y), nthreads or threads())
    return y


def w8a8_gemm_f64(xq, sx, wq, sw, rows=None, nthreads=None, bias=None):
    """(y, yabs) fp64 [len(rows)][N]: the quantized product dequantized in
    fp64, and the sum of its terms' magnitudes."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    sx = np.ascontiguousarray(sx, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    y = np.empty((len(rows), N))
    ya = np.empty((len(rows), N))
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
    lib().orc_w8a8_gemm_f64(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(bias), M, N, K, _ptr(rows),
                            len(rows), _ptr(y), _ptr(ya), nthreads or threads())
    return y, ya
