"""Host-side checks of the C-ABI library: it loads without a GPU, exports every
function include/ssa.h declares, and rejects bad arguments before any HIP call
(so these run on a CPU-only machine)."""
import ctypes as C
import os
import re

import pytest

import bit_sparse_attention_amd as ssa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssa.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\**\s+\**([a-z_][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("sage_quant_qk", "sla_block_mask", "sage_sla_attn_fwd", "sage_sla_fwd",
              "sage_sla_attn_bwd", "sage_quant_qk_noalloc",
              "sage_qk_int32_tiles", "w8a8_quant", "w8a8_gemm",
              "ssa_workspace_bytes", "ssa_keep_blocks", "ssa_status_str", "ssa_last_error",
              "ssa_num_q_blocks", "ssa_num_k_blocks"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    L = C.CDLL(ssa.lib_path())
    for n in _declared_functions():
        assert hasattr(L, n), f"libssa.so does not export {n}"


def test_block_counts_and_keep():
    assert ssa.num_q_blocks(75600) == 591 and ssa.num_k_blocks(75600) == 1182
    assert ssa.keep_blocks(75600, 0.1) == 118
    assert ssa.keep_blocks(32760, 0.1) == 51
    assert ssa.keep_blocks(269280, 0.05) == 210
    assert ssa.keep_blocks(1024, 0.0) == 1 and ssa.keep_blocks(1024, 5.0) == 16
    assert ssa.keep_blocks(0, 0.1) == 0


def test_keep_matches_oracle(orc):
    for N in (1, 63, 64, 65, 1000, 32760, 75600, 269280):
        for topk in (0.0, 0.05, 0.1, 0.15, 0.5, 1.0):
            assert ssa.keep_blocks(N, topk) == orc.keep_blocks(N, topk)


def test_workspace_sizes():
    s = (1, 40, 75600, 128)
    assert ssa.workspace_bytes(ssa.OP_QUANT, s) >= 40 * 1182 * 128 * 4
    dense = ssa.workspace_bytes(ssa.OP_ATTN, s, 1182, ssa.SPARSE | ssa.LINEAR)
    sparse = ssa.workspace_bytes(ssa.OP_ATTN, s, 118, ssa.SPARSE)
    lin = ssa.workspace_bytes(ssa.OP_ATTN, s, 118, ssa.SPARSE | ssa.LINEAR)
    assert dense == sparse < lin  # all blocks kept: no linear states needed
    assert ssa.workspace_bytes(ssa.OP_ATTN, (1, 1, 100, 64), 1, 1) == 0  # D != 128
    assert ssa.workspace_bytes(7, s) == 0
    # the one-call step holds the attention's workspace, the pooled means and
    # the K-mean partials
    for keep, br in ((1182, 3), (118, 1), (118, 3)):
        step = ssa.workspace_bytes(ssa.OP_STEP, s, keep, br)
        assert step >= (ssa.workspace_bytes(ssa.OP_ATTN, s, keep, br) + ssa.pool_bytes(s)
                        + ssa.workspace_bytes(ssa.OP_QUANT, s))


def _L():
    return ssa._load()


def _shape(B=1, H=1, N=1000, D=128):
    return ssa.Shape(B, H, N, D)


# Fake, never dereferenced device addresses: validation must reject each call
# before it touches the GPU.
A = 1 << 40


def _p(off=0):
    return C.c_void_p(A + off)


def test_quant_rejects_bad_arguments():
    L = _L()
    GB = 1 << 30
    ok = [_p(0), _p(GB), _shape(), _p(2 * GB), _p(3 * GB), _p(4 * GB), _p(5 * GB), _p(6 * GB),
          None, _p(7 * GB), 1 << 24, None]

    def call(**kw):
        args = list(ok)
        names = ["q", "k", "s", "q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "pool", "ws", "n",
                 "st"]
        for k_, v_ in kw.items():
            args[names.index(k_)] = v_
        return L.sage_quant_qk(*args)

    assert call(q=None) == 1
    assert call(q=_p(8)) == 1  # misaligned
    assert call(s=_shape(D=64)) == 2
    assert call(s=_shape(N=0)) == 1
    assert call(s=_shape(N=(1 << 19) + 1)) == 2
    assert call(ws=None) == 3
    assert call(n=16) == 3
    assert call(ws=_p(7 * GB + 16)) == 3  # workspace misaligned
    assert call(q_i8=_p(0)) == 1  # output aliases input q
    assert call(k_mean=_p(2 * GB + 64)) == 1  # two outputs overlap
    assert b"overlap" in L.ssa_last_error()
    assert call(pool=_p(8 * GB + 16)) == 1  # pool misaligned
    assert call(pool=_p(GB)) == 1  # pool overlaps input k
    assert b"overlap" in L.ssa_last_error()


def test_mask_rejects_bad_keep():
    L = _L()
    GB = 1 << 30
    s = _shape(N=1000)  # 16 key blocks
    for keep, want in ((0, 1), (17, 1), (16, 3)):
        st = L.sla_block_mask(_p(0), _p(GB), s, keep, None, _p(2 * GB), None, None, 0, None)
        assert st == want, (keep, st)


def test_mask_with_pool_needs_no_workspace_nor_inputs():
    L = _L()
    GB = 1 << 30
    s = _shape(N=1000)
    # with a pool, q, k and the workspace are not needed; a bad keep is still caught
    assert L.sla_block_mask(None, None, s, 0, _p(GB), _p(2 * GB), None, None, 0, None) == 1
    assert L.sla_block_mask(None, None, s, 4, _p(GB + 16), _p(2 * GB), None, None, 0, None) == 1
    assert b"pool" in L.ssa_last_error()
    # kidx inside the pool
    assert L.sla_block_mask(None, None, s, 4, _p(GB), _p(GB + 256), None, None, 0, None) == 1
    assert b"overlap" in L.ssa_last_error()


def test_pool_bytes():
    L = _L()
    assert L.ssa_pool_bytes(_shape(N=75600)) > 0
    assert L.ssa_pool_bytes(_shape(N=0)) == 0


def test_attn_rejects_bad_arguments():
    L = _L()
    GB = 1 << 30
    s = _shape(N=1000)

    def call(kidx=_p(6 * GB), keep=4, branches=3, sm=0.0, out=_p(7 * GB), lse=None, ws=None, n=0):
        return L.sage_sla_attn_fwd(_p(0), _p(GB), _p(2 * GB), s, _p(3 * GB), _p(4 * GB),
                                   _p(5 * GB), _p(5 * GB + (1 << 20)), kidx, keep, branches,
                                   sm, out, None, lse, ws, n, None)

    assert call(branches=0) == 1
    assert call(branches=4) == 1
    assert call(keep=0) == 1
    assert call(kidx=None, keep=4) == 1  # dense needs keep == Nkb
    assert call(sm=float("nan")) == 1
    assert call(out=_p(2 * GB)) == 1  # out aliases v
    assert call(lse=_p(8 * GB + 2)) == 1  # lse misaligned
    assert call(lse=_p(7 * GB + 64)) == 1  # lse overlaps out
    assert call() == 3  # workspace missing
    assert b"workspace" in L.ssa_last_error()


def test_step_rejects_bad_arguments():
    L = _L()
    GB = 1 << 30
    s = _shape(N=1000)  # 16 key blocks
    names = ["q", "k", "v", "s", "keep", "branches", "sm", "q_i8", "q_scale", "k_i8", "k_scale",
             "k_mean", "kidx", "mask", "out", "out32", "lse", "ws", "n", "st"]
    ok = [_p(0), _p(GB), _p(2 * GB), s, 4, 3, 0.0, _p(3 * GB), _p(4 * GB), _p(5 * GB),
          _p(6 * GB), _p(6 * GB + (1 << 20)), _p(7 * GB), None, _p(8 * GB), None, None,
          _p(9 * GB), 1 << 30, None]

    def call(**kw):
        args = list(ok)
        for k_, v_ in kw.items():
            args[names.index(k_)] = v_
        return L.sage_sla_fwd(*args)

    assert call(branches=0) == 1
    assert call(branches=4) == 1
    assert call(keep=0) == 1
    assert call(keep=17) == 1
    assert call(kidx=None) == 1  # dense needs keep == Nkb
    assert call(kidx=None, keep=16, mask=_p(10 * GB)) == 1  # a mask needs the selection
    assert b"mask" in L.ssa_last_error()
    assert call(sm=float("inf")) == 1
    assert call(q=None) == 1
    assert call(v=_p(2 * GB + 8)) == 1  # misaligned
    assert call(k_mean=None) == 1
    assert call(s=_shape(N=1000, D=64)) == 2
    assert call(out=_p(2 * GB)) == 1  # out aliases v
    assert call(kidx=_p(5 * GB + 64)) == 1  # kidx overlaps k_i8
    assert call(mask=_p(9 * GB)) == 1  # mask inside the workspace
    assert b"overlap" in L.ssa_last_error()
    assert call(lse=_p(8 * GB)) == 1  # lse aliases out
    assert call(ws=None) == 3
    assert call(n=1 << 10) == 3
    assert call(ws=_p(9 * GB + 16)) == 3  # workspace misaligned


def test_bwd_rejects_bad_arguments():
    L = _L()
    GB = 1 << 30
    s = _shape(N=1000)  # 16 key blocks

    def call(kidx=_p(8 * GB), keep=4, branches=3, sm=0.0, dq=_p(9 * GB), ws=_p(12 * GB),
             n=1 << 34, dout=_p(7 * GB), out32=None, lse=None):
        return L.sage_sla_attn_bwd(_p(0), _p(GB), _p(2 * GB), s, _p(3 * GB), _p(4 * GB),
                                   _p(5 * GB), _p(6 * GB), kidx, keep, branches, sm, dout, out32,
                                   lse, dq, _p(10 * GB), _p(11 * GB), ws, n, None)

    assert call(branches=0) == 1 and call(branches=4) == 1
    assert call(keep=0) == 1 and call(keep=17) == 1
    assert call(kidx=None) == 1  # dense needs keep == Nkb
    assert call(sm=float("nan")) == 1
    assert call(dout=None) == 1
    assert call(dq=_p(9 * GB + 8)) == 1  # misaligned
    assert call(dq=_p(7 * GB)) == 1  # dq aliases dout
    assert b"overlap" in L.ssa_last_error()
    assert call(out32=_p(13 * GB)) == 1  # out32 without lse
    assert call(lse=_p(13 * GB)) == 1  # lse without out32
    assert call(out32=_p(13 * GB), lse=_p(9 * GB)) == 1  # lse aliases dq
    assert call(ws=None) == 3
    assert call(n=1 << 10) == 3
    s2 = _shape(N=1000)
    assert L.ssa_workspace_bytes(ssa.OP_BWD, s2, 4, 3) > L.ssa_workspace_bytes(ssa.OP_BWD, s2, 4, 1)
    assert L.ssa_workspace_bytes(ssa.OP_BWD, s2, 16, 3) == L.ssa_workspace_bytes(ssa.OP_BWD, s2, 16, 1)


def test_tiles_reject_bad_count():
    L = _L()
    GB = 1 << 30
    assert L.sage_qk_int32_tiles(_p(0), _p(GB), _shape(), _p(2 * GB), 0, _p(3 * GB), None) == 1


def test_w8a8_quant_rejects_bad_arguments():
    L = _L()
    GB = 1 << 30

    def call(x=_p(0), rows=300, cols=384, q=_p(GB), sc=_p(2 * GB)):
        return L.w8a8_quant(x, rows, cols, q, sc, None)

    assert call(rows=0) == 1
    assert call(rows=(1 << 20) + 1) == 1
    assert call(cols=100) == 1  # not a multiple of 128
    assert call(cols=0) == 1
    assert call(x=None) == 1
    assert call(x=_p(8)) == 1  # misaligned
    assert call(q=_p(GB + 4)) == 1
    assert call(sc=_p(2 * GB + 2)) == 1
    assert call(q=_p(16)) == 1  # q overlaps x
    assert b"overlap" in L.ssa_last_error()
    assert call(sc=_p(GB + 64)) == 1  # scale inside q
    assert b"overlap" in L.ssa_last_error()


def test_w8a8_gemm_rejects_bad_arguments():
    L = _L()
    GB = 1 << 30

    def call(xq=_p(0), sx=_p(GB), wq=_p(2 * GB), sw=_p(3 * GB), M=300, N=256, K=384,
             y=_p(4 * GB), y32=None, bias=None):
        return L.w8a8_gemm(xq, sx, wq, sw, bias, M, N, K, y, y32, None)

    assert call(M=0) == 1
    assert call(M=(1 << 20) + 1) == 1
    assert call(N=200) == 1 and call(K=200) == 1  # not multiples of 128
    assert call(N=0) == 1 and call(K=0) == 1
    assert call(xq=None) == 1 and call(wq=None) == 1 and call(y=None) == 1
    assert call(sx=None) == 1 and call(sw=None) == 1
    assert call(xq=_p(8)) == 1  # misaligned
    assert call(y32=_p(5 * GB + 8)) == 1
    assert call(y=_p(2 * GB + 64)) == 1  # output overlaps wq
    assert b"overlap" in L.ssa_last_error()
    assert call(y32=_p(4 * GB + 1024)) == 1  # the two outputs overlap
    assert b"overlap" in L.ssa_last_error()
    assert call(bias=_p(6 * GB + 4)) == 1  # misaligned bias
    assert call(bias=_p(4 * GB + 256)) == 1  # bias inside the output
    assert b"overlap" in L.ssa_last_error()


def test_shapes_beyond_the_launch_grids_are_rejected():
    # B*H rides on the grid's y dimension (at most 65535); the attention grid
    # has one 256-thread workgroup per head and query block (fewer than 2^24);
    # both must fail in validation, before anything is enqueued
    L = _L()
    GB = 1 << 30
    for shape, ok in (((1, 65000, 64), True), ((1, 65100, 64), False), ((1, 65536, 64), False),
                      ((2, 40000, 64), False),
                      ((1, 4095, 1 << 19), True), ((1, 4096, 1 << 19), False),
                      ((64, 64, 1 << 19), False)):
        s = _shape(*shape)
        want_ws = L.ssa_workspace_bytes(ssa.OP_QUANT, s, 0, 0)
        assert (want_ws > 0) == ok, shape
        st = L.sage_quant_qk(_p(0), _p(16 * GB), s, _p(32 * GB), _p(48 * GB), _p(64 * GB),
                             _p(80 * GB), _p(96 * GB), None, _p(112 * GB), 1 << 40, None)
        if not ok:
            assert st == 2, (shape, st)
            assert b"exceeds" in L.ssa_last_error() or b"too large" in L.ssa_last_error()
        st = L.sage_sla_attn_fwd(_p(0), _p(16 * GB), _p(32 * GB), s, _p(48 * GB), _p(64 * GB),
                                 _p(80 * GB), _p(96 * GB), None, ssa.num_k_blocks(shape[2]),
                                 ssa.SPARSE, 0.0, _p(112 * GB), None, None, _p(128 * GB), 0, None)
        if not ok:
            assert st == 2, (shape, st)


def test_w8a8_gemm_rejects_a_grid_too_large():
    # ceil(M/256) * N/128 workgroups of 1024 threads: at most 2^22 per launch
    L = _L()
    GB = 1 << 30
    M = N = 1 << 20
    st = L.w8a8_gemm(_p(0), _p(GB), _p(2 * GB), _p(3 * GB), None, M, N, 128, _p(4 * GB), None,
                     None)
    assert st == 2 and b"workgroups" in L.ssa_last_error()


def test_status_strings():
    L = _L()
    for st in range(5):
        assert L.ssa_status_str(st)
    assert L.ssa_status_str(99) == b"unknown status"


def test_python_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        ssa.sage_quant_qk(q, q)
