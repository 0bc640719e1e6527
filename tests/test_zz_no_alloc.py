"""The allocation-free quantization call (sage_quant_qk_noalloc) against
sage_quant_qk with a caller workspace: every output bit for bit, on two calls
in a row whose second input is smaller (the fixed scratch keeps the first
call's partials, which the second must not read), each with and without the
pooled-means buffer. Called through the C ABI."""
import ctypes as C

import numpy as np
import pytest
import torch

import bit_sparse_attention_amd as ssa
from bit_sparse_attention_amd.workloads import make_qkv
from gpu_common import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _outputs(B, H, N):
    e = dict(device=DEV)
    return {
        "q_i8": torch.full((B, H, N, 128), 99, dtype=torch.int8, **e),
        "q_scale": torch.full((B, H, ssa.num_q_blocks(N)), -1.0, dtype=torch.float32, **e),
        "k_i8": torch.full((B, H, N, 128), 99, dtype=torch.int8, **e),
        "k_scale": torch.full((B, H, ssa.num_k_blocks(N)), -1.0, dtype=torch.float32, **e),
        "k_mean": torch.full((B, H, 128), -1.0, dtype=torch.float32, **e),
    }


def _call_noalloc(q, k, outs, pool):
    L = ssa._load()
    B, H, N, D = q.shape
    p = lambda t: None if t is None else C.c_void_p(t.data_ptr())  # noqa: E731
    st = L.sage_quant_qk_noalloc(p(q), p(k), ssa.Shape(B, H, N, D), p(outs["q_i8"]),
                                 p(outs["q_scale"]), p(outs["k_i8"]), p(outs["k_scale"]),
                                 p(outs["k_mean"]), p(pool),
                                 C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.ssa_last_error().decode()


@pytest.mark.parametrize("with_pool", [False, True])
def test_noalloc_quant_matches_workspace_call(with_pool):
    for B, H, N, seed in ((1, 3, 4100, 21), (1, 2, 1000, 22)):  # the second input is smaller
        say(f"[noalloc] B={B} H={H} N={N} pool={with_pool}")
        q, k, _ = make_qkv(B, H, N, 128, seed=seed, spikes=True)
        qd, kd = q.to(DEV), k.to(DEV)
        pool_a = ssa.new_pool(qd) if with_pool else None
        ref = ssa.sage_quant_qk(qd, kd, pool_a)
        outs = _outputs(B, H, N)
        pool_b = ssa.new_pool(qd).fill_(7) if with_pool else None
        _call_noalloc(qd, kd, outs, pool_b)
        torch.cuda.synchronize()
        for name, want in zip(("q_i8", "q_scale", "k_i8", "k_scale", "k_mean"), ref):
            assert torch.equal(outs[name].view(torch.uint8), want.view(torch.uint8)), name
        if with_pool:
            # the defined parts of the pool: qbar [BH][Nqb][128] fp32 at 0, then
            # (256-byte aligned) kbar^T [BH][128][ldk] fp32, columns below Nkb
            nqb, nkb = ssa.num_q_blocks(N), ssa.num_k_blocks(N)
            ldk = (nkb + 15) // 16 * 16
            nq = B * H * nqb * 128
            off = (nq * 4 + 255) // 256 * 256 // 4
            fa, fb = pool_a.view(torch.float32), pool_b.view(torch.float32)
            assert torch.equal(fa[:nq].view(torch.int32), fb[:nq].view(torch.int32)), "qbar"
            ka = fa[off:off + B * H * 128 * ldk].view(B * H * 128, ldk)[:, :nkb]
            kb_ = fb[off:off + B * H * 128 * ldk].view(B * H * 128, ldk)[:, :nkb]
            assert torch.equal(ka.contiguous().view(torch.int32), kb_.contiguous().view(torch.int32)), "kbar"


def test_noalloc_rejects_more_than_its_scratch():
    # B*H*Nkb above 65536 is refused before anything is enqueued
    L = ssa._load()
    q = torch.zeros(16, dtype=torch.uint8, device=DEV)
    p = C.c_void_p(q.data_ptr())
    N = 64 * 1025  # 1025 key blocks
    st = L.sage_quant_qk_noalloc(p, p, ssa.Shape(1, 64, N, 128), p, p, p, p, p, None, None)
    assert st == 2 and b"scratch" in L.ssa_last_error()
    np.testing.assert_equal(q.cpu().numpy(), np.zeros(16, np.uint8))
