"""The one-call step (sage_sla_fwd) against the three staged calls and the
oracle. The step gets the K-mean partials and the pooled key means from the
V-layout / linear-states pass instead of a pass of its own, so every output it
writes must equal, bit for bit, what sage_quant_qk (with a pool),
sla_block_mask (from that pool) and sage_sla_attn_fwd write; the staged calls
are checked against the oracle elsewhere, and one ragged case here checks the
step against the oracle directly."""
import numpy as np
import pytest
import torch

import bit_sparse_attention_amd as ssa
from bit_sparse_attention_amd.workloads import make_qkv
from gpu_common import bits, check_attn, flat, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _staged(qd, kd, vd, topk, branches, want_mask):
    N = qd.shape[2]
    pool = None if topk is None else ssa.new_pool(qd)
    q_i8, q_scale, k_i8, k_scale, k_mean = ssa.sage_quant_qk(qd, kd, pool)
    kidx = mask = None
    keep = ssa.num_k_blocks(N)
    if topk is not None:
        keep = ssa.keep_blocks(N, topk)
        r = ssa.sla_block_mask(qd, kd, keep, return_mask=want_mask, pool=pool)
        kidx, mask = r if want_mask else (r, None)
    out, out32 = ssa.sage_sla_attn_fwd(qd, kd, vd, q_i8, q_scale, k_i8, k_scale, kidx, keep,
                                       branches, 0.0, return_f32=True)
    return dict(q_i8=q_i8, q_scale=q_scale, k_i8=k_i8, k_scale=k_scale, k_mean=k_mean,
                kidx=kidx, mask=mask, out=out, out32=out32)


# (B, H, N, topk, linear): ragged query and key tails, a single token, one key
# block, more than one group of 16 key blocks with a ragged last group, dense,
# and a keep fraction that keeps every block
CASES = [(1, 1, 1, None, False), (1, 1, 64, 0.5, True), (1, 1, 129, 0.5, True),
         (1, 2, 1000, 0.25, True), (2, 1, 3000, 0.2, False), (1, 1, 4100, 0.1, True),
         (1, 3, 2100, None, False), (1, 1, 1500, 1.0, True), (1, 1, 17000, 0.15, True)]


@pytest.mark.parametrize("B,H,N,topk,linear", CASES)
def test_step_equals_staged_calls(B, H, N, topk, linear):
    q, k, v = make_qkv(B, H, N, 128, seed=N + 11 * H + (3 if linear else 0))
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    branches = ssa.SPARSE | (ssa.LINEAR if (linear and topk is not None) else 0)
    say(f"[step] B{B}H{H}N{N} topk={topk} branches={branches}")
    want_mask = topk is not None
    ref = _staged(qd, kd, vd, topk, branches, want_mask)
    out, out32, mask, got = ssa.sage_sla_fwd(qd, kd, vd, topk, linear=linear, return_f32=True,
                                             return_mask=True, return_all=True)
    torch.cuda.synchronize()
    got = dict(got, out=out, out32=out32, mask=mask)
    for name, want in ref.items():
        if want is None:
            assert got.get(name) is None, name
            continue
        assert torch.equal(got[name].view(torch.uint8), want.view(torch.uint8)), name


def test_step_parity_with_oracle(orc):
    B, H, N = 1, 2, 2500  # 20 query blocks (last 68 tokens), 40 key blocks (last 4)
    q, k, v = make_qkv(B, H, N, 128, seed=29)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    out, out32, got = ssa.sage_sla_fwd(qd, kd, vd, 0.2, return_f32=True, return_all=True)
    torch.cuda.synchronize()
    qb, kb, vb = bits(q), bits(k), bits(v)
    oqi, oqs, oki, oks, omu = orc.quant_qk(qb, kb)
    assert np.array_equal(flat(got["k_mean"]).view(np.uint32), omu.view(np.uint32))
    assert np.array_equal(flat(got["q_scale"]).view(np.uint32), oqs.view(np.uint32))
    assert np.array_equal(flat(got["k_scale"]).view(np.uint32), oks.view(np.uint32))
    assert np.array_equal(flat(got["q_i8"]), oqi)
    assert np.array_equal(flat(got["k_i8"]), oki)
    keep = ssa.keep_blocks(N, 0.2)
    kidx = flat(got["kidx"])
    nqb = ssa.num_q_blocks(N)
    quant = (oqi, oqs, oki, oks)
    g32, g16 = flat(out32), flat(out.float())
    for bh in range(B * H):
        okidx, _ = orc.block_mask_head(qb, kb, bh, keep, np.arange(nqb))
        assert np.array_equal(kidx[bh], okidx), bh
        ref = orc.sagesla_rows(qb, kb, vb, quant, bh, np.arange(N), okidx, branches=3)
        rel, mx, _ = check_attn(g32[bh], g16[bh], ref, f"step bh={bh}")
        say(f"    bh={bh} rel-L2={rel:.2e} max={mx:.2e}")


def test_plan_fused_and_staged_agree():
    B, H, N = 1, 2, 3000
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, N, 128, seed=5))
    a = ssa.SageSLAPlan(B, H, N, 0.25, device=DEV, want_f32=True).bind(q, k, v)
    b = ssa.SageSLAPlan(B, H, N, 0.25, device=DEV, want_f32=True, fused=False).bind(q, k, v)
    a.run()
    b.run()
    torch.cuda.synchronize()
    for name in ("q_i8", "k_i8", "q_scale", "k_scale", "k_mean", "kidx", "out", "out32"):
        assert torch.equal(getattr(a, name).view(torch.uint8),
                           getattr(b, name).view(torch.uint8)), name
