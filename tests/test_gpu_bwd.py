"""GPU parity of the SageSLA backward (sage_sla_attn_bwd, through the C ABI)
against the oracle's fp64 gradients, on the dense 1024-token case, on ragged
sparse shapes with every branch mix, and at the benchmarked size (40 heads x
75600 tokens, as bench.py --bwd runs it) on sampled rows.

Every reference is built from the oracle's own quantized tensors and block
selection, each first asserted equal to the GPU's.

Tolerance, from the arithmetic: each gradient element is a sum of products in
which one factor (P for dV, dS for dQ and dK) is rounded to bf16 before the
matrix-core product, a relative error uniform in +-2^-9 (RMS 2^-9/sqrt(3) =
1.13e-3) that is independent across the summed terms, so each gradient's
relative L2 error is about 1.1e-3, plus the forward statistics' own bf16
rounding (its row sums and D come from the rounded P), of the same order:
1.6e-3 to 1.8e-3 measured. The linear branch runs in fp32 with its state
products carried on two bf16 stacks (~16 bits), 1e-7 to 1e-5. Gate: relative
L2 <= 3e-3 per gradient tensor, and every element within 1e-2 of the tensor's
largest magnitude."""
import numpy as np
import pytest
import torch

import bit_sparse_attention_amd as ssa
from bit_sparse_attention_amd.workloads import BENCH_WORKLOAD, WORKLOADS, make_qkv, make_workload
from gpu_common import bits, flat, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REL_L2 = 3e-3
MAX_FRAC = 1e-2


def _dout(B, H, N, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(B, H, N, 128, generator=g).to(torch.bfloat16)


def _check_grads(got, want, what):
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        err = np.abs(g - w)
        scale = max(np.abs(w).max(), 1e-30)
        rel = np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-30)
        say(f"    {what} {name}: rel-L2={rel:.2e} max-err/max={err.max() / scale:.2e}")
        assert np.isfinite(g).all(), f"{what} {name}: non-finite"
        assert rel <= REL_L2, f"{what} {name}: rel-L2 {rel:.3e}"
        assert err.max() <= MAX_FRAC * scale, f"{what} {name}: max error {err.max():.3e}"


BWD_CASES = [(1, 1, 1024, None, 1),      # the dense 1024-token workload
             (1, 2, 1000, 0.25, 1), (1, 2, 1000, 0.25, 2), (1, 2, 1000, 0.25, 3),
             (2, 1, 3000, 0.2, 3), (1, 1, 200, 0.5, 3), (1, 1, 2000, 0.8, 3),
             (1, 1, 64, None, 1), (1, 1, 130, 0.5, 2)]


@pytest.mark.parametrize("saved", [False, True], ids=["recomputed-stats", "forward-stats"])
@pytest.mark.parametrize("B,H,N,topk,branches", BWD_CASES)
def test_bwd_parity(orc, B, H, N, topk, branches, saved):
    # saved: the forward's fp32 output and row statistics are handed over;
    # otherwise the backward recomputes them
    q, k, v = make_qkv(B, H, N, 128, seed=3 * N + branches)
    dout = _dout(B, H, N, seed=N + 17)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    label = f"B{B}H{H}N{N} topk={topk} branches={branches} saved={saved}"
    say(f"[bwd] {label}")
    q_i8, q_scale, k_i8, k_scale, _ = ssa.sage_quant_qk(qd, kd)
    if topk is None:
        kidx, keep = None, ssa.num_k_blocks(N)
    else:
        keep = ssa.keep_blocks(N, topk)
        kidx = ssa.sla_block_mask(qd, kd, keep)
    fwd = {}
    if saved:
        _, fwd["out32"], fwd["lse"] = ssa.sage_sla_attn_fwd(
            qd, kd, vd, q_i8, q_scale, k_i8, k_scale, kidx, keep, branches, return_f32=True,
            return_lse=True)
    dq, dk, dv = ssa.sage_sla_attn_bwd(qd, kd, vd, q_i8, q_scale, k_i8, k_scale, gd, kidx, keep,
                                       branches, **fwd)
    torch.cuda.synchronize()
    qb, kb, vb, gb = bits(q), bits(k), bits(v), bits(dout)
    oqi, oqs, oki, oks, _ = orc.quant_qk(qb, kb)
    assert np.array_equal(flat(q_i8), oqi) and np.array_equal(flat(k_i8), oki)
    assert np.array_equal(flat(q_scale).view(np.uint32), oqs.view(np.uint32))
    assert np.array_equal(flat(k_scale).view(np.uint32), oks.view(np.uint32))
    okidx = None
    if kidx is not None:
        okidx, _ = orc.block_mask(qb, kb, keep)
        assert np.array_equal(flat(kidx), okidx)
    got = [flat(t) for t in (dq, dk, dv)]
    for bh in range(B * H):
        want = orc.sagesla_bwd(qb, kb, vb, (oqi, oqs, oki, oks), bh, gb,
                               None if okidx is None else okidx[bh], branches)
        _check_grads([g[bh] for g in got], want, f"{label} bh={bh}")


def test_forward_lse_is_the_statistics_the_backward_recomputes():
    # the forward's lse and the backward's own statistics pass are the same
    # expression over the same sums: handing lse over changes nothing in P,
    # so the sparse-only gradients differ from the recomputed ones only
    # through D (dO . out from the fp32 output instead of dO . o_s in the
    # statistics pass), within fp32 rounding
    B, H, N = 1, 2, 1500
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, N, 128, seed=4))
    gd = _dout(B, H, N, seed=5).to(DEV)
    qq = ssa.sage_quant_qk(q, k)[:4]
    keep = ssa.keep_blocks(N, 0.3)
    kidx = ssa.sla_block_mask(q, k, keep)
    _, out32, lse = ssa.sage_sla_attn_fwd(q, k, v, *qq, kidx, keep, ssa.SPARSE, return_f32=True,
                                          return_lse=True)
    a = ssa.sage_sla_attn_bwd(q, k, v, *qq, gd, kidx, keep, ssa.SPARSE)
    b = ssa.sage_sla_attn_bwd(q, k, v, *qq, gd, kidx, keep, ssa.SPARSE, out32=out32, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()
    for x, y in zip(a, b):
        rel = ((x - y).norm() / y.norm()).item()
        assert rel < 1e-5, rel


def test_bwd_repeat_runs_bit_identical():
    B, H, N = 1, 2, 1500
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, N, 128, seed=2))
    gd = _dout(B, H, N, seed=9).to(DEV)
    qq = ssa.sage_quant_qk(q, k)[:4]
    keep = ssa.keep_blocks(N, 0.3)
    kidx = ssa.sla_block_mask(q, k, keep)
    runs = [ssa.sage_sla_attn_bwd(q, k, v, *qq, gd, kidx, keep, 3) for _ in range(2)]
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_bwd_at_the_benchmarked_size(orc):
    # the call bench.py --bwd times: the plan's one-call forward, then the
    # backward on its quantized tensors and selection with the same seeded dO.
    # Heads 0 and H-1: the oracle's quantization and selection checked equal
    # to the GPU's, then dq at the first and last token of every query block
    # and dk, dv at every key of the first, a middle and the ragged last key
    # block, each computed by the oracle one row at a time.
    w = WORKLOADS[BENCH_WORKLOAD]
    say(f"[bwd-full] {w.name}: generating B={w.B} H={w.H} N={w.N}")
    q, k, v = make_workload(w)
    plan = ssa.SageSLAPlan(w.B, w.H, w.N, w.topk, linear=True, device=DEV, want_f32=True,
                           want_lse=True)
    plan.bind(*(t.to(DEV) for t in (q, k, v)))
    plan.run()
    g = torch.Generator().manual_seed(1)
    dout = torch.randn(w.B, w.H, w.N, 128, generator=g).to(torch.bfloat16)
    grads = ssa.sage_sla_attn_bwd(plan.q, plan.k, plan.v, plan.q_i8, plan.q_scale, plan.k_i8,
                                  plan.k_scale, dout.to(DEV), plan.kidx, plan.keep, plan.branches,
                                  plan.sm_scale, out32=plan.out32, lse=plan.lse)
    BH, N, nqb, nkb = w.B * w.H, w.N, plan.nqb, plan.nkb
    heads = [0, BH - 1]
    sel = torch.tensor(heads, device=DEV)
    got = [t.reshape(BH, N, 128).index_select(0, sel).cpu().numpy() for t in grads]
    gq8, gk8 = (t.reshape(BH, N, 128).index_select(0, sel).cpu().numpy()
                for t in (plan.q_i8, plan.k_i8))
    gqs, gks = (t.reshape(BH, -1)[heads].cpu().numpy() for t in (plan.q_scale, plan.k_scale))
    gkidx = plan.kidx.reshape(BH, nqb, plan.keep)[heads].cpu().numpy()
    del grads
    say(f"[bwd-full] {w.name}: GPU done; oracle quantization and selection of heads {heads}")
    qb, kb, vb, gb = (bits(t).reshape(BH, N, 128)[heads] for t in (q, k, v, dout))
    oqi, oqs, oki, oks, _ = orc.quant_qk(qb, kb)
    assert np.array_equal(gq8, oqi) and np.array_equal(gk8, oki)
    assert np.array_equal(gqs.view(np.uint32), oqs.view(np.uint32))
    assert np.array_equal(gks.view(np.uint32), oks.view(np.uint32))
    starts = 128 * np.arange(nqb)
    qrows = np.unique(np.concatenate([starts, np.minimum(starts + 127, N - 1)]))
    kcols = np.concatenate([np.arange(64 * j, min(64 * j + 64, N)) for j in (0, nkb // 2, nkb - 1)])
    for x, bh in enumerate(heads):
        okidx, _ = orc.block_mask_head(qb, kb, x, plan.keep)
        assert np.array_equal(gkidx[x], okidx), bh
        say(f"[bwd-full] {w.name}: oracle backward of head {bh} on {len(qrows)} query rows "
            f"and {len(kcols)} keys")
        want = orc.sagesla_bwd(qb, kb, vb, (oqi, oqs, oki, oks), x, gb, okidx, plan.branches,
                               plan.sm_scale, qrows=qrows, kcols=kcols)
        _check_grads([got[0][x][qrows], got[1][x][kcols], got[2][x][kcols]],
                     [want[0][qrows], want[1][kcols], want[2][kcols]], f"{w.name} bh={bh}")
