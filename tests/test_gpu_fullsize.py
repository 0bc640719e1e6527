"""GPU parity at the full workload sizes, in the launch configuration the bench
times (SageSLAPlan.run: the one-call step on one stream), and the staged calls
against it.

Integer outputs are compared whole where the oracle is cheap (quantized
tensors, scales, K mean) and on samples otherwise (block-mask rows, int32
tiles including every tail position); attention outputs on sampled tokens of
the first and last head, which the oracle computes one row at a time."""
import numpy as np
import pytest
import torch

import bit_sparse_attention_amd as ssa
from bit_sparse_attention_amd.workloads import WORKLOADS, make_workload
from gpu_common import bits, check_attn, flat, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity(orc, name):
    w = WORKLOADS[name]
    say(f"[full] {name}: generating B={w.B} H={w.H} N={w.N}")
    q, k, v = make_workload(w)
    plan = ssa.SageSLAPlan(w.B, w.H, w.N, w.topk, linear=True, device=DEV, want_f32=True)
    plan.bind(*(t.to(DEV) for t in (q, k, v)))
    plan.run()
    torch.cuda.synchronize()
    say(f"[full] {name}: GPU done, checking quantization")
    BH, N = w.B * w.H, w.N
    qb, kb, vb = bits(q), bits(k), bits(v)
    oqi, oqs, oki, oks, omu = orc.quant_qk(qb, kb)
    assert np.array_equal(flat(plan.k_mean).view(np.uint32), omu.view(np.uint32))
    assert np.array_equal(flat(plan.q_scale).view(np.uint32), oqs.view(np.uint32))
    assert np.array_equal(flat(plan.k_scale).view(np.uint32), oks.view(np.uint32))
    assert np.array_equal(flat(plan.q_i8), oqi)
    assert np.array_equal(flat(plan.k_i8), oki)

    nqb, nkb = plan.nqb, plan.nkb
    heads = sorted({0, BH - 1})
    rng = np.random.default_rng(0)
    kidx_np = None if plan.dense else flat(plan.kidx)
    if not plan.dense:
        say(f"[full] {name}: checking sampled mask rows (keep={plan.keep})")
        for bh in heads:
            rows = np.unique(np.concatenate([[0, nqb - 1], rng.integers(0, nqb, 6)]))
            okidx, _ = orc.block_mask_head(qb, kb, bh, plan.keep, rows)
            assert np.array_equal(kidx_np[bh][rows], okidx), (bh, rows)

    say(f"[full] {name}: checking sampled int32 tiles")
    trip = [(bh, i, j) for bh in heads for i, j in ((0, 0), (nqb - 1, nkb - 1), (0, nkb - 1),
                                                    (nqb - 1, 0), (nqb // 2, nkb // 3))]
    tiles = torch.tensor(trip, dtype=torch.int32, device=DEV)
    out = ssa.sage_qk_int32_tiles(plan.q_i8, plan.k_i8, tiles).cpu().numpy()
    for t, (bh, i, j) in enumerate(trip):
        assert np.array_equal(out[t], orc.qk_tile(oqi, oki, bh, i, j)), (bh, i, j)

    say(f"[full] {name}: checking sampled attention rows")
    g32, g16 = flat(plan.out32), flat(plan.out.float())
    quant = (oqi, oqs, oki, oks)
    for bh in heads:
        toks = np.unique(np.concatenate([[0, 1, 127, 128, N - 1, N - 2, (nqb - 1) * 128],
                                         rng.integers(0, N, 17)]))
        ref = orc.sagesla_rows(qb, kb, vb, quant, bh, toks,
                               None if kidx_np is None else kidx_np[bh],
                               branches=plan.branches)
        rel, mx, rel_ex = check_attn(g32[bh][toks], g16[bh][toks], ref, f"{name} bh={bh}")
        flips = int((ref["amb"] > 0).sum())
        say(f"    bh={bh} rows={len(toks)} rel-L2={rel:.2e} max={mx:.2e} "
            f"vs-exact={rel_ex:.2e} rows-with-flip-bound={flips}")

    # the staged calls write the same buffers bit for bit
    say(f"[full] {name}: staged calls against the one-call step")
    names = ("q_i8", "k_i8", "q_scale", "k_scale", "k_mean", "kidx", "out", "out32")
    ref = {n: getattr(plan, n).clone() for n in names if getattr(plan, n) is not None}
    plan.run_staged()
    torch.cuda.synchronize()
    for n, want in ref.items():
        assert torch.equal(getattr(plan, n).view(torch.uint8), want.view(torch.uint8)), n
