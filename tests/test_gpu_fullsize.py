"""GPU parity at the full workload sizes, in the launch configuration the bench
times (SageSLAPlan.run: the one-call step on one stream), and the staged calls
against it.

Every reference is built from the oracle's own intermediates, each first
checked equal to the GPU's: the quantized tensors, scales and K mean of every
head, and the block selection of every query block of the first and last
head. Attention outputs of those two heads are then compared row by row:
every row where the oracle finishes in seconds (the sparse workloads up to
75600 tokens), 8 rows of every query block for the dense 32760-token one, and
at 269280 tokens the sparse branch (a separate sparse-only call on the same
buffers) at the first and last token of every query block, plus the whole
output on sampled query blocks."""
import numpy as np
import pytest
import torch

import bit_sparse_attention_amd as ssa
from bit_sparse_attention_amd.workloads import WORKLOADS, make_workload
from gpu_common import bits, check_attn, flat, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check_rows(orc, name, bh, toks, g32, g16, qb, kb, vb, quant, okidx_h, branches):
    ref = orc.sagesla_rows(qb, kb, vb, quant, bh, toks, okidx_h, branches=branches)
    rel, mx, rel_ex = check_attn(g32[bh][toks], g16[bh][toks], ref,
                                 f"{name} bh={bh} branches={branches}")
    flips = int((ref["amb"] > 0).sum())
    say(f"    bh={bh} branches={branches} rows={len(toks)} rel-L2={rel:.2e} max={mx:.2e} "
        f"vs-exact={rel_ex:.2e} rows-with-flip-bound={flips}")


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity(orc, name):
    w = WORKLOADS[name]
    say(f"[full] {name}: generating B={w.B} H={w.H} N={w.N}")
    q, k, v = make_workload(w)
    plan = ssa.SageSLAPlan(w.B, w.H, w.N, w.topk, linear=True, device=DEV, want_f32=True)
    plan.bind(*(t.to(DEV) for t in (q, k, v)))
    plan.run()
    torch.cuda.synchronize()
    say(f"[full] {name}: GPU done, checking quantization of every head")
    BH, N = w.B * w.H, w.N
    qb, kb, vb = bits(q), bits(k), bits(v)
    oqi, oqs, oki, oks, omu = orc.quant_qk(qb, kb)
    assert np.array_equal(flat(plan.k_mean).view(np.uint32), omu.view(np.uint32))
    assert np.array_equal(flat(plan.q_scale).view(np.uint32), oqs.view(np.uint32))
    assert np.array_equal(flat(plan.k_scale).view(np.uint32), oks.view(np.uint32))
    assert np.array_equal(flat(plan.q_i8), oqi)
    assert np.array_equal(flat(plan.k_i8), oki)
    quant = (oqi, oqs, oki, oks)

    nqb, nkb = plan.nqb, plan.nkb
    heads = sorted({0, BH - 1})
    okidx = {bh: None for bh in heads}
    if not plan.dense:
        say(f"[full] {name}: every selection row of heads {heads} (keep={plan.keep})")
        kidx_np = flat(plan.kidx)
        for bh in heads:
            okidx[bh], _ = orc.block_mask_head(qb, kb, bh, plan.keep)
            assert np.array_equal(kidx_np[bh], okidx[bh]), bh

    say(f"[full] {name}: sampled int32 tiles")
    trip = [(bh, i, j) for bh in heads for i, j in ((0, 0), (nqb - 1, nkb - 1), (0, nkb - 1),
                                                    (nqb - 1, 0), (nqb // 2, nkb // 3))]
    tiles = torch.tensor(trip, dtype=torch.int32, device=DEV)
    out = ssa.sage_qk_int32_tiles(plan.q_i8, plan.k_i8, tiles).cpu().numpy()
    for t, (bh, i, j) in enumerate(trip):
        assert np.array_equal(out[t], orc.qk_tile(oqi, oki, bh, i, j)), (bh, i, j)

    g32, g16 = flat(plan.out32), flat(plan.out.float())
    rng = np.random.default_rng(0)
    starts = 128 * np.arange(nqb)
    ends = np.minimum(starts + 127, N - 1)
    if w.N <= 80000 and (not plan.dense or w.N <= 4096):
        say(f"[full] {name}: every attention row of heads {heads}")
        for bh in heads:
            _check_rows(orc, name, bh, np.arange(N), g32, g16, qb, kb, vb, quant, okidx[bh],
                        plan.branches)
    elif plan.dense:
        say(f"[full] {name}: 8 rows of every query block of heads {heads}")
        for bh in heads:
            pick = [starts, ends] + [np.minimum(starts + rng.integers(0, 128, nqb), N - 1)
                                     for _ in range(6)]
            toks = np.unique(np.concatenate(pick))
            _check_rows(orc, name, bh, toks, g32, g16, qb, kb, vb, quant, None, plan.branches)
    else:
        # the sparse branch alone, from the same quantized tensors and selection
        say(f"[full] {name}: sparse branch at the first and last token of every query block")
        s16, s32 = ssa.sage_sla_attn_fwd(plan.q, plan.k, plan.v, plan.q_i8, plan.q_scale,
                                         plan.k_i8, plan.k_scale, plan.kidx, plan.keep,
                                         ssa.SPARSE, plan.sm_scale, return_f32=True)
        torch.cuda.synchronize()
        sg32, sg16 = flat(s32), flat(s16.float())
        del s16, s32
        toks = np.unique(np.concatenate([starts, ends]))
        for bh in heads:
            _check_rows(orc, name, bh, toks, sg32, sg16, qb, kb, vb, quant, okidx[bh], ssa.SPARSE)
        say(f"[full] {name}: whole output on sampled query blocks")
        for bh in heads:
            blocks = np.unique(np.concatenate([[0, nqb - 1], rng.integers(0, nqb, 10)]))
            toks = np.unique(np.concatenate([starts[blocks], ends[blocks],
                                             np.minimum(starts[blocks] + 64, N - 1)]))
            _check_rows(orc, name, bh, toks, g32, g16, qb, kb, vb, quant, okidx[bh],
                        plan.branches)

    # the staged calls write the same buffers bit for bit
    say(f"[full] {name}: staged calls against the one-call step")
    names = ("q_i8", "k_i8", "q_scale", "k_scale", "k_mean", "kidx", "out", "out32")
    ref = {n: getattr(plan, n).clone() for n in names if getattr(plan, n) is not None}
    plan.run_staged()
    torch.cuda.synchronize()
    for n, want in ref.items():
        assert torch.equal(getattr(plan, n).view(torch.uint8), want.view(torch.uint8)), n
