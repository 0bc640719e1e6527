"""The largest sequence the library takes (N = 2^19 tokens) with enough heads
that every bf16 tensor holds more than 2^31 elements, so every offset into Q,
K, V, the quantized tensors, the outputs and the workspaces needs 64 bits.
The last head (the largest offsets) is checked against the oracle: quantized
tensors, scales and K mean whole; the block-mask rows of every query block
that holds a checked token (the reference uses the oracle's rows), int32 tiles
and attention rows. The staged calls must agree with the one-call step."""
import numpy as np
import pytest
import torch

import bit_sparse_attention_amd as ssa
from bit_sparse_attention_amd.workloads import make_qkv
from gpu_common import bits, check_attn, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_max_sequence_beyond_32bit_offsets(orc):
    B, H, N, topk = 1, 34, 1 << 19, 0.05
    assert B * H * N * 128 > 2**31
    say(f"[max] generating B={B} H={H} N={N}")
    q, k, v = make_qkv(B, H, N, 128, seed=3)
    plan = ssa.SageSLAPlan(B, H, N, topk, linear=True, device=DEV, want_f32=True)
    plan.bind(*(t.to(DEV) for t in (q, k, v)))
    say(f"[max] one-call step, keep={plan.keep} of {plan.nkb} key blocks")
    plan.run()
    torch.cuda.synchronize()

    bh = H - 1
    qh, kh, vh = (bits(t)[bh:bh + 1] for t in (q, k, v))
    say(f"[max] oracle quantization of head {bh}")
    oqi, oqs, oki, oks, omu = orc.quant_qk(qh, kh)
    assert np.array_equal(plan.k_mean[0, bh].cpu().numpy().view(np.uint32), omu[0].view(np.uint32))
    assert np.array_equal(plan.q_scale[0, bh].cpu().numpy().view(np.uint32), oqs[0].view(np.uint32))
    assert np.array_equal(plan.k_scale[0, bh].cpu().numpy().view(np.uint32), oks[0].view(np.uint32))
    assert np.array_equal(plan.q_i8[0, bh].cpu().numpy(), oqi[0])
    assert np.array_equal(plan.k_i8[0, bh].cpu().numpy(), oki[0])

    nqb, nkb = plan.nqb, plan.nkb
    toks = np.unique(np.concatenate([[0, 1, 127, N - 129, N - 2, N - 1],
                                     np.random.default_rng(3).integers(0, N, 8)]))
    # the selection of every query block that holds a checked token (and the
    # middle ones), from the oracle; the GPU's rows must equal them
    rows = np.unique(np.concatenate([toks // 128, [nqb // 2, nqb - 2]]))
    kidx = plan.kidx[0, bh].cpu().numpy()
    say(f"[max] oracle mask rows {rows.tolist()}")
    okrows, _ = orc.block_mask_head(qh, kh, 0, plan.keep, rows)
    assert np.array_equal(kidx[rows], okrows)
    okidx = np.zeros_like(kidx)
    okidx[rows] = okrows

    say("[max] int32 tiles at the end of the head")
    trip = [(i, j) for i, j in ((nqb - 1, nkb - 1), (nqb - 1, 0), (0, nkb - 1), (nqb // 2, nkb // 3))]
    tiles = torch.tensor([(bh, i, j) for i, j in trip], dtype=torch.int32, device=DEV)
    out = ssa.sage_qk_int32_tiles(plan.q_i8, plan.k_i8, tiles).cpu().numpy()
    for t, (i, j) in enumerate(trip):
        assert np.array_equal(out[t], orc.qk_tile(oqi, oki, 0, i, j)), (i, j)

    say(f"[max] oracle attention rows of head {bh}: {len(toks)} tokens")
    ref = orc.sagesla_rows(qh, kh, vh, (oqi, oqs, oki, oks), 0, toks, okidx, branches=3)
    g32 = plan.out32[0, bh].cpu().numpy()[toks]
    g16 = plan.out[0, bh].float().cpu().numpy()[toks]
    rel, mx, _ = check_attn(g32, g16, ref, "max-size last head")
    say(f"    rel-L2={rel:.2e} max={mx:.2e}")

    say("[max] staged calls against the one-call step")
    ref32 = plan.out32.clone()
    plan.run_staged()
    torch.cuda.synchronize()
    assert torch.equal(plan.out32.view(torch.int32), ref32.view(torch.int32))
