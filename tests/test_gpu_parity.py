"""GPU parity of the HIP path against the CPU oracle, element by element, at
sizes the oracle finishes in seconds (several tiles and ragged tails), plus the
edge cases of the method. Every call goes through the C ABI (libssa.so)."""
import numpy as np
import pytest
import torch

import bit_sparse_attention_amd as ssa
from bit_sparse_attention_amd.workloads import make_qkv
from gpu_common import bits, check_attn, flat, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gpu(*ts):
    return [t.to(DEV) for t in ts]


def _quant_and_check(orc, q, k, label):
    qd, kd = _gpu(q, k)
    say(f"[quant] {label} shape={tuple(q.shape)}")
    q_i8, q_scale, k_i8, k_scale, k_mean = ssa.sage_quant_qk(qd, kd)
    torch.cuda.synchronize()
    qb, kb = bits(q), bits(k)
    oq_i8, oq_s, ok_i8, ok_s, omu = orc.quant_qk(qb, kb)
    assert np.array_equal(flat(k_mean).view(np.uint32), omu.view(np.uint32)), "k_mean"
    assert np.array_equal(flat(q_scale).view(np.uint32), oq_s.view(np.uint32)), "q_scale"
    assert np.array_equal(flat(k_scale).view(np.uint32), ok_s.view(np.uint32)), "k_scale"
    assert np.array_equal(flat(q_i8), oq_i8), "q_i8"
    assert np.array_equal(flat(k_i8), ok_i8), "k_i8"
    return (q_i8, q_scale, k_i8, k_scale), (oq_i8, oq_s, ok_i8, ok_s)


@pytest.mark.parametrize("B,H,N", [(1, 1, 1024), (1, 2, 1000), (2, 1, 300), (1, 1, 64),
                                   (1, 1, 1), (1, 3, 4100), (1, 1, 129)])
def test_quant_bitexact(orc, B, H, N):
    q, k, v = make_qkv(B, H, N, 128, seed=N)
    _quant_and_check(orc, q, k, f"B{B}H{H}N{N}")


def test_quant_ties_zero_block_and_spikes(orc):
    # hand-built ties (amax 127 -> scale 1), an all-zero Q block, and x20 K spikes
    q, k, v = make_qkv(1, 1, 700, 128, seed=5, spikes=True)
    qf = q.float()
    qf[0, 0, 0, :10] = torch.tensor([127.0, -127.0, 2.5, -3.5, 0.5, 1.5, -0.5, 126.5, -2.5, 3.25])
    qf[0, 0, 1:128] = 0.0
    qf[0, 0, 0, 10:] = 0.0
    qf[0, 0, 128:256] = 0.0  # an all-zero block
    q = qf.to(torch.bfloat16)
    (qi, qs, _, _), _ = _quant_and_check(orc, q, k, "ties/zero/spikes")
    assert qs[0, 0, 0].item() == 1.0 and qs[0, 0, 1].item() == 0.0
    assert qi[0, 0, 0, :10].tolist() == [127, -127, 2, -4, 0, 2, 0, 126, -2, 3]


def _with_denormals(x, rows, count, seed):
    """x (bf16, [B,H,N,D]) with `count` elements of each given token row set to
    bf16 denormals of random sign (bit patterns 1 .. 127 in the mantissa)."""
    g = torch.Generator().manual_seed(seed)
    xb = x.contiguous().view(torch.int16).clone()
    for t in rows:
        cols = torch.randperm(x.shape[-1], generator=g)[:count]
        mant = torch.randint(1, 128, (count,), generator=g, dtype=torch.int16)
        sign = torch.randint(0, 2, (count,), generator=g, dtype=torch.int16) * -32768
        xb[0, 0, t, cols] = mant | sign
    return xb.view(torch.bfloat16)


def test_quant_tiny_scales_and_denormals(orc):
    # Q blocks (128 tokens): block 0 scaled by 2^-100 and block 3 by 2^-88
    # (scales below 2^-90, where the kernel divides), block 1 by 2^-80 and
    # block 2 unscaled (the reciprocal path), blocks 1 and 2 with denormal
    # elements; K scaled by 2^-100 throughout (tiny smoothed blocks)
    q, k, v = make_qkv(1, 1, 512, 128, seed=21)
    qf = q.float()
    qf[0, 0, 0:128] *= 2.0 ** -100
    qf[0, 0, 128:256] *= 2.0 ** -80
    qf[0, 0, 384:512] *= 2.0 ** -88
    q = _with_denormals(qf.to(torch.bfloat16), range(128, 384, 5), 16, seed=3)
    kt = (k.float() * 2.0 ** -100).to(torch.bfloat16)
    (qi, qs, _, ks), _ = _quant_and_check(orc, q, kt, "tiny scales / denormals")
    s = qs.flatten().cpu()
    assert s[0] < 2.0 ** -90 and s[3] < 2.0 ** -90 and s[1] > 2.0 ** -90 and s[2] > 2.0 ** -90
    assert float(ks.max()) < 2.0 ** -90
    # and unscaled K with denormals in Q only: the reciprocal path for both
    _quant_and_check(orc, q, k, "denormals, normal K")
    # an infinite element in Q block 2: an infinite scale, which must divide
    qi16 = q.contiguous().view(torch.int16).clone()
    qi16[0, 0, 300, 7] = 0x7F80
    (qi, qs, _, _), _ = _quant_and_check(orc, qi16.view(torch.bfloat16), k, "infinite element")
    assert torch.isinf(qs.flatten()[2].cpu())


@pytest.mark.parametrize("B,H,N,topk", [(1, 2, 1000, 0.25), (1, 1, 4100, 0.1), (1, 2, 8192, 0.05),
                                        (1, 1, 1000, 1.0), (1, 1, 1000, 0.0), (1, 1, 64, 0.5),
                                        (2, 1, 3000, 0.3)])
def test_mask_bitexact(orc, B, H, N, topk):
    q, k, v = make_qkv(B, H, N, 128, seed=N + 1)
    keep = ssa.keep_blocks(N, topk)
    say(f"[mask] B{B}H{H}N{N} keep={keep}")
    qd, kd = _gpu(q, k)
    kidx, mask = ssa.sla_block_mask(qd, kd, keep, return_mask=True)
    # the same selection from the pooled means sage_quant_qk hands over
    pool = ssa.new_pool(qd)
    ssa.sage_quant_qk(qd, kd, pool)
    kidx_p, mask_p = ssa.sla_block_mask(qd, kd, keep, return_mask=True, pool=pool)
    torch.cuda.synchronize()
    okidx, omask = orc.block_mask(bits(q), bits(k), keep)
    assert np.array_equal(flat(kidx), okidx)
    assert np.array_equal(flat(mask), omask)
    assert np.array_equal(flat(kidx_p), okidx)
    assert np.array_equal(flat(mask_p), omask)


def test_mask_ties_break_to_lower_block(orc):
    # every key block is a copy of the first one: all scores of a row tie and
    # the kept set must be the lowest `keep` blocks
    q, k, v = make_qkv(1, 1, 1024, 128, seed=9)
    k = k[:, :, :64].repeat(1, 1, 16, 1).contiguous()
    keep = 5
    kidx = ssa.sla_block_mask(*_gpu(q, k), keep)
    okidx, _ = orc.block_mask(bits(q), bits(k), keep)
    assert np.array_equal(flat(kidx), okidx)
    assert np.array_equal(okidx[0], np.tile(np.arange(keep), (8, 1)))


def test_qk_int32_tiles_bitexact(orc):
    B, H, N = 1, 2, 1000
    q, k, v = make_qkv(B, H, N, 128, seed=11)
    (q_i8, _, k_i8, _), (oqi, _, oki, _) = _quant_and_check(orc, q, k, "tiles")
    trip = [(bh, i, j) for bh in range(2) for i in range(8) for j in range(16)]
    trip += [(2, 0, 0), (0, 8, 0), (0, 0, 16), (-1, 0, 0)]  # out of range -> zero tile
    tiles = torch.tensor(trip, dtype=torch.int32, device=DEV)
    say(f"[tiles] {len(trip)} tiles")
    out = ssa.sage_qk_int32_tiles(q_i8, k_i8, tiles).cpu().numpy()
    for t, (bh, i, j) in enumerate(trip):
        if 0 <= bh < 2 and 0 <= i < 8 and 0 <= j < 16:
            assert np.array_equal(out[t], orc.qk_tile(oqi, oki, bh, i, j)), (bh, i, j)
        else:
            assert not out[t].any()


ATTN_CASES = [(1, 1, 1024, None), (1, 2, 1000, 0.25), (1, 1, 4100, 0.1), (2, 1, 3000, 0.2),
              (1, 1, 200, 0.5), (1, 1, 64, None), (1, 1, 1, None)]


# dense attention (topk None) has no linear branch: only branches == 1
ATTN_PARAMS = [(B, H, N, topk, br) for (B, H, N, topk) in ATTN_CASES for br in (1, 2, 3)
               if topk is not None or br == 1]


def _oracle_intermediates(orc, q_i8, q_scale, k_i8, k_scale, kidx, qb, kb, keep, label):
    """The oracle's quantized tensors, scales and selection for the same
    inputs, after asserting the GPU's equal them bit for bit: the attention
    reference is then built from the oracle's values only."""
    oqi, oqs, oki, oks, _ = orc.quant_qk(qb, kb)
    assert np.array_equal(flat(q_i8), oqi), f"{label}: q_i8"
    assert np.array_equal(flat(k_i8), oki), f"{label}: k_i8"
    assert np.array_equal(flat(q_scale).view(np.uint32), oqs.view(np.uint32)), f"{label}: q_scale"
    assert np.array_equal(flat(k_scale).view(np.uint32), oks.view(np.uint32)), f"{label}: k_scale"
    okidx = None
    if kidx is not None:
        okidx, _ = orc.block_mask(qb, kb, keep)
        assert np.array_equal(flat(kidx), okidx), f"{label}: kidx"
    return (oqi, oqs, oki, oks), okidx


@pytest.mark.parametrize("B,H,N,topk,branches", ATTN_PARAMS)
def test_attn_parity(orc, B, H, N, topk, branches):
    q, k, v = make_qkv(B, H, N, 128, seed=7 * N + branches)
    qd, kd, vd = _gpu(q, k, v)
    label = f"B{B}H{H}N{N} topk={topk} branches={branches}"
    say(f"[attn] {label}")
    q_i8, q_scale, k_i8, k_scale, _ = ssa.sage_quant_qk(qd, kd)
    if topk is None:
        kidx, keep = None, ssa.num_k_blocks(N)
    else:
        keep = ssa.keep_blocks(N, topk)
        kidx = ssa.sla_block_mask(qd, kd, keep)
    out, out32 = ssa.sage_sla_attn_fwd(qd, kd, vd, q_i8, q_scale, k_i8, k_scale, kidx, keep,
                                       branches, 0.0, return_f32=True)
    torch.cuda.synchronize()
    qb, kb, vb = bits(q), bits(k), bits(v)
    quant, okidx = _oracle_intermediates(orc, q_i8, q_scale, k_i8, k_scale, kidx, qb, kb, keep,
                                         label)
    g32, g16 = flat(out32), flat(out.float())
    toks = np.arange(N)
    for bh in range(B * H):
        ref = orc.sagesla_rows(qb, kb, vb, quant, bh, toks,
                               None if okidx is None else okidx[bh], branches=branches)
        if branches == 2:
            ref = {"decl": ref["linear"], "exact": ref["linear"], "amb": np.zeros(N)}
            if keep == ssa.num_k_blocks(N):
                assert not g32[bh].any()
                continue
        rel, mx, rel_ex = check_attn(g32[bh], g16[bh], ref, f"{label} bh={bh}")
        say(f"    bh={bh} rel-L2={rel:.2e} max={mx:.2e} rel-L2 vs exact={rel_ex:.2e}")


@pytest.mark.parametrize("topk", [0.4, 0.6, 0.9, 0.97])
def test_linear_branch_high_keep(orc, topk):
    # The complement states subtract the kept blocks from the total while
    # fewer than half are kept, and sum the non-kept blocks directly beyond
    # that; either way only the smaller set carries bf16 rounding. Linear
    # branch alone on every row, both branches on two rows per query block.
    B, H, N = 1, 1, 32760
    q, k, v = make_qkv(B, H, N, 128, seed=41)
    qd, kd, vd = _gpu(q, k, v)
    label = f"N{N} topk={topk}"
    say(f"[linear-high-keep] {label}")
    qq = ssa.sage_quant_qk(qd, kd)[:4]
    keep = ssa.keep_blocks(N, topk)
    kidx = ssa.sla_block_mask(qd, kd, keep)
    lin32 = ssa.sage_sla_attn_fwd(qd, kd, vd, *qq, kidx, keep, ssa.LINEAR, return_f32=True)[1]
    out, out32 = ssa.sage_sla_attn_fwd(qd, kd, vd, *qq, kidx, keep, 3, return_f32=True)
    torch.cuda.synchronize()
    qb, kb, vb = bits(q), bits(k), bits(v)
    quant, okidx = _oracle_intermediates(orc, *qq, kidx, qb, kb, keep, label)
    h, z = orc.linear_states(kb, vb, 0)
    ol = orc.linear_rows(qb, h, z, 0, np.arange(N), okidx[0])
    g = flat(lin32)[0]
    rel = np.linalg.norm(g - ol) / np.linalg.norm(ol)
    err = np.abs(g - ol).max()
    say(f"    linear branch rel-L2={rel:.2e} max={err:.2e}")
    assert rel <= 1e-3 and err <= 2e-3, (rel, err)
    nqb = ssa.num_q_blocks(N)
    toks = np.unique(np.concatenate([128 * np.arange(nqb),
                                     np.minimum(128 * np.arange(nqb) + 77, N - 1)]))
    ref = orc.sagesla_rows(qb, kb, vb, quant, 0, toks, okidx[0], branches=3)
    rel3, mx3, _ = check_attn(flat(out32)[0][toks], flat(out.float())[0][toks], ref, label)
    say(f"    both branches rows={len(toks)} rel-L2={rel3:.2e} max={mx3:.2e}")


def test_dense_equals_all_blocks_kept():
    q, k, v = make_qkv(1, 2, 1000, 128, seed=3)
    qd, kd, vd = _gpu(q, k, v)
    qq = ssa.sage_quant_qk(qd, kd)[:4]
    nkb = ssa.num_k_blocks(1000)
    kidx = torch.arange(nkb, dtype=torch.int32, device=DEV).repeat(1, 2, 8, 1).contiguous()
    a = ssa.sage_sla_attn_fwd(qd, kd, vd, *qq, None, None, ssa.SPARSE)
    b = ssa.sage_sla_attn_fwd(qd, kd, vd, *qq, kidx, nkb, ssa.SPARSE | ssa.LINEAR)
    assert torch.equal(a, b)


def test_repeat_runs_bit_identical():
    q, k, v = make_qkv(1, 2, 3000, 128, seed=4)
    qd, kd, vd = _gpu(q, k, v)
    outs = [ssa.sagesla(qd, kd, vd, topk=0.2, return_f32=True)[1] for _ in range(3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_branch_sum(orc):
    q, k, v = make_qkv(1, 1, 2000, 128, seed=8)
    qd, kd, vd = _gpu(q, k, v)
    qq = ssa.sage_quant_qk(qd, kd)[:4]
    keep = ssa.keep_blocks(2000, 0.2)
    kidx = ssa.sla_block_mask(qd, kd, keep)
    s = ssa.sage_sla_attn_fwd(qd, kd, vd, *qq, kidx, keep, 1, return_f32=True)[1]
    lin = ssa.sage_sla_attn_fwd(qd, kd, vd, *qq, kidx, keep, 2, return_f32=True)[1]
    both = ssa.sage_sla_attn_fwd(qd, kd, vd, *qq, kidx, keep, 3, return_f32=True)[1]
    d = (both - (s + lin)).abs()
    assert d.max().item() <= 2 * torch.finfo(torch.float32).eps * (s.abs() + lin.abs()).max().item()


def test_explicit_sm_scale(orc):
    N = 1500
    q, k, v = make_qkv(1, 1, N, 128, seed=12)
    qd, kd, vd = _gpu(q, k, v)
    qq = ssa.sage_quant_qk(qd, kd)[:4]
    keep = ssa.keep_blocks(N, 0.3)
    kidx = ssa.sla_block_mask(qd, kd, keep)
    out, out32 = ssa.sage_sla_attn_fwd(qd, kd, vd, *qq, kidx, keep, 3, 0.05, return_f32=True)
    torch.cuda.synchronize()
    qb, kb = bits(q), bits(k)
    quant, okidx = _oracle_intermediates(orc, *qq, kidx, qb, kb, keep, "sm_scale=0.05")
    ref = orc.sagesla_rows(qb, kb, bits(v), quant, 0, np.arange(N), okidx[0], branches=3,
                           sm_scale=0.05)
    check_attn(flat(out32)[0], flat(out.float())[0], ref, "sm_scale=0.05")


def test_workspace_too_small_is_reported():
    q, k, v = make_qkv(1, 1, 256, 128, seed=1)
    qd, kd = _gpu(q, k)
    L = ssa._load()
    dummy = torch.empty(16, dtype=torch.uint8, device=DEV)
    outs = [torch.empty(256 * 128, dtype=torch.int8, device=DEV) for _ in range(2)]
    sc = [torch.empty(8, dtype=torch.float32, device=DEV) for _ in range(2)]
    mu = torch.empty(128, dtype=torch.float32, device=DEV)
    st = L.sage_quant_qk(qd.data_ptr(), kd.data_ptr(), ssa.Shape(1, 1, 256, 128),
                         outs[0].data_ptr(), sc[0].data_ptr(), outs[1].data_ptr(),
                         sc[1].data_ptr(), mu.data_ptr(), None, dummy.data_ptr(), 16, None)
    assert st == 3
