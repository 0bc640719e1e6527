"""GPU parity of the W8A8 linear layer (page 5, "Four Technical Pillars",
Pillar Three: INT8 weights and activations, block-wise 128x128) against the
CPU oracle: quantized tensors and scales bit-exact, and the fp32 product
bit-exact too (the oracle follows the same exact int32 block sums and the
same fmaf chain over the K blocks); the bf16 output is the RNE of the fp32
one. Beside the bit-exact chain, the product is also gated against the
dequantization carried in fp64 (exact int32 block sums times the fp64 product
of the two scales): each of the nkb = K/128 steps of the fp32 chain rounds
twice (the scale product and the fma), so |y32 - y64| <= (nkb + 2) 2^-24
sum_kb |I_kb| sx sw per element."""
import numpy as np
import pytest
import torch

import bit_sparse_attention_amd as ssa
from bit_sparse_attention_amd.workloads import (LINEAR_WORKLOADS, bf16_bits, make_linear,
                                                make_linear_workload)

from gpu_common import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _u16(t):
    return bf16_bits(t.detach().cpu()).reshape(t.shape)


def _check_quant(orc, x, what):
    xd = x.to(DEV)
    q, s = ssa.w8a8_quant(xd)
    torch.cuda.synchronize()
    oq, os_ = orc.w8a8_quant(_u16(x))
    assert np.array_equal(q.cpu().numpy(), oq), f"{what}: int8 differs"
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32)), f"{what}: scales differ"
    return q, s, oq, os_


@pytest.mark.parametrize("rows,cols", [(1, 128), (127, 256), (300, 384), (1000, 512)])
def test_w8a8_quant_bitexact(orc, rows, cols):
    say(f"[w8a8 quant] {rows}x{cols}")
    x, _ = make_linear(rows, 128, cols, seed=rows + cols, outliers=True)
    _check_quant(orc, x, f"{rows}x{cols}")


def test_w8a8_quant_zero_block(orc):
    x, _ = make_linear(200, 128, 256, seed=1)
    x[:128, 128:] = 0  # one all-zero block: scale 0, q 0
    q, s, _, _ = _check_quant(orc, x, "zero block")
    assert float(s[0, 1]) == 0.0 and int(q[:128, 128:].abs().max()) == 0


def test_w8a8_quant_tiny_scales_and_denormals(orc):
    # 128x128 blocks scaled by 2^-100 and 2^-88 (scales below 2^-90: the kernel
    # divides) and by 2^-80 or not at all (the reciprocal path), with bf16
    # denormals sprinkled into the latter: bytes and scales bit-exact
    x, _ = make_linear(256, 128, 256, seed=4)
    xf = x.float()
    xf[:128, :128] *= 2.0 ** -100
    xf[:128, 128:] *= 2.0 ** -88
    xf[128:, :128] *= 2.0 ** -80
    xb = xf.to(torch.bfloat16).view(torch.int16).clone()
    g = torch.Generator().manual_seed(7)
    idx = torch.randint(0, 256 * 256, (600,), generator=g)
    rows, cols = idx // 256, idx % 256
    keep = rows >= 128  # the two blocks of the reciprocal path
    mant = torch.randint(1, 128, (600,), generator=g, dtype=torch.int16)
    xb[rows[keep], cols[keep]] = mant[keep]
    xb[200, 200] = 0x7F80  # +inf: block [1][1] gets an infinite scale (the division path)
    xb[201, 201] = -0x80   # -inf (0xFF80) in the same block
    xb[150, 20] = 0x7FC0   # a NaN in block [1][0] (finite scale, the reciprocal path)
    x = xb.view(torch.bfloat16)
    say("[w8a8 quant] tiny scales / denormals / infinities")
    q, s, _, _ = _check_quant(orc, x, "tiny scales / denormals / infinities")
    sc = s.cpu()
    assert sc[0, 0] < 2.0 ** -90 and sc[0, 1] < 2.0 ** -90 and sc[1, 0] > 2.0 ** -90
    assert torch.isinf(sc[1, 1])


@pytest.mark.parametrize("M,N,K,with_bias", [(1, 128, 128, False), (300, 256, 384, False),
                                             (700, 384, 1280, False), (257, 128, 640, False),
                                             (300, 256, 384, True), (1, 128, 640, True)])
def test_w8a8_gemm_bitexact(orc, M, N, K, with_bias):
    say(f"[w8a8 gemm] M={M} N={N} K={K} bias={with_bias}")
    x, w = make_linear(M, N, K, seed=M * 7 + K, outliers=True)
    xq, sx, oxq, osx = _check_quant(orc, x, "x")
    wq, sw, owq, osw = _check_quant(orc, w, "w")
    bias = (torch.randn(N, generator=torch.Generator().manual_seed(N + K)) * 0.5
            if with_bias else None)
    y, y32 = ssa.w8a8_gemm(xq, sx, wq, sw, return_f32=True,
                           bias=None if bias is None else bias.to(DEV))
    torch.cuda.synchronize()
    oy = orc.w8a8_gemm(oxq, osx, owq, osw, bias=None if bias is None else bias.numpy())
    got = y32.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oy.view(np.uint32)), \
        f"max |diff| {np.abs(got - oy).max():.3e}"
    assert torch.equal(y.cpu(), y32.cpu().to(torch.bfloat16))


def test_w8a8_linear_matches_the_two_calls(orc):
    x, w = make_linear(300, 256, 384, seed=3, outliers=True)
    xd, wd = x.to(DEV), w.to(DEV)
    bias = torch.linspace(-1.0, 1.0, 256, device=DEV)
    wq, sw = ssa.w8a8_quant(wd)
    y1 = ssa.w8a8_linear(xd, wq, sw)
    y1b = ssa.w8a8_linear(xd, wq, sw, bias=bias)
    xq, sx = ssa.w8a8_quant(xd)
    y2 = ssa.w8a8_gemm(xq, sx, wq, sw)
    y2b = ssa.w8a8_gemm(xq, sx, wq, sw, bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1b, y2b)
    assert not torch.equal(y1, y1b)


def test_w8a8_fullsize_sampled(orc):
    wl = LINEAR_WORKLOADS["w8a8_m75600_k5120_n5120"]
    say(f"[w8a8 full] {wl.name}: generating")
    x, w = make_linear_workload(wl)
    xq, sx, oxq, osx = _check_quant(orc, x, "x full")
    wq, sw, owq, osw = _check_quant(orc, w, "w full")
    say(f"[w8a8 full] {wl.name}: quantization bit-exact; GEMM")
    y, y32 = ssa.w8a8_gemm(xq, sx, wq, sw, return_f32=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 4), np.arange(wl.M - 4, wl.M),
                                     np.random.default_rng(0).integers(0, wl.M, 16)]))
    oy = orc.w8a8_gemm(oxq, osx, owq, osw, rows=rows)
    got = y32[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oy.view(np.uint32))
    say(f"[w8a8 full] {len(rows)} sampled rows bit-exact")


def test_w8a8_beyond_32bit_offsets(orc):
    """The most rows the library takes (2^20) at K = 2304, so x holds more than
    2^31 elements and its offsets need 64 bits: the quantization whole and
    rows at both ends of the product bit-exact."""
    M, N, K = 1 << 20, 256, 2304
    assert M * K > 2**31
    say(f"[w8a8 max] generating {M}x{K}, {N} outputs")
    x, w = make_linear(M, N, K, seed=5, outliers=True)
    xq, sx, oxq, osx = _check_quant(orc, x, "x max")
    wq, sw, owq, osw = _check_quant(orc, w, "w max")
    say("[w8a8 max] quantization bit-exact; GEMM")
    y, y32 = ssa.w8a8_gemm(xq, sx, wq, sw, return_f32=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 2), np.arange(M - 130, M - 126),
                                     np.arange(M - 4, M),
                                     np.random.default_rng(1).integers(0, M, 8)]))
    oy = orc.w8a8_gemm(oxq, osx, owq, osw, rows=rows)
    got = y32[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oy.view(np.uint32))
    want16 = torch.from_numpy(got).to(torch.bfloat16)
    assert torch.equal(y[torch.from_numpy(rows).to(DEV)].cpu(), want16)
    say(f"[w8a8 max] {len(rows)} sampled rows bit-exact")


@pytest.mark.parametrize("M,N,K,full", [(1000, 512, 5120, False), (75600, 5120, 5120, True)])
def test_w8a8_gemm_within_the_fp64_dequantization_bound(orc, M, N, K, full):
    if full:
        x, w = make_linear_workload(LINEAR_WORKLOADS["w8a8_m75600_k5120_n5120"])
    else:
        x, w = make_linear(M, N, K, seed=13, outliers=True)
    say(f"[w8a8 fp64] M={M} N={N} K={K}")
    xq, sx, oxq, osx = _check_quant(orc, x, "x")
    wq, sw, owq, osw = _check_quant(orc, w, "w")
    y, y32 = ssa.w8a8_gemm(xq, sx, wq, sw, return_f32=True)
    torch.cuda.synchronize()
    rows = (np.unique(np.concatenate([np.arange(0, 4), np.arange(M - 4, M),
                                      np.random.default_rng(1).integers(0, M, 24)]))
            if full else np.arange(M))
    y64, yabs = orc.w8a8_gemm_f64(oxq, osx, owq, osw, rows=rows)
    got = y32[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    bound = (K // 128 + 2) * 2.0**-24 * yabs
    err = np.abs(got - y64)
    assert np.all(err <= bound), f"max excess {(err - bound).max():.3e}"
    rel = np.linalg.norm(got - y64) / np.linalg.norm(y64)
    say(f"    rows={len(rows)} rel-L2 vs fp64 = {rel:.2e}, max err / bound = {(err / bound).max():.3f}")

