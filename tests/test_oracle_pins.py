"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, exact rational arithmetic, brute force on tiny inputs, library
routines for special cases, and hand-derived values under tests/golden/.

The method is the one on the TurboDiffusion pages (page 5, "Four Technical
Pillars", Pillars One and Two; "Hands-On Tutorial" flags --attention_type
sagesla and --sla_topk).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from bit_sparse_attention_amd.workloads import bf16_bits, make_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits(t):
    return bf16_bits(t.to(torch.bfloat16))


def _f(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()


def round_rational(fr: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Exact round-to-nearest-even of a rational to a binary format with
    `mant_bits` significant bits and smallest exponent of the last bit `emin`."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length() - mant_bits
    while a / Fraction(2) ** e >= 2 ** mant_bits:
        e += 1
    while a / Fraction(2) ** e < 2 ** (mant_bits - 1):
        e -= 1
    e = max(e, emin)
    m = a / Fraction(2) ** e
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * Fraction(n) * Fraction(2) ** e


def f32_of(fr: Fraction) -> float:
    return float(round_rational(fr, 24, -149))


# --------------------------------------------------------------------------
# block counts and keep (page 5, "Hands-On Tutorial": --sla_topk 0.1 keeps 10%)

def test_keep_blocks(orc):
    assert orc.nqb(32760) == 256 and orc.nkb(32760) == 512
    assert orc.nqb(75600) == 591 and orc.nkb(75600) == 1182
    assert orc.nqb(269280) == 2104 and orc.nkb(269280) == 4208
    assert orc.keep_blocks(32760, 0.1) == 51
    assert orc.keep_blocks(75600, 0.1) == 118
    assert orc.keep_blocks(269280, 0.05) == 210
    assert orc.keep_blocks(1024, 0.0) == 1
    assert orc.keep_blocks(1024, 1.0) == 16
    assert orc.keep_blocks(1024, 0.5) == 8
    assert orc.keep_blocks(1024, 0.15) == 2  # 2.4 -> 2


# --------------------------------------------------------------------------
# bf16 rounding helpers, against torch's conversion and exact rationals

def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(2000).astype(np.float32) * 10 ** rng.uniform(-40, 38, 2000))
    # exact ties: lower 16 bits = 0x8000 with even and odd kept lsb
    for hi in (0x3F80, 0x3F81, 0xBF80, 0xBF81, 0x0001, 0x0002, 0x7F7E, 0x7F7F):
        for lo in (0x8000, 0x7FFF, 0x8001):
            vals.append(np.array([(hi << 16) | lo], np.uint32).view(np.float32)[0])
    vals += [np.float32(1e-45), np.float32(-3e-39), np.float32(0.0), np.float32(-0.0)]
    x = np.array(vals, np.float32)
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16_bits(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, want)


def test_round_bf16_double_exact(orc):
    rng = np.random.default_rng(2)
    xs = list(rng.uniform(0, 1, 500)) + list(2.0 ** rng.uniform(-140, -120, 100))
    xs += [1 + 2 ** -8, 1 + 3 * 2 ** -8, 0.5 + 2 ** -9, 2 ** -126 * (1 + 2 ** -8)]
    for x in xs:
        want = float(round_rational(Fraction(x), 8, -133))
        assert orc.round_bf16(x) == want, x


# --------------------------------------------------------------------------
# K smoothing mean (page 5, Pillar One: "smoothing" of outliers)

def test_k_mean_close_to_fp64(orc):
    q, k, v = make_qkv(1, 2, 1000, 128, seed=3)
    kb = _bits(k).reshape(2, 1000, 128)
    mu = orc.k_mean(kb)
    ref = _f(kb).astype(np.float64).mean(axis=1)
    assert np.all(np.abs(mu - ref) <= 1e-6 * (np.abs(ref) + 1))


def test_k_mean_exact_on_integers(orc):
    rng = np.random.default_rng(4)
    N, D = 300, 128  # ragged: 4 full key blocks + 44 tokens
    ki = rng.integers(-20, 21, size=(1, N, D)).astype(np.float32)
    kb = _bits(torch.from_numpy(ki))
    mu = orc.k_mean(kb)
    # every partial sum is an exact small integer, so mu = fl32(sum / N)
    want = (ki.sum(axis=1, dtype=np.float64)).astype(np.float32) / np.float32(N)
    assert np.array_equal(mu, want)


def test_smoothing_reading_is_softmax_invariant():
    # The reading behind smoothing: subtracting a per-channel mean mu from every
    # key shifts all scores of a query row by q.mu, which softmax ignores.
    rng = np.random.default_rng(5)
    q = rng.standard_normal((7, 16))
    k = rng.standard_normal((33, 16)) + 3 * rng.standard_normal(16)
    v = rng.standard_normal((33, 16))
    mu = rng.standard_normal(16) * 5

    def attn(kk):
        s = q @ kk.T
        p = np.exp(s - s.max(axis=1, keepdims=True))
        return (p / p.sum(axis=1, keepdims=True)) @ v

    assert np.max(np.abs(attn(k) - attn(k - mu))) < 1e-12


# --------------------------------------------------------------------------
# INT8 quantization (page 5, Pillar One)

def _check_quant_invariants(x, xq, sc, blk):
    BH, N, D = x.shape
    for bh in range(BH):
        for b in range(sc.shape[1]):
            t0, t1 = b * blk, min(N, (b + 1) * blk)
            xb = x[bh, t0:t1].astype(np.float64)
            qb = xq[bh, t0:t1].astype(np.int64)
            s = float(sc[bh, b])
            amax = np.abs(xb).max()
            assert s == np.float32(np.float32(amax) / np.float32(127.0))
            assert np.all(np.abs(qb) <= 127)
            if amax == 0:
                assert s == 0 and np.all(qb == 0)
                continue
            assert np.abs(qb).max() == 127
            # rint acts on fl32(x/s), whose rounding (<= 2^-17 at |x/s| <= 127)
            # can move a value just past a half-integer: |x - q s| <= s (1/2 + 2^-17)
            assert np.all(np.abs(xb - qb * s) <= s / 2 * (1 + 2 ** -15))


def test_quant_invariants_q_and_k(orc):
    q, k, v = make_qkv(1, 2, 1000, 128, seed=6)
    qb, kb = _bits(q).reshape(2, 1000, 128), _bits(k).reshape(2, 1000, 128)
    qi, qs, ki, ks, mu = orc.quant_qk(qb, kb)
    assert qs.shape == (2, 8) and ks.shape == (2, 16)
    _check_quant_invariants(_f(qb), qi, qs, 128)
    kp = (_f(kb) - mu[:, None, :]).astype(np.float32)  # one fp32 subtraction
    _check_quant_invariants(kp, ki, ks, 64)


def test_quant_golden_ties(orc):
    g = _golden("quant_ties.json")
    x = np.zeros((1, 128, 128), np.float32)
    x[0, 0, : len(g["x"])] = g["x"]
    xb = _bits(torch.from_numpy(x))
    assert np.array_equal(_f(xb), x)  # all values are exact in bf16
    qi, qs = orc.quant(xb, None, 128)
    assert qs[0, 0] == 1.0
    assert list(qi[0, 0, : len(g["q"])]) == g["q"]
    # K path: rows in +/- pairs give a zero channel mean, so K' = K exactly
    kx = np.zeros((1, 64, 128), np.float32)
    kx[0, 0, : len(g["x"])] = g["x"]
    kx[0, 1, : len(g["x"])] = [-a for a in g["x"]]
    kb = _bits(torch.from_numpy(kx))
    mu = orc.k_mean(kb)
    assert np.all(mu == 0)
    ki, ks = orc.quant(kb, mu, 64)
    assert ks[0, 0] == 1.0
    assert list(ki[0, 0, : len(g["q"])]) == g["q"]
    assert list(ki[0, 1, : len(g["q"])]) == [-a for a in g["q"]]


def test_quant_block_boundaries(orc):
    # one large value moves only the scale of the block that holds it
    N = 300
    for blk, pos, want_block in ((128, 127, 0), (128, 128, 1), (128, 299, 2), (64, 63, 0),
                                 (64, 64, 1), (64, 299, 4)):
        x = np.full((1, N, 128), 0.25, np.float32)
        x[0, pos, 5] = 100.0
        xb = _bits(torch.from_numpy(x))
        xq, sc = orc.quant(xb, None, blk)
        big = np.float32(np.float32(100.0) / np.float32(127.0))
        small = np.float32(np.float32(0.25) / np.float32(127.0))
        for b in range(sc.shape[1]):
            assert sc[0, b] == (big if b == want_block else small), (blk, pos, b)


def test_quant_zero_block(orc):
    x = np.zeros((1, 200, 128), np.float32)
    x[0, 150:, :] = 1.0
    xq, sc = orc.quant(_bits(torch.from_numpy(x)), None, 128)
    assert sc[0, 0] == 0 and np.all(xq[0, :128] == 0)
    assert sc[0, 1] == np.float32(1.0) / np.float32(127.0) and np.all(xq[0, 150:] == 127)


def test_quant_non_finite_elements(orc):
    # Reading (the pages do not cover non-finite inputs): the clamp to +-127 is
    # IEEE minNum/maxNum, so a NaN quotient becomes -127. An infinite element
    # makes its block's scale infinite: every finite element then quantizes to
    # 0 and the infinite ones (inf/inf = NaN) to -127; a NaN element in a finite
    # block does not change the scale and also gives -127.
    x = np.zeros((1, 256, 128), np.float32)
    x[0, :128, :] = 0.5
    x[0, 3, 7] = np.inf
    x[0, 4, 9] = -np.inf
    x[0, 128:, :] = 2.0
    x[0, 130, 1] = np.nan
    xq, sc = orc.quant(_bits(torch.from_numpy(x)), None, 128)
    assert np.isinf(sc[0, 0]) and sc[0, 1] == np.float32(2.0) / np.float32(127.0)
    assert xq[0, 3, 7] == -127 and xq[0, 4, 9] == -127
    blk0 = xq[0, :128].copy()
    blk0[3, 7] = blk0[4, 9] = 0
    assert np.all(blk0 == 0)
    assert xq[0, 130, 1] == -127 and xq[0, 129, 1] == 127
    q, s = orc.w8a8_quant(_bits(torch.from_numpy(x[0, :128])))
    assert np.isinf(s[0, 0]) and q[3, 7] == -127 and q[4, 9] == -127 and q[0, 0] == 0


# --------------------------------------------------------------------------
# int32 scores

def test_qk_tile_matches_int64_matmul(orc):
    rng = np.random.default_rng(7)
    N, D = 200, 128
    qi = rng.integers(-127, 128, size=(2, N, D), dtype=np.int8)
    ki = rng.integers(-127, 128, size=(2, N, D), dtype=np.int8)
    qi[0, 0, :] = 127
    ki[0, 0, :] = 127  # extreme value 128 * 127^2 fits int32
    for bh, i, j in ((0, 0, 0), (1, 1, 2), (0, 1, 3), (1, 0, 3)):
        tile = orc.qk_tile(qi, ki, bh, i, j)
        ref = np.zeros((128, 64), np.int64)
        t0, u0 = i * 128, j * 64
        qa = qi[bh, t0:min(N, t0 + 128)].astype(np.int64)
        ka = ki[bh, u0:min(N, u0 + 64)].astype(np.int64)
        ref[: qa.shape[0], : ka.shape[0]] = qa @ ka.T
        assert np.array_equal(tile, ref)


# --------------------------------------------------------------------------
# block mask (page 5, Pillar Two; --sla_topk = fraction kept)

def test_pool_means(orc):
    q, k, v = make_qkv(1, 1, 300, 128, seed=8)
    qb = _bits(q).reshape(1, 300, 128)
    p = orc.pool(qb, 0, 128)
    x = _f(qb)[0].astype(np.float64)
    ref = np.stack([x[0:128].mean(0), x[128:256].mean(0), x[256:300].mean(0)])
    assert np.all(np.abs(p - ref) <= 1e-6 * (np.abs(ref) + 1))
    # exact on small integers: fl32(sum / n) with the tail's valid count
    xi = np.random.default_rng(9).integers(-5, 6, size=(1, 300, 128)).astype(np.float32)
    p = orc.pool(_bits(torch.from_numpy(xi)), 0, 64)
    for b, (t0, t1) in enumerate(((0, 64), (64, 128), (128, 192), (192, 256), (256, 300))):
        want = xi[0, t0:t1].sum(0).astype(np.float32) / np.float32(t1 - t0)
        assert np.array_equal(p[b], want)


def test_block_scores_are_an_exact_fma_chain(orc):
    rng = np.random.default_rng(10)
    D = 24
    qbar = rng.standard_normal((3, D)).astype(np.float32)
    kbar = (rng.standard_normal((5, D)) * 3).astype(np.float32)
    sc = orc.block_scores(qbar, kbar, [0, 1, 2])
    for r in range(3):
        for j in range(5):
            acc = Fraction(0)
            for d in range(D):  # one rounding per fused multiply-add
                acc = Fraction(f32_of(Fraction(float(qbar[r, d])) * Fraction(float(kbar[j, d]))
                                      + acc))
            assert sc[r, j] == np.float32(float(acc))
            assert abs(float(sc[r, j]) - float(qbar[r] @ kbar[j].astype(np.float64))) < 1e-4


def _brute_topk(s, keep):
    """Unique kept set under the order (score desc, index asc), by enumeration."""
    n = len(s)
    found = []
    for sub in itertools.combinations(range(n), keep):
        subset = set(sub)
        ok = all((s[a] > s[b]) or (s[a] == s[b] and a < b)
                 for a in subset for b in range(n) if b not in subset)
        if ok:
            found.append(sub)
    return found


def test_topk_bruteforce_with_ties(orc):
    rng = np.random.default_rng(11)
    for trial in range(60):
        n = int(rng.integers(1, 13))
        keep = int(rng.integers(1, n + 1))
        s = rng.integers(-3, 4, size=n).astype(np.float32)  # many ties
        if trial % 3 == 0:
            s[s == 0] = np.where(rng.random((s == 0).sum()) < 0.5, -0.0, 0.0)
        kidx, mask = orc.topk(s[None, :], keep)
        found = _brute_topk([float(a) for a in s], keep)
        assert len(found) == 1
        assert list(kidx[0]) == list(found[0])
        assert mask[0].sum() == keep and all(mask[0][list(found[0])] == 1)


def test_topk_nested_and_full(orc):
    rng = np.random.default_rng(12)
    s = rng.standard_normal((4, 40)).astype(np.float32)
    prev = None
    for keep in range(1, 41):
        kidx, _ = orc.topk(s, keep)
        assert np.all(np.diff(kidx, axis=1) > 0)
        if prev is not None:
            for r in range(4):
                assert set(prev[r]) <= set(kidx[r])
        prev = kidx
    assert np.array_equal(prev, np.tile(np.arange(40), (4, 1)))


def test_mask_from_raw_k_matches_smoothed_k_when_separated(orc):
    # q.mu is the same for every key block of a query row, so ranking with raw
    # K or with K - mu agrees (exactly in exact arithmetic; checked here on
    # well separated scores).
    q, k, v = make_qkv(1, 1, 2048, 128, seed=13)
    qb, kb = _bits(q).reshape(1, 2048, 128), _bits(k).reshape(1, 2048, 128)
    qbar, kbar = orc.pool(qb, 0, 128), orc.pool(kb, 0, 64)
    mu = kbar.astype(np.float64).mean(0)
    s_raw = qbar.astype(np.float64) @ kbar.astype(np.float64).T
    s_sm = qbar.astype(np.float64) @ (kbar.astype(np.float64) - mu).T
    kidx, _ = orc.topk(orc.block_scores(qbar, kbar, range(16)), 5)
    for i in range(16):
        order = np.argsort(-s_sm[i], kind="stable")
        gap = np.sort(s_raw[i])[::-1]
        if gap[4] - gap[5] > 1e-4:
            assert sorted(order[:5]) == list(kidx[i])


# --------------------------------------------------------------------------
# sparse softmax branch (page 5, Pillars One and Two)

def test_sparse_golden_small(orc):
    g = _golden("sparse_decl_small.json")
    N, D = 3, 128
    qi = np.zeros((1, N, D), np.int8)
    qi[0, :, 0] = 1
    ki = np.zeros((1, N, D), np.int8)
    ki[0, :, 0] = g["S"]
    v = np.zeros((1, N, D), np.float32)
    for u in range(3):
        v[0, u, u] = 1.0
    vb = _bits(torch.from_numpy(v))
    sm = float(np.float32(math.log(2.0)))
    assert np.float32(sm * 1.4426950408889634) == 1.0
    res = orc.sparse_rows(qi, np.ones((1, 1), np.float32), ki,
                          np.full((1, 1), g["k_scale"], np.float32), vb, 0, [0], sm_scale=sm)
    assert np.allclose(res["decl"][0, :3], g["o"], rtol=0, atol=1e-15)
    assert np.all(res["decl"][0, 3:] == 0)
    # exact arithmetic: p = exp((S*0.5) * ln2 - max) = 2^((S-3)/2) up to fl32(ln 2)
    pe = 2.0 ** ((np.array(g["S"]) - 3) / 2.0)
    assert np.allclose(res["exact"][0, :3], pe / pe.sum(), rtol=1e-7)


def test_sparse_uniform_when_q_is_zero(orc):
    # q = 0 gives every score 0: both numerics reduce to the plain mean of V
    # over the valid tokens of the kept blocks.
    q, k, v = make_qkv(1, 1, 300, 128, seed=14)
    qb, kb, vb = (_bits(t).reshape(1, 300, 128) for t in (torch.zeros_like(q), k, v))
    qi, qs, ki, ks, mu = orc.quant_qk(qb, kb)
    kidx = np.array([[0, 4], [1, 2], [3, 4]], np.int32)  # block 4 is the 44-token tail
    toks = [0, 130, 299]
    res = orc.sparse_rows(qi, qs, ki, ks, vb, 0, toks, kidx_head=kidx)
    vf = _f(vb)[0].astype(np.float64)
    for r, t in enumerate(toks):
        sel = np.concatenate([np.arange(j * 64, min(300, j * 64 + 64)) for j in kidx[t // 128]])
        want = vf[sel].mean(0)
        assert np.allclose(res["decl"][r], want, atol=1e-12)
        assert np.allclose(res["exact"][r], want, atol=1e-12)


def test_sparse_equals_dense_on_gathered_blocks(orc):
    # The sparse branch over kept blocks equals the dense branch run on a
    # problem whose keys are exactly those blocks (same int8 rows and scales).
    q, k, v = make_qkv(1, 1, 1000, 128, seed=15)
    qb, kb, vb = (_bits(t).reshape(1, 1000, 128) for t in (q, k, v))
    qi, qs, ki, ks, mu = orc.quant_qk(qb, kb)
    kidx = np.array([[1, 5, 15]] * 8, np.int32)  # block 15 = tokens 960..999 (tail)
    toks = [3, 500, 999]
    res = orc.sparse_rows(qi, qs, ki, ks, vb, 0, toks, kidx_head=kidx)
    sel = np.concatenate([np.arange(64, 128), np.arange(320, 384), np.arange(960, 1000)])
    ks2 = ks[:, [1, 5, 15]].copy()
    for r, t in enumerate(toks):
        # a problem of exactly the 168 gathered keys (blocks of 64, 64, 40),
        # with the query row placed at its token 0 and run densely
        q3 = np.zeros((1, len(sel), 128), np.int8)
        q3[0, 0] = qi[0, t]
        res3 = orc.sparse_rows(q3, np.full((1, 2), qs[0, t // 128], np.float32),
                               ki[:, sel].copy(), ks2, vb[:, sel].copy(), 0, [0])
        assert np.allclose(res["decl"][r], res3["decl"][0], rtol=0, atol=1e-15)
        assert np.allclose(res["exact"][r], res3["exact"][0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("N", [256, 1000])
def test_full_density_close_to_fp64_dense_attention(orc, N):
    # BASELINE pin: at 100% block density with the linear branch off, both
    # numerics stay within cosine 0.999 of fp64 softmax attention on the
    # unquantized inputs.
    q, k, v = make_qkv(1, 2, N, 128, seed=16)
    qb, kb, vb = (_bits(t).reshape(2, N, 128) for t in (q, k, v))
    qi, qs, ki, ks, mu = orc.quant_qk(qb, kb)
    toks = np.arange(N)
    for bh in range(2):
        res = orc.sparse_rows(qi, qs, ki, ks, vb, bh, toks)
        ref = orc.dense_rows(qb, kb, vb, bh, toks)
        for key in ("decl", "exact"):
            a, b = res[key].ravel(), ref.ravel()
            cos = a @ b / np.linalg.norm(a) / np.linalg.norm(b)
            assert cos >= 0.999, (key, cos)


def test_smoothing_reduces_quantization_error(orc):
    # With outlier channels in K, quantizing K - mean is more accurate than
    # quantizing K itself (the purpose of the smoothing on page 5, Pillar One).
    N = 512
    q, k, v = make_qkv(1, 1, N, 128, seed=17, offset_std=8.0)
    qb, kb, vb = (_bits(t).reshape(1, N, 128) for t in (q, k, v))
    qi, qs, ki, ks, mu = orc.quant_qk(qb, kb)
    ki0, ks0 = orc.quant(kb, np.zeros_like(mu), 64)
    toks = np.arange(0, N, 3)
    ref = orc.dense_rows(qb, kb, vb, 0, toks)
    e_sm = np.linalg.norm(orc.sparse_rows(qi, qs, ki, ks, vb, 0, toks)["exact"] - ref)
    e_raw = np.linalg.norm(orc.sparse_rows(qi, qs, ki0, ks0, vb, 0, toks)["exact"] - ref)
    assert e_sm < 0.5 * e_raw, (e_sm, e_raw)


def test_dense_fp64_matches_torch_sdpa(orc):
    q, k, v = make_qkv(1, 1, 200, 128, seed=18)
    qb, kb, vb = (_bits(t).reshape(1, 200, 128) for t in (q, k, v))
    toks = np.arange(200)
    got = orc.dense_rows(qb, kb, vb, 0, toks)
    qd, kd, vd = (t.reshape(1, 1, 200, 128).double() for t in (q, k, v))
    sm = float(np.float32(1.0 / math.sqrt(128)))  # the oracle's default scale is fp32
    want = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, scale=sm)[0, 0].numpy()
    assert np.max(np.abs(got - want)) < 1e-12


def test_amb_flags_a_near_midpoint(orc):
    # c chosen so that 2^(c - 1) sits within 2^-24 of the bf16 midpoint
    # 200.5/256: that p may round either way on a GPU, so amb > 0; a row whose
    # p are exact powers of two has amb = 0.
    N, D = 2, 128
    qi = np.zeros((1, N, D), np.int8)
    qi[0, :, 0] = 1
    ki = np.zeros((1, N, D), np.int8)
    ki[0, 0, 0] = 1
    ki[0, 1, 0] = 0
    v = np.zeros((1, N, D), np.float32)
    v[0, 0, 0] = 1.0
    vb = _bits(torch.from_numpy(v))
    sm = float(np.float32(math.log(2.0)))
    c = np.float32(1.0 + math.log2(200.5 / 256))
    res = orc.sparse_rows(qi, np.ones((1, 1), np.float32), ki, np.full((1, 1), c, np.float32),
                          vb, 0, [0], sm_scale=sm)
    assert res["amb"][0] > 0
    res = orc.sparse_rows(qi, np.ones((1, 1), np.float32), ki, np.ones((1, 1), np.float32),
                          vb, 0, [0], sm_scale=sm)
    assert res["amb"][0] == 0


def _bf16_round_array(x):
    """RNE of float64 values in the normal range straight to bf16."""
    _, e = np.frexp(x)
    q = e - 8
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


@pytest.mark.parametrize("lag", [0, 16, 64])
def test_flip_window_covers_a_lagging_normalizer(orc, lag):
    # A GPU forms y = fma(S, c, -m') in fp32 against an integer normalizer m'
    # that may sit up to 64 below the row's m = ceil(max), takes 2^y with about
    # one fp32 ulp of error and rounds to bf16; scaling by 2^(m' - m) is exact.
    # Emulated here exactly (S*c is exact in fp64, one rounding to fp32), on p
    # placed within 2^-17 of bf16 midpoints: every p whose rounding differs
    # from the oracle's must lie inside the oracle's flip window.
    rng = np.random.default_rng(2)
    n = 60000
    b = 128 + rng.integers(0, 128, n)
    tgt = np.log2((b + 0.5) / 256.0 * (1 + rng.uniform(-2**-17, 2**-17, n)))
    c = 2.0**-21
    x = np.rint(tgt / c) * c                  # x = S c, S an integer
    m = 0.0
    yg = (x - (m - lag)).astype(np.float32).astype(np.float64)
    po = _bf16_round_array(np.exp2(x - m))
    flips = 0
    for sgn in (-1, 1):
        pg = _bf16_round_array(np.exp2(yg) * (1 + sgn * 2**-23)) * 2.0**-lag
        idx = np.nonzero(pg != po)[0]
        flips += len(idx)
        for a in idx:
            pe = 2.0**(x[a] - m)
            assert orc.p_ambiguous(pe, abs(x[a]), abs(x[a]), m) > 0, (lag, x[a])
    assert flips > 0
    if lag == 64:
        # the window without the lag term is too narrow here: the pin bites
        pe = np.exp2(x - m)
        _, e = np.frexp(pe)
        ulp = np.ldexp(1.0, e - 8)
        dist = np.abs(pe / ulp - np.floor(pe / ulp) - 0.5) * ulp
        narrow = dist <= pe * (2**-20 + 2**-23 * (2 * np.abs(x) + 2.0))
        pg = _bf16_round_array(np.exp2(yg) * (1 - 2**-23)) * 2.0**-lag
        assert np.any((pg != po) & ~narrow)


# --------------------------------------------------------------------------
# linear branch (page 5, Pillar Two: the linear-attention term)

def _phi(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def test_phi_values():
    assert _phi(np.array([0.0]))[0] == 1.0 and _phi(np.array([1.0]))[0] == 2.0
    assert abs(_phi(np.array([-1.0]))[0] - math.exp(-1)) < 1e-16


def test_linear_branch_equals_token_level_linear_attention(orc):
    N = 700  # 11 key blocks, the last one 60 tokens; 6 query blocks
    q, k, v = make_qkv(1, 2, N, 128, seed=19)
    qb, kb, vb = (_bits(t).reshape(2, N, 128) for t in (q, k, v))
    keep = 3
    kidx, _ = orc.block_mask(qb, kb, keep)
    toks = np.array([0, 1, 127, 128, 400, 650, 699])
    for bh in range(2):
        h, z = orc.linear_states(kb, vb, bh)
        got = orc.linear_rows(qb, h, z, bh, toks, kidx[bh])
        qf, kf, vf = (_f(x)[bh].astype(np.float64) for x in (qb, kb, vb))
        for r, t in enumerate(toks):
            kept = set(kidx[bh][t // 128])
            comp = [u for u in range(N) if (u // 64) not in kept]
            w = _phi(kf[comp]) @ _phi(qf[t])  # phi(q).phi(k_u) per complement token
            want = (w[:, None] * vf[comp]).sum(0) / w.sum()
            assert np.max(np.abs(got[r] - want)) < 1e-12 * (1 + np.max(np.abs(want)))


def test_linear_branch_zero_when_everything_kept(orc):
    N = 300
    q, k, v = make_qkv(1, 1, N, 128, seed=20)
    qb, kb, vb = (_bits(t).reshape(1, N, 128) for t in (q, k, v))
    h, z = orc.linear_states(kb, vb, 0)
    kidx = np.tile(np.arange(5, dtype=np.int32), (3, 1))
    got = orc.linear_rows(qb, h, z, 0, [0, 200, 299], kidx)
    assert np.all(got == 0)
    got = orc.linear_rows(qb, h, z, 0, [0, 200], None)
    assert np.all(got == 0)


def test_linear_states_sum_to_global_linear_attention(orc):
    # With no block kept the branch is global linear attention over all keys.
    N = 260
    q, k, v = make_qkv(1, 1, N, 128, seed=21)
    qb, kb, vb = (_bits(t).reshape(1, N, 128) for t in (q, k, v))
    h, z = orc.linear_states(kb, vb, 0)
    qf, kf, vf = (_f(x)[0].astype(np.float64) for x in (qb, kb, vb))
    fk = _phi(kf)
    assert np.allclose(h.sum(0), fk.T @ vf, rtol=1e-13, atol=1e-10)
    assert np.allclose(z.sum(0), fk.sum(0), rtol=1e-13)


# ---------------------------------------------------------------------------
# W8A8 linear layer (page 5, Pillar Three: INT8 weights and activations,
# block-wise 128x128). y = x . w^T with x [M][K], w [N][K].

def _bf16_matrix(a):
    """float array -> bf16 bit patterns (RNE), as numpy uint16."""
    return _bits(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)))


def test_w8a8_quant_golden_ties(orc):
    # one 128x128 block whose amax is 127 has scale 1.0 exactly: the quantized
    # values are the round-half-even integers of the inputs
    x = np.zeros((128, 256), np.float32)
    x[0, 0] = 127.0
    vals = [2.5, -3.5, 0.5, 1.5, -0.5, 126.5, -127.0]
    want = [2, -4, 0, 2, 0, 126, -127]
    for n, v in enumerate(vals):
        x[1 + n, 3 + n] = v
    x[5, 200] = 3.0  # second column block: amax 3, scale 3/127
    q, s = orc.w8a8_quant(_bf16_matrix(x))
    assert s.shape == (1, 2)
    assert s[0, 0] == np.float32(1.0)
    assert s[0, 1] == np.float32(3.0) / np.float32(127.0)
    for n, w in enumerate(want):
        assert q[1 + n, 3 + n] == w
    assert q[0, 0] == 127 and q[5, 200] == 127
    assert np.count_nonzero(q) == len([w for w in want if w]) + 2


def test_w8a8_quant_partial_row_block_and_invariants(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((300, 384)).astype(np.float32)
    x[256:, 128:256] *= 40.0  # the partial last row block alone is large
    xb = _bf16_matrix(x)
    q, s = orc.w8a8_quant(xb)
    xf = _f(xb)
    assert s.shape == (3, 3)
    for rb in range(3):
        for cb in range(3):
            blk = xf[128 * rb:128 * (rb + 1), 128 * cb:128 * (cb + 1)]
            qb = q[128 * rb:128 * (rb + 1), 128 * cb:128 * (cb + 1)].astype(np.float64)
            amax = np.float32(np.abs(blk).max())
            assert s[rb, cb] == amax / np.float32(127.0)  # only the block's own rows count
            assert np.abs(qb).max() == 127
            err = np.abs(blk.astype(np.float64) - qb * float(s[rb, cb]))
            assert err.max() <= float(s[rb, cb]) / 2 * (1 + 2.0 ** -20)


def test_w8a8_gemm_is_the_exact_fma_chain(orc):
    # independent recomputation in exact rational arithmetic: int64 block sums,
    # s = fl32(sx * sw), then y = fl32(I * s + y) per column block in order
    rng = np.random.default_rng(5)
    M, K, N = 5, 384, 128
    x = _bf16_matrix(rng.standard_normal((M, K)) * 3)
    w = _bf16_matrix(rng.standard_normal((N, K)) * 0.05)
    xq, sx = orc.w8a8_quant(x)
    wq, sw = orc.w8a8_quant(w)
    y = orc.w8a8_gemm(xq, sx, wq, sw)
    for m in range(M):
        for n in range(0, N, 7):
            acc = Fraction(0)
            for kb in range(K // 128):
                sl = slice(128 * kb, 128 * (kb + 1))
                i = int(np.dot(xq[m, sl].astype(np.int64), wq[n, sl].astype(np.int64)))
                s = f32_of(Fraction(float(sx[m // 128, kb])) * Fraction(float(sw[n // 128, kb])))
                acc = Fraction(f32_of(Fraction(i) * Fraction(s) + acc))
            assert y[m, n] == np.float32(float(acc)), (m, n)


def test_w8a8_gemm_bias_is_one_fp32_add(orc):
    # the bias enters after the chain as one IEEE single add (numpy float32
    # arithmetic, an implementation independent of the oracle's C), and a
    # bias equal to the negated product gives exact zeros
    rng = np.random.default_rng(9)
    M, K, N = 7, 256, 256
    x = _bf16_matrix(rng.standard_normal((M, K)))
    w = _bf16_matrix(rng.standard_normal((N, K)) * 0.05)
    xq, sx = orc.w8a8_quant(x)
    wq, sw = orc.w8a8_quant(w)
    y = orc.w8a8_gemm(xq, sx, wq, sw)
    bias = (rng.standard_normal(N) * 3).astype(np.float32)
    yb = orc.w8a8_gemm(xq, sx, wq, sw, bias=bias)
    assert np.array_equal(yb.view(np.uint32), (y + bias[None, :]).astype(np.float32).view(np.uint32))
    assert np.all(orc.w8a8_gemm(xq, sx, wq, sw, rows=[3], bias=-y[3]) == 0.0)


def test_w8a8_gemm_power_of_two_scales_is_an_integer_product(orc):
    # every block's amax is 127 * 2^e, so every scale is a power of two, every
    # quantized value is x / scale exactly, and the product is exact integers
    rng = np.random.default_rng(7)
    M, K, N = 130, 256, 256
    ex = rng.integers(-3, 3, size=(2, 2))
    ew = rng.integers(-3, 3, size=(2, 2))
    xi = rng.integers(-127, 128, size=(M, K))
    wi = rng.integers(-127, 128, size=(N, K))
    for rb in range(2):
        for cb in range(2):
            xi[128 * rb, 128 * cb] = 127
            wi[128 * rb, 128 * cb] = -127
    x = np.zeros((M, K)); w = np.zeros((N, K))
    for rb in range(2):
        for cb in range(2):
            rs, cs = slice(128 * rb, 128 * (rb + 1)), slice(128 * cb, 128 * (cb + 1))
            x[rs, cs] = xi[rs, cs] * 2.0 ** ex[rb, cb]
            w[rs, cs] = wi[rs, cs] * 2.0 ** ew[rb, cb]
    xq, sx = orc.w8a8_quant(_bf16_matrix(x))
    wq, sw = orc.w8a8_quant(_bf16_matrix(w))
    assert np.array_equal(xq, xi) and np.array_equal(wq, wi)
    y = orc.w8a8_gemm(xq, sx, wq, sw)
    want = np.zeros((M, N))
    for kb in range(2):
        cs = slice(128 * kb, 128 * (kb + 1))
        prod = xi[:, cs].astype(np.int64) @ wi[:, cs].astype(np.int64).T
        scale = (2.0 ** ex[(np.arange(M) // 128), kb])[:, None] * (2.0 ** ew[(np.arange(N) // 128), kb])[None, :]
        want += prod * scale
    assert np.array_equal(y.astype(np.float64), want)


def test_w8a8_gemm_close_to_fp64_product(orc):
    # the quantized product stays within the 8-bit quantization error of the
    # plain fp64 product of the bf16 operands
    rng = np.random.default_rng(11)
    M, K, N = 200, 512, 256
    x = _bf16_matrix(rng.standard_normal((M, K)))
    w = _bf16_matrix(rng.standard_normal((N, K)) * 0.02)
    xq, sx = orc.w8a8_quant(x)
    wq, sw = orc.w8a8_quant(w)
    y = orc.w8a8_gemm(xq, sx, wq, sw).astype(np.float64)
    ref = _f(x).astype(np.float64) @ _f(w).astype(np.float64).T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 2e-2, rel


# --------------------------------------------------------------------------
# backward (page 5: SLA is trainable; the quantizer passes gradients straight
# through, the block selection is held fixed)

def _bwd_case(orc, N, D, topk, seed, branches=3):
    q, k, v = make_qkv(1, 1, N, D, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    dout = torch.randn(1, 1, N, D, generator=g).to(torch.bfloat16)
    qb, kb, vb, gb = (_bits(t).reshape(1, N, D) for t in (q, k, v, dout))
    qi, qs, ki, ks, _ = orc.quant_qk(qb, kb)
    kidx = None
    if topk is not None:
        keep = orc.keep_blocks(N, topk)
        kidx, _ = orc.block_mask(qb, kb, keep)
        kidx = kidx[0]
    dq, dk, dv = orc.sagesla_bwd(qb, kb, vb, (qi, qs, ki, ks), 0, gb, kidx, branches)
    # the continuous inputs the gradient is taken in
    qh = qi[0].astype(np.float64) * np.repeat(qs[0].astype(np.float64), 128)[:N, None]
    kh = ki[0].astype(np.float64) * np.repeat(ks[0].astype(np.float64), 64)[:N, None]
    f = lambda t: t.float().numpy().reshape(N, D).astype(np.float64)  # noqa: E731
    return dict(q=f(q), k=f(k), v=f(v), dout=f(dout), qh=qh, kh=kh, kidx=kidx,
                dq=dq, dk=dk, dv=dv, branches=branches)


@pytest.mark.parametrize("N,topk,branches", [(200, 0.5, 3), (200, 0.5, 1), (200, 0.5, 2),
                                             (130, None, 1)])
def test_backward_matches_central_differences(orc, N, topk, branches):
    # D = 32 keeps the loss cheap; every formula is generic in D. Each checked
    # entry moves the sparse and the linear input of Q (or K) together: the
    # straight-through reading.
    D = 32
    c = _bwd_case(orc, N, D, topk, seed=N + branches, branches=branches)
    sm = float(np.float32(1.0 / np.sqrt(D)))
    args = dict(kidx_head=c["kidx"], branches=branches, sm=sm)

    def loss(qh, kh, vv, ql, kl):
        return orc.sagesla_loss(qh, kh, vv, ql, kl, c["dout"], **args)

    rng = np.random.default_rng(7)
    h = 1e-5
    for name in ("dq", "dk", "dv"):
        for _ in range(6):
            t, d = int(rng.integers(0, N)), int(rng.integers(0, D))
            ins = {n: c[n].copy() for n in ("qh", "kh", "v", "q", "k")}
            pairs = {"dq": ("qh", "q"), "dk": ("kh", "k"), "dv": ("v",)}[name]
            vals = []
            for sgn in (1, -1):
                x = {n: a.copy() for n, a in ins.items()}
                for n in pairs:
                    x[n][t, d] += sgn * h
                vals.append(loss(x["qh"], x["kh"], x["v"], x["q"], x["k"]))
            fd = (vals[0] - vals[1]) / (2 * h)
            an = c[name][t, d]
            scale = max(1.0, np.abs(c[name]).max())
            assert abs(fd - an) <= 1e-6 * scale, (name, t, d, fd, an)


def test_backward_sparse_dense_matches_torch_autograd(orc):
    # full density, sparse branch: the gradient of sum(dO * softmax(sm qh kh^T) v)
    # by torch's fp64 autograd on the dequantized operands
    N, D = 300, 64
    c = _bwd_case(orc, N, D, None, seed=5, branches=1)
    sm = float(np.float32(1.0 / np.sqrt(D)))
    qh = torch.tensor(c["qh"], requires_grad=True)
    kh = torch.tensor(c["kh"], requires_grad=True)
    vv = torch.tensor(c["v"], requires_grad=True)
    o = torch.softmax(sm * qh @ kh.T, dim=-1) @ vv
    (o * torch.tensor(c["dout"])).sum().backward()
    for got, want in ((c["dq"], qh.grad), (c["dk"], kh.grad), (c["dv"], vv.grad)):
        want = want.numpy()
        assert np.abs(got - want).max() <= 1e-10 * max(1.0, np.abs(want).max())


def test_backward_invariants(orc):
    # every query row's dS sums to zero over its keys, so the sparse dK summed
    # over all keys vanishes; its softmax weights sum to one, so the sparse dV
    # summed over all keys equals dO summed over all queries (each query block
    # keeps at least one block); zero dO gives zero gradients; with every block
    # kept the linear branch contributes nothing
    N, D = 640, 32
    c = _bwd_case(orc, N, D, 0.3, seed=11, branches=1)
    assert np.abs(c["dk"].sum(axis=0)).max() <= 1e-10 * np.abs(c["dk"]).max()
    assert np.allclose(c["dv"].sum(axis=0), c["dout"].sum(axis=0), rtol=0, atol=1e-9)
    q, k, v = make_qkv(1, 1, N, D, seed=3)
    qb, kb, vb = (_bits(t).reshape(1, N, D) for t in (q, k, v))
    quant = orc.quant_qk(qb, kb)[:4]
    zero = np.zeros_like(qb)
    keep = orc.keep_blocks(N, 0.3)
    kidx = orc.block_mask(qb, kb, keep)[0][0]
    for g in orc.sagesla_bwd(qb, kb, vb, quant, 0, zero, kidx, 3):
        assert not g.any()
    gb = _bits(torch.randn(1, N, D).to(torch.bfloat16)).reshape(1, N, D)
    nkb = orc.nkb(N)
    allk = np.tile(np.arange(nkb, dtype=np.int32), (orc.nqb(N), 1))
    a = orc.sagesla_bwd(qb, kb, vb, quant, 0, gb, allk, 3)
    b = orc.sagesla_bwd(qb, kb, vb, quant, 0, gb, None, 1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("topk,branches", [(0.3, 3), (None, 1)])
def test_backward_sampled_rows_equal_the_full_backward(orc, topk, branches):
    # restricting the work to sampled rows and keys leaves those rows bit for
    # bit as the full computation gives them
    N, D = 700, 64
    q, k, v = make_qkv(1, 1, N, D, seed=21)
    qb, kb, vb = (_bits(t).reshape(1, N, D) for t in (q, k, v))
    quant = orc.quant_qk(qb, kb)[:4]
    kidx = None
    if topk is not None:
        kidx = orc.block_mask(qb, kb, orc.keep_blocks(N, topk))[0][0]
    g = torch.Generator().manual_seed(22)
    dout = _bits(torch.randn(1, N, D, generator=g).to(torch.bfloat16)).reshape(1, N, D)
    full = orc.sagesla_bwd(qb, kb, vb, quant, 0, dout, kidx, branches=branches)
    qrows = np.array([0, 5, 127, 128, 300, N - 1])
    kcols = np.array([1, 63, 64, 200, 640, N - 1])
    part = orc.sagesla_bwd(qb, kb, vb, quant, 0, dout, kidx, branches=branches, qrows=qrows,
                           kcols=kcols)
    assert np.array_equal(part[0][qrows], full[0][qrows])
    for n in (1, 2):
        assert np.array_equal(part[n][kcols], full[n][kcols])


def test_w8a8_gemm_f64_is_the_exact_block_dequantization(orc):
    # an int64 matmul per K block (numpy), times the fp64 product of the two
    # fp32 scales, summed over blocks; and the fp32 chain stays within its
    # rounding bound of it
    M, N, K = 200, 256, 384
    rng = np.random.default_rng(4)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((N, K)) * 0.05).astype(np.float32)).to(torch.bfloat16)
    xq, sx = orc.w8a8_quant(_bits(x).reshape(M, K))
    wq, sw = orc.w8a8_quant(_bits(w).reshape(N, K))
    y, ya = orc.w8a8_gemm_f64(xq, sx, wq, sw)
    want = np.zeros((M, N))
    want_abs = np.zeros((M, N))
    for kb in range(K // 128):
        sl = slice(128 * kb, 128 * kb + 128)
        I = xq[:, sl].astype(np.int64) @ wq[:, sl].astype(np.int64).T
        s = sx[np.arange(M) // 128, kb].astype(np.float64)[:, None] * \
            sw[np.arange(N) // 128, kb].astype(np.float64)[None, :]
        want += I * s
        want_abs += np.abs(I) * s
    assert np.allclose(y, want, rtol=1e-13, atol=0) and np.allclose(ya, want_abs, rtol=1e-13)
    y32 = orc.w8a8_gemm(xq, sx, wq, sw).astype(np.float64)
    nkb = K // 128
    assert np.all(np.abs(y32 - y) <= (nkb + 2) * 2.0**-24 * ya)
