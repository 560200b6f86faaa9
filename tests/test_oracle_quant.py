"""Pins of the oracle's 4-bit K/V codes (CPU only).

* The page's number: 4-bit codes plus an fp16 norm per head vector take
  3.88x less memory than bf16 at head_dim 128 (Dendrite page, TurboQuant).
* The quantizer table is the 16-level Lloyd-Max quantizer of the unit
  normal: decision levels are midpoints of neighbouring reconstruction
  levels, each reconstruction level is the mean of the normal over its cell
  (computed here with scipy), and the distortion is the published 0.009497.
* The rotation is orthogonal and the code of each coordinate is the nearest
  reconstruction level of the rotated, scaled coordinate (brute force).
* Symmetries: negating a vector mirrors its codes, doubling it doubles the
  norm and keeps the codes.
* Gaussian vectors come back with the quantizer's distortion; attention
  over the codes equals textbook attention over the dequantized vectors and
  stays close to attention over the original ones.
"""

import math

import numpy as np
import pytest
from scipy import stats

import synth
from oracle import PoolModel, bf16_bits_to_f64, decode
from oracle.quant import (DECISION_POS, LEVELS, MAX_MSE, RECON_POS, decode_q4, dequantize,
                          fp16_nearest_sqrt, hadamard, quantize, rotation)


def bits(rng, shape, scale=1.0):
    return synth.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))


def test_compression_ratio_matches_the_page():
    d = 128
    bf16_bytes = 2 * d
    q4_bytes = d // 2 + 2          # 4-bit codes + fp16 norm
    assert round(bf16_bytes / q4_bytes, 2) == 3.88


def test_table_is_the_lloyd_max_quantizer_of_the_normal():
    r = np.array(RECON_POS)
    b = np.array((0.0,) + DECISION_POS + (np.inf,))
    # decision levels: midpoints
    assert np.allclose(DECISION_POS, (r[:-1] + r[1:]) / 2, atol=6e-5)
    # reconstruction levels: conditional means of N(0,1) over their cells
    lo, hi = b[:-1], b[1:]
    mean = (stats.norm.pdf(lo) - stats.norm.pdf(hi)) / (stats.norm.cdf(hi) - stats.norm.cdf(lo))
    assert np.allclose(r, mean, atol=2e-4)
    # distortion: E (X - Q(X))^2 over both halves
    mse = 0.0
    for a, c, rr in zip(lo, hi, r):
        m2 = lambda t: stats.norm.expect(lambda x: (x - rr) ** 2, lb=a, ub=t)
        mse += 2 * m2(c)
    assert abs(mse - MAX_MSE) < 1e-5      # the table is printed to 4 decimals
    assert LEVELS == tuple(sorted(LEVELS)) and len(LEVELS) == 16


@pytest.mark.parametrize("d", [8, 64, 128])
def test_rotation_is_orthogonal(d):
    h = hadamard(d)
    assert np.array_equal(h @ h.T, d * np.eye(d))
    s = np.random.default_rng(d).choice([-1.0, 1.0], size=d)
    r = rotation(s)
    assert np.allclose(r @ r.T, np.eye(d), atol=1e-14)


@pytest.mark.parametrize("d", [64, 128])
def test_codes_are_nearest_levels(d):
    rng = np.random.default_rng(d + 1)
    s = rng.choice([-1, 1], size=d)
    x = bits(rng, (200, d))
    codes, _ = quantize(x, s)
    xf = bf16_bits_to_f64(x)
    u = (xf @ rotation(s).T) * math.sqrt(d) / np.linalg.norm(xf, axis=1, keepdims=True)
    lv = np.array(LEVELS)
    near = np.abs(u[..., None] - lv).argmin(axis=-1)
    edge = np.min(np.abs(np.abs(u[..., None]) - np.array((0.0,) + DECISION_POS)), axis=-1) < 1e-4
    assert np.all((codes == near) | edge)


def test_symmetries():
    rng = np.random.default_rng(3)
    s = rng.choice([-1, 1], size=64)
    x = bits(rng, (50, 64))
    c, n = quantize(x, s)
    cneg, nneg = quantize(x ^ np.uint16(0x8000), s)
    nonzero = np.abs((bf16_bits_to_f64(x) * s) @ hadamard(64).T) > 0
    assert np.array_equal(cneg[nonzero], (15 - c)[nonzero]) and np.array_equal(nneg, n)
    x2 = synth.f32_to_bf16_bits(bf16_bits_to_f64(x).astype(np.float32) * np.float32(2))
    c2, n2 = quantize(x2, s)
    assert np.array_equal(c2, c)
    assert np.array_equal(n2.view(np.float16).astype(np.float64), 2 * n.view(np.float16).astype(np.float64))


@pytest.mark.parametrize("d", [64, 128])
def test_gaussian_vectors_come_back_with_the_quantizer_distortion(d):
    rng = np.random.default_rng(d + 7)
    s = rng.choice([-1, 1], size=d)
    x = bits(rng, (4000, d))
    xf = bf16_bits_to_f64(x)
    xh = dequantize(*quantize(x, s), s)
    rel = ((xh - xf) ** 2).sum(-1) / (xf ** 2).sum(-1)
    assert abs(rel.mean() - MAX_MSE) < 0.1 * MAX_MSE


def test_attention_over_codes():
    rng = np.random.default_rng(11)
    L, Hkv, D, B, Hq = 2, 2, 64, 16, 8
    s = rng.choice([-1, 1], size=D)
    pool = PoolModel(64, B, L, Hkv, D)
    a = pool.allocate()
    k, v = bits(rng, (L, 1, 300, Hkv, D)), bits(rng, (L, 1, 300, Hkv, D))
    pool.append([a], 300, k, v)
    b = pool.fork(a)
    pool.append([b], 5, bits(rng, (L, 1, 5, Hkv, D)), bits(rng, (L, 1, 5, Hkv, D)))
    q = bits(rng, (2, Hq, D))
    for layer in range(L):
        out, lse = decode_q4(pool, layer, [a, b], q, 0.125, s)
        exact, _ = decode(pool, layer, [a, b], q, 0.125)
        # the same attention written out per token from the codes
        kb, vb = pool.gather_bits(b, layer)
        kc, kn = quantize(kb, s)
        vc, vn = quantize(vb, s)
        lv = np.array(LEVELS)
        qf = bf16_bits_to_f64(q[1])
        for h in range(Hq):
            g = h // (Hq // Hkv)
            qh = hadamard(D) @ (s * qf[h])
            z = np.array([0.125 * kn[t, g].view(np.float16) / D * (qh * lv[kc[t, g]]).sum()
                          for t in range(kc.shape[0])])
            p = np.exp(z - z.max())
            acc = (p[:, None] * vn[:, g].view(np.float16).astype(np.float64)[:, None]
                   * lv[vc[:, g]]).sum(0)
            o = s * (hadamard(D) @ acc) / D / p.sum()
            assert np.allclose(out[1, h], o, atol=1e-12)
            assert math.isclose(lse[1, h], z.max() + math.log(p.sum()), abs_tol=1e-12)
        # close to attention over the original bf16 vectors
        assert np.abs(out - exact).mean() < 0.05


def test_norm_is_the_nearest_fp16_of_the_square_root():
    """Brute force over every positive finite fp16: the stored norm of S is
    the fp16 closest to sqrt(S) (exact rational comparison), ties to even."""
    from fractions import Fraction
    rng = np.random.default_rng(5)
    all_h = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    # S from bf16 sums of squares, plus exact squares of fp16 values and of midpoints
    x = bits(rng, (300, 64)).astype(np.uint32) << 16
    S = list((x.view(np.float32).astype(np.float64) ** 2).sum(-1))
    S += [v * v for v in all_h[::97]]
    S += [(0.5 * (a + b)) ** 2 for a, b in zip(all_h[:-1:211], all_h[1::211])]
    got = fp16_nearest_sqrt(np.array(S)).view(np.float16).astype(np.float64)
    for s_, g in zip(S, got):
        fs = Fraction(s_)
        i = np.searchsorted(all_h, np.sqrt(s_))
        cands = [c for c in all_h[max(0, i - 2):i + 2]]
        # |c - sqrt(S)| compared through (c^2 - S) signs: pick by squared midpoints
        best = min(cands, key=lambda c: (abs(Fraction(c) ** 2 - fs) / (Fraction(c) + Fraction(np.sqrt(s_)))))
        if best != g:
            # only a tie may differ, and then g must have the even mantissa
            lo, hi = sorted([best, g])
            mid = (Fraction(lo) + Fraction(hi)) / 2
            assert mid * mid == fs
            assert int(np.float16(g).view(np.uint16)) % 2 == 0
