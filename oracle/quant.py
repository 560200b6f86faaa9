"""4-bit K/V codes and attention over them, in float64 (test infrastructure).

What the pages fix: the Dendrite page compresses the KV cache to 4 bits
(TurboQuant) for 3.88x less memory and computes from the quantized indices
instead of dequantizing the cache on every call (Dendrite page, summary and
the "TurboQuant Integration" line; glossary "Quantization").  They give no
format.  The plain reading taken here, one that lands exactly on 3.88x at
head_dim 128:

* each token's K (and V) vector of one kv head, x in R^D, is stored as its
  norm ||x|| in fp16 plus D 4-bit codes: 2 + D/2 bytes against 2D bytes of
  bf16, 256 / 66 = 3.879 at D = 128;
* the direction is rotated before it is quantized, so every coordinate is
  close to N(0, 1/D) whatever x looks like (the rotate-then-scalar-quantize
  construction of vector quantizers such as TurboQuant): R = H diag(s) / sqrt(D)
  with H the Sylvester Hadamard matrix (H[i][j] = (-1)^popcount(i & j)) and
  s a seeded vector of random signs, handed in by the caller;
* each rotated coordinate, times sqrt(D), goes through the 16-level
  Lloyd-Max quantizer of the unit normal (J. Max, "Quantizing for minimum
  distortion", IRE Trans. Information Theory, 1960, table for 16 levels):
  reconstruction levels +-0.1284, 0.3881, 0.6568, 0.9423, 1.2562, 1.6180,
  2.0690, 2.7326 and decision levels 0, +-0.2582, 0.5224, 0.7996, 1.0993,
  1.4371, 1.8435, 2.4008 (mean squared error 0.009497);
* code j in 0..15 names level LEVELS[j] (ascending); a coordinate y of
  y_vec = H (s * x) is compared with the decision levels scaled by ||x||,
  y >= 0: code 8 + #{k : y^2 > b_k^2 S}, y < 0: code 7 - #{k : y^2 > b_k^2 S},
  S = sum x^2, b_k the positive decision levels -- all in float64, where
  y, y^2 and S are exact for bf16 inputs of ordinary range, so both sides
  take the same decision;
* the norm is stored as the fp16 value nearest to sqrt(S), ties to even
  (decided exactly: S and the squares of fp16 midpoints are exact in
  float64).

Dequantized vector: x_hat = n * R^T (LEVELS[code] / sqrt(D))
                          = n * s * (H LEVELS[code]) / D.
Attention over a 4-bit cache is textbook attention over the dequantized K
and V (the kernel computes the same thing from the codes: q.x_hat =
n / D * sum_d (H (s * q))_d LEVELS[code_d]).
"""

from __future__ import annotations

import numpy as np

from .attention import attend, bf16_bits_to_f64, _group
from .pool import ArgError, EmptyError

# Max (1960), 16 levels, unit-variance Gaussian: positive half
RECON_POS = (0.1284, 0.3881, 0.6568, 0.9423, 1.2562, 1.6180, 2.0690, 2.7326)
DECISION_POS = (0.2582, 0.5224, 0.7996, 1.0993, 1.4371, 1.8435, 2.4008)
LEVELS = tuple(-r for r in reversed(RECON_POS)) + RECON_POS     # code 0..15, ascending
MAX_MSE = 0.009497


def hadamard(d):
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1."""
    i = np.arange(d)
    pop = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pop % 2 == 0, 1.0, -1.0)


def rotation(signs):
    """R = H diag(s) / sqrt(D) (orthogonal)."""
    s = np.asarray(signs, dtype=np.float64)
    d = s.size
    return hadamard(d) * s[None, :] / np.sqrt(d)


def quantize(bits, signs):
    """bf16 bits [..., D] -> (codes uint8 [..., D], norm fp16 bits uint16 [...])."""
    x = bf16_bits_to_f64(bits)
    s = np.asarray(signs, dtype=np.float64)
    d = x.shape[-1]
    if s.shape != (d,):
        raise ArgError("one sign per dimension")
    y = (s * x) @ hadamard(d).T                      # H (s * x), exact for bf16 inputs
    S = (x * x).sum(axis=-1, keepdims=True)
    y2 = y * y
    level = np.zeros(y.shape, dtype=np.int64)
    for b in DECISION_POS:
        level += y2 > (b * b) * S
    codes = np.where(y >= 0, 8 + level, 7 - level).astype(np.uint8)
    return codes, fp16_nearest_sqrt(S[..., 0])


def fp16_nearest_sqrt(S):
    """Bits of the fp16 nearest to sqrt(S) (ties to even), for exact S >= 0.

    Start from float16(float64 sqrt) and step to a neighbour while S lies
    beyond the squared midpoint towards it.
    """
    S = np.asarray(S, dtype=np.float64)
    h = np.sqrt(S).astype(np.float16).view(np.uint16).astype(np.int64)
    val = lambda b: np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)
    for _ in range(2):
        v = val(h)
        lo = 0.5 * (v + val(np.maximum(h - 1, 0)))
        hi = 0.5 * (v + val(np.minimum(h + 1, 0x7BFF)))
        down = (h > 0) & ((S < lo * lo) | ((S == lo * lo) & (h % 2 == 1)))
        up = ~down & (h < 0x7BFF) & ((S > hi * hi) | ((S == hi * hi) & (h % 2 == 1)))
        h = h - down + up
    return h.astype(np.uint16)


def dequantize(codes, norm_bits, signs):
    """Codes [..., D] + fp16 norm bits [...] -> float64 vectors [..., D]."""
    lv = np.asarray(LEVELS, dtype=np.float64)[np.asarray(codes, dtype=np.int64)]
    n = np.asarray(norm_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    d = lv.shape[-1]
    return n[..., None] * (lv @ rotation(signs))  / np.sqrt(d)


def decode_q4(pool, layer, seqs, q_bits, sm_scale, signs):
    """Decode attention over the 4-bit codes of each sequence's K and V.

    Same rule as :func:`oracle.attention.decode` (the query attends to every
    cached token, its own included), with every cached K/V vector replaced by
    its dequantized 4-bit form.
    """
    q = bf16_bits_to_f64(q_bits)
    n, hq, d = q.shape
    g = _group(hq, pool.Hkv)
    out = np.empty((n, hq, d))
    lse = np.empty((n, hq))
    for i, sid in enumerate(seqs):
        kb, vb = pool.gather_bits(sid, layer)
        if kb.shape[0] == 0:
            raise EmptyError("decode on an empty sequence")
        k = dequantize(*quantize(kb, signs), signs)
        v = dequantize(*quantize(vb, signs), signs)
        for kvh in range(pool.Hkv):
            rows = slice(kvh * g, (kvh + 1) * g)
            out[i, rows], lse[i, rows] = attend(q[i, rows], k[:, kvh], v[:, kvh], sm_scale)
    return out, lse
