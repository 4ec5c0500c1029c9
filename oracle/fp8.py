"""FP8 (E4M3) attention (oracle; test infrastructure).

The Sparse VideoGen verdict page (pith_extraction.core_discovery and
forward_implications; skeptic_critique.rationale) reports an optional FP8
quantization of attention, worth about 1.3x on HunyuanVideo, and gives no
scheme.  Readings taken here, the plainest FP8 attention that leaves the
block mask and the softmax as they are:
  * format: OCP FP8 E4M3 -- 1 sign bit, 4 exponent bits with bias 7, 3
    mantissa bits, subnormals, no infinities, largest finite 448, NaN only
    as S.1111.111 -- with round to nearest, ties to even;
  * Q, K and V are quantized per (batch, head) with a power-of-two factor
    2^e: e is the largest integer with amax * 2^e <= 448, amax the largest
    |x| over the head's tokens and channels (e = 0 when amax = 0), clamped
    to [-32, 32];
  * scores are the dequantized product s = scale * (q8 . k8) * 2^-(e_q+e_k);
  * probabilities are quantized too, against the power of two at or above
    the row maximum: with t = s * log2(e) and r = ceil(max t) over the
    row's kept keys, p8 = E4M3(2^(t - r + 8)), so every p8 <= 256;
  * O = 2^-e_v * sum_j p8_j v8_j / sum_j p8_j (the normalisation uses the
    quantized probabilities that multiply V).
Everything is computed in fp64 on the exact dequantized values; a power of
two times an E4M3 value is exact in fp64.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
EXP_CLAMP = 32


def e4m3_decode(codes):
    """Values of E4M3 codes (uint8 array) from the bit fields; NaN codes
    give NaN."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_round(x):
    """Round fp64 values to the nearest E4M3 value, ties to even mantissa.

    Below 2^-6 the grid is the subnormal one (spacing 2^-9); in the binade
    [2^E, 2^(E+1)) it is 2^(E-3).  Values must satisfy |x| <= 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(~np.isfinite(a)) or np.any(a > E4M3_MAX):
        raise ValueError("E4M3 rounding needs finite |x| <= 448")
    _, ex = np.frexp(a)                       # a = m * 2^ex, m in [0.5, 1)
    E = np.maximum(ex - 1, -6)                # binade exponent (subnormals share -6)
    quantum = np.exp2(E - 3.0)
    n = np.rint(a / quantum)                  # exact quotient; rint ties to even
    return np.copysign(n * quantum, x)


def e4m3_encode(x):
    """E4M3 codes of fp64 values (|x| <= 448), round to nearest even: the
    bit fields of the rounded value (exponent field E + 7 and mantissa
    8 * (a / 2^E - 1) for a >= 2^-6; exponent field 0 and mantissa a / 2^-9
    below)."""
    r = e4m3_round(x)
    a = np.abs(r)
    _, ex = np.frexp(a)
    E = ex - 1
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, E + 7, 0)
    man = np.where(normal, (np.ldexp(a, -E) - 1.0) * 8.0, np.ldexp(a, 9))
    codes = (exp_field.astype(np.int64) << 3) | man.astype(np.int64)
    # the sign survives rounding to zero (-0 is 0x80), as in IEEE rounding
    return (codes | np.where(np.signbit(r), 0x80, 0)).astype(np.uint8)


def scale_exponent(amax):
    """Largest integer e with amax * 2^e <= 448 (0 for amax = 0), clamped
    to [-32, 32].  Found by exact comparisons (ldexp is exact)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    _, ex = np.frexp(amax)
    e = 9 - int(ex)
    while np.ldexp(amax, e) > E4M3_MAX:
        e -= 1
    while np.ldexp(amax, e + 1) <= E4M3_MAX:
        e += 1
    return int(min(max(e, -EXP_CLAMP), EXP_CLAMP))


def quantize_head(x):
    """x [N, d] (one head, values exact in fp64).  Returns (codes uint8
    [N, d], e)."""
    x = np.asarray(x, dtype=np.float64)
    e = scale_exponent(np.abs(x).max() if x.size else 0.0)
    return e4m3_encode(np.ldexp(x, e)), e


def prob_exponents(q8v, k8v, eq, ek, scale):
    """t = s * log2(e) for dequantized-code inputs q8v [nq, d], k8v [nk, d]
    (the decoded E4M3 values before the 2^-e factors), fp64."""
    s = (np.asarray(q8v, np.float64) @ np.asarray(k8v, np.float64).T) * np.ldexp(1.0, -(eq + ek)) * scale
    return s / np.log(2.0)


def quantized_probs(t):
    """Per row: r = ceil(max t), p8 = E4M3(2^(t - r + 8)).  Returns
    (p_exact, p8, r) with p_exact = 2^(t - r + 8) before rounding."""
    t = np.asarray(t, dtype=np.float64)
    r = np.ceil(t.max(axis=1, keepdims=True))
    p = np.exp2(t - r + 8.0)
    return p, e4m3_round(p), r


def fp8_attention_dense(q8v, k8v, v8v, eq, ek, ev, scale):
    """O [nq, d] of one query set over its kept keys (all rows of k8v,
    v8v), from decoded codes and the head's exponents."""
    t = prob_exponents(q8v, k8v, eq, ek, scale)
    _, p8, _ = quantized_probs(t)
    l = p8.sum(axis=1, keepdims=True)
    return np.ldexp((p8 @ np.asarray(v8v, np.float64)) / l, -ev)


def quantize_qkv(q, k, v):
    """Per-head quantization of one head's q, k, v ([N, d] each).  Returns
    decoded values (q8v, k8v, v8v), codes (qc, kc, vc) and exponents
    (eq, ek, ev)."""
    qc, eq = quantize_head(q)
    kc, ek = quantize_head(k)
    vc, ev = quantize_head(v)
    return (e4m3_decode(qc), e4m3_decode(kc), e4m3_decode(vc)), (qc, kc, vc), (eq, ek, ev)


def block_sparse_fp8_attention(q, k, v, members, rows, query_tiles=None, scale=None):
    """One head, FP8 path.  q, k, v [N, d] (bf16 values as fp64);
    rows[i] = kept key tiles of query tile i.  Returns fp64 O [N, d]."""
    N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    (q8v, k8v, v8v), _, (eq, ek, ev) = quantize_qkv(q, k, v)
    out = np.zeros((N, d), dtype=np.float64)
    tiles = range(len(members)) if query_tiles is None else query_tiles
    for i in tiles:
        if not rows[i]:
            continue
        qi = members[i]
        keys = np.concatenate([members[j] for j in rows[i]])
        out[qi] = fp8_attention_dense(q8v[qi], k8v[keys], v8v[keys], eq, ek, ev, scale)
    return out
