"""Pins of the FP8 oracle (oracle/fp8.py) against things other than itself.

E4M3 facts come from the OCP 8-bit floating point format definition (bias
7, 3 mantissa bits, subnormals, largest finite 448, NaN S.1111.111); the
rounding is checked against torch's float8_e4m3fn conversion (a library
routine) and hand-worked ties; the attention reduces to the pinned softmax
oracle when quantization is exact, and hand-computed probability
quantizations catch a wrong reference power or a dropped rounding.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, fp8


def _torch_codes(x):
    return torch.tensor(np.asarray(x, np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_format_facts():
    assert fp8.e4m3_decode(0x38) == 1.0
    assert fp8.e4m3_decode(0x7E) == 448.0          # largest finite
    assert fp8.e4m3_decode(0x08) == 2.0 ** -6      # smallest normal
    assert fp8.e4m3_decode(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert fp8.e4m3_decode(0x01) == 2.0 ** -9      # smallest subnormal
    assert fp8.e4m3_decode(0xB8) == -1.0
    assert math.isnan(fp8.e4m3_decode(0x7F)) and math.isnan(fp8.e4m3_decode(0xFF))
    assert np.signbit(fp8.e4m3_decode(0x80)) and fp8.e4m3_decode(0x80) == 0.0
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    assert len(set(fp8.e4m3_decode(np.array(finite)).tolist())) == 253  # +0 and -0 compare equal


def test_encode_inverts_decode_on_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


def test_encode_matches_torch_on_random_values_and_midpoints():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000) * np.exp2(rng.uniform(-14, 8, 100000))
    x = np.clip(x, -448, 448)
    assert np.array_equal(fp8.e4m3_encode(x), _torch_codes(x))
    v = np.sort(fp8.e4m3_decode(np.arange(0, 0x7F)))
    mids = (v[:-1] + v[1:]) / 2
    ties = np.concatenate([mids, -mids])
    assert np.array_equal(fp8.e4m3_encode(ties), _torch_codes(ties))


def test_ties_go_to_even_mantissa():
    assert fp8.e4m3_round(1.0625) == 1.0          # between 1 and 1.125 -> even 1.0
    assert fp8.e4m3_round(1.1875) == 1.25         # between 1.125 and 1.25 -> even 1.25
    assert fp8.e4m3_round(2.0 ** -10) == 0.0      # half the smallest subnormal -> 0
    assert fp8.e4m3_round(3 * 2.0 ** -10) == 2.0 ** -8
    assert fp8.e4m3_round(240.0) == 240.0 and fp8.e4m3_round(248.0) == 256.0
    with pytest.raises(ValueError):
        fp8.e4m3_round(449.0)


def test_scale_exponent_edges():
    assert fp8.scale_exponent(448.0) == 0
    assert fp8.scale_exponent(449.0) == -1
    assert fp8.scale_exponent(1.0) == 8           # 256 <= 448 < 512
    assert fp8.scale_exponent(0.875) == 9         # 0.875 * 512 = 448 exactly
    assert fp8.scale_exponent(0.0) == 0
    assert fp8.scale_exponent(2.0 ** -40) == 32   # clamped
    rng = np.random.default_rng(1)
    for a in np.exp2(rng.uniform(-20, 20, 500)):
        e = fp8.scale_exponent(a)
        assert a * 2.0 ** e <= 448 < a * 2.0 ** (e + 1)


def test_quantize_head_codes_match_torch():
    rng = np.random.default_rng(2)
    x = torch.tensor(rng.standard_normal((64, 32)) * 3).to(torch.bfloat16).double().numpy()
    codes, e = fp8.quantize_head(x)
    assert e == fp8.scale_exponent(np.abs(x).max())
    assert np.array_equal(codes, _torch_codes(np.ldexp(x, e)))


def test_exact_quantization_reduces_to_softmax_attention():
    # q in {0,1,2}, k in {-1,0,1}, v in {-3..3}: every scaled value lies on
    # the E4M3 grid, and with scale = ln 2 every t = q.k is an integer, so
    # every 2^(t - r + 8) is an exact power of two >= 2^-8.
    rng = np.random.default_rng(3)
    d, nq, nk = 4, 6, 40
    q = rng.integers(0, 3, (nq, d)).astype(np.float64)
    k = rng.integers(-1, 2, (nk, d)).astype(np.float64)
    v = rng.integers(-3, 4, (nk, d)).astype(np.float64)
    q[0, 0], v[0, 0] = 2.0, 3.0
    (q8v, k8v, v8v), _, (eq, ek, ev) = fp8.quantize_qkv(q, k, v)
    assert np.array_equal(np.ldexp(q8v, -eq), q) and np.array_equal(np.ldexp(v8v, -ev), v)
    got = fp8.fp8_attention_dense(q8v, k8v, v8v, eq, ek, ev, math.log(2.0))
    want = attention.attention_dense(q, k, v, scale=math.log(2.0))
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_probability_quantization_by_hand():
    one = np.array([[1.0]])
    k = np.array([[0.0], [-1.0]])
    v = np.array([[1.0], [3.0]])
    # t = (0, -0.1): r = 0, p = (256, 256 * 2^-0.1 = 238.9 -> 240)
    got = fp8.fp8_attention_dense(one, k, v, 0, 0, 0, 0.1 * math.log(2.0))
    assert got[0, 0] == pytest.approx((256 * 1 + 240 * 3) / 496, rel=1e-15)
    # t = (0.3, 0.2): r = ceil(0.3) = 1, p = (2^7.3 = 157.6 -> 160, 2^7.2 = 147.0 -> 144)
    k2 = np.array([[3.0], [2.0]])
    got = fp8.fp8_attention_dense(one, k2, v, 0, 0, 0, 0.1 * math.log(2.0))
    assert got[0, 0] == pytest.approx((160 * 1 + 144 * 3) / 304, rel=1e-15)
    # the exponents scale what they should: 2^-(eq+ek) on scores, 2^-ev on O
    got = fp8.fp8_attention_dense(one, k2 * 4, v, 1, 1, 3, 0.1 * math.log(2.0))
    assert got[0, 0] == pytest.approx((160 * 1 + 144 * 3) / 304 / 8, rel=1e-15)
    # subnormal probabilities: t - r + 8 = -9.5 -> 2^-9.5 = 0.00138 -> 2^-9
    p, p8, r = fp8.quantized_probs(np.array([[0.0, -17.5, -16.0]]))
    assert r[0, 0] == 0 and p8[0, 0] == 256 and p8[0, 1] == 2.0 ** -9 and p8[0, 2] == 2.0 ** -8


def test_block_sparse_fp8_close_to_exact_attention():
    # quantization error only: the FP8 result stays near the exact one
    rng = np.random.default_rng(4)
    N, d = 64, 32
    q, k, v = (torch.tensor(rng.standard_normal((N, d))).to(torch.bfloat16).double().numpy() for _ in range(3))
    members = [np.arange(0, 32), np.arange(32, 64)]
    rows = [[0, 1], [1]]
    got = fp8.block_sparse_fp8_attention(q, k, v, members, rows)
    want = attention.block_sparse_attention(q, k, v, members, rows)
    assert np.abs(got - want).max() < 0.1
    assert np.abs(got - want).mean() < 0.02
