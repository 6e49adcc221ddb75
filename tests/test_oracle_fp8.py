"""Pins of the oracle's V quantization (OCP FP8 E4M3, power-of-two scale per head and channel).

Fixed independently of the oracle's code by:
  * a library routine: torch's float8_e4m3fn conversion (round to nearest, ties to
    even) encodes a large sample of float32 values, ties, subnormals and the range
    ends exactly as the oracle does, and decodes all 256 codes to the same values;
  * closed forms of the format: 448 = 0x7e, 2^-6 = 0x08, 2^-9 = 0x01, 1 = 0x38,
    -0 = 0x80, the NaN codes, and hand-worked ties;
  * the scale rule by brute force over candidate exponents;
  * the quantization error bound of a 3-bit mantissa (half a unit in the last
    place: 2^-4 relative, or 2^-10 times the scale below the normal range), and
    values that the format holds exactly coming back unchanged;
  * quantized attention: with values the format holds exactly it equals the plain
    attention; with constant values it returns the constant;
  * the weight-rounding bound of attention_tile_spread, by perturbing the weights
    (at random and adversarially) within the stated relative error.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import absh_oracle as O


def torch_encode(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_decode(codes):
    return torch.tensor(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def test_encode_matches_library_conversion():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.normal(0, 50, 20000), rng.normal(0, 1e-2, 20000), rng.uniform(-464, 464, 20000),
        # exact ties: midpoints between neighbouring codes, normal and subnormal
        (torch_decode(np.arange(0, 126)).astype(np.float64) + torch_decode(np.arange(1, 127))) / 2,
        -(torch_decode(np.arange(0, 126)).astype(np.float64) + torch_decode(np.arange(1, 127))) / 2,
        [0.0, -0.0, 448.0, -448.0, 464.0, -464.0, 2.0 ** -6, 2.0 ** -9, 2.0 ** -10, 2.0 ** -11, 1e-30],
    ]).astype(np.float32)
    got = O.e4m3_encode(x)
    want = torch_encode(x)
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:10]


def test_decode_matches_library_and_closed_forms():
    codes = np.arange(256)
    got = O.e4m3_decode(codes)
    want = torch_decode(codes).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.isnan(got).sum() == 2
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0
    assert got[0x80] == 0.0 and math.copysign(1.0, got[0x80]) == -1.0
    assert got[0x07] == 7 * 2.0 ** -9 and got[0x0F] == 1.875 * 2.0 ** -6   # largest subnormal, 2nd binade top


def test_worked_ties():
    # 1.0625 lies halfway between 1.0 (mantissa 000) and 1.125 (001): the even one wins
    # subnormal ties: 1.5 and 0.5 quanta (2^-9) go to 2 and 0 quanta
    assert O.e4m3_encode([1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10, 464.0]).tolist() == [0x38, 0x3A, 0x02, 0x00, 0x7E]
    with pytest.raises(ValueError):
        O.e4m3_encode([465.0])


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F])
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes)


@settings(max_examples=200, deadline=None)
@given(st.floats(min_value=1e-30, max_value=1e30, allow_nan=False, allow_infinity=False))
def test_scale_exponent_is_smallest(amax):
    amax = float(np.float32(amax))
    e = int(O.v_scale_exponent(amax))
    assert math.ldexp(amax, -e) <= 448.0 < math.ldexp(amax, -(e - 1))
    assert int(O.v_scale_exponent(0.0)) == 0


def test_quantization_error_bound():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((500, 16)) * np.exp(rng.uniform(-20, 20, 16))[None, :]).astype(np.float32)
    v[:, 3] = 0.0
    codes, e = O.quantize_v(v)
    vt = O.dequantize_v(codes, e)
    amax = np.abs(v).max(axis=0)
    live = amax > 0
    top = amax[live] * np.ldexp(1.0, -e[live])
    assert (top > 224.0).all() and (top <= 448.0).all()        # one binade of headroom at most
    err = np.abs(vt - v)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, np.ldexp(1.0, e - 10)[None, :])
    assert (err <= bound).all()
    assert (vt[:, 3] == 0).all() and e[3] == 0


def test_representable_values_come_back_exactly():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 0x7F, size=(64, 8))
    v = O.e4m3_decode(codes) * 2.0 ** 5
    v[0] = 448.0 * 2.0 ** 5                                     # pins the scale to 2^5
    c2, e = O.quantize_v(v)
    assert (e == 5).all() and np.array_equal(O.dequantize_v(c2, e), v)


def test_quantized_attention_special_cases():
    rng = np.random.default_rng(5)
    B, N, H, d = 1, 30, 2, 8
    q = rng.standard_normal((B, N, H, d)).astype(np.float32)
    k = rng.standard_normal((B, N, H, d)).astype(np.float32)
    perm, _ = O.hilbert_perm(2, 3, 5)
    # values the format holds exactly (small integers) are unchanged by the quantization
    v_int = rng.integers(-8, 9, size=(B, N, H, d)).astype(np.float32)
    v_int[0, 0, :, :] = 8.0
    assert np.array_equal(O.quantized_v(v_int), v_int)
    a = O.attention(q, k, O.quantized_v(v_int), perm, 4)
    assert np.array_equal(a, O.attention(q, k, v_int, perm, 4))
    # constant values: the output is the (quantized) constant, whatever the weights
    v_c = np.full((B, N, H, d), 0.3, np.float32)
    vq = O.quantized_v(v_c)
    assert np.allclose(O.attention(q, k, vq, perm, 4), vq[0, 0, 0, 0], rtol=0, atol=1e-12)
    assert abs(vq[0, 0, 0, 0] - 0.3) <= 0.3 * 2.0 ** -4


def test_spread_bounds_weight_rounding():
    rng = np.random.default_rng(6)
    N, d, block = 40, 6, 8
    q = rng.standard_normal((N, d)) * 2
    k = rng.standard_normal((N, d)) * 2
    v = rng.standard_normal((N, d)) + 3.0
    kv = [0, 2, 3]
    O_, A1, A2, As = O.attention_tile_spread(q, k, v, block, 1, kv, small=0.02)
    assert np.allclose(O_, O.attention_tile(q, k, v, block, 1, kv), rtol=0, atol=1e-13)
    keys = np.concatenate([np.arange(j * block, (j + 1) * block) for j in kv])
    s = q[block:2 * block] @ k[keys].T / math.sqrt(d)
    P = np.exp(s - s.max(axis=1, keepdims=True))
    u = 2.0 ** -4
    for trial in range(50):
        delta = rng.uniform(-u, u, P.shape)
        Pt = P * (1 + delta)
        Ot = (Pt @ v[keys]) / Pt.sum(axis=1, keepdims=True)
        assert (np.abs(Ot - O_) <= u / (1 - u) * A1 + 1e-12).all()
    # adversarial: push every weight of values above the output up, the others down
    for c in range(d):
        sign = np.sign(v[keys][None, :, c] - O_[:, c][:, None])
        Pt = P * (1 + u * sign)
        Ot = (Pt @ v[keys][:, c]) / Pt.sum(axis=1)
        assert (np.abs(Ot - O_[:, c]) <= u / (1 - u) * A1[:, c] + 1e-12).all()
        assert (np.abs(Ot - O_[:, c]) >= 0.5 * u * A1[:, c]).all()   # the bound is within a factor ~2 of tight
    # absolute changes of at most a in the normalised weights at or below `small`
    a = 1e-3
    w = P / P.sum(axis=1, keepdims=True)
    for trial in range(50):
        dw = np.where(w <= 0.02, rng.uniform(-a, a, w.shape), 0.0)
        Ot = ((w + dw) @ v[keys]) / (w + dw).sum(axis=1, keepdims=True)
        lo = 1 - a * (w <= 0.02).sum(axis=1, keepdims=True)     # the renormalisation
        assert (np.abs(Ot - O_) <= a * As / lo + 1e-12).all()
    # a single key: no spread
    one = O.attention_tile_spread(q[:1], k[:1], v[:1], 1, 0, [0], small=1.0)
    assert (one[1] == 0).all() and (one[2] == 0).all() and (one[3] == 0).all()
    assert (A2 <= A1 + 1e-15).all()
    # every key counted when small >= 1, none when small < min weight
    full = O.attention_tile_spread(q, k, v, block, 1, kv, small=1.0)[3]
    assert np.allclose(full, np.abs(v[keys][None, :, :] - O_[:, None, :]).sum(axis=1), rtol=1e-12, atol=0)
    assert (O.attention_tile_spread(q, k, v, block, 1, kv, small=0.0)[3] == 0).all()
