"""Pins of the oracle's group quantizer against what the pages and the arithmetic fix.

- invariants: codes in 0..L; every element within s/2 (plus two binary32 roundings) of its decoded value;
- closed forms: exact ties round to the even level; grid-exact groups reproduce their integers exactly;
- brute force: the code is the nearest level except within 2^-20 of a tie;
- special cases: constant groups, the smallest subnormal range (coverage guard), -0 minimum, +-65504 extremes;
- an exact-rational second path (fractions.Fraction and a textbook round-to-nearest-even into binary32/binary16)
  that must agree bit for bit with the numpy casts the oracle uses;
- grouping axes: keys per channel over 32 tokens and values per token over 32 channels (KIVI page, paragraph on
  the cache contents), checked through equivariance and isolation properties rather than by recomputation.
"""
import zlib
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant

F16_MIN_SUB = 2.0 ** -24


def _groups(rng, n, kind):
    if kind == "normal":
        x = rng.standard_normal((n, 32))
    elif kind == "outlier":
        x = rng.standard_normal((n, 32)) * np.where(rng.random((n, 1)) < 0.3, 20.0, 1.0)
    elif kind == "wide":
        x = rng.uniform(-60000, 60000, (n, 32))
    elif kind == "tiny":
        x = rng.standard_normal((n, 32)) * 1e-6
    elif kind == "subnormal":
        x = rng.integers(-40, 40, (n, 32)) * F16_MIN_SUB
    elif kind == "offset":
        x = 1000.0 + rng.standard_normal((n, 32)) * 0.5
    else:
        raise ValueError(kind)
    return x.astype(np.float16)


KINDS = ["normal", "outlier", "wide", "tiny", "subnormal", "offset"]


# ------------------------------------------------------------------ exact-rational second path
def _round_binary(x: Fraction, precision: int, emin: int) -> Fraction:
    """Round a rational to the nearest value of a binary format (precision bits, min normal exponent emin),
    ties to even, subnormals included (no overflow handling needed for the inputs used here)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - precision + 1)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def rn32(x):
    return _round_binary(x, 24, -126)


def rn16(x):
    return _round_binary(x, 11, -14)


def _next16_up(s: Fraction) -> Fraction:
    v = np.float16(float(s))
    return Fraction(float(np.nextafter(v, np.float16(np.inf))))


def exact_quantize(xs, bits):
    L = (1 << bits) - 1
    x = [Fraction(float(v)) for v in xs]
    mn, mx = min(x), max(x)
    r = rn32(mx - mn)
    s = rn16(rn32(r / L))
    if (L + Fraction(1, 2)) * s < r:
        s = _next16_up(s)
    z = mn
    if s == 0:
        return [0] * len(x), s, z
    codes = []
    for v in x:
        t = rn32(rn32(v - z) / s)
        q = round(t)                      # Fraction rounding: half to even
        codes.append(min(max(q, 0), L))
    return codes, s, z


@pytest.mark.parametrize("bits", [2, 4])
def test_rounding_chain_matches_exact_rationals(bits):
    rng = np.random.default_rng(7 + bits)
    groups = np.concatenate([_groups(rng, 60, k) for k in KINDS])
    special = np.array([
        [-65504.0, 65504.0] + [0.0] * 30,
        [0.0, F16_MIN_SUB] + [0.0] * 30,
        [-0.0] * 32,
        [1.0] * 31 + [np.nextafter(np.float16(1.0), np.float16(2.0))],
        [0.0, 3.0, 0.5, 1.5, 2.5] + [0.0] * 27,
        [-1.0, 2.0] + [0.5] * 30,
    ], np.float16)
    groups = np.concatenate([groups, special])
    codes, scale, zero = quant.quantize_groups(groups, bits)
    for i, g in enumerate(groups):
        c, s, z = exact_quantize(g, bits)
        assert list(codes[i]) == c, i
        assert Fraction(float(scale[i])) == s, i
        assert Fraction(float(zero[i])) == z, i
        assert not np.signbit(zero[i]) or zero[i] != 0


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("kind", KINDS)
def test_codes_in_range_and_error_bound(bits, kind):
    rng = np.random.default_rng(zlib.crc32(kind.encode()) + bits)
    x = _groups(rng, 4000, kind)
    codes, scale, zero = quant.quantize_groups(x, bits)
    L = (1 << bits) - 1
    assert codes.dtype == np.uint8 and codes.max() <= L
    xhat = quant.dequantize_groups(codes, scale, zero)
    err = np.abs(x.astype(np.float64) - xhat)
    bound = scale.astype(np.float64)[:, None] * (0.5 + 2.0 ** -21)
    assert np.all(err <= bound)
    # the minimum always gets code 0 and decodes exactly
    amin = x.astype(np.float64).argmin(axis=1)
    assert np.all(codes[np.arange(len(x)), amin] == 0)
    # with a normal-range binary16 scale, the maximum gets the top level
    normal = scale.astype(np.float64) >= 2.0 ** -14
    amax = x.astype(np.float64).argmax(axis=1)
    assert np.all(codes[np.arange(len(x)), amax][normal] == L)


def test_exact_ties_round_to_even():
    # s = 1, z = 0: endpoints 0 and 3; x = k + 1/2 lies exactly between two levels
    x = np.array([[0.0, 3.0, 0.5, 1.5, 2.5, 0.5, 1.5, 2.5] + [1.0] * 24], np.float16)
    codes, scale, zero = quant.quantize_groups(x, 2)
    assert float(scale[0]) == 1.0 and float(zero[0]) == 0.0
    assert list(codes[0, :8]) == [0, 3, 0, 2, 2, 0, 2, 2]
    # the same with s = 2^-3 and z = -4
    x2 = (x.astype(np.float64) / 8 - 4).astype(np.float16)
    c2, s2, z2 = quant.quantize_groups(x2, 2)
    assert float(s2[0]) == 0.125 and float(z2[0]) == -4.0
    assert np.array_equal(c2, codes)


@pytest.mark.parametrize("bits", [2, 4])
def test_grid_exact_groups_reproduce_integers(bits):
    rng = np.random.default_rng(3)
    L = (1 << bits) - 1
    for e in range(-20, 10):
        s = 2.0 ** e
        k = rng.integers(0, L + 1, 32)
        k[rng.integers(0, 32)] = 0
        k[(rng.integers(0, 31) + 1 + np.argmin(k)) % 32] = L
        z = s * rng.integers(-50, 50)
        x = (z + k * s).astype(np.float16)
        assert np.array_equal(x.astype(np.float64), z + k * s)   # representable exactly
        codes, scale, zero = quant.quantize_groups(x, bits)
        if L * s > 2.0 ** -14 * L:                              # normal-range scale
            assert float(scale) == s and float(zero) == z
            assert np.array_equal(codes, k)
        assert np.array_equal(quant.dequantize_groups(codes, scale, zero), x.astype(np.float64))


@pytest.mark.parametrize("kind", ["normal", "outlier", "offset"])
def test_nearest_level_brute_force(kind):
    rng = np.random.default_rng(11)
    x = _groups(rng, 3000, kind)
    codes, scale, zero = quant.quantize_groups(x, 2)
    s = scale.astype(np.float64)[:, None]
    z = zero.astype(np.float64)[:, None]
    levels = z[..., None] + np.arange(4) * s[..., None]                # [n, 1, 4]
    dist = np.abs(x.astype(np.float64)[..., None] - levels)
    nearest = dist.argmin(-1)
    t_exact = (x.astype(np.float64) - z) / s
    near_tie = np.abs(t_exact - np.floor(t_exact) - 0.5) < 2.0 ** -20
    agree = (nearest == codes) | near_tie
    assert np.all(agree)
    # at (near-)ties the code is one of the two neighbouring levels
    lo = np.floor(t_exact)
    assert np.all(((codes == lo) | (codes == lo + 1))[near_tie])


def test_constant_groups_and_guard():
    for c in [0.0, -0.0, 1.0, -3.5, 65504.0, F16_MIN_SUB]:
        x = np.full((1, 32), c, np.float16)
        codes, scale, zero = quant.quantize_groups(x, 2)
        assert float(scale[0]) == 0.0 and np.all(codes == 0)
        assert np.array_equal(quant.dequantize_groups(codes, scale, zero), x.astype(np.float64))
        assert not np.signbit(zero[0]) or float(zero[0]) != 0.0
    # range of one subnormal step: RN16(r / 3) underflows to 0, the guard raises s to the smallest subnormal
    x = np.array([[0.0, F16_MIN_SUB] + [0.0] * 30], np.float16)
    codes, scale, zero = quant.quantize_groups(x, 2)
    assert float(scale[0]) == F16_MIN_SUB
    assert list(codes[0, :2]) == [0, 1]
    # c and the next float16 above it
    c = np.float16(1.0)
    x = np.array([[c] * 31 + [np.nextafter(c, np.float16(2))]], np.float16)
    codes, scale, zero = quant.quantize_groups(x, 2)
    err = np.abs(quant.dequantize_groups(codes, scale, zero) - x.astype(np.float64))
    assert np.all(err <= float(scale[0]) / 2 * (1 + 2.0 ** -20))


def test_negative_zero_minimum_is_stored_positive():
    x = np.array([[-0.0, 0.5, 1.0] + [0.25] * 29], np.float16)
    _, _, zero = quant.quantize_groups(x, 2)
    assert float(zero[0]) == 0.0 and not np.signbit(zero[0])


def test_non_finite_rejected():
    x = np.zeros((1, 32), np.float16)
    x[0, 3] = np.inf
    with pytest.raises(ValueError):
        quant.quantize_groups(x, 2)


# ------------------------------------------------------------------ grouping axes
OUTLIER_CH = [3, 40, 77, 100]        # one per 32-channel group


def _k(rng, t=64, d=128):
    k = rng.standard_normal((t, d)).astype(np.float32)
    k[:, OUTLIER_CH] *= 20
    return k.astype(np.float16)


def test_keys_grouped_along_tokens_of_one_channel():
    rng = np.random.default_rng(5)
    k = _k(rng)
    codes, scale, zero = quant.quantize_keys_per_channel(k)
    assert codes.shape == (64, 128) and scale.shape == (2, 128)
    # scaling one channel by 4 (exact) scales only that channel's scale/zero; nothing else moves
    k2 = k.copy()
    k2[:, 10] = (k2[:, 10].astype(np.float32) * 4).astype(np.float16)
    c2, s2, z2 = quant.quantize_keys_per_channel(k2)
    others = np.arange(128) != 10
    assert np.array_equal(c2[:, others], codes[:, others]) and np.array_equal(s2[:, others], scale[:, others])
    assert np.array_equal(c2[:, 10], codes[:, 10])
    assert np.array_equal(s2[:, 10].astype(np.float64), scale[:, 10].astype(np.float64) * 4)
    # tokens of another 32-token tile do not influence a tile
    k3 = k.copy()
    k3[40] = k3[40] * np.float16(8)
    c3, s3, z3 = quant.quantize_keys_per_channel(k3)
    assert np.array_equal(c3[:32], codes[:32]) and np.array_equal(s3[0], scale[0]) and np.array_equal(z3[0], zero[0])
    # permuting tokens inside a tile permutes codes and keeps the per-channel scale
    perm = rng.permutation(32)
    c4, s4, z4 = quant.quantize_keys_per_channel(np.concatenate([k[:32][perm], k[32:]]))
    assert np.array_equal(c4[:32], codes[:32][perm]) and np.array_equal(s4, scale) and np.array_equal(z4, zero)
    # permuting channels permutes everything the same way
    pc = rng.permutation(128)
    c5, s5, z5 = quant.quantize_keys_per_channel(k[:, pc])
    assert np.array_equal(c5, codes[:, pc]) and np.array_equal(s5, scale[:, pc]) and np.array_equal(z5, zero[:, pc])


def test_values_grouped_along_channels_of_one_token():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((64, 128)).astype(np.float16)
    codes, scale, zero = quant.quantize_values_per_token(v)
    assert scale.shape == (64, 4)
    # changing one token leaves every other token untouched
    v2 = v.copy()
    v2[7] = v2[7] * np.float16(16)
    c2, s2, z2 = quant.quantize_values_per_token(v2)
    rows = np.arange(64) != 7
    assert np.array_equal(c2[rows], codes[rows]) and np.array_equal(s2[rows], scale[rows])
    # changing channel group 1 of a token leaves its groups 0, 2, 3 untouched
    v3 = v.copy()
    v3[9, 32:64] = v3[9, 32:64] * np.float16(4)
    c3, s3, z3 = quant.quantize_values_per_token(v3)
    assert np.array_equal(s3[9, [0, 2, 3]], scale[9, [0, 2, 3]])
    assert np.array_equal(c3[9, 32:64], codes[9, 32:64])


def test_per_channel_keys_confine_outlier_error():
    """The mechanism the KIVI page gives for per-channel keys: a token-wise group containing an outlier channel
    crushes the normal channels, a channel-wise group keeps the error in the outlier channel."""
    rng = np.random.default_rng(9)
    k = _k(rng, 256)
    normal = np.setdiff1d(np.arange(128), OUTLIER_CH)
    c, s, z = quant.quantize_keys_per_channel(k)
    err_ch = np.abs(quant.dequantize_keys(c, s, z) - k.astype(np.float64))[:, normal].mean()
    c2, s2, z2 = quant.quantize_values_per_token(k)          # the same tensor grouped per token
    err_tok = np.abs(quant.dequantize_values(c2, s2, z2) - k.astype(np.float64))[:, normal].mean()
    assert err_tok > 4 * err_ch
