"""Pins for the oracle's scalar codecs: E4M3 decode/encode, the exponential, bf16.

Each check ties the oracle to something other than itself: the OCP E4M3 definition's
closed-form values, torch's independent float8_e4m3fn conversion, an exhaustive
nearest-value search, a second exp2 route through long double, and decimal arithmetic.
"""
import decimal

import numpy as np
import pytest
import torch

import workloads as W


def _all_bf16_finite():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = W.bf16_to_f32(bits)
    return f[np.isfinite(f)]


def test_e4m3_decode_closed_forms(orc):
    t = orc.e4m3_decode_table()
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9  # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9  # largest subnormal
    assert t[0x08] == 2.0 ** -6  # smallest normal
    assert t[0x38] == 1.0 and t[0x40] == 2.0 and t[0x78] == 256.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0  # largest finite
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    pos = t[:127]
    assert np.all(np.diff(pos) > 0), "non-negative codes must decode in ascending order"
    assert np.array_equal(t[128:255], -t[:127])


def test_e4m3_decode_matches_torch(orc):
    t = orc.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = ~np.isnan(ref)
    assert np.array_equal(np.isnan(t), ~finite)
    assert np.array_equal(t[finite], ref[finite])


def test_e4m3_encode_all_bf16_vs_torch(orc):
    """Every finite bf16 value with |x| <= 464 (torch does not saturate above)."""
    f = _all_bf16_finite()
    f = f[np.abs(f) <= 464.0]
    ours = orc.e4m3_encode(f)
    ref = torch.from_numpy(f.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_random_fp32_vs_bruteforce(orc):
    """Exhaustive nearest-value search over all finite codes, ties to even mantissa."""
    rng = np.random.default_rng(7)
    # random magnitudes over the whole range plus exact midpoints and their neighbours
    mags = np.exp2(rng.uniform(-14, 9.5, 20000)).astype(np.float32)
    t = orc.e4m3_decode_table()
    pos = t[:127]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    x = np.concatenate([mags, -mags, near, -near, np.float32([0.0, -0.0, 447.9, 448.0, 460.0, 1e6, -1e6])])
    x = x.astype(np.float32)
    ours = orc.e4m3_encode(x)
    a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    dist = np.abs(a[:, None] - pos[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among tied candidates take the even code
    codes = np.arange(127)
    even_pick = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 999).min(axis=1)
    any_pick = np.where(cand, codes[None, :], 999).min(axis=1)
    pick = np.where(cand.sum(axis=1) > 1, even_pick, any_pick)
    ref = (pick | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)
    assert np.array_equal(ours, ref)


def test_e4m3_roundtrip_and_sign(orc):
    t = orc.e4m3_decode_table()
    finite = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.int64)
    vals = t[finite].astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(vals), finite.astype(np.uint8))
    assert orc.e4m3_encode(np.float32([-0.0]))[0] == 0x80
    assert orc.e4m3_encode(np.float32([np.nan]))[0] == 0x7F
    assert orc.e4m3_encode(np.float32([1e30, -1e30]))[0] == 0x7E


def test_exp2_integers_exact(orc):
    n = np.arange(-126, 128, dtype=np.float32)
    assert np.array_equal(orc.exp2(n), np.ldexp(np.float32(1), n.astype(np.int32)).astype(np.float32))
    assert orc.exp2(np.float32([-np.inf]))[0] == 0.0


def _exp2_cr_decimal(x: float) -> np.float32:
    """2^x correctly rounded to fp32 by 50-digit decimal arithmetic."""
    decimal.getcontext().prec = 50
    ln2 = decimal.Decimal(2).ln()
    exact = (decimal.Decimal(float(x)) * ln2).exp()
    f = np.float32(float(exact))
    lo, hi = np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))
    best = min((f, lo, hi), key=lambda c: (abs(decimal.Decimal(float(c)) - exact), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


def test_exp2_correctly_rounded_samples(orc):
    rng = np.random.default_rng(11)
    # grid exponents x = u - 80 (exact in fp32) for random grid arguments u in [40, 88],
    # plus plain random x
    u = rng.uniform(40.0, 88.0, 1500).astype(np.float32)  # x in [-40, 8]: P up to 256
    x = np.concatenate([(u - np.float32(80.0)).astype(np.float32), rng.uniform(-30, 8, 500).astype(np.float32)])
    got = orc.exp2(x)
    ref = np.array([_exp2_cr_decimal(v) for v in x], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.slow
def test_exp2_grid_settled_by_long_double(orc):
    """Over every softmax grid argument (all fp32 u in [16, 96)), P' = 2^(u - 80) rounds
    to the same fp32 through double and through long double: the oracle's P' is the
    correctly rounded power there (an ambiguous case would need 2^(u - 80) within
    2^-52 of an fp32 midpoint)."""
    lo = int(np.float32(16.0).view(np.uint32))
    hi = int(np.float32(96.0).view(np.uint32))
    assert orc.exp2_check_grid(lo, hi) == 0


def test_p8_code_grid_properties(orc):
    """P8 code of 2^(u - 80) is a monotone step function of u with the right anchors."""
    lo = int(np.float32(16.0).view(np.uint32))
    hi = int(np.float32(96.0).view(np.uint32))
    codes = orc.p8_codes_grid(lo, hi)
    assert np.all(np.diff(codes.astype(np.int32)) >= 0)
    u = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
    at = lambda val: codes[np.searchsorted(u, np.float32(val))]
    assert at(88.0) == 0x78  # x = 8 -> 256
    assert at(80.0) == 0x38  # x = 0 -> 1
    assert at(80.0 - 9.0) == 0x01  # x = -9 -> 2^-9
    assert at(80.0 - 10.0) == 0x00  # 2^-10: half the smallest subnormal, ties to even (0)
    assert at(80.0 - 11.0) == 0x00  # below half the smallest subnormal
    assert codes.max() <= 0x7E  # the oracle's encoder saturates at 448
    assert (codes[u > np.float32(88.81)] == 0x7E).all()  # P' = 2^(u - 80) > 448: saturated


def _exponent_arguments(rng, n, m_mag):
    """u = fl32(acc * c + fl32(88 - m_s)) for rows whose running max m_s = fl32(acc_max * c)
    has magnitude about m_mag (the softmax's exponent argument, computed exactly in
    fractions-free double arithmetic: acc * c is exact in double, the sum is rounded once
    to double and then to fp32, which cannot cross an fp32 rounding boundary here)."""
    acc_max = rng.integers(1 << 20, 1 << 21, n)
    acc = acc_max - rng.integers(0, 4, n)  # keys at or just below the row maximum
    sign = rng.choice([-1, 1], n)
    c = (m_mag / acc_max * rng.uniform(0.5, 2.0, n)).astype(np.float32)
    acc_max, acc = acc_max * sign, acc * sign
    m_s = (acc_max.astype(np.float64) * c.astype(np.float64)).astype(np.float32)
    m_s = np.maximum(m_s, (acc.astype(np.float64) * c.astype(np.float64)).astype(np.float32))
    b = (np.float32(88.0) - m_s).astype(np.float32)
    u = (acc.astype(np.float64) * c.astype(np.float64) + b.astype(np.float64)).astype(np.float32)
    return u, m_s


def test_exponent_argument_bound():
    """The bound the fused kernel's two softmax forms rest on: while |m_s| < 2^22 the
    exponent argument u exceeds 88 by at most (ulp(m_s) + ulp(88 - m_s)) / 2 + ulp(u) / 2
    <= 0.375 + 2^-17, so P' = 2^(u - 80) < 448 and no P code saturates; for larger |m_s|
    the argument passes 88.81 (saturated codes), which is why the kernel switches to its
    saturating form there."""
    rng = np.random.default_rng(11)
    for mag in (1.0, 2.0 ** 10, 2.0 ** 20, 2.0 ** 21.9):
        u, m_s = _exponent_arguments(rng, 200_000, mag)
        keep = np.abs(m_s) < 2.0 ** 22
        assert keep.sum() > 50_000
        assert u[keep].max() <= 88.375 + 2.0 ** -17, mag
    u, m_s = _exponent_arguments(rng, 200_000, 2.0 ** 24)
    assert (u > 88.81).any()  # reachable: the saturating form is needed


def test_bf16_rounding(orc):
    """Output rounding fp32 -> bf16: round to nearest even, checked against torch."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.exp2(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ours = np.array([orc.lib().orc_f32_to_bf16(float(v)) for v in x[:4000]], dtype=np.uint16)
    ref = torch.from_numpy(x[:4000].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_bits(x), torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
