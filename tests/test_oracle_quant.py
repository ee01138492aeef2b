"""Pins for the oracle's preparation steps: K mean, INT8 blocks, E4M3 V, cache requant.

Closed forms (reconstruction bounds, absmax maps to the top code, zero blocks, padding),
exact rational arithmetic for the mean, brute-force nearest codes, and the bit-exact
shift invariance of K smoothing on a dyadic construction.
"""
import fractions

import numpy as np

import workloads as W


def _bf16(x):
    return W.bf16_bits(np.asarray(x, dtype=np.float32))


def test_k_mean_exact_rational(orc):
    rng = np.random.default_rng(5)
    B, N, H, D = 2, 77, 3, 8
    k = _bf16(rng.standard_normal((B, N, H, D)) * 3 + 1)
    mean, inexact = orc.k_mean(k)
    assert inexact == 0
    kf = W.bf16_to_f32(k).astype(np.float64)
    for b in range(B):
        for h in range(H):
            for c in range(D):
                s = sum(fractions.Fraction(float(v)) for v in kf[b, :, h, c])
                # contract: fp64 sum (exact here), one fp64 division, one fp32 rounding
                ref = np.float32(float(s) / N)
                assert float(s) == fractions.Fraction(float(s)) == s  # the fp64 sum is exact
                assert mean[b, h, c] == ref


def test_k_mean_strided_view(orc):
    """A projection-strided view [B,N,3,H,D][:, :, 1] gives the same mean as a copy."""
    rng = np.random.default_rng(6)
    qkv = _bf16(rng.standard_normal((1, 50, 3, 2, 16)))
    k_view = qkv[:, :, 1]
    m1, _ = orc.k_mean(k_view)
    m2, _ = orc.k_mean(np.ascontiguousarray(k_view))
    assert np.array_equal(m1, m2)


def _check_i8(orc, xf, codes, scales, N):
    """xf: fp32 values actually quantized [B,N,H,D]; codes [B,H,Npad,D]; scales [B,H,nblk]."""
    B, _, H, D = xf.shape
    npad = codes.shape[2]
    for b in range(B):
        for h in range(H):
            for blk in range(npad // 64):
                r0, r1 = blk * 64, min(N, blk * 64 + 64)
                s = scales[b, h, blk]
                cb = codes[b, h, blk * 64:blk * 64 + 64].astype(np.int32)
                if r1 <= r0:
                    assert s == 0 and not cb.any()
                    continue
                x = xf[b, r0:r1, h, :]
                a = np.float32(np.abs(x).max())
                if a == 0:
                    assert s == 0 and not cb.any()
                    continue
                assert s == np.float32(a / np.float32(127.0))
                c = cb[: r1 - r0]
                # reconstruction bound: |x - code*s| <= s/2 (plus fp32 slack of the reciprocal)
                err = np.abs(x.astype(np.float64) - c * np.float64(s))
                assert np.all(err <= 0.5 * s * (1 + 1e-5) + 1e-30)
                # the absmax element maps to +-127
                idx = np.unravel_index(np.argmax(np.abs(x)), x.shape)
                assert abs(c[idx]) == 127
                # padding rows are zero codes
                assert not cb[r1 - r0:].any()
                # brute force: nearest integer of fl32(x * fl32(127/a)), ties to even
                r = np.float32(np.float32(127.0) / a)
                t = (x * r).astype(np.float32).astype(np.float64)
                ks = np.arange(-127, 128, dtype=np.float64)
                d = np.abs(t[..., None] - ks)
                best = d.min(axis=-1, keepdims=True)
                cand = d == best
                pick_even = np.where(cand & (ks % 2 == 0), ks, 999).min(axis=-1)
                pick_any = np.where(cand, ks, 999).min(axis=-1)
                ref = np.where(cand.sum(axis=-1) > 1, pick_even, pick_any)
                assert np.array_equal(c, ref.astype(np.int32))


def test_quant_q_blocks_closed_forms(orc):
    rng = np.random.default_rng(8)
    B, N, H, D = 1, 150, 2, 64  # 3 blocks, ragged last block (22 rows)
    q = _bf16(rng.standard_normal((B, N, H, D)) * np.exp2(rng.uniform(-3, 3, (B, N, H, 1))))
    q[0, 64:128, 1, :] = 0  # an all-zero block
    codes, scales = orc.quant_i8_blocks(q)
    assert codes.shape == (1, 2, 192, 64) and scales.shape == (1, 2, 3)
    assert scales[0, 1, 1] == 0
    _check_i8(orc, W.bf16_to_f32(q), codes, scales, N)


def test_quant_k_smoothed_closed_forms(orc):
    rng = np.random.default_rng(9)
    B, N, H, D = 1, 100, 2, 32
    off = rng.uniform(-2, 2, (1, 1, H, D)).astype(np.float32)
    k = _bf16(rng.standard_normal((B, N, H, D)).astype(np.float32) + off)
    mean, _ = orc.k_mean(k)
    codes, scales = orc.quant_i8_blocks(k, mean)
    kf = W.bf16_to_f32(k)
    ks = (kf - mean[:, None, :, :]).astype(np.float32)  # fl32(K - mu)
    _check_i8(orc, ks, codes, scales, N)
    # the smoothed values have (near) zero channel means
    assert np.abs(ks.mean(axis=1)).max() < 1e-5


def test_smoothing_shift_invariance_bit_exact(orc):
    """Dyadic construction: K values k/16 (|k| < 256) and a per-channel shift c (multiple of
    1/16, |K + c| < 16).  Then K + c, the fp64 sum, the mean and K' are all exact, so the
    INT8 codes, the scales and the attention output are bit-identical with and without c."""
    rng = np.random.default_rng(10)
    B, N, H, D = 1, 256, 2, 64
    kint = rng.integers(-100, 100, (B, N, H, D))
    shift = rng.integers(-60, 60, (1, 1, H, D))
    k0 = _bf16(kint / 16.0)
    k1 = _bf16((kint + shift) / 16.0)
    assert np.array_equal(W.bf16_to_f32(k1).astype(np.float64) * 16, (kint + shift).astype(np.float64))
    q = _bf16(rng.standard_normal((B, N, H, D)))
    v = _bf16(rng.standard_normal((B, N, H, D)))
    o0, it0 = orc.fwd(q, k0, v)
    o1, it1 = orc.fwd(q, k1, v)
    assert np.array_equal(it0["k8"], it1["k8"]) and np.array_equal(it0["k_scale"], it1["k_scale"])
    assert np.array_equal(o0, o1)
    assert not np.array_equal(it0["k_mean"], it1["k_mean"])


def test_quant_v_closed_forms(orc):
    rng = np.random.default_rng(13)
    B, N, H, D = 1, 90, 2, 16
    v = _bf16(rng.standard_normal((B, N, H, D)) * np.exp2(rng.uniform(-4, 4, (1, 1, H, D))))
    v[0, :, 1, 3] = 0  # a zero channel
    v[0, 5, 0, 2] = _bf16(-0.0)
    v8t, vs = orc.quant_v(v)
    assert v8t.shape == (1, 2, 16, 128)
    dec = orc.e4m3_decode_table()
    vf = W.bf16_to_f32(v)
    for h in range(H):
        for c in range(D):
            x = vf[0, :, h, c]
            a = np.float32(np.abs(x).max())
            col = v8t[0, h, c]
            assert not col[N:].any()  # padding
            if a == 0:
                assert vs[0, h, c] == 0 and not col.any()
                continue
            assert vs[0, h, c] == np.float32(a / np.float32(448.0))
            # absmax maps to +-448 exactly
            i = int(np.argmax(np.abs(x)))
            assert col[i] in (0x7E, 0xFE)
            # relative error of normal codes <= 2^-4 after undoing the scale
            y = (x * np.float32(np.float32(448.0) / a)).astype(np.float32).astype(np.float64)
            d = dec[col[:N]]
            normal = np.abs(y) >= 2.0 ** -6
            assert np.all(np.abs(d[normal] - y[normal]) <= np.abs(y[normal]) * 2.0 ** -4)
            assert np.all(np.abs(d[~normal] - y[~normal]) <= 2.0 ** -10)
    assert v8t[0, 0, 2, 5] == 0x80 or vf[0, 5, 0, 2] != 0  # -0 keeps its sign


def test_requant_v_cache(orc):
    rng = np.random.default_rng(14)
    H, Nk, D = 2, 70, 16
    vc, vts = W.int8_cache(3, 6, H, Nk, D)
    v8t, vs = orc.requant_v_cache(vc, vts)
    vf = (vc.astype(np.float32) * vts[:, :, None]).astype(np.float32)  # fl32(code * s_tok)
    dec = orc.e4m3_decode_table()
    for h in range(H):
        a = np.abs(vf[h]).max(axis=0).astype(np.float32)
        assert np.array_equal(vs[h], (a / np.float32(448.0)).astype(np.float32))
        r = (np.float32(448.0) / a).astype(np.float32)
        y = (vf[h] * r[None, :]).astype(np.float32)
        assert np.array_equal(v8t[h][:, :Nk].T, orc.e4m3_encode(y))
        assert not v8t[h][:, Nk:].any()
        assert np.all(np.abs(dec[v8t[h][:, :Nk]]).max(axis=1) == 448.0)


def test_reciprocal_overflow_clamped(orc):
    """A block whose absmax is below 127/FLT_MAX: the reciprocal saturates at FLT_MAX
    instead of overflowing, so codes stay finite (rne(x * FLT_MAX)) and no NaN appears."""
    fmax = np.float32(np.finfo(np.float32).max)
    tiny = np.float32(2.0 ** -127)  # a bf16-representable subnormal
    x = np.zeros((1, 64, 1, 64), np.float32)
    x[0, :, 0, 0] = tiny
    x[0, :, 0, 1] = -tiny / 2
    codes, scales = orc.quant_i8_blocks(W.bf16_bits(x))
    assert scales[0, 0, 0] == np.float32(tiny / np.float32(127.0))
    assert np.all(codes[0, 0, :, 0] == np.int8(np.rint(np.float32(tiny * fmax))))
    assert np.all(codes[0, 0, :, 1] == np.int8(np.rint(np.float32(-tiny / 2 * fmax))))
    v8t, vs = orc.quant_v(W.bf16_bits(x))
    assert v8t[0, 0, 0, 0] == orc.e4m3_encode(np.float32([tiny * fmax]))[0]
    assert v8t[0, 0, 2, 0] == 0x00
