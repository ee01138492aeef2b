"""Pins for the oracle's fused loop (INT8 QK, tile-ordered online softmax, FP8 PV, epilogue).

* closed forms: Q = 0 (uniform weights -> per-channel mean of V), causal Q = 0 (prefix
  means), Nk = 1, one-hot scores;
* exact brute force on the 1-4-tile boundary shapes: scores, weights and partial sums
  are exact by construction, so the oracle must equal FP64 softmax attention to the
  last bit of its single final rounding (this catches dropped or duplicated keys, wrong
  scale indices, masking and rescaling errors);
* V = 1: the normalized FP8 weights of every row sum to 1 within the FP8 error;
* FP64 softmax attention on the dequantized operands (rel-L2 <= 0.03) on random
  1-4-tile shapes, the tiny dense workload and a small prefill over an int8 cache.
"""
import numpy as np
import pytest

import workloads as W

TILE = 64
SHAPES = [1, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256]


def _npad(n):
    return (n + TILE - 1) // TILE * TILE


def _v_codes(orc, rng, H, D, Nk, values=(1.0, 1.5, 2.0, 3.0)):
    vals = np.array(values + tuple(-v for v in values), dtype=np.float32)
    codes = orc.e4m3_encode(vals)
    v8t = np.zeros((1, H, D, _npad(Nk)), dtype=np.uint8)
    v8t[..., :Nk] = codes[rng.integers(0, len(codes), (1, H, D, Nk))]
    vs = np.exp2(-rng.integers(0, 4, (1, H, D))).astype(np.float32)
    return v8t, vs


def _vd(orc, v8t, vs, Nk):
    dec = orc.e4m3_decode_table()
    return dec[v8t[..., :Nk]].transpose(0, 1, 3, 2) * vs[:, :, None, :]  # [1,H,Nk,D]


def test_q_zero_gives_channel_mean(orc):
    rng = np.random.default_rng(20)
    H, D, Nq, Nk = 2, 64, 70, 200
    q8 = np.zeros((1, H, _npad(Nq), D), np.int8)
    qs = np.ones((1, H, _npad(Nq) // TILE), np.float32)
    k8 = rng.integers(-127, 128, (1, H, _npad(Nk), D)).astype(np.int8)
    ks = rng.uniform(0.01, 0.05, (1, H, _npad(Nk) // TILE)).astype(np.float32)
    v8t, vs = _v_codes(orc, rng, H, D, Nk, values=(0.25, 1.0, 3.5, 100.0))
    out = orc.attn(q8, qs, k8, ks, v8t, vs, Nq, Nk, lam=0.3)
    ref = _vd(orc, v8t, vs, Nk).mean(axis=2)  # [1,H,D]
    for h in range(H):
        np.testing.assert_allclose(out[0, :, h, :], np.broadcast_to(ref[0, h], (Nq, D)), rtol=2e-6, atol=0)


def test_causal_q_zero_gives_prefix_means(orc):
    rng = np.random.default_rng(21)
    H, D, Nq, Nk = 1, 64, 100, 300
    q8 = np.zeros((1, H, _npad(Nq), D), np.int8)
    qs = np.ones((1, H, _npad(Nq) // TILE), np.float32)
    k8 = rng.integers(-127, 128, (1, H, _npad(Nk), D)).astype(np.int8)
    ks = np.full((1, H, _npad(Nk) // TILE), 0.02, np.float32)
    v8t, vs = _v_codes(orc, rng, H, D, Nk)
    for pos_off in (Nk - Nq, 17):
        out = orc.attn(q8, qs, k8, ks, v8t, vs, Nq, Nk, lam=1.0, causal=True, pos_off=pos_off)
        vd = _vd(orc, v8t, vs, Nk)[0, 0]
        csum = np.cumsum(vd, axis=0)
        for i in range(Nq):
            last = min(Nk - 1, i + pos_off)
            np.testing.assert_allclose(out[0, i, 0], csum[last] / (last + 1), rtol=3e-6, atol=1e-7)


def test_causal_fully_masked_rows_are_zero(orc):
    """Bottom-right alignment with Nq > Nk: rows i < Nq - Nk see no key and output 0."""
    rng = np.random.default_rng(22)
    H, D, Nq, Nk = 1, 64, 130, 70
    q8 = rng.integers(-127, 128, (1, H, _npad(Nq), D)).astype(np.int8)
    qs = np.full((1, H, _npad(Nq) // TILE), 0.01, np.float32)
    k8 = rng.integers(-127, 128, (1, H, _npad(Nk), D)).astype(np.int8)
    ks = np.full((1, H, _npad(Nk) // TILE), 0.01, np.float32)
    v8t, vs = _v_codes(orc, rng, H, D, Nk)
    out = orc.attn(q8, qs, k8, ks, v8t, vs, Nq, Nk, lam=1.0, causal=True)
    assert not out[0, : Nq - Nk].any()
    assert np.all(np.abs(out[0, Nq - Nk:]).sum(axis=-1) > 0)


def test_single_key(orc):
    """Nk = 1: the output is that key's dequantized V.  With arbitrary scales the row max
    is subtracted on the 2^-16 grid of the exponent argument, so P' of the only key is
    256 * 2^e with |e| <= 2^-16; with an integer score the result is exact."""
    rng = np.random.default_rng(23)
    H, D, Nq, Nk = 2, 128, 5, 1
    q8 = rng.integers(-127, 128, (1, H, 64, D)).astype(np.int8)
    qs = np.full((1, H, 1), 0.02, np.float32)
    k8 = rng.integers(-127, 128, (1, H, 64, D)).astype(np.int8)
    ks = np.full((1, H, 1), 0.03, np.float32)
    v8t, vs = _v_codes(orc, rng, H, D, Nk, values=(0.5, 7.0, 448.0))
    ref = _vd(orc, v8t, vs, 1)[0, :, 0, :]  # [H,D]
    out = orc.attn(q8, qs, k8, ks, v8t, vs, Nq, Nk, lam=0.7)
    for h in range(H):
        np.testing.assert_allclose(out[0, :, h, :], np.broadcast_to(ref[h], (Nq, D)), rtol=2.0 ** -15, atol=0)
    qs1 = np.ones((1, H, 1), np.float32)
    ks1 = np.ones((1, H, 1), np.float32)
    out = orc.attn(q8, qs1, k8, ks1, v8t, vs, Nq, Nk, lam=1.0)
    for h in range(H):
        assert np.array_equal(out[0, :, h, :], np.broadcast_to(ref[h].astype(np.float32), (Nq, D)))


def test_one_hot_scores(orc):
    """One key scores 40 (log2 units) above every other: P of the rest underflows FP8."""
    rng = np.random.default_rng(24)
    H, D, Nq, Nk = 1, 64, 64, 190
    q8 = np.zeros((1, H, 64, D), np.int8)
    q8[0, 0, :, 0] = 1
    k8 = np.zeros((1, H, _npad(Nk), D), np.int8)
    hot = rng.integers(0, Nk, Nq)
    qs = np.ones((1, H, 1), np.float32)
    ks = np.ones((1, H, _npad(Nk) // TILE), np.float32)
    out = np.zeros((1, Nq, H, D), np.float32)
    v8t, vs = _v_codes(orc, rng, H, D, Nk)
    vd = _vd(orc, v8t, vs, Nk)[0, 0]
    for i in range(Nq):
        k8[:] = 0
        k8[0, 0, hot[i], 0] = 40
        o = orc.attn(q8, qs, k8, ks, v8t, vs, Nq, Nk, lam=1.0, rows=[i])
        assert np.array_equal(o[0, 0, 0], vd[hot[i]].astype(np.float32))


def _exact_case(orc, rng, Nq, Nk, D, causal, H=1):
    """Operands whose scores are small integers: s_q in {1,2} per 64-row block, s_k in
    {1, 1/2} per 64-key block, one-hot Q codes and K codes chosen so every score is in
    {-2, -1, 0}; V values in {+-1, +-1.5, +-2, +-3} times a power of two per channel.
    Every P is then a power of two (exact in FP8) and every partial sum is exact."""
    nqb, nkb = _npad(Nq) // TILE, _npad(Nk) // TILE
    qs = rng.choice(np.float32([1.0, 2.0]), (1, H, nqb)).astype(np.float32)
    ks = rng.choice(np.float32([1.0, 0.5]), (1, H, nkb)).astype(np.float32)
    q8 = np.zeros((1, H, _npad(Nq), D), np.int8)
    ch = rng.integers(0, D, (H, Nq))
    for h in range(H):
        q8[0, h, np.arange(Nq), ch[h]] = 1
    k8 = np.zeros((1, H, _npad(Nk), D), np.int8)
    for h in range(H):
        for kb in range(nkb):
            vals = np.int8([-1, 0]) if ks[0, h, kb] == 1.0 else np.int8([-2, 0])
            k8[0, h, kb * TILE:(kb + 1) * TILE] = rng.choice(vals, (TILE, D))
    k8[0, :, Nk:] = 0
    v8t, vs = _v_codes(orc, rng, H, D, Nk)
    return q8, qs, k8, ks, v8t, vs


def _exact_ref(orc, q8, qs, k8, ks, v8t, vs, Nq, Nk, causal, pos_off):
    H = q8.shape[1]
    vd = _vd(orc, v8t, vs, Nk)
    out = np.zeros((1, Nq, H, q8.shape[-1]), np.float32)
    for h in range(H):
        qd = q8[0, h, :Nq].astype(np.float64) * np.repeat(qs[0, h], TILE)[:Nq, None]
        kd = k8[0, h, :Nk].astype(np.float64) * np.repeat(ks[0, h], TILE)[:Nk, None]
        s = qd @ kd.T  # lambda = 1 (log2 domain)
        if causal:
            s = np.where(np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + pos_off, s, -np.inf)
        w = np.exp2(s - np.max(np.where(np.isfinite(s), s, -1e300), axis=1, keepdims=True))
        w = np.where(np.isfinite(s), w, 0.0)
        den = w.sum(axis=1, keepdims=True)
        o = (w @ vd[0, h]) / np.where(den > 0, den, 1.0)
        out[0, :, h, :] = np.where(den > 0, o, 0.0).astype(np.float32)
    return out


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_exact_tile_boundary_shapes(orc, D, causal):
    rng = np.random.default_rng(30 + D + causal)
    for Nk in SHAPES:
        for Nq in ([1, 64, 65, 193, 256] if D == 64 else [63, 129, 255]):
            if causal and Nq > Nk:
                continue
            q8, qs, k8, ks, v8t, vs = _exact_case(orc, rng, Nq, Nk, D, causal)
            pos_off = Nk - Nq
            out = orc.attn(q8, qs, k8, ks, v8t, vs, Nq, Nk, lam=1.0, causal=causal, pos_off=pos_off)
            ref = _exact_ref(orc, q8, qs, k8, ks, v8t, vs, Nq, Nk, causal, pos_off)
            ulp = np.abs(out.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
            assert ulp.max() <= 1, (Nq, Nk, D, causal, ulp.max())


def test_exact_detects_scale_index_mixup(orc):
    """Guard for the exact construction itself: swapping two K block scales must break it."""
    rng = np.random.default_rng(40)
    Nq, Nk, D = 130, 193, 64
    for _ in range(10):
        q8, qs, k8, ks, v8t, vs = _exact_case(orc, rng, Nq, Nk, D, False)
        if ks[0, 0, 0] != ks[0, 0, 1]:
            break
    ref = _exact_ref(orc, q8, qs, k8, ks, v8t, vs, Nq, Nk, False, 0)
    ks_bad = ks.copy()
    ks_bad[0, 0, [0, 1]] = ks_bad[0, 0, [1, 0]]
    out_bad = orc.attn(q8, qs, k8, ks_bad, v8t, vs, Nq, Nk, lam=1.0)
    assert not np.array_equal(out_bad, ref)


def test_v_ones_rows_sum_to_one(orc):
    rng = np.random.default_rng(41)
    B, N, H, D = 1, 300, 2, 64
    q = W.bf16_bits(rng.standard_normal((B, N, H, D)).astype(np.float32) * 2)
    k = W.bf16_bits(rng.standard_normal((B, N, H, D)).astype(np.float32))
    v = W.bf16_bits(np.ones((B, N, H, D), np.float32))
    out, it = orc.fwd(q, k, v)
    assert np.all(it["v8t"][..., :N] == 0x7E)
    # out = sum dec(P8) * 448 * (1/448) / d' ; FP8 P is within 2^-4 of fp32 P
    assert np.all(np.abs(out - 1.0) <= 2.0 ** -4)
    assert np.abs(out - 1.0).max() > 0  # d sums fp32 P, not FP8 P


def _rel_l2_readings(orc, q, k, v, out, it, Nq, Nk, rows=None, causal=False):
    lam = it["lam"]
    qd, kd, vd = orc.dequant_operands(it["q8"], it["q_scale"], it["k8"], it["k_scale"], it["v8t"], it["v_scale"], Nq, Nk)
    B, _, H, D = out.shape
    rows = np.arange(Nq) if rows is None else np.asarray(rows)
    num_a = num_b = den_a = den_b = 0.0
    for b in range(B):
        for h in range(H):
            refa = orc.attention_fp64(qd[b, h], kd[b, h], vd[b, h], lam * np.log(2.0), causal, Nk - Nq, rows)
            refb = orc.attention_fp64(W.bf16_to_f32(q[b, :, h]), W.bf16_to_f32(k[b, :, h]), W.bf16_to_f32(v[b, :, h]),
                                      1.0 / np.sqrt(D), causal, Nk - Nq, rows)
            o = out[b, :, h].astype(np.float64)
            num_a += ((o - refa) ** 2).sum(); den_a += (refa ** 2).sum()
            num_b += ((o - refb) ** 2).sum(); den_b += (refb ** 2).sum()
    return np.sqrt(num_a / den_a), np.sqrt(num_b / den_b)


def test_random_tile_shapes_vs_fp64(orc):
    rng = np.random.default_rng(50)
    for Nq, Nk, D in [(65, 129, 64), (193, 256, 128), (1, 191, 64), (127, 63, 128)]:
        q = W.bf16_bits(rng.standard_normal((1, Nq, 2, D)).astype(np.float32))
        k = W.bf16_bits(rng.standard_normal((1, Nk, 2, D)).astype(np.float32) + 1.0)
        v = W.bf16_bits(rng.standard_normal((1, Nk, 2, D)).astype(np.float32))
        out, it = orc.fwd(q, k, v)
        ra, rb = _rel_l2_readings(orc, q, k, v, out, it, Nq, Nk)
        assert ra <= 0.03, (Nq, Nk, D, ra)
        assert rb <= 0.05, (Nq, Nk, D, rb)


def test_tiny_workload_fp64_readings(orc):
    w = W.TINY
    q, k, v = W.dense_inputs(w)
    out, it = orc.fwd(q, k, v)
    ra, rb = _rel_l2_readings(orc, q, k, v, out, it, w.Nq, w.Nk)
    assert ra <= 0.03
    assert rb <= 0.045  # reading B (original bf16 inputs) is reported, not gated


def test_i8kv_small_vs_fp64(orc):
    rng = np.random.default_rng(60)
    H, D, Nq, Nk, pos0 = 2, 128, 100, 700, 600
    q = W.bf16_bits(rng.standard_normal((Nq, H, D)).astype(np.float32))
    kc, kts = W.int8_cache(77, 5, H, Nk, D)
    vc, vts = W.int8_cache(77, 6, H, Nk, D)
    out, it = orc.fwd_i8kv(q, kc, kts, vc, vts, pos0)
    dec = orc.e4m3_decode_table()
    num = den = 0.0
    for h in range(H):
        qd = it["q8"][h, :Nq].astype(np.float64) * np.repeat(it["q_scale"][h], TILE)[:Nq, None]
        kd = kc[h].astype(np.float64) * kts[h][:, None]
        vd = dec[it["v8t"][h, :, :Nk]].T * it["v_scale"][h][None, :]
        ref = orc.attention_fp64(qd, kd, vd, it["lam"] * np.log(2.0), causal=True, pos_off=pos0)
        num += ((out[:, h].astype(np.float64) - ref) ** 2).sum()
        den += (ref ** 2).sum()
    assert np.sqrt(num / den) <= 0.03
    # a query at position pos0+i never sees keys beyond pos0+i: perturbing them changes nothing
    vc2 = vc.copy()
    vc2[:, pos0 + Nq:] = 0
    kc2 = kc.copy()
    kc2[:, pos0 + Nq:] = 0
    vts2 = vts.copy()
    out2, it2 = orc.fwd_i8kv(q, kc2, kts, vc2, vts2, pos0)
    # the V channel scales are taken over the whole cache, so keep them identical
    if np.array_equal(it2["v_scale"], it["v_scale"]):
        assert np.array_equal(out2, out)
