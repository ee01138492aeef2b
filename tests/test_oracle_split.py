"""Pins for the oracle's split-KV path (key tiles cut into contiguous ranges, each run
from m = -inf, combined in split order with weights 2^(m_s - M)).

* exact closed form: per-tile constant integer scores, so every P', weight, rescale and
  partial sum is an exact small binary number; the result must equal the exactly
  computed weighted mean sum_j 2^(a_j) v_j / sum_j 2^(a_j) to the final rounding, for
  split counts that leave some ranges empty for some rows (causal) or for all of them;
* one split reduces bit for bit to the unsplit loop;
* FP64 softmax attention on the dequantized operands (rel-L2 <= 0.03) and on the bf16
  inputs (<= 0.05) with random data, causal and not, several split counts.
"""
import numpy as np
import pytest

TILE = 64


def _npad(n):
    return (n + TILE - 1) // TILE * TILE


def test_split_bounds_cover_the_tiles(orc):
    for T in (0, 1, 5, 64, 513):
        for S in (1, 2, 3, 7, 8):
            b = orc.split_bounds(T, S)
            assert b[0][0] == 0 and b[-1][1] == T
            assert all(b[i][1] == b[i + 1][0] for i in range(S - 1))
            assert all(lo <= hi for lo, hi in b)
    assert orc.key_tiles(100, 1000, True, 30) == 3  # last visible key 129 -> 3 tiles
    assert orc.key_tiles(100, 1000, False, 0) == 16


def _tile_constant_ops(orc, rng, H, D, Nq, Nk, a_tile):
    """Query rows are e_0 (one-hot); key j's channel 0 is a_tile[j // 64]: scores are the
    integers a_tile[t] (c = 1, lambda = 1)."""
    q8 = np.zeros((1, H, _npad(Nq), D), np.int8)
    q8[0, :, :Nq, 0] = 1
    qs = np.ones((1, H, _npad(Nq) // TILE), np.float32)
    k8 = np.zeros((1, H, _npad(Nk), D), np.int8)
    for j in range(Nk):
        k8[0, :, j, 0] = a_tile[j // TILE]
    ks = np.ones((1, H, _npad(Nk) // TILE), np.float32)
    vals = np.float32([1.0, 1.5, 2.0, 3.0, -1.0, -1.5, -2.0, -3.0])
    codes = orc.e4m3_encode(vals)
    v8t = np.zeros((1, H, D, _npad(Nk)), np.uint8)
    v8t[..., :Nk] = codes[rng.integers(0, 8, (1, H, D, Nk))]
    vs = np.ones((1, H, D), np.float32)
    return q8, qs, k8, ks, v8t, vs


@pytest.mark.parametrize("causal", [False, True])
def test_split_exact_weighted_mean(orc, causal):
    rng = np.random.default_rng(40)
    H, D, Nq, Nk = 2, 64, 70, 7 * TILE - 5
    a_tile = [2, 5, 1, 6, 6, 0, 3]  # integer scores per tile; within 8 of each other
    ops = _tile_constant_ops(orc, rng, H, D, Nq, Nk, a_tile)
    pos_off = Nk - Nq if not causal else 200
    dec = orc.e4m3_decode_table()
    v = dec[ops[4][..., :Nk]].astype(np.float64)  # [1,H,D,Nk]
    w = np.exp2(np.array([a_tile[j // TILE] for j in range(Nk)], np.float64))
    for S in (1, 2, 3, 5, 9):
        out = orc.attn(*ops, Nq, Nk, lam=1.0, causal=causal, pos_off=pos_off, kv_splits=S)
        for i in range(Nq):
            last = min(Nk - 1, i + pos_off) if causal else Nk - 1
            ref = (v[0, :, :, :last + 1] * w[:last + 1]).sum(-1) / w[:last + 1].sum()  # [H,D]
            got = out[0, i].astype(np.float64)
            # every partial sum is exact; only the final division rounds
            np.testing.assert_allclose(got, ref, rtol=2 ** -23, atol=0, err_msg=f"S={S} row {i}")


def test_one_split_is_the_unsplit_loop(orc):
    rng = np.random.default_rng(41)
    H, D, Nq, Nk = 2, 128, 90, 333
    q8 = rng.integers(-127, 128, (1, H, _npad(Nq), D)).astype(np.int8)
    qs = rng.uniform(0.005, 0.02, (1, H, _npad(Nq) // TILE)).astype(np.float32)
    k8 = rng.integers(-127, 128, (1, H, Nk, D)).astype(np.int8)
    ks = rng.uniform(0.005, 0.02, (1, H, Nk)).astype(np.float32)
    v8t = rng.integers(0, 256, (1, H, D, _npad(Nk))).astype(np.uint8)
    v8t[(v8t & 0x7F) == 0x7F] = 0  # no NaN codes
    vs = rng.uniform(0.5, 2, (1, H, D)).astype(np.float32)
    kw = dict(causal=True, pos_off=Nk - Nq, k_scale_per_token=True)
    a = orc.attn(q8, qs, k8, ks, v8t, vs, Nq, Nk, 0.18, **kw)
    b = orc.attn(q8, qs, k8, ks, v8t, vs, Nq, Nk, 0.18, kv_splits=1, **kw)
    # a single range through the partial/combine route: weights 2^0 = 1
    T = orc.key_tiles(Nq, Nk, True, Nk - Nq)
    L = orc.lib()
    for h in range(H):
        op = np.empty((1, Nq, D), np.float32)
        mp = np.empty((1, Nq), np.float32)
        dp = np.empty((1, Nq), np.float32)
        L.orc_attn_rows_part(orc._ptr(np.ascontiguousarray(q8[0, h])), orc._ptr(np.ascontiguousarray(qs[0, h])),
                             orc._ptr(np.ascontiguousarray(k8[0, h])), orc._ptr(np.ascontiguousarray(ks[0, h])), 1,
                             orc._ptr(np.ascontiguousarray(v8t[0, h])), v8t.shape[-1], Nq, Nk, D, 0.18, 1, Nk - Nq, 0,
                             Nq, 0, T, orc._ptr(op), orc._ptr(mp), orc._ptr(dp))
        c = np.empty((Nq, D), np.float32)
        L.orc_combine_rows(1, orc._ptr(op), orc._ptr(mp), orc._ptr(dp), orc._ptr(np.ascontiguousarray(vs[0, h])), Nq,
                           D, orc._ptr(c))
        assert np.array_equal(c.view(np.uint32), a[0, :, h].view(np.uint32))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("causal,S", [(False, 2), (False, 5), (True, 3), (True, 8)])
def test_split_matches_fp64_attention(orc, causal, S):
    rng = np.random.default_rng(42 + S)
    H, D, Nq, Nk = 2, 64, 100, 600
    q = rng.standard_normal((1, Nq, H, D)).astype(np.float32)
    k = rng.standard_normal((1, Nk, H, D)).astype(np.float32)
    v = rng.standard_normal((1, Nk, H, D)).astype(np.float32)
    import workloads as W
    qb, kb, vb = W.bf16_bits(q), W.bf16_bits(k), W.bf16_bits(v)
    q8, qs, k8, ks, _ = orc.quant_qk(qb, kb)
    v8t, vs = orc.quant_v(vb)
    lam = orc.default_lambda(D)
    out = orc.attn(q8, qs, k8, ks, v8t, vs, Nq, Nk, lam, causal=causal, kv_splits=S)
    # reading A: the dequantized operands (the softmax and FP8 P error alone) <= 0.03;
    # reading B: the bf16 inputs (all quantization) <= 0.05
    qd, kd, vd = orc.dequant_operands(q8, qs, k8, ks, v8t, vs, Nq, Nk)
    qf, kf, vf = W.bf16_to_f32(qb), W.bf16_to_f32(kb), W.bf16_to_f32(vb)
    na = nb = da = db = 0.0
    for h in range(H):
        ra = orc.attention_fp64(qd[0, h], kd[0, h], vd[0, h], lam * np.log(2.0), causal, Nk - Nq)
        rb = orc.attention_fp64(qf[0, :, h], kf[0, :, h], vf[0, :, h], 1 / np.sqrt(D), causal, Nk - Nq)
        o = out[0, :, h].astype(np.float64)
        na += ((o - ra) ** 2).sum(); da += (ra ** 2).sum()
        nb += ((o - rb) ** 2).sum(); db += (rb ** 2).sum()
    assert np.sqrt(na / da) <= 0.03
    assert np.sqrt(nb / db) <= 0.05
