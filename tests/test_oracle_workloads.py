"""The oracle against unquantized FP64 softmax attention on the five workloads.

Two FP64 references (the method is an approximation, so the oracle is checked against
plain attention within the method's own error, rel-L2 = ||out - ref|| / ||ref||):

* reading A: FP64 softmax attention on the dequantized operands the fused loop consumes
  (q8 * s_q, k8 * s_k, dec(v8) * s_v; for the prefill workloads the cached K as stored) --
  gated at rel-L2 <= 0.03;
* reading B: FP64 softmax attention on the original bf16 inputs (for the prefill
  workloads, the dequantized cache) -- reported; it adds the quantization error of the
  inputs themselves (INT8 Q/K, e4m3 V, e4m3 P), about 0.035-0.041 on these white-noise
  inputs, and is asserted only against a loose bound.

Sampling (the FP64 references and the oracle run on whole 64-row query blocks of a few
heads; the quantizers always see every token of those heads, as the method needs):
  tiny 256 x 2 heads: every row of both heads;
  dense 4,096 x 16 heads: 4 heads x 8 query blocks;
  prefill 32K x 1,024 and 64K x 512: 4 of 32 heads x every query row;
  video 37,810 x 24 heads: 3 heads x 8 query blocks (the ragged last block included).
"""
import numpy as np
import pytest

import workloads as W

TILE = 64


def _blocks(nq, nblk, seed):
    """nblk distinct 64-row query blocks (the last, possibly ragged one included)."""
    nb = (nq + TILE - 1) // TILE
    rng = np.random.default_rng(seed)
    pick = sorted(set(rng.choice(nb - 1, size=min(nblk - 1, nb - 1), replace=False).tolist()) | {nb - 1})
    return np.concatenate([np.arange(b * TILE, min(nq, b * TILE + TILE)) for b in pick])


def _accumulate(acc, o, ref):
    o = np.asarray(o, np.float64)
    acc[0] += ((o - ref) ** 2).sum()
    acc[1] += (ref ** 2).sum()


def _dense_readings(orc, w, heads, rows):
    q, k, v = W.dense_inputs(w)
    sel = (slice(None), slice(None), heads)
    q, k, v = q[sel], k[sel], v[sel]
    out, it = orc.fwd(q, k, v, rows=rows)
    qd, kd, vd = orc.dequant_operands(it["q8"], it["q_scale"], it["k8"], it["k_scale"], it["v8t"], it["v_scale"],
                                      w.Nq, w.Nk)
    lam = it["lam"]
    ra, rb = [0.0, 0.0], [0.0, 0.0]
    for h in range(len(heads)):
        refa = orc.attention_fp64(qd[0, h], kd[0, h], vd[0, h], lam * np.log(2.0), w.causal, w.Nk - w.Nq, rows)
        refb = orc.attention_fp64(W.bf16_to_f32(q[0, :, h]), W.bf16_to_f32(k[0, :, h]), W.bf16_to_f32(v[0, :, h]),
                                  1.0 / np.sqrt(w.D), w.causal, w.Nk - w.Nq, rows)
        _accumulate(ra, out[0, :, h], refa)
        _accumulate(rb, out[0, :, h], refb)
    return np.sqrt(ra[0] / ra[1]), np.sqrt(rb[0] / rb[1])


def _i8kv_readings(orc, w, heads):
    q, kc, kts, vc, vts = W.i8kv_inputs(w)
    q, kc, kts, vc, vts = q[:, heads], kc[heads], kts[heads], vc[heads], vts[heads]
    S = _kv_splits(w.H, w.Nq, w.Nk, w.pos0)
    out, it = orc.fwd_i8kv(q, kc, kts, vc, vts, w.pos0, kv_splits=S)
    dec = orc.e4m3_decode_table()
    lam = it["lam"]
    ra, rb = [0.0, 0.0], [0.0, 0.0]
    for h in range(len(heads)):
        qd = it["q8"][h, :w.Nq].astype(np.float64) * np.repeat(it["q_scale"][h], TILE)[:w.Nq, None]
        kd = kc[h].astype(np.float64) * kts[h][:, None]
        vd = dec[it["v8t"][h, :, :w.Nk]].T * it["v_scale"][h][None, :]
        refa = orc.attention_fp64(qd, kd, vd, lam * np.log(2.0), causal=True, pos_off=w.pos0)
        vsrc = vc[h].astype(np.float64) * vts[h][:, None]
        refb = orc.attention_fp64(W.bf16_to_f32(q[:, h]), kd, vsrc, 1.0 / np.sqrt(w.D), causal=True, pos_off=w.pos0)
        _accumulate(ra, out[:, h], refa)
        _accumulate(rb, out[:, h], refb)
    return np.sqrt(ra[0] / ra[1]), np.sqrt(rb[0] / rb[1])


def _kv_splits(H, Nq, Nk, pos0):
    """The key-range count the library's rule gives for the whole workload (the prefill
    result depends on it, so the oracle runs at the same count): one workgroup of 256
    query rows per CU over 256 CUs, ranges of at least 16 key tiles, at most 64."""
    wgs = H * ((Nq + 255) // 256)
    T = (min(Nk, pos0 + Nq) + TILE - 1) // TILE
    return max(1, min((256 + wgs - 1) // wgs, T // 16, 64))


CASES = [
    ("tiny_b1_h2_n256_d64", [0, 1], None),
    ("dense_b1_h16_n4096_d128", [0, 5, 10, 15], 8),
    ("prefill_i8kv_h32_d128_q1024_ctx32768", [0, 9, 18, 31], None),
    ("prefill_i8kv_h32_d128_q512_ctx65536", [3, 12, 21, 30], None),
    ("video_dit_b1_h24_n37810_d128", [0, 11, 23], 8),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,heads,nblk", CASES, ids=[c[0] for c in CASES])
def test_fp64_readings_on_workloads(orc, name, heads, nblk):
    w = W.BY_NAME[name]
    if w.kind == "dense":
        rows = np.arange(w.Nq) if nblk is None else _blocks(w.Nq, nblk, w.seed)
        ra, rb = _dense_readings(orc, w, heads, rows)
    else:
        ra, rb = _i8kv_readings(orc, w, heads)
    print(f"{name}: rel-L2 reading A {ra:.4f}, reading B {rb:.4f}", flush=True)
    assert ra <= 0.03, (name, ra)
    assert rb <= 0.05, (name, rb)
