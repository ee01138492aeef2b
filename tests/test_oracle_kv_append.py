"""Pins for the oracle's KV-cache append quantizer (per (token, head) INT8 rows).

* exact worked rows (a = 127 gives s = 1 and the codes are the rounded values, ties to
  even; a power-of-two rescaling of the row keeps the codes and scales the scale; a zero
  row gives s = 0 and zero codes);
* invariants on random rows: |code| = 127 at the row's largest magnitude, the
  dequantized value is within half a step, signs are kept, rows outside [pos, pos+n)
  are untouched;
* agreement with the (separately pinned) 64-row block quantizer on inputs whose every
  64-row block holds a single nonzero row.
"""
import numpy as np

import workloads as W


def _bf16(vals):
    return W.bf16_bits(np.asarray(vals, dtype=np.float32))


def test_worked_rows(orc):
    H, D, Nmax = 1, 64, 8
    row = np.zeros(D, np.float32)
    row[:6] = [127.0, -63.5, 0.5, -0.5, 1.5, -2.5]
    x = np.stack([row, row * np.float32(2.0 ** -3), np.zeros(D, np.float32)])[:, None, :]  # [3, 1, D]
    cache = np.full((H, Nmax, D), 55, np.int8)
    ts = np.full((H, Nmax), -1.0, np.float32)
    c, s = orc.kv_append_i8(_bf16(x), cache, ts, pos=2)
    want = np.zeros(D, np.int8)
    want[:6] = [127, -64, 0, 0, 2, -2]  # ties to even: -63.5 -> -64, 0.5 -> 0, 1.5 -> 2, -2.5 -> -2
    assert np.array_equal(c[0, 2], want) and s[0, 2] == 1.0
    assert np.array_equal(c[0, 3], want) and s[0, 3] == np.float32(0.125)
    assert not c[0, 4].any() and s[0, 4] == 0.0
    # untouched rows
    assert (c[0, :2] == 55).all() and (c[0, 5:] == 55).all()
    assert (s[0, :2] == -1).all() and (s[0, 5:] == -1).all()


def test_random_rows_invariants(orc):
    rng = np.random.default_rng(70)
    for D in (64, 128):
        H, Nnew, Nmax, pos = 3, 50, 80, 17
        x = _bf16(rng.standard_normal((Nnew, H, D)).astype(np.float32) * np.exp2(rng.uniform(-20, 20, (Nnew, H, 1))))
        c, s = orc.kv_append_i8(x, np.zeros((H, Nmax, D), np.int8), np.zeros((H, Nmax), np.float32), pos)
        xf = W.bf16_to_f32(x).astype(np.float64)  # [Nnew, H, D]
        for n in range(Nnew):
            for h in range(H):
                code = c[h, pos + n].astype(np.float64)
                sc = float(s[h, pos + n])
                a = np.abs(xf[n, h]).max()
                assert abs(sc - a / 127) <= 2 ** -23 * (a / 127)
                assert abs(code[np.argmax(np.abs(xf[n, h]))]) == 127
                # half a step, plus the relative error of the rounded reciprocal r = fl32(127 / a)
                # and of the product, which can move a value within ~|x| 2^-22 of a tie
                assert np.all(np.abs(code * sc - xf[n, h]) <= 0.5 * sc + np.abs(xf[n, h]) * 2 ** -21)
                big = np.abs(xf[n, h]) >= sc
                assert np.all(np.sign(code[big]) == np.sign(xf[n, h][big]))
        assert not c[:, :pos].any() and not c[:, pos + Nnew:].any()


def test_agrees_with_block_quantizer(orc):
    rng = np.random.default_rng(71)
    H, D, n = 2, 128, 9
    rows = _bf16(rng.standard_normal((n, H, D)).astype(np.float32) * 3)
    xb = np.zeros((1, 64 * n, H, D), np.uint16)  # one nonzero row per 64-row block
    xb[0, ::64] = rows
    codes, scales = orc.quant_i8_blocks(xb)
    c, s = orc.kv_append_i8(rows, np.zeros((H, n, D), np.int8), np.zeros((H, n), np.float32), 0)
    for h in range(H):
        assert np.array_equal(c[h], codes[0, h, ::64])
        assert np.array_equal(s[h], scales[0, h])
