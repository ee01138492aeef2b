"""GPU parity: the HIP path (through the C-ABI binding) against the CPU oracle.

* codes and scales (q8, k8, v8t, their scales, the K mean, the prefill workspace) are
  compared bit for bit;
* attention outputs (fp32) must satisfy max|gpu - oracle| <= 2e-3 * RMS(oracle); bf16
  outputs must be the round-to-nearest-even of the GPU's own fp32 result;
* full-size workloads are checked on sampled query blocks (rows are independent).
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
TOL = 2e-3


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def qa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_attention_qattn_amd as qa

    oracle.build(force=False)
    return qa


def dev_bf16(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt((ref ** 2).mean())
    err = np.abs(gpu - ref).max()
    assert np.isfinite(gpu).all(), what
    assert err <= TOL * rms, f"{what}: max abs err {err:.3e} > {TOL} * rms {rms:.3e} (ratio {err / rms:.2e})"
    return err / rms


def bf16_of(f32: np.ndarray) -> np.ndarray:
    return W.bf16_bits(f32)


# ----------------------------------------------------------------------------------
# preparation: bit-exact
# ----------------------------------------------------------------------------------
QK_SHAPES = [(1, 2, 256, 256, 64), (2, 3, 150, 77, 128), (1, 1, 1, 1, 64), (1, 2, 65, 300, 128), (1, 1, 700, 1100, 64)]


@pytest.mark.parametrize("B,H,Nq,Nk,D", QK_SHAPES)
def test_quant_qk_bit_exact(qa, B, H, Nq, Nk, D):
    say(f"quant_qk B={B} H={H} Nq={Nq} Nk={Nk} D={D}")
    rng = np.random.default_rng(100 + Nq + Nk + D)
    q = W.bf16_bits(rng.standard_normal((B, Nq, H, D)).astype(np.float32) * 3)
    k = W.bf16_bits(rng.standard_normal((B, Nk, H, D)).astype(np.float32) + rng.uniform(-2, 2, (B, 1, H, D)).astype(np.float32))
    t = qa.quant_qk(dev_bf16(q), dev_bf16(k))
    torch.cuda.synchronize()
    q8, qs, k8, ks, mean = oracle.quant_qk(q, k)
    assert np.array_equal(host(t["k_mean"]), mean)
    assert np.array_equal(host(t["q8"]), q8)
    assert np.array_equal(host(t["q_scale"]).view(np.uint32), qs.view(np.uint32))
    assert np.array_equal(host(t["k8"]), k8)
    assert np.array_equal(host(t["k_scale"]).view(np.uint32), ks.view(np.uint32))


def test_quant_qk_strided_views(qa):
    """Q and K as projection-strided views of one packed [B, N, 3, H, D] tensor."""
    say("quant_qk strided views")
    rng = np.random.default_rng(7)
    B, N, H, D = 2, 130, 4, 128
    qkv = W.bf16_bits(rng.standard_normal((B, N, 3, H, D)).astype(np.float32))
    dq = dev_bf16(qkv)
    t = qa.quant_qk(dq[:, :, 0], dq[:, :, 1])
    torch.cuda.synchronize()
    q8, qs, k8, ks, mean = oracle.quant_qk(qkv[:, :, 0], qkv[:, :, 1])
    assert np.array_equal(host(t["q8"]), q8) and np.array_equal(host(t["k8"]), k8)
    assert np.array_equal(host(t["k_mean"]), mean) and np.array_equal(host(t["k_scale"]), ks)
    v = qa.quant_v(dq[:, :, 2])
    torch.cuda.synchronize()
    v8t, vs = oracle.quant_v(qkv[:, :, 2])
    assert np.array_equal(host(v["v8t"]), v8t) and np.array_equal(host(v["v_scale"]), vs)


@pytest.mark.parametrize("B,H,Nq,Nk,D", QK_SHAPES)
def test_quant_v_bit_exact(qa, B, H, Nq, Nk, D):
    say(f"quant_v B={B} H={H} Nk={Nk} D={D}")
    rng = np.random.default_rng(200 + Nk + D)
    v = W.bf16_bits(rng.standard_normal((B, Nk, H, D)).astype(np.float32) * np.exp2(rng.uniform(-3, 3, (1, 1, H, D))).astype(np.float32))
    v[:, :, 0, 1] = 0  # a zero channel
    t = qa.quant_v(dev_bf16(v))
    torch.cuda.synchronize()
    v8t, vs = oracle.quant_v(v)
    assert np.array_equal(host(t["v8t"]), v8t)
    assert np.array_equal(host(t["v_scale"]).view(np.uint32), vs.view(np.uint32))
    assert np.array_equal(host(t["vbf"]), host(vbf_of(v8t)))  # the codes' exact bf16 values


@pytest.mark.parametrize("B,H,Nq,Nk,D", QK_SHAPES)
def test_prep_bit_exact(qa, B, H, Nq, Nk, D):
    """The fused preparation (one call, four launches) against the oracle's steps 1-2."""
    say(f"prep B={B} H={H} Nq={Nq} Nk={Nk} D={D}")
    rng = np.random.default_rng(300 + Nq + Nk + D)
    q = W.bf16_bits(rng.standard_normal((B, Nq, H, D)).astype(np.float32) * 3)
    k = W.bf16_bits(rng.standard_normal((B, Nk, H, D)).astype(np.float32) + rng.uniform(-2, 2, (B, 1, H, D)).astype(np.float32))
    v = W.bf16_bits(rng.standard_normal((B, Nk, H, D)).astype(np.float32) * np.exp2(rng.uniform(-3, 3, (1, 1, H, D))).astype(np.float32))
    v[:, :, 0, 1] = 0  # a zero channel
    t = qa.prep(dev_bf16(q), dev_bf16(k), dev_bf16(v))
    torch.cuda.synchronize()
    q8, qs, k8, ks, mean = oracle.quant_qk(q, k)
    v8t, vs = oracle.quant_v(v)
    assert np.array_equal(host(t["k_mean"]).view(np.uint32), mean.view(np.uint32))
    assert np.array_equal(host(t["q8"]), q8)
    assert np.array_equal(host(t["q_scale"]).view(np.uint32), qs.view(np.uint32))
    assert np.array_equal(host(t["k8"]), k8)
    assert np.array_equal(host(t["k_scale"]).view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(host(t["v8t"]), v8t)
    assert np.array_equal(host(t["v_scale"]).view(np.uint32), vs.view(np.uint32))
    assert np.array_equal(host(t["vbf"]), host(vbf_of(v8t)))


def test_prep_strided_views(qa):
    """Q, K and V as projection-strided views of one packed [B, N, 3, H, D] tensor."""
    say("prep strided views")
    rng = np.random.default_rng(8)
    B, N, H, D = 2, 300, 3, 64
    qkv = W.bf16_bits(rng.standard_normal((B, N, 3, H, D)).astype(np.float32))
    dq = dev_bf16(qkv)
    t = qa.prep(dq[:, :, 0], dq[:, :, 1], dq[:, :, 2])
    torch.cuda.synchronize()
    q8, qs, k8, ks, mean = oracle.quant_qk(qkv[:, :, 0], qkv[:, :, 1])
    v8t, vs = oracle.quant_v(qkv[:, :, 2])
    assert np.array_equal(host(t["q8"]), q8) and np.array_equal(host(t["k8"]), k8)
    assert np.array_equal(host(t["k_mean"]), mean) and np.array_equal(host(t["k_scale"]), ks)
    assert np.array_equal(host(t["q_scale"]), qs)
    assert np.array_equal(host(t["v8t"]), v8t) and np.array_equal(host(t["v_scale"]), vs)


def test_prep_same_bytes_as_separate_calls(qa):
    """Identical bytes from qattn_prep and from qattn_quant_qk + qattn_quant_v, also where
    the fp64 channel sums round (K channels mixing magnitudes 2^40 and 2^-40): both
    paths add the same partial sums in the same order."""
    say("prep vs separate calls")
    rng = np.random.default_rng(11)
    B, H, Nq, Nk, D = 1, 2, 1000, 1500, 128
    q = W.bf16_bits(rng.standard_normal((B, Nq, H, D)).astype(np.float32))
    kf = rng.standard_normal((B, Nk, H, D)).astype(np.float32)
    kf *= np.exp2(rng.choice([-40.0, 0.0, 40.0], size=kf.shape)).astype(np.float32)
    k = W.bf16_bits(kf)
    v = W.bf16_bits(rng.standard_normal((B, Nk, H, D)).astype(np.float32))
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    fused = qa.prep(dq, dk, dv)
    sep = {**qa.quant_qk(dq, dk), **qa.quant_v(dv)}
    torch.cuda.synchronize()
    for name in ["q8", "q_scale", "k8", "k_scale", "k_mean", "v8t", "v_scale", "vbf"]:
        assert torch.equal(fused[name].view(torch.uint8), sep[name].view(torch.uint8)), name


def test_quant_v_every_bf16_value(qa):
    """Channel 0 holds every bf16 value with |v| <= 448 (amax 448, so fl32(v * 1) is
    encoded as is): the GPU's e4m3 encoder must match the oracle's on all of them."""
    say("quant_v every bf16 value")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = W.bf16_to_f32(bits)
    vals = bits[np.isfinite(f) & (np.abs(f) <= 448.0)]
    N = len(vals)
    rng = np.random.default_rng(3)
    v = W.bf16_bits(rng.standard_normal((1, N, 1, 64)).astype(np.float32))
    v[0, :, 0, 0] = vals
    t = qa.quant_v(dev_bf16(v))
    torch.cuda.synchronize()
    v8t, vs = oracle.quant_v(v)
    assert vs[0, 0, 0] == 1.0
    assert np.array_equal(host(t["v8t"]), v8t)


def _p8_codes_gpu(qa, u: torch.Tensor, saturating: bool) -> np.ndarray:
    codes = torch.empty(u.numel(), dtype=torch.uint8, device="cuda")
    qa.qattn_selftest_p8_codes(u, codes, saturating)
    torch.cuda.synchronize()
    return host(codes)


@pytest.mark.parametrize("saturating,u_hi", [(False, 88.5), (True, 96.0)])
def test_p8_codes_whole_grid(qa, saturating, u_hi):
    """The fused kernel's P8 code of P' = 2^(u - 80) equals the oracle's code of the
    correctly rounded power (saturating at 448) for EVERY fp32 u in [16, u_hi).

    The kernel's argument is u = fl32(acc * c + fl32(88 - m_s)).  It exceeds 88 by at
    most (ulp(m_s) + ulp(88 - m_s)) / 2 + ulp(u) / 2, i.e. by at most 0.375 + 2^-17 while
    every row of the wave has |m_s| < 2^22: the ordinary form is checked up to 88.5.
    Beyond, u is unbounded (it passed 89 in a CPU emulation at |m_s| ~ 2^24) and the
    wave uses the large-score form, which must give the saturated code 0x7E for every
    u above 88.81: checked over the whole grid up to 96, then at larger and infinite
    powers.  Below u = 16, P' < 2^-64: zero codes, including -inf for masked keys."""
    lo = int(np.float32(16.0).view(np.uint32))
    hi = int(np.float32(u_hi).view(np.uint32))
    say(f"p8 codes over {hi - lo} grid arguments (saturating={saturating})")
    u = torch.arange(lo, hi, dtype=torch.int64, device="cuda").to(torch.int32).view(torch.float32)
    got = _p8_codes_gpu(qa, u, saturating)
    ref = oracle.p8_codes_grid(lo, hi)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} mismatches, first u bits {[hex(lo + int(i)) for i in bad[:5]]}"
    tail = [0.0, 1.0, 15.9, -5.0, -1e30, float("-inf")]
    assert not _p8_codes_gpu(qa, torch.tensor(tail, dtype=torch.float32, device="cuda"), saturating).any()
    if saturating:
        big = torch.tensor([96.0, 127.99, 128.0, 200.0, 1e30, float("inf")], dtype=torch.float32, device="cuda")
        assert (_p8_codes_gpu(qa, big, True) == 0x7E).all()


# ----------------------------------------------------------------------------------
# fused loop
# ----------------------------------------------------------------------------------
def vbf_of(v8t: np.ndarray) -> torch.Tensor:
    """The bf16 values of e4m3 codes (exact), as qattn_quant_v's vbf output holds them."""
    dec = oracle.e4m3_decode_table().astype(np.float32)
    return dev_bf16(W.bf16_bits(dec[v8t]))


def i8kv_workspace(wsh: np.ndarray, H: int, Nq: int, Nk: int, D: int) -> dict:
    """The sections of a qattn_fwd_i8kv workspace (host copy), as the header lays them out."""
    nqp, nkp = oracle.npad(Nq), oracle.npad(Nk)
    r = lambda n: (n + 255) // 256 * 256
    out, off = {}, 0
    for name, nbytes, dt, shape in [("v_scale", H * D * 4, np.float32, (H, D)), ("q8", H * nqp * D, np.int8, (H, nqp, D)),
                                    ("q_scale", H * (nqp // 64) * 4, np.float32, (H, nqp // 64)),
                                    ("vbf", H * D * nkp * 2, np.uint16, (H, D, nkp))]:
        out[name] = wsh[off: off + nbytes].view(dt).reshape(shape)
        off += r(nbytes)
    return out


def run_fwd(qa, ops, Nq, Nk, lam, causal, out_dtype=torch.float32):
    q8, qs, k8, ks, vs = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (ops[0], ops[1], ops[2], ops[3], ops[5])]
    vbf = vbf_of(np.ascontiguousarray(ops[4]))
    B, H, _, D = q8.shape
    out = torch.empty((B, Nq, H, D), dtype=out_dtype, device="cuda")
    qa.qattn_fwd(q8, qs, k8, ks, vbf, vs, Nq, Nk, out, lam, causal)
    torch.cuda.synchronize()
    return host(out)


def test_fwd_tiny_workload(qa):
    w = W.TINY
    say(f"fwd {w.name}")
    q, k, v = W.dense_inputs(w)
    out32, inter = qa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), out_dtype=torch.float32)
    out16, _ = qa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, it = oracle.fwd(q, k, v)
    assert np.array_equal(host(inter["q8"]), it["q8"]) and np.array_equal(host(inter["v8t"]), it["v8t"])
    r = assert_close(host(out32), ref, w.name)
    say(f"  max err / rms = {r:.2e}")
    assert np.array_equal(host(out16), bf16_of(host(out32)))


def _exact_ops(rng, Nq, Nk, D, H=2):
    """Operands whose scores are small integers (see the oracle's exact pins)."""
    npq, npk = oracle.npad(Nq), oracle.npad(Nk)
    qs = rng.choice(np.float32([1.0, 2.0]), (1, H, npq // 64)).astype(np.float32)
    ks = rng.choice(np.float32([1.0, 0.5]), (1, H, npk // 64)).astype(np.float32)
    q8 = np.zeros((1, H, npq, D), np.int8)
    for h in range(H):
        q8[0, h, np.arange(Nq), rng.integers(0, D, Nq)] = 1
    k8 = np.zeros((1, H, npk, D), np.int8)
    for h in range(H):
        for kb in range(npk // 64):
            vals = np.int8([-1, 0]) if ks[0, h, kb] == 1.0 else np.int8([-2, 0])
            k8[0, h, kb * 64:(kb + 1) * 64] = rng.choice(vals, (64, D))
    k8[0, :, Nk:] = 0
    codes = oracle.e4m3_encode(np.float32([1, 1.5, 2, 3, -1, -1.5, -2, -3]))
    v8t = np.zeros((1, H, D, npk), np.uint8)
    v8t[..., :Nk] = codes[rng.integers(0, 8, (1, H, D, Nk))]
    vs = np.exp2(-rng.integers(0, 4, (1, H, D))).astype(np.float32)
    return q8, qs, k8, ks, v8t, vs


SHAPES = [1, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_exact_tile_boundary_shapes(qa, D, causal):
    """1-4-tile boundary shapes with exact scores: GPU == oracle within 2 ulp."""
    rng = np.random.default_rng(1000 + D + causal)
    for Nk in SHAPES:
        for Nq in [1, 63, 65, 129, 256]:
            if causal and Nq > Nk:
                continue
            say(f"exact Nq={Nq} Nk={Nk} D={D} causal={causal}")
            ops = _exact_ops(rng, Nq, Nk, D)
            got = run_fwd(qa, ops, Nq, Nk, 1.0, causal)
            ref = oracle.attn(*ops, Nq, Nk, 1.0, causal=causal)
            ulp = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
            assert ulp.max() <= 2, (Nq, Nk, D, causal, ulp.max())


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_random_tile_shapes(qa, D, causal):
    rng = np.random.default_rng(2000 + D + causal)
    for Nq, Nk in [(1, 1), (65, 129), (193, 256), (127, 63), (300, 555), (64, 1000)]:
        if causal and Nq > Nk:
            Nq, Nk = Nk, Nq
        say(f"random Nq={Nq} Nk={Nk} D={D} causal={causal}")
        q = W.bf16_bits(rng.standard_normal((1, Nq, 3, D)).astype(np.float32))
        k = W.bf16_bits(rng.standard_normal((1, Nk, 3, D)).astype(np.float32) + 1)
        v = W.bf16_bits(rng.standard_normal((1, Nk, 3, D)).astype(np.float32))
        out, _ = qa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, out_dtype=torch.float32)
        torch.cuda.synchronize()
        ref, _ = oracle.fwd(q, k, v, causal=causal)
        assert_close(host(out), ref, f"Nq={Nq} Nk={Nk}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_large_scores(qa, D, causal):
    """Scores far beyond the ordinary range (through a large softmax scale, up to |S| of
    about 2^27): the exponent argument passes 88.81 (saturated P codes) once |m| >= 2^22,
    and 2^u then exceeds 2^88.  Element by element against the oracle, which saturates
    every such code at 448; the outputs must stay finite.  (Beyond |S| ~ 2^28 the fp32
    sum d' itself may overflow, in the oracle as in the kernel: outside the contract.)"""
    rng = np.random.default_rng(3000 + D + causal)
    Nq, Nk, H = 200, 333, 3
    q = W.bf16_bits(rng.standard_normal((1, Nq, H, D)).astype(np.float32))
    k = W.bf16_bits(rng.standard_normal((1, Nk, H, D)).astype(np.float32) + 1)
    v = W.bf16_bits(rng.standard_normal((1, Nk, H, D)).astype(np.float32))
    ops_t = qa.prep(dev_bf16(q), dev_bf16(k), dev_bf16(v))
    torch.cuda.synchronize()
    q8, qs, k8, ks, mean = oracle.quant_qk(q, k)
    v8t, vs = oracle.quant_v(v)
    for lam in (2.0 ** 10, 2.0 ** 16, 2.0 ** 18, 2.0 ** 20, 2.0 ** 22):
        say(f"large scores D={D} causal={causal} lambda=2^{np.log2(lam):.0f}")
        out = torch.empty((1, Nq, H, D), dtype=torch.float32, device="cuda")
        qa.qattn_fwd(ops_t["q8"], ops_t["q_scale"], ops_t["k8"], ops_t["k_scale"], ops_t["vbf"], ops_t["v_scale"], Nq,
                     Nk, out, lam, causal)
        torch.cuda.synchronize()
        ref = oracle.attn(q8, qs, k8, ks, v8t, vs, Nq, Nk, lam, causal=causal)
        got = host(out)
        assert np.isfinite(ref).all()
        assert_close(got, ref, f"lambda=2^{np.log2(lam):.0f}")


def test_fwd_large_score_form_switch(qa):
    """A row whose running max crosses 2^22 between two tiles while the earlier tile's
    keys still weigh in (ties at scores just below and just above 2^22): the kernel
    switches to its large-score form mid-row and rescales the partial sums it holds."""
    D, H, Nq, Nk = 64, 2, 64, 192
    q8 = np.zeros((1, H, 64, D), np.int8)
    q8[..., :Nq, :] = 1
    k8 = np.ones((1, H, Nk, D), np.int8)  # every score of a tile is acc * c with acc = 64
    qs = np.ones((1, H, 1), np.float32)
    # tile 0 just below 2^22, tile 1 just above, tile 2 well above (its keys dominate)
    ks = np.float32([(2.0 ** 22 - 2) / 64, (2.0 ** 22 + 1) / 64, (2.0 ** 22 + 40) / 64])
    ks = np.broadcast_to(ks, (1, H, 3)).copy()
    rng = np.random.default_rng(7)
    codes = oracle.e4m3_encode(np.float32([1, 1.5, 2, 3, -1, -1.5, -2, -3]))
    v8t = codes[rng.integers(0, 8, (1, H, D, Nk))]
    vs = np.full((1, H, D), 0.25, np.float32)
    ops = (q8, qs, k8, ks, v8t, vs)
    for last in (2, 3):  # without and with the dominating third tile
        n = 64 * last
        sub = (q8, qs, np.ascontiguousarray(k8[:, :, :n]), np.ascontiguousarray(ks[:, :, :last]),
               np.ascontiguousarray(v8t[..., :n]), vs)
        got = run_fwd(qa, sub, Nq, n, 1.0, False)
        ref = oracle.attn(*sub, Nq, n, 1.0)
        assert np.isfinite(got).all()
        assert_close(got, ref, f"form switch, {last} tiles")
    del ops


def test_i8kv_large_scores(qa):
    """The per-token-scale loop (prefill over an INT8 cache) with scores far beyond the
    ordinary range, against the oracle."""
    rng = np.random.default_rng(61)
    H, D, Nq, Nk, pos0 = 2, 128, 100, 700, 600
    q = W.bf16_bits(rng.standard_normal((Nq, H, D)).astype(np.float32))
    kc, kts = W.int8_cache(int(rng.integers(1 << 30)), 5, H, Nk, D)
    vc, vts = W.int8_cache(int(rng.integers(1 << 30)), 6, H, Nk, D)
    for lam in (2.0 ** 16, 2.0 ** 20, 2.0 ** 22):
        for S in (1, 3):
            say(f"i8kv large scores lambda=2^{np.log2(lam):.0f} splits={S}")
            out, _ = qa.attention_i8kv(dev_bf16(q), torch.from_numpy(kc).cuda(), torch.from_numpy(kts).cuda(),
                                       torch.from_numpy(vc).cuda(), torch.from_numpy(vts).cuda(), pos0,
                                       scale_log2=lam, out_dtype=torch.float32, kv_splits=S)
            torch.cuda.synchronize()
            ref, _ = oracle.fwd_i8kv(q, kc, kts, vc, vts, pos0, lam=lam, kv_splits=S)
            assert np.isfinite(ref).all()
            assert_close(host(out), ref, f"i8kv lambda=2^{np.log2(lam):.0f} S={S}")


def test_fwd_causal_fully_masked_rows(qa):
    say("causal Nq > Nk")
    rng = np.random.default_rng(5)
    Nq, Nk, D = 200, 70, 64
    q = W.bf16_bits(rng.standard_normal((1, Nq, 2, D)).astype(np.float32))
    k = W.bf16_bits(rng.standard_normal((1, Nk, 2, D)).astype(np.float32))
    v = W.bf16_bits(rng.standard_normal((1, Nk, 2, D)).astype(np.float32))
    out, _ = qa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.fwd(q, k, v, causal=True)
    o = host(out)
    assert not o[:, : Nq - Nk].any()
    assert_close(o, ref, "causal Nq>Nk")


def test_fwd_deterministic_and_stream(qa):
    say("determinism + side stream")
    w = W.TINY
    q, k, v = W.dense_inputs(w)
    a, _ = qa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b, _ = qa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v))
    torch.cuda.synchronize()
    assert np.array_equal(host(a), host(b))


def test_i8kv_small(qa):
    say("i8kv small")
    rng = np.random.default_rng(60)
    for H, D, Nq, Nk, pos0 in [(2, 128, 100, 700, 600), (3, 64, 64, 64, 0), (2, 128, 1, 129, 128), (1, 64, 130, 1000, 17)]:
        q = W.bf16_bits(rng.standard_normal((Nq, H, D)).astype(np.float32))
        kc, kts = W.int8_cache(int(rng.integers(1 << 30)), 5, H, Nk, D)
        vc, vts = W.int8_cache(int(rng.integers(1 << 30)), 6, H, Nk, D)
        out, ws = qa.attention_i8kv(dev_bf16(q), torch.from_numpy(kc).cuda(), torch.from_numpy(kts).cuda(),
                                    torch.from_numpy(vc).cuda(), torch.from_numpy(vts).cuda(), pos0,
                                    out_dtype=torch.float32)
        torch.cuda.synchronize()
        S = qa.qattn_fwd_i8kv_kv_splits(H, Nq, Nk, pos0)
        ref, it = oracle.fwd_i8kv(q, kc, kts, vc, vts, pos0, kv_splits=S)
        sec = i8kv_workspace(host(ws), H, Nq, Nk, D)
        assert np.array_equal(sec["v_scale"], it["v_scale"])
        assert np.array_equal(sec["q8"], it["q8"])
        assert np.array_equal(sec["vbf"], host(vbf_of(it["v8t"])))  # the V codes, bit for bit
        assert_close(host(out), ref, f"i8kv H={H} Nq={Nq} Nk={Nk} pos0={pos0}")


@pytest.mark.parametrize("D", [64, 128])
def test_i8kv_kv_splits(qa, D):
    """Explicit key-range counts: ranges empty for some rows (causal diagonal), for whole
    workgroups (ranges past a query block's last visible tile) and for every row (more
    ranges than tiles); each against the oracle's split loop and combine."""
    rng = np.random.default_rng(62 + D)
    for H, Nq, Nk, pos0, S in [(2, 100, 700, 600, 2), (2, 300, 1000, 17, 3), (3, 64, 200, 136, 5),
                               (1, 1, 129, 128, 16), (2, 513, 1500, 987, 7), (2, 40, 2048, 1000, 64)]:
        say(f"  i8kv split H={H} D={D} Nq={Nq} Nk={Nk} pos0={pos0} S={S}")
        q = W.bf16_bits(rng.standard_normal((Nq, H, D)).astype(np.float32))
        kc, kts = W.int8_cache(int(rng.integers(1 << 30)), 5, H, Nk, D)
        vc, vts = W.int8_cache(int(rng.integers(1 << 30)), 6, H, Nk, D)
        outs = []
        for od in (torch.float32, torch.bfloat16):
            out, _ = qa.attention_i8kv(dev_bf16(q), torch.from_numpy(kc).cuda(), torch.from_numpy(kts).cuda(),
                                       torch.from_numpy(vc).cuda(), torch.from_numpy(vts).cuda(), pos0,
                                       out_dtype=od, kv_splits=S)
            outs.append(out)
        torch.cuda.synchronize()
        ref, _ = oracle.fwd_i8kv(q, kc, kts, vc, vts, pos0, kv_splits=S)
        assert_close(host(outs[0]), ref, f"i8kv split H={H} Nq={Nq} Nk={Nk} pos0={pos0} S={S}")
        assert np.array_equal(host(outs[1]), bf16_of(host(outs[0])))


@pytest.mark.parametrize("D", [64, 128])
def test_kv_append_bit_exact(qa, D):
    """Codes and per-token scales bit for bit against the oracle: random rows over a wide
    range of magnitudes, zero rows, bf16 extremes, a projection-strided view, two appends
    into one cache; rows outside each append keep their previous bytes."""
    rng = np.random.default_rng(80 + D)
    H, Nmax = 3, 700
    cache = np.full((H, Nmax, D), 77, np.int8)
    ts = np.full((H, Nmax), -1.0, np.float32)
    dc, dts = torch.from_numpy(cache.copy()).cuda(), torch.from_numpy(ts.copy()).cuda()
    for pos, Nnew in [(5, 300), (305, 333)]:
        say(f"  kv append D={D} pos={pos} Nnew={Nnew}")
        x = rng.standard_normal((Nnew, 3, H, D)).astype(np.float32) * np.exp2(rng.uniform(-30, 30, (Nnew, 1, H, 1)))
        packed = W.bf16_bits(x)
        packed[0, 1] = 0  # zero rows
        packed[1, 1, 0, 0] = 0x7F7F  # largest finite bf16
        packed[2, 1, 1, :] = 0x0001  # smallest subnormal bf16
        dx = dev_bf16(packed)[:, 1]  # K projection of [N, 3, H, D]: strides {3 H D, D}
        qa.qattn_kv_append_i8(dx, dc, dts, pos)
        torch.cuda.synchronize()
        cache, ts = oracle.kv_append_i8(packed[:, 1], cache, ts, pos)
        assert np.array_equal(host(dc), cache)
        assert np.array_equal(host(dts).view(np.uint32), ts.view(np.uint32))


def test_i8kv_on_appended_cache(qa):
    """End to end: K and V appended to the caches by the library in two chunks, then the
    prefill over the caches; each step against the oracle's."""
    rng = np.random.default_rng(85)
    H, D, Nk, Nq = 4, 128, 1500, 200
    pos0 = Nk - Nq
    kx = W.bf16_bits(rng.standard_normal((Nk, H, D)).astype(np.float32))
    vx = W.bf16_bits(rng.standard_normal((Nk, H, D)).astype(np.float32))
    q = W.bf16_bits(rng.standard_normal((Nq, H, D)).astype(np.float32))
    kc = torch.zeros((H, Nk, D), dtype=torch.int8, device="cuda")
    vc = torch.zeros((H, Nk, D), dtype=torch.int8, device="cuda")
    kts = torch.zeros((H, Nk), dtype=torch.float32, device="cuda")
    vts = torch.zeros((H, Nk), dtype=torch.float32, device="cuda")
    okc, okts = np.zeros((H, Nk, D), np.int8), np.zeros((H, Nk), np.float32)
    ovc, ovts = okc.copy(), okts.copy()
    for lo, hi in [(0, 1000), (1000, Nk)]:
        qa.qattn_kv_append_i8(dev_bf16(kx[lo:hi]), kc, kts, lo)
        qa.qattn_kv_append_i8(dev_bf16(vx[lo:hi]), vc, vts, lo)
        okc, okts = oracle.kv_append_i8(kx[lo:hi], okc, okts, lo)
        ovc, ovts = oracle.kv_append_i8(vx[lo:hi], ovc, ovts, lo)
    out, _ = qa.attention_i8kv(dev_bf16(q), kc, kts, vc, vts, pos0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(host(kc), okc) and np.array_equal(host(vts), ovts)
    S = qa.qattn_fwd_i8kv_kv_splits(H, Nq, Nk, pos0)
    ref, _ = oracle.fwd_i8kv(q, okc, okts, ovc, ovts, pos0, kv_splits=S)
    assert_close(host(out), ref, "i8kv on appended cache")


# ----------------------------------------------------------------------------------
# many heads (grids of several hundred 256-row workgroups, every XCD busy)
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_many_heads_exact(qa, D, causal):
    """Exact-score operands over 256 heads: GPU == oracle within 2 ulp."""
    rng = np.random.default_rng(3000 + D + causal)
    H = 256
    for Nk in [1, 64, 65, 200, 333]:
        for Nq in [1, 129, 300]:
            if causal and Nq > Nk:
                continue
            say(f"many heads exact Nq={Nq} Nk={Nk} D={D} causal={causal}")
            ops = _exact_ops(rng, Nq, Nk, D, H=H)
            got = run_fwd(qa, ops, Nq, Nk, 1.0, causal)
            ref = oracle.attn(*ops, Nq, Nk, 1.0, causal=causal)
            ulp = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
            assert ulp.max() <= 2, (Nq, Nk, D, causal, ulp.max())


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_many_heads_random(qa, D, causal):
    rng = np.random.default_rng(4000 + D + causal)
    B, H = 2, 128
    for Nq, Nk in [(257, 129), (300, 555), (600, 64), (64, 700)]:
        if causal and Nq > Nk:
            Nq, Nk = Nk, Nq
        say(f"many heads random B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal}")
        q = W.bf16_bits(rng.standard_normal((B, Nq, H, D)).astype(np.float32))
        k = W.bf16_bits(rng.standard_normal((B, Nk, H, D)).astype(np.float32) + 1)
        v = W.bf16_bits(rng.standard_normal((B, Nk, H, D)).astype(np.float32))
        out, _ = qa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, out_dtype=torch.float32)
        torch.cuda.synchronize()
        ref, _ = oracle.fwd(q, k, v, causal=causal)
        assert_close(host(out), ref, f"B={B} H={H} Nq={Nq} Nk={Nk}")


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_head_split_bit_identical(qa, causal):
    """Rows are independent: one call over 256 heads and the same heads in calls of 16
    (other grid sizes, other workgroup-to-XCD mapping) give bit-identical outputs."""
    rng = np.random.default_rng(77 + causal)
    H, Nq, Nk, D, step = 256, 700, 1500, 128, 16
    say(f"head split H={H} Nq={Nq} Nk={Nk} causal={causal}")
    q = dev_bf16(W.bf16_bits(rng.standard_normal((1, Nq, H, D)).astype(np.float32)))
    k = dev_bf16(W.bf16_bits(rng.standard_normal((1, Nk, H, D)).astype(np.float32)))
    v = dev_bf16(W.bf16_bits(rng.standard_normal((1, Nk, H, D)).astype(np.float32)))
    t = qa.alloc_qk(1, H, Nq, Nk, D)
    tv = qa.alloc_v(1, H, Nk, D)
    qa.qattn_quant_qk(q, k, t["q8"], t["q_scale"], t["k8"], t["k_scale"], t["k_mean"])
    qa.qattn_quant_v(v, tv["v8t"], tv["v_scale"], tv["vbf"])
    whole = torch.empty((1, Nq, H, D), dtype=torch.float32, device="cuda")
    parts = torch.empty_like(whole)
    qa.qattn_fwd(t["q8"], t["q_scale"], t["k8"], t["k_scale"], tv["vbf"], tv["v_scale"], Nq, Nk, whole, 0.0, causal)
    for h in range(0, H, step):
        sl = slice(h, h + step)
        qa.qattn_fwd(t["q8"][:, sl], t["q_scale"][:, sl], t["k8"][:, sl], t["k_scale"][:, sl], tv["vbf"][:, sl],
                     tv["v_scale"][:, sl], Nq, Nk, parts[:, :, sl], 0.0, causal)
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int32), parts.view(torch.int32))


def test_binding_rejects_strided_code_buffers(qa):
    """Code buffers are passed by base pointer: a head slice of a B = 2 buffer is not
    dense and must be refused before any launch."""
    t = qa.alloc_qk(2, 4, 64, 64, 64)
    tv = qa.alloc_v(2, 4, 64, 64)
    out = torch.empty((2, 64, 2, 64), dtype=torch.float32, device="cuda")
    sl = slice(0, 2)
    with pytest.raises(ValueError):
        qa.qattn_fwd(t["q8"][:, sl], t["q_scale"][:, sl], t["k8"][:, sl], t["k_scale"][:, sl], tv["vbf"][:, sl],
                     tv["v_scale"][:, sl], 64, 64, out)


def test_i8kv_many_heads(qa):
    say("i8kv over many heads")
    rng = np.random.default_rng(61)
    for H, D, Nq, Nk, pos0 in [(256, 128, 100, 700, 600), (256, 64, 300, 1000, 17), (128, 128, 513, 600, 87)]:
        say(f"  H={H} D={D} Nq={Nq} Nk={Nk} pos0={pos0}")
        q = W.bf16_bits(rng.standard_normal((Nq, H, D)).astype(np.float32))
        kc, kts = W.int8_cache(int(rng.integers(1 << 30)), 5, H, Nk, D)
        vc, vts = W.int8_cache(int(rng.integers(1 << 30)), 6, H, Nk, D)
        out, _ = qa.attention_i8kv(dev_bf16(q), torch.from_numpy(kc).cuda(), torch.from_numpy(kts).cuda(),
                                   torch.from_numpy(vc).cuda(), torch.from_numpy(vts).cuda(), pos0,
                                   out_dtype=torch.float32)
        torch.cuda.synchronize()
        S = qa.qattn_fwd_i8kv_kv_splits(H, Nq, Nk, pos0)
        ref, _ = oracle.fwd_i8kv(q, kc, kts, vc, vts, pos0, kv_splits=S)
        assert_close(host(out), ref, f"i8kv H={H} Nq={Nq} Nk={Nk} pos0={pos0} S={S}")


# ----------------------------------------------------------------------------------
# full-size workloads, sampled outputs
# ----------------------------------------------------------------------------------
def _sample_rows(Nq, rng, nblk=3):
    blocks = sorted(set([0, (Nq - 1) // 64] + list(rng.integers(0, (Nq + 63) // 64, nblk))))
    rows = [r for b in blocks for r in range(b * 64, min(Nq, b * 64 + 64))]
    return np.array(rows)


@pytest.mark.parametrize("name", ["video_dit_b1_h24_n74000_d128", "causal_b1_h24_n37810_d128"])
def test_dense_workload_full_size(qa, name):
    """The two further dense workloads (74,000 tokens; causal at 37,810): every code, and
    the outputs of sampled query blocks of three heads (the five main workloads are
    compared in full by the whole-workload tests)."""
    w = W.BY_NAME[name]
    say(f"full-size {w.name}: generating inputs")
    q, k, v = W.dense_inputs(w)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    out, inter = qa.attention(dq, dk, dv, causal=w.causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    say("  oracle quantizers")
    q8, qs, k8, ks, mean = oracle.quant_qk(q, k)
    v8t, vs = oracle.quant_v(v)
    assert np.array_equal(host(inter["k_mean"]), mean)
    assert np.array_equal(host(inter["q8"]), q8) and np.array_equal(host(inter["q_scale"]), qs)
    assert np.array_equal(host(inter["k8"]), k8) and np.array_equal(host(inter["k_scale"]), ks)
    assert np.array_equal(host(inter["v8t"]), v8t) and np.array_equal(host(inter["v_scale"]), vs)
    rng = np.random.default_rng(9)
    rows = _sample_rows(w.Nq, rng, nblk=2 if w.Nq > 10000 else 3)
    heads = sorted(set([0, w.H - 1, int(rng.integers(w.H))]))
    say(f"  oracle attention on {len(rows)} rows x {len(heads)} heads")
    lam = oracle.default_lambda(w.D)
    sel = (slice(None), heads)
    ref = oracle.attn(q8[sel], qs[sel], k8[sel], ks[sel], v8t[sel], vs[sel], w.Nq, w.Nk, lam, causal=w.causal,
                      rows=rows)
    got = host(out)[:, rows][:, :, heads]
    r = assert_close(got, ref, w.name)
    say(f"  max err / rms = {r:.2e}")
    out16, _ = qa.attention(dq, dk, dv, causal=w.causal, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(host(out16)[:, rows][:, :, heads], bf16_of(host(out)[:, rows][:, :, heads]))


