"""Whole-workload parity on the GPU: every code, scale and output element of each of the
five workloads, in the launch configuration the benchmark times (qattn_prep then
qattn_fwd for the dense workloads; qattn_fwd_i8kv with the library's key-range rule for
the prefill ones), against the CPU oracle.

* codes and scales: bit for bit (the prefill workspace's q codes, V scales and V values
  included);
* outputs: max |gpu - oracle| <= 2e-3 * RMS(oracle) on the fp32 output, over every row
  and head; the bf16 output equals the round-to-nearest-even of the GPU's fp32 output.

The oracle's attention for the 37,810-token workload runs in six parts of four heads
each (one test per part), so that every test ends within a minute or so.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
TOL = 2e-3
_cache = {}


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def qa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_attention_qattn_amd as qa

    oracle.build(force=False)
    yield qa
    _cache.clear()


def dev_bf16(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _gpu_dense(qa, w):
    q, k, v = W.dense_inputs(w)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    t = {**qa.alloc_qk(w.B, w.H, w.Nq, w.Nk, w.D), **qa.alloc_v(w.B, w.H, w.Nk, w.D)}
    qa.qattn_prep(dq, dk, dv, t["q8"], t["q_scale"], t["k8"], t["k_scale"], t["k_mean"], t["v8t"], t["v_scale"],
                  t["vbf"])
    o32 = torch.empty((w.B, w.Nq, w.H, w.D), dtype=torch.float32, device="cuda")
    o16 = torch.empty((w.B, w.Nq, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    for o in (o32, o16):
        qa.qattn_fwd(t["q8"], t["q_scale"], t["k8"], t["k_scale"], t["vbf"], t["v_scale"], w.Nq, w.Nk, o, 0.0,
                     w.causal)
    torch.cuda.synchronize()
    res = {n: host(x) for n, x in t.items()}
    res.update(out32=host(o32), out16=host(o16), inputs=(q, k, v))
    return res


def _gpu_i8kv(qa, w):
    q, kc, kts, vc, vts = W.i8kv_inputs(w)
    S = qa.qattn_fwd_i8kv_kv_splits(w.H, w.Nq, w.Nk, w.pos0)
    args = [torch.from_numpy(x).cuda() for x in (kc, kts, vc, vts)]
    ws = torch.empty(qa.qattn_fwd_i8kv_workspace_bytes(w.H, w.Nq, w.Nk, w.D, S), dtype=torch.uint8, device="cuda")
    o32 = torch.empty((w.Nq, w.H, w.D), dtype=torch.float32, device="cuda")
    o16 = torch.empty((w.Nq, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    sections = None
    for o in (o32, o16):
        qa.qattn_fwd_i8kv(dev_bf16(q), *args, w.pos0, ws, o, kv_splits=S)
        torch.cuda.synchronize()
        if sections is None:
            sections = host(ws).copy()
    return dict(out32=host(o32), out16=host(o16), ws=sections, S=S, inputs=(q, kc, kts, vc, vts))


def _gpu(qa, w):
    if w.name not in _cache:
        _cache.clear()
        say(f"GPU run of {w.name}")
        _cache[w.name] = _gpu_dense(qa, w) if w.kind == "dense" else _gpu_i8kv(qa, w)
    return _cache[w.name]


def _vbf_bits(v8t: np.ndarray) -> np.ndarray:
    dec = oracle.e4m3_decode_table().astype(np.float32)
    return W.bf16_bits(dec[v8t])


def _ws_sections(wsh, H, Nq, Nk, D):
    nqp, nkp = oracle.npad(Nq), oracle.npad(Nk)
    r = lambda n: (n + 255) // 256 * 256
    out, off = {}, 0
    for name, nbytes, dt, shape in [("v_scale", H * D * 4, np.float32, (H, D)), ("q8", H * nqp * D, np.int8, (H, nqp, D)),
                                    ("q_scale", H * (nqp // 64) * 4, np.float32, (H, nqp // 64)),
                                    ("vbf", H * D * nkp * 2, np.uint16, (H, D, nkp))]:
        out[name] = wsh[off: off + nbytes].view(dt).reshape(shape)
        off += r(nbytes)
    return out


NAMES = ["tiny_b1_h2_n256_d64", "dense_b1_h16_n4096_d128", "prefill_i8kv_h32_d128_q1024_ctx32768",
         "prefill_i8kv_h32_d128_q512_ctx65536", "video_dit_b1_h24_n37810_d128"]


def _check_codes(g, w):
    """Every code and scale of the workload, bit for bit."""
    if w.kind == "dense":
        q, k, v = g["inputs"]
        q8, qs, k8, ks, mean = oracle.quant_qk(q, k)
        v8t, vs = oracle.quant_v(v)
        for n, ref in dict(q8=q8, q_scale=qs, k8=k8, k_scale=ks, k_mean=mean, v8t=v8t, v_scale=vs).items():
            assert np.array_equal(g[n].view(np.uint8), ref.view(np.uint8)), n
        assert np.array_equal(g["vbf"], _vbf_bits(v8t))
    else:
        q, kc, kts, vc, vts = g["inputs"]
        q8, qs = oracle.quant_i8_blocks(q[None])
        v8t, vs = oracle.requant_v_cache(vc, vts)
        sec = _ws_sections(g["ws"], w.H, w.Nq, w.Nk, w.D)
        assert np.array_equal(sec["q8"], q8[0]) and np.array_equal(sec["q_scale"].view(np.uint32), qs[0].view(np.uint32))
        assert np.array_equal(sec["v_scale"].view(np.uint32), vs.view(np.uint32))
        assert np.array_equal(sec["vbf"], _vbf_bits(v8t))


def _parts():
    """(workload, first head, end head): the codes first (h0 = -1), then the outputs."""
    out = []
    for name in NAMES:
        w = W.BY_NAME[name]
        step = 4 if w.Nq * w.Nk * w.H > 2e10 else w.H
        out += [(name, -1, -1)] + [(name, h, min(w.H, h + step)) for h in range(0, w.H, step)]
    return out


@pytest.mark.parametrize("name,h0,h1", _parts(),
                         ids=[f"{n}-codes" if a < 0 else f"{n}-heads{a}-{b}" for n, a, b in _parts()])
def test_whole_workload(qa, name, h0, h1):
    """h0 < 0: every code and scale, bit for bit.  Otherwise every output element of heads
    [h0, h1): fp32 within 2e-3 * RMS of the oracle, bf16 = RNE of the GPU's own fp32."""
    w = W.BY_NAME[name]
    g = _gpu(qa, w)
    if h0 < 0:
        _check_codes(g, w)
        return
    heads = list(range(h0, h1))
    if w.kind == "dense":
        q, k, v = g["inputs"]
        sel = (slice(None), slice(None), heads)
        ref, _ = oracle.fwd(q[sel], k[sel], v[sel], causal=w.causal)
        got = g["out32"][:, :, h0:h1]
        got16 = g["out16"][:, :, h0:h1]
    else:
        q, kc, kts, vc, vts = g["inputs"]
        ref, _ = oracle.fwd_i8kv(q[:, heads], kc[heads], kts[heads], vc[heads], vts[heads], w.pos0,
                                 kv_splits=g["S"])
        got = g["out32"][:, h0:h1]
        got16 = g["out16"][:, h0:h1]
    assert np.isfinite(got).all()
    ref64 = ref.astype(np.float64)
    rms = np.sqrt((ref64 ** 2).mean())
    err = np.abs(got.astype(np.float64) - ref64).max()
    rel = np.linalg.norm(got.astype(np.float64) - ref64) / np.linalg.norm(ref64)
    say(f"{name} heads {h0}-{h1}: max|err|/rms = {err / rms:.3e}, rel-L2 vs oracle = {rel:.3e}")
    assert err <= TOL * rms, f"{name} heads {h0}-{h1}: max abs err {err:.3e} > {TOL} * rms {rms:.3e}"
    assert np.array_equal(got16, W.bf16_bits(got))
