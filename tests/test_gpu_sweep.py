"""GPU parity over seeded random configurations: shapes (batch, heads, ragged query and key
counts from 1 to ~1,500, D in {64, 128}), causal and not, softmax scales from 1/16 to 64
times the default, value distributions (normal, heavy-tailed, per-channel offsets, tiny and
large magnitudes), and prefill chunks over an INT8 cache with random positions and key
range counts.  Each case: codes and scales bit for bit against the oracle, fp32 output
within 2e-3 * RMS of the oracle, bf16 output the round-to-nearest-even of the fp32 one."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
TOL = 2e-3
DENSE_CASES = 40
I8KV_CASES = 24


@pytest.fixture(scope="module")
def qa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_attention_qattn_amd as qa

    oracle.build(force=False)
    return qa


def _dev_bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(torch.bfloat16)


def _host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _close(gpu, ref, what):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.isfinite(gpu).all(), what
    rms = np.sqrt((ref ** 2).mean())
    err = np.abs(gpu - ref).max()
    assert err <= TOL * rms, f"{what}: max abs err {err:.3e} > {TOL} * rms {rms:.3e}"


def _count(rng, lo, hi):
    """Log-uniform integer in [lo, hi]."""
    return int(np.clip(np.round(np.exp(rng.uniform(np.log(lo), np.log(hi + 1)))) - 0, lo, hi))


def _values(rng, shape, kind):
    if kind == "normal":
        x = rng.standard_normal(shape)
    elif kind == "heavy":
        x = rng.standard_t(3, shape)
    elif kind == "offset":  # per-channel offsets, as the pages' K
        x = rng.standard_normal(shape) + rng.uniform(-4, 4, shape[-1])
    elif kind == "tiny":
        x = rng.standard_normal(shape) * 1e-3
    else:  # "large"
        x = rng.standard_normal(shape) * 30.0
    return W.bf16_bits(x.astype(np.float32))


def dense_case(qa, rng, tag=""):
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 7))
    D = int(rng.choice([64, 128]))
    Nq, Nk = _count(rng, 1, 1500), _count(rng, 1, 1500)
    causal = bool(rng.integers(0, 2))
    kinds = [str(rng.choice(["normal", "heavy", "offset", "tiny", "large"])) for _ in range(3)]
    # the library takes the scale as fp32: draw it as an fp32 value
    lam = float(np.float32(oracle.default_lambda(D) * np.exp2(rng.uniform(-4, 6)))) if rng.integers(0, 2) else None
    what = f"{tag} B={B} H={H} D={D} Nq={Nq} Nk={Nk} causal={causal} kinds={kinds} lam={lam}"
    print(what, flush=True)
    q = _values(rng, (B, Nq, H, D), kinds[0])
    k = _values(rng, (B, Nk, H, D), kinds[1])
    v = _values(rng, (B, Nk, H, D), kinds[2])
    t = qa.prep(_dev_bf16(q), _dev_bf16(k), _dev_bf16(v))
    outs = {}
    for od in (torch.float32, torch.bfloat16):
        outs[od] = torch.empty((B, Nq, H, D), dtype=od, device="cuda")
        qa.fwd_from(t, Nq, Nk, outs[od], 0.0 if lam is None else lam, causal)
    torch.cuda.synchronize()
    ref, it = oracle.fwd(q, k, v, lam=lam, causal=causal)
    nqp, nkp = oracle.npad(Nq), oracle.npad(Nk)
    assert np.array_equal(_host(t["q8"]).reshape(it["q8"].shape), it["q8"]), what
    assert np.array_equal(_host(t["k8"]).reshape(it["k8"].shape), it["k8"]), what
    assert np.array_equal(_host(t["q_scale"]).reshape(it["q_scale"].shape), it["q_scale"]), what
    assert np.array_equal(_host(t["k_scale"]).reshape(it["k_scale"].shape), it["k_scale"]), what
    assert np.array_equal(_host(t["v8t"]).reshape(it["v8t"].shape), it["v8t"]), what
    assert np.array_equal(_host(t["v_scale"]).reshape(it["v_scale"].shape), it["v_scale"]), what
    assert (nqp, nkp) == (it["q8"].shape[2], it["k8"].shape[2]), what
    _close(_host(outs[torch.float32]), ref, what)
    assert np.array_equal(_host(outs[torch.bfloat16]), W.bf16_bits(_host(outs[torch.float32]))), what


def i8kv_case(qa, rng, tag=""):
    H = int(rng.integers(1, 5))
    D = int(rng.choice([64, 128]))
    Nk = _count(rng, 1, 3000)
    Nq = _count(rng, 1, min(Nk, 600))
    pos0 = int(rng.integers(0, Nk - Nq + 1))
    S = int(rng.choice([0, 1, int(rng.integers(2, 17))]))
    # the library takes the scale as fp32: draw it as an fp32 value
    lam = float(np.float32(oracle.default_lambda(D) * np.exp2(rng.uniform(-4, 6)))) if rng.integers(0, 2) else None
    what = f"{tag} i8kv H={H} D={D} Nq={Nq} Nk={Nk} pos0={pos0} S={S} lam={lam}"
    print(what, flush=True)
    q = _values(rng, (Nq, H, D), str(rng.choice(["normal", "heavy", "large"])))
    kc, kts = W.int8_cache(int(rng.integers(1 << 30)), 5, H, Nk, D)
    vc, vts = W.int8_cache(int(rng.integers(1 << 30)), 6, H, Nk, D)
    args = [torch.from_numpy(x).cuda() for x in (kc, kts, vc, vts)]
    outs = {}
    for od in (torch.float32, torch.bfloat16):
        outs[od], _ = qa.attention_i8kv(_dev_bf16(q), *args, pos0, scale_log2=0.0 if lam is None else lam,
                                        out_dtype=od, kv_splits=S)
    torch.cuda.synchronize()
    S_used = S if S > 0 else qa.qattn_fwd_i8kv_kv_splits(H, Nq, Nk, pos0)
    ref, _ = oracle.fwd_i8kv(q, kc, kts, vc, vts, pos0, lam=lam, kv_splits=S_used)
    _close(_host(outs[torch.float32]), ref, what)
    assert np.array_equal(_host(outs[torch.bfloat16]), W.bf16_bits(_host(outs[torch.float32]))), what


def test_dense_random_configurations(qa):
    rng = np.random.default_rng(90210)
    for c in range(DENSE_CASES):
        dense_case(qa, rng, f"[{c}]")


def test_i8kv_random_configurations(qa):
    rng = np.random.default_rng(31337)
    for c in range(I8KV_CASES):
        i8kv_case(qa, rng, f"[{c}]")
