"""The allocation-free prefill entry point (qattn_fwd_i8kv_noalloc) against the one with
a caller workspace (qattn_fwd_i8kv), through the C-ABI: two calls in a row, the second
with a smaller input, each bit-identical to the workspace call (the same kernels and key
ranges) and within the accuracy bar of the oracle; a call needing more than the static
array is refused before any launch."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module")
def qa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_attention_qattn_amd as qa

    oracle.build(force=False)
    return qa


def _dev_bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(torch.bfloat16)


def test_noalloc_matches_workspace_call(qa):
    rng = np.random.default_rng(808)
    for H, D, Nq, Nk, pos0 in [(8, 128, 300, 3000, 2700), (4, 64, 100, 700, 600)]:
        print(f"noalloc H={H} D={D} Nq={Nq} Nk={Nk} pos0={pos0}", flush=True)
        q = W.bf16_bits(rng.standard_normal((Nq, H, D)).astype(np.float32))
        kc, kts = W.int8_cache(int(rng.integers(1 << 30)), 5, H, Nk, D)
        vc, vts = W.int8_cache(int(rng.integers(1 << 30)), 6, H, Nk, D)
        args = [torch.from_numpy(x).cuda() for x in (kc, kts, vc, vts)]
        dq = _dev_bf16(q)
        ref_out, _ = qa.attention_i8kv(dq, *args, pos0, out_dtype=torch.float32)
        got = torch.empty((Nq, H, D), dtype=torch.float32, device="cuda")
        qa.qattn_fwd_i8kv_noalloc(dq, *args, pos0, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), ref_out.view(torch.int32))
        S = qa.qattn_fwd_i8kv_kv_splits(H, Nq, Nk, pos0)
        ref, _ = oracle.fwd_i8kv(q, kc, kts, vc, vts, pos0, kv_splits=S)
        g, r = got.cpu().numpy().astype(np.float64), ref.astype(np.float64)
        assert np.abs(g - r).max() <= TOL * np.sqrt((r ** 2).mean())


def test_noalloc_refuses_beyond_the_scratch(qa):
    H, D, Nq, Nk, pos0 = 32, 128, 1024, 65536, 64512
    assert qa.qattn_fwd_i8kv_workspace_bytes(H, Nq, Nk, D, qa.qattn_fwd_i8kv_kv_splits(H, Nq, Nk, pos0)) > \
        qa.QATTN_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((Nq, H, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((H, Nk, D), dtype=torch.int8, device="cuda")
    ks = torch.zeros((H, Nk), dtype=torch.float32, device="cuda")
    out = torch.empty((Nq, H, D), dtype=torch.float32, device="cuda")
    with pytest.raises(qa.QattnError) as e:
        qa.qattn_fwd_i8kv_noalloc(q, kc, ks, kc, ks, pos0, out)
    assert e.value.status == qa.QATTN_ESCRATCH
