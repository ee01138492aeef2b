"""C-ABI checks that need no GPU: the library loads, exports every function the header
declares, and rejects bad arguments before any HIP call (so nothing is launched)."""
import ctypes as ct
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qattn.h")
LIB = os.path.join(ROOT, "quantized_attention_qattn_amd", "libqattn.so")

EINVAL, EUNSUP, EWS = -1, -2, -3
I64x3 = ct.c_int64 * 3
I64x2 = ct.c_int64 * 2
A = 0x10000000  # an aligned, never-dereferenced address (validation fails before use)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import importlib.util

        spec = importlib.util.spec_from_file_location("qattn_build", os.path.join(os.path.dirname(LIB), "_build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()
    L = ct.CDLL(LIB)
    P, I, F = ct.c_void_p, ct.c_int, ct.c_float
    L.qattn_quant_qk.argtypes = [P, I64x3, P, I64x3, I, I, I, I, I, P, P, P, P, P, P]
    L.qattn_quant_v.argtypes = [P, I64x3, I, I, I, I, P, P, P, P]
    L.qattn_fwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, P, I64x3, I, P]
    L.qattn_prep.argtypes = [P, I64x3, P, I64x3, P, I64x3, I, I, I, I, I, P, P, P, P, P, P, P, P, P]
    L.qattn_fwd_i8kv.argtypes = [P, I64x2, P, P, P, P, I, I, I, I, I, F, I, P, ct.c_size_t, P, I64x2, I, P]
    L.qattn_fwd_i8kv_workspace_bytes.argtypes = [I, I, I, I, I]
    L.qattn_fwd_i8kv_workspace_bytes.restype = ct.c_size_t
    L.qattn_fwd_i8kv_kv_splits.argtypes = [I, I, I, I]
    L.qattn_fwd_i8kv_kv_splits.restype = I
    L.qattn_selftest_p8_codes.argtypes = [P, P, ct.c_int64, ct.c_int, P]
    L.qattn_kv_append_i8.argtypes = [P, I64x2, I, I, I, P, P, I, I, P]
    L.qattn_fwd_i8kv_noalloc.argtypes = [P, I64x2, P, P, P, P, I, I, I, I, I, F, I, P, I64x2, I, P]
    L.qattn_status_string.argtypes = [I]
    L.qattn_status_string.restype = ct.c_char_p
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(qattn_[a-z0-9_]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["qattn_quant_qk", "qattn_quant_v", "qattn_prep", "qattn_fwd", "qattn_fwd_i8kv", "qattn_fwd_i8kv_workspace_bytes",
              "qattn_fwd_i8kv_kv_splits", "qattn_kv_append_i8", "qattn_status_string", "qattn_selftest_p8_codes"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5):
        assert lib.qattn_status_string(s)
    assert b"unknown" in lib.qattn_status_string(7)


def test_workspace_bytes(lib):
    # H*D*4 + H*Nq_pad*D + H*Nq_pad/64*4 + H*D*Nk_pad*2, each rounded up to 256 bytes
    H, Nq, Nk, D = 32, 1024, 32768, 128
    expect = H * D * 4 + H * Nq * D + ((H * Nq // 64 * 4 + 255) // 256) * 256 + H * D * Nk * 2
    assert lib.qattn_fwd_i8kv_workspace_bytes(H, Nq, Nk, D, 1) == expect
    # split-KV adds S*H*Nq_pad*D*4 (partial O) + S*H*Nq_pad*8 (m, d')
    assert lib.qattn_fwd_i8kv_workspace_bytes(H, Nq, Nk, D, 4) == expect + 4 * H * Nq * D * 4 + 4 * H * Nq * 8
    assert lib.qattn_fwd_i8kv_workspace_bytes(2, 1, 1, 64, 1) == 512 + 2 * 64 * 64 + 256 + 2 * 64 * 64 * 2
    assert lib.qattn_fwd_i8kv_workspace_bytes(0, 1, 1, 64, 1) == 0
    assert lib.qattn_fwd_i8kv_workspace_bytes(2, 1, 1, 96, 1) == 0
    assert lib.qattn_fwd_i8kv_workspace_bytes(2, 1, 1, 64, 0) == 0
    assert lib.qattn_fwd_i8kv_workspace_bytes(2, 1, 1, 64, 65) == 0


def test_kv_split_rule(lib):
    # ceil(256 / (H * ceil(Nq / 256))), at least 16 key tiles per range, at most 64, at least 1
    assert lib.qattn_fwd_i8kv_kv_splits(32, 1024, 32768, 31744) == 2  # 128 workgroups, 512 tiles
    assert lib.qattn_fwd_i8kv_kv_splits(32, 512, 65536, 65024) == 4  # 64 workgroups, 1024 tiles
    assert lib.qattn_fwd_i8kv_kv_splits(2, 64, 128, 64) == 1  # 2 tiles: no split
    assert lib.qattn_fwd_i8kv_kv_splits(1, 1, 65536, 100) == 1  # 2 visible tiles
    assert lib.qattn_fwd_i8kv_kv_splits(1, 1, 65536, 65535) == 64  # one query, 1024 tiles: capped at 64
    assert lib.qattn_fwd_i8kv_kv_splits(1, 1, 65536, 0) == 1  # the query sees 1 key
    assert lib.qattn_fwd_i8kv_kv_splits(8, 256, 8192, 2000) == 2  # 36 visible tiles: 2 ranges of >= 16
    assert lib.qattn_fwd_i8kv_kv_splits(2, 64, 128, 65) == 0  # pos0 + Nq > Nk
    assert lib.qattn_fwd_i8kv_kv_splits(0, 64, 128, 0) == 0


def _qk(lib, **kw):
    a = dict(q=A, qs=I64x3(1024, 128, 64), k=A, ks=I64x3(1024, 128, 64), B=1, H=2, Nq=64, Nk=64, D=64,
             q8=A, q_scale=A, k8=A, k_scale=A, k_mean=A)
    a.update(kw)
    return lib.qattn_quant_qk(a["q"], a["qs"], a["k"], a["ks"], a["B"], a["H"], a["Nq"], a["Nk"], a["D"], a["q8"],
                              a["q_scale"], a["k8"], a["k_scale"], a["k_mean"], None)


def test_quant_qk_validation(lib):
    assert _qk(lib, q=None) == EINVAL
    assert _qk(lib, k_mean=None) == EINVAL
    assert _qk(lib, D=96) == EUNSUP
    assert _qk(lib, Nq=0) == EINVAL
    assert _qk(lib, B=-1) == EINVAL
    assert _qk(lib, q=A + 2) == EINVAL  # bf16 view not 16-byte aligned
    assert _qk(lib, qs=I64x3(1024, 129, 64)) == EINVAL  # stride not a multiple of 8 elements
    assert _qk(lib, k8=A + 16) == EINVAL  # code buffer not 256-byte aligned
    assert _qk(lib, Nk=1 << 29) == EINVAL


def test_quant_v_validation(lib):
    st = I64x3(1024, 128, 64)
    assert lib.qattn_quant_v(None, st, 1, 2, 64, 64, A, A, None, None) == EINVAL
    assert lib.qattn_quant_v(A, st, 1, 2, 64, 80, A, A, None, None) == EUNSUP
    assert lib.qattn_quant_v(A, st, 1, 2, 64, 64, A + 1, A, None, None) == EINVAL
    assert lib.qattn_quant_v(A, st, 1, 2, 64, 64, A, A, A + 16, None) == EINVAL  # vbf not 256-byte aligned


def test_prep_validation(lib):
    # the fused preparation rejects what either separate call rejects, before any launch
    st = I64x3(1024, 128, 64)
    ok = dict(q=A, qs=st, k=A, ks=st, v=A, vs=st, B=1, H=2, Nq=64, Nk=64, D=64, q8=A, q_scale=A, k8=A, k_scale=A,
              k_mean=A, v8t=A, v_scale=A, vbf=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.qattn_prep(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["B"], a["H"], a["Nq"], a["Nk"],
                              a["D"], a["q8"], a["q_scale"], a["k8"], a["k_scale"], a["k_mean"], a["v8t"],
                              a["v_scale"], a["vbf"], None)

    assert call(v=None) == EINVAL
    assert call(v8t=None) == EINVAL  # neither the codes nor their bf16 values requested
    assert call(v8t=None, vbf=A + 16) == EINVAL  # vbf alone, but not 256-byte aligned
    assert call(k_mean=None) == EINVAL
    assert call(D=96) == EUNSUP
    assert call(Nk=0) == EINVAL
    assert call(H=1 << 17) == EINVAL
    assert call(v=A + 2) == EINVAL  # bf16 view not 16-byte aligned
    assert call(vs=I64x3(1024, 129, 64)) == EINVAL  # stride not a multiple of 8 elements
    assert call(v8t=A + 16) == EINVAL  # code buffer not 256-byte aligned
    assert call(vbf=A + 16) == EINVAL  # vbf not 256-byte aligned
    assert call(v_scale=A + 2) == EINVAL


def test_fwd_validation(lib):
    st = I64x3(1024, 128, 64)
    ok = dict(q8=A, qs=A, k8=A, ks=A, v8=A, vs=A, B=1, H=2, Nq=64, Nk=64, D=64, sl=0.0, causal=0, out=A, st=st, od=1)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.qattn_fwd(a["q8"], a["qs"], a["k8"], a["ks"], a["v8"], a["vs"], a["B"], a["H"], a["Nq"], a["Nk"],
                             a["D"], a["sl"], a["causal"], a["out"], a["st"], a["od"], None)

    assert call(v8=None) == EINVAL
    assert call(D=256) == EUNSUP
    assert call(od=7) == EINVAL
    assert call(out=A + 4) == EINVAL  # f32 output base must be 16-byte aligned
    assert call(st=I64x3(1024, 130, 64)) == EINVAL
    assert call(sl=float("nan")) == EINVAL
    assert call(H=0) == EINVAL
    assert call(Nq=0) == EINVAL  # empty inputs are refused, not launched
    assert call(Nk=0) == EINVAL
    assert call(Nk=(1 << 28) + 1) == EINVAL  # beyond the largest token count
    assert call(Nk=1 << 24, D=128) == EINVAL  # a (b, h) slice of 2^31 code bytes: past 32-bit offsets
    assert call(Nk=1 << 25, D=64) == EINVAL


def test_i8kv_validation(lib):
    qs = I64x2(128, 64)
    os_ = I64x2(128, 64)
    need = lib.qattn_fwd_i8kv_workspace_bytes(2, 64, 128, 64, 1)
    need2 = lib.qattn_fwd_i8kv_workspace_bytes(2, 64, 128, 64, 2)

    def call(pos0=64, ws=A, wsb=need, D=64, Nq=64, Nk=128, k=A, S=0):
        return lib.qattn_fwd_i8kv(A, qs, k, A, A, A, 2, Nq, Nk, D, pos0, 0.0, S, ws, wsb, A, os_, 0, None)

    assert call(pos0=65) == EINVAL  # pos0 + Nq > Nk
    assert call(pos0=-1) == EINVAL
    assert call(wsb=need - 1) == EWS
    assert call(ws=A + 128) == EINVAL
    assert call(D=32) == EUNSUP
    assert call(k=None) == EINVAL
    assert call(S=65) == EINVAL
    assert call(S=-1) == EINVAL
    assert call(S=2, wsb=need2 - 1) == EWS  # the partial results need room


def test_kv_append_validation(lib):
    st = I64x2(3 * 2 * 64, 64)  # one projection of a packed [N, 3, H=2, D=64] tensor

    def call(x=A, s=st, Nnew=10, H=2, D=64, cache=A, ts=A, Nmax=100, pos=0):
        return lib.qattn_kv_append_i8(x, s, Nnew, H, D, cache, ts, Nmax, pos, None)

    assert call(cache=None) == EINVAL
    assert call(ts=None) == EINVAL
    assert call(D=96) == EUNSUP
    assert call(pos=91) == EINVAL  # pos + Nnew > Nmax
    assert call(pos=-1) == EINVAL
    assert call(x=A + 2) == EINVAL  # bf16 view not 16-byte aligned
    assert call(s=I64x2(3 * 2 * 64, 63)) == EINVAL  # head stride not a multiple of 8 elements
    assert call(cache=A + 4) == EINVAL  # cache not 8-byte aligned
    assert call(Nnew=0) == EINVAL
    assert call(Nmax=0) == EINVAL


def test_p8_codes_validation(lib):
    assert lib.qattn_selftest_p8_codes(None, A, 10, 0, None) == EINVAL
    assert lib.qattn_selftest_p8_codes(A, A, 0, 0, None) == EINVAL
    assert lib.qattn_selftest_p8_codes(A, A, 10, 2, None) == EINVAL


def test_product_path_does_not_use_the_oracle():
    """The binding and the HIP sources never import, load or name the oracle."""
    pkg = os.path.join(ROOT, "quantized_attention_qattn_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text and "qattn_oracle" not in text, f


def test_noalloc_validation(lib):
    """The allocation-free prefill call checks its arguments like qattn_fwd_i8kv and
    refuses a call whose workspace exceeds its static array, all before any HIP call."""
    st = I64x2(32 * 128, 128)

    def call(H=32, Nq=1024, Nk=65536, D=128, pos0=64512, q=A, k=A, out=A):
        return lib.qattn_fwd_i8kv_noalloc(q, st, k, A, A, A, H, Nq, Nk, D, pos0, 0.0, 0, out, st, 1, None)

    assert call() == -5  # 32 heads over 64K cached tokens: beyond the static workspace
    assert call(q=None) == EINVAL
    assert call(pos0=65000) == EINVAL  # pos0 + Nq > Nk
    assert call(D=96) == EUNSUP
    assert call(out=A + 4) == EINVAL
