"""CPU oracle for the quantized attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import this package.  The product path (``quantized_attention_qattn_amd``) never
imports it and fails loudly when its HIP library is missing.

The arithmetic lives in ``qattn_oracle.c`` (plain C, fp32 operations written out,
``-ffp-contract=off``); this module builds it, marshals numpy arrays to it, runs
independent (b, h, row-chunk) pieces on a thread pool (rows are independent), and adds
the FP64 reference attention used by the pins.

Parity status of each function (what pins it) is listed in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import concurrent.futures as _cf
import ctypes as _ct
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qattn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libqattn_oracle.so")
TILE = 64

_lock = threading.Lock()
_lib = None

_CFLAGS = ["-O3", "-march=x86-64-v3", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            L = _ct.CDLL(_LIB_PATH)
            P = _ct.c_void_p
            i32, i64, f32 = _ct.c_int, _ct.c_int64, _ct.c_float
            L.orc_bf16_to_f32.argtypes = [_ct.c_uint16]
            L.orc_bf16_to_f32.restype = f32
            L.orc_f32_to_bf16.argtypes = [f32]
            L.orc_f32_to_bf16.restype = _ct.c_uint16
            L.orc_e4m3_decode.argtypes = [_ct.c_uint8]
            L.orc_e4m3_decode.restype = _ct.c_double
            L.orc_e4m3_encode.argtypes = [f32]
            L.orc_e4m3_encode.restype = _ct.c_uint8
            L.orc_exp2.argtypes = [f32]
            L.orc_exp2.restype = f32
            L.orc_k_mean.argtypes = [P, P, i32, i32, i32, i32, P]
            L.orc_k_mean.restype = _ct.c_long
            L.orc_quant_i8_blocks.argtypes = [P, P, P, i32, i32, i32, i32, P, P]
            L.orc_quant_i8_blocks.restype = None
            L.orc_quant_v.argtypes = [P, P, i32, i32, i32, i32, P, P]
            L.orc_quant_v.restype = None
            L.orc_requant_v_cache.argtypes = [P, P, i32, i32, i32, P, P]
            L.orc_requant_v_cache.restype = None
            L.orc_attn_rows.argtypes = [P, P, P, P, i32, P, i64, P, i32, i32, i32, f32, i32, i64, i32, i32, P]
            L.orc_attn_rows.restype = None
            L.orc_attn_rows_part.argtypes = [P, P, P, P, i32, P, i64, i32, i32, i32, f32, i32, i64, i32, i32, i32,
                                             i32, P, P, P]
            L.orc_attn_rows_part.restype = None
            L.orc_combine_rows.argtypes = [i32, P, P, P, P, i32, i32, P]
            L.orc_combine_rows.restype = None
            L.orc_kv_append_i8.argtypes = [P, P, i32, i32, i32, P, P, i32, i32]
            L.orc_kv_append_i8.restype = None
            L.orc_default_lambda.argtypes = [i32]
            L.orc_default_lambda.restype = f32
            L.orc_exp2_check_grid.argtypes = [_ct.c_uint32, _ct.c_uint32]
            L.orc_exp2_check_grid.restype = _ct.c_long
            L.orc_p8_codes_grid.argtypes = [_ct.c_uint32, _ct.c_uint32, P]
            L.orc_p8_codes_grid.restype = None
            L.orc_e4m3_encode_n.argtypes = [P, _ct.c_long, P]
            L.orc_e4m3_encode_n.restype = None
            L.orc_exp2_n.argtypes = [P, _ct.c_long, P]
            L.orc_exp2_n.restype = None
            _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _estrides(a: np.ndarray):
    st = np.array([s // a.itemsize for s in a.strides], dtype=np.int64)
    return st


def npad(n: int) -> int:
    return (n + TILE - 1) // TILE * TILE


def default_workers() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


# ----------------------------------------------------------------------------------
# scalar codecs
# ----------------------------------------------------------------------------------
def e4m3_decode_table() -> np.ndarray:
    L = lib()
    return np.array([L.orc_e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_e4m3_encode_n(_ptr(x), x.size, _ptr(out))
    return out


def exp2(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.float32)
    lib().orc_exp2_n(_ptr(x), x.size, _ptr(out))
    return out


def default_lambda(D: int) -> float:
    return float(np.float32(lib().orc_default_lambda(D)))


def p8_codes_grid(lo_bits: int, hi_bits: int) -> np.ndarray:
    out = np.empty(hi_bits - lo_bits, dtype=np.uint8)
    lib().orc_p8_codes_grid(lo_bits, hi_bits, _ptr(out))
    return out


def exp2_check_grid(lo_bits: int, hi_bits: int, workers: int | None = None) -> int:
    """Count grid arguments where the double and long-double exp2 routes disagree."""
    L = lib()
    workers = workers or default_workers()
    edges = np.linspace(lo_bits, hi_bits, workers + 1).astype(np.int64)
    with _cf.ThreadPoolExecutor(workers) as ex:
        futs = [ex.submit(L.orc_exp2_check_grid, int(edges[i]), int(edges[i + 1])) for i in range(workers)]
        return sum(f.result() for f in futs)


# ----------------------------------------------------------------------------------
# a1-a3: preparation
# ----------------------------------------------------------------------------------
def _check_bshd(x: np.ndarray, name: str):
    if x.dtype != np.uint16 or x.ndim != 4:
        raise ValueError(f"{name}: expected bf16 bits (uint16) of rank 4 [B,N,H,D], got {x.dtype} {x.shape}")
    if x.strides[3] != 2:
        raise ValueError(f"{name}: innermost (D) stride must be 1 element")


def k_mean(k: np.ndarray):
    """a1: fp32 mean [B,H,D] and the number of inexact fp64 additions."""
    _check_bshd(k, "k")
    B, N, H, D = k.shape
    st = _estrides(k)[:3].copy()
    mean = np.empty((B, H, D), dtype=np.float32)
    inexact = lib().orc_k_mean(_ptr(k), _ptr(st), B, H, N, D, _ptr(mean))
    return mean, int(inexact)


def quant_i8_blocks(x: np.ndarray, mean: np.ndarray | None = None):
    """a2: INT8 codes [B,H,N_pad,D] and per-64-row scales [B,H,N_pad/64]."""
    _check_bshd(x, "x")
    B, N, H, D = x.shape
    st = _estrides(x)[:3].copy()
    codes = np.empty((B, H, npad(N), D), dtype=np.int8)
    scales = np.empty((B, H, npad(N) // TILE), dtype=np.float32)
    m = None if mean is None else np.ascontiguousarray(mean, dtype=np.float32)
    lib().orc_quant_i8_blocks(_ptr(x), _ptr(st), None if m is None else _ptr(m), B, H, N, D, _ptr(codes), _ptr(scales))
    return codes, scales


def quant_qk(q: np.ndarray, k: np.ndarray):
    """Step 1: (q8, q_scale, k8, k_scale, k_mean) for bf16 Q and K views [B,N,H,D]."""
    mean, _ = k_mean(k)
    q8, qs = quant_i8_blocks(q)
    k8, ks = quant_i8_blocks(k, mean)
    return q8, qs, k8, ks, mean


def quant_v(v: np.ndarray):
    """Step 2: (v8t [B,H,D,N_pad] e4m3 bytes, v_scale [B,H,D])."""
    _check_bshd(v, "v")
    B, N, H, D = v.shape
    st = _estrides(v)[:3].copy()
    v8t = np.empty((B, H, D, npad(N)), dtype=np.uint8)
    vs = np.empty((B, H, D), dtype=np.float32)
    lib().orc_quant_v(_ptr(v), _ptr(st), B, H, N, D, _ptr(v8t), _ptr(vs))
    return v8t, vs


def kv_append_i8(x: np.ndarray, cache: np.ndarray, tok_scale: np.ndarray, pos: int):
    """Tokens x (bf16 bits [Nnew, H, D]) quantized into rows pos.. of copies of the int8
    cache [H, Nmax, D] and its per-token scales [H, Nmax]; returns (cache, tok_scale)."""
    Nnew, H, D = x.shape
    Hc, Nmax, Dc = cache.shape
    if (Hc, Dc) != (H, D) or tok_scale.shape != (H, Nmax) or pos < 0 or pos + Nnew > Nmax:
        raise ValueError("kv_append_i8: shapes or position out of range")
    x = np.ascontiguousarray(x, dtype=np.uint16)
    cache = np.array(cache, dtype=np.int8, copy=True)
    tok_scale = np.array(tok_scale, dtype=np.float32, copy=True)
    st = np.array([H * D, D], dtype=np.int64)
    lib().orc_kv_append_i8(_ptr(x), _ptr(st), Nnew, H, D, _ptr(cache), _ptr(tok_scale), Nmax, int(pos))
    return cache, tok_scale


def requant_v_cache(v_cache: np.ndarray, v_tok_scale: np.ndarray):
    """Int8 V cache [H,Nk,D] with per-token scales [H,Nk] -> (v8t [H,D,Nk_pad], v_scale [H,D])."""
    H, Nk, D = v_cache.shape
    vc = np.ascontiguousarray(v_cache, dtype=np.int8)
    vt = np.ascontiguousarray(v_tok_scale, dtype=np.float32)
    v8t = np.empty((H, D, npad(Nk)), dtype=np.uint8)
    vs = np.empty((H, D), dtype=np.float32)
    lib().orc_requant_v_cache(_ptr(vc), _ptr(vt), H, Nk, D, _ptr(v8t), _ptr(vs))
    return v8t, vs


# ----------------------------------------------------------------------------------
# a4-a6: fused loop
# ----------------------------------------------------------------------------------
def _chunks(rows, chunk):
    rows = sorted(set(int(r) for r in rows))
    out, cur = [], []
    for r in rows:
        if cur and (r != cur[-1] + 1 or len(cur) >= chunk):
            out.append((cur[0], cur[-1] + 1))
            cur = []
        cur.append(r)
    if cur:
        out.append((cur[0], cur[-1] + 1))
    return out


def key_tiles(Nq: int, Nk: int, causal: bool, pos_off: int) -> int:
    """Key tiles any query can see: ceil(min(Nk, Nq + pos_off) / 64) when causal."""
    last = min(Nk, Nq + pos_off) if causal else Nk
    return max(0, (last + TILE - 1) // TILE)


def split_bounds(T: int, S: int):
    """Split s of S covers key tiles [s*T//S, (s+1)*T//S) (see orc_combine_rows)."""
    return [(s * T // S, (s + 1) * T // S) for s in range(S)]


def attn(q8, q_scale, k8, k_scale, v8t, v_scale, Nq: int, Nk: int, lam: float, causal: bool = False,
         pos_off: int | None = None, k_scale_per_token: bool = False, rows=None, workers: int | None = None,
         kv_splits: int = 1):
    """Steps 3-5 on prequantized operands.

    q8 [B,H,Nq_pad,D]; q_scale [B,H,Nq_pad/64]; k8 [B,H,>=Nk,D]; k_scale [B,H,Nk_pad/64] or
    [B,H,Nk] (per token); v8t [B,H,D,ldv]; v_scale [B,H,D].
    kv_splits > 1: the key tiles are cut into that many ranges, each run on its own, and
    the partial results combined (orc_combine_rows).
    Returns fp32 out [B, len(rows), H, D] for the requested query rows (all rows if None).
    """
    B, H, _, D = q8.shape
    if pos_off is None:
        pos_off = Nk - Nq
    rows = np.arange(Nq) if rows is None else np.asarray(rows)
    row_list = sorted(set(int(r) for r in rows))
    if any(r < 0 or r >= Nq for r in row_list):
        raise ValueError("row out of range")
    index = {r: i for i, r in enumerate(row_list)}
    out = np.zeros((B, len(row_list), H, D), dtype=np.float32)
    q8 = np.ascontiguousarray(q8)
    k8 = np.ascontiguousarray(k8)
    v8t = np.ascontiguousarray(v8t)
    q_scale = np.ascontiguousarray(q_scale, dtype=np.float32)
    k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
    v_scale = np.ascontiguousarray(v_scale, dtype=np.float32)
    ldv = v8t.shape[-1]
    L = lib()
    workers = workers or default_workers()
    jobs = []
    for b in range(B):
        for h in range(H):
            for (i0, i1) in _chunks(row_list, 16):
                jobs.append((b, h, i0, i1))

    bounds = split_bounds(key_tiles(Nq, Nk, causal, int(pos_off)), int(kv_splits)) if kv_splits > 1 else None

    def run(job):
        b, h, i0, i1 = job
        buf = np.empty((i1 - i0, D), dtype=np.float32)
        if bounds is None:
            L.orc_attn_rows(_ptr(q8[b, h]), _ptr(q_scale[b, h]), _ptr(k8[b, h]), _ptr(k_scale[b, h]),
                            1 if k_scale_per_token else 0, _ptr(v8t[b, h]), ldv, _ptr(v_scale[b, h]), Nq, Nk, D,
                            float(lam), 1 if causal else 0, int(pos_off), i0, i1, _ptr(buf))
            return job, buf
        S, n = len(bounds), i1 - i0
        op = np.empty((S, n, D), dtype=np.float32)
        mp = np.empty((S, n), dtype=np.float32)
        dp = np.empty((S, n), dtype=np.float32)
        for s, (t_lo, t_hi) in enumerate(bounds):
            L.orc_attn_rows_part(_ptr(q8[b, h]), _ptr(q_scale[b, h]), _ptr(k8[b, h]), _ptr(k_scale[b, h]),
                                 1 if k_scale_per_token else 0, _ptr(v8t[b, h]), ldv, Nq, Nk, D, float(lam),
                                 1 if causal else 0, int(pos_off), i0, i1, t_lo, t_hi, _ptr(op[s]), _ptr(mp[s]),
                                 _ptr(dp[s]))
        L.orc_combine_rows(S, _ptr(op), _ptr(mp), _ptr(dp), _ptr(v_scale[b, h]), n, D, _ptr(buf))
        return job, buf

    with _cf.ThreadPoolExecutor(workers) as ex:
        for (b, h, i0, i1), buf in ex.map(run, jobs):
            out[b, index[i0]:index[i0] + (i1 - i0), h, :] = buf
    return out


def fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, lam: float | None = None, causal: bool = False, rows=None,
        workers: int | None = None):
    """End to end on bf16 views [B,N,H,D]: returns (out fp32 [B,len(rows),H,D], intermediates dict)."""
    B, Nq, H, D = q.shape
    Nk = k.shape[1]
    q8, qs, k8, ks, mean = quant_qk(q, k)
    v8t, vs = quant_v(v)
    lam = default_lambda(D) if lam is None else lam
    out = attn(q8, qs, k8, ks, v8t, vs, Nq, Nk, lam, causal=causal, rows=rows, workers=workers)
    return out, dict(q8=q8, q_scale=qs, k8=k8, k_scale=ks, k_mean=mean, v8t=v8t, v_scale=vs, lam=lam)


def fwd_i8kv(q: np.ndarray, k_cache: np.ndarray, k_tok_scale: np.ndarray, v_cache: np.ndarray,
             v_tok_scale: np.ndarray, pos0: int, lam: float | None = None, rows=None, workers: int | None = None,
             kv_splits: int = 1):
    """Prefill over an int8 KV cache: q bf16 [Nq,H,D]; caches [H,Nk,D]; scales [H,Nk]."""
    Nq, H, D = q.shape
    Nk = k_cache.shape[1]
    if pos0 + Nq > Nk:
        raise ValueError("pos0 + Nq must not exceed Nk")
    q8, qs = quant_i8_blocks(q[None])
    v8t, vs = requant_v_cache(v_cache, v_tok_scale)
    lam = default_lambda(D) if lam is None else lam
    out = attn(q8, qs, k_cache[None], k_tok_scale[None], v8t[None], vs[None], Nq, Nk, lam, causal=True,
               pos_off=pos0, k_scale_per_token=True, rows=rows, workers=workers, kv_splits=kv_splits)
    return out[0], dict(q8=q8[0], q_scale=qs[0], v8t=v8t, v_scale=vs, lam=lam)


# ----------------------------------------------------------------------------------
# FP64 references (plain definitions, used by the pins)
# ----------------------------------------------------------------------------------
def attention_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool = False,
                   pos_off: int = 0, rows=None) -> np.ndarray:
    """softmax(scale * q k^T) v in float64 for one head: q [Nq,D], k [Nk,D], v [Nk,D].

    Causal: key j visible iff j <= i + pos_off.  Fully masked rows give 0."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq, Nk = q.shape[0], k.shape[0]
    rows = np.arange(Nq) if rows is None else np.asarray(rows)
    s = (q[rows] @ k.T) * scale
    if causal:
        j = np.arange(Nk)[None, :]
        s = np.where(j <= rows[:, None] + pos_off, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    p = np.exp(s - mx)
    den = p.sum(axis=1, keepdims=True)
    o = p @ v
    return np.where(den > 0, o / np.where(den > 0, den, 1.0), 0.0)


def dequant_operands(q8, q_scale, k8, k_scale, v8t, v_scale, Nq: int, Nk: int, k_scale_per_token: bool = False):
    """Per (b,h): fp64 dequantized operands the fused loop consumes (reading A of the FP64 check).

    Returns arrays qd [B,H,Nq,D], kd [B,H,Nk,D], vd [B,H,Nk,D]."""
    dec = e4m3_decode_table()
    qd = q8[:, :, :Nq, :].astype(np.float64) * np.repeat(q_scale, TILE, axis=2)[:, :, :Nq, None]
    if k_scale_per_token:
        kd = k8[:, :, :Nk, :].astype(np.float64) * k_scale[:, :, :Nk, None]
    else:
        kd = k8[:, :, :Nk, :].astype(np.float64) * np.repeat(k_scale, TILE, axis=2)[:, :, :Nk, None]
    vd = dec[v8t[:, :, :, :Nk]].transpose(0, 1, 3, 2) * v_scale[:, :, None, :]
    return qd, kd, vd


def rel_l2(a: np.ndarray, ref: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(a - ref) / max(np.linalg.norm(ref), 1e-300))
