"""Python binding of libqattn (quantized attention forward for MI355X / gfx950).

The functions below carry the C-ABI's names and only marshal arguments: torch tensors'
device pointers, element strides and the current HIP stream go to ``libqattn.so``;
every step of the computation runs in the library's HIP kernels.  torch provides the
device memory and the stream, nothing else.  Importing this package fails loudly when
the library has not been built (``python quantized_attention_qattn_amd/_build.py``);
there is no fallback.

Layouts (N_pad = ceil(N / 64) * 64):
  q, k, v   bf16 [B, N, H, D] (any strides with a unit innermost stride)
  q8, k8    int8 [B, H, N_pad, D];  q_scale, k_scale f32 [B, H, N_pad / 64]
  k_mean    f32 [B, H, D]
  v8t       uint8 (e4m3fn codes) [B, H, D, N_pad];  v_scale f32 [B, H, D]
  vbf       bf16 [B, H, D, N_pad]: the values of the v8t codes, the V operand of qattn_fwd
  out       bf16 or f32 [B, Nq, H, D]
"""
from __future__ import annotations

import contextlib as _contextlib
import ctypes as _ct
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqattn.so")

QATTN_OK, QATTN_EINVAL, QATTN_EUNSUPPORTED, QATTN_EWORKSPACE, QATTN_EHIP, QATTN_ESCRATCH = 0, -1, -2, -3, -4, -5
QATTN_NOALLOC_SCRATCH_BYTES = 256 << 20  # the static workspace of qattn_fwd_i8kv_noalloc, per GPU
QATTN_OUT_BF16, QATTN_OUT_F32 = 0, 1
BLOCK = 64
# The matrix instruction of the fused loop's P.V product, and the bytes per V element of
# the operand it reads (the bf16 values of the V codes, written by the preparation).
PV_INSTRUCTION = "v_mfma_f32_32x32x16_bf16"
V_OPERAND_BYTES = 2

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python quantized_attention_qattn_amd/_build.py`")

_lib = _ct.CDLL(LIB_PATH)
_P, _I, _I64, _F, _SZ = _ct.c_void_p, _ct.c_int, _ct.c_int64, _ct.c_float, _ct.c_size_t
_I64x3 = _ct.c_int64 * 3
_I64x2 = _ct.c_int64 * 2
_lib.qattn_quant_qk.argtypes = [_P, _I64x3, _P, _I64x3, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
_lib.qattn_quant_qk.restype = _I
_lib.qattn_quant_v.argtypes = [_P, _I64x3, _I, _I, _I, _I, _P, _P, _P, _P]
_lib.qattn_quant_v.restype = _I
_lib.qattn_prep.argtypes = [_P, _I64x3, _P, _I64x3, _P, _I64x3, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                            _P]
_lib.qattn_prep.restype = _I
_lib.qattn_fwd.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _I64x3, _I, _P]
_lib.qattn_fwd.restype = _I
_lib.qattn_fwd_i8kv.argtypes = [_P, _I64x2, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _SZ, _P, _I64x2, _I, _P]
_lib.qattn_fwd_i8kv.restype = _I
_lib.qattn_fwd_i8kv_noalloc.argtypes = [_P, _I64x2, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _I64x2, _I, _P]
_lib.qattn_fwd_i8kv_noalloc.restype = _I
_lib.qattn_fwd_i8kv_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
_lib.qattn_fwd_i8kv_workspace_bytes.restype = _SZ
_lib.qattn_fwd_i8kv_kv_splits.argtypes = [_I, _I, _I, _I]
_lib.qattn_fwd_i8kv_kv_splits.restype = _I
_lib.qattn_kv_append_i8.argtypes = [_P, _I64x2, _I, _I, _I, _P, _P, _I, _I, _P]
_lib.qattn_kv_append_i8.restype = _I
_lib.qattn_selftest_p8_codes.argtypes = [_P, _P, _I64, _I, _P]
_lib.qattn_selftest_p8_codes.restype = _I
_lib.qattn_status_string.argtypes = [_I]
_lib.qattn_status_string.restype = _ct.c_char_p


class QattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {qattn_status_string(status)} (status {status})")
        self.status = status


def qattn_status_string(status: int) -> str:
    return _lib.qattn_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != QATTN_OK:
        raise QattnError(status, where)


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda:
        raise TypeError(f"{name}: expected a {dtype} CUDA tensor")


def _buf(t: torch.Tensor, dtype, shape, name: str):
    """A code, scale or workspace buffer: the C ABI takes its base pointer and assumes the
    dense layout, so its dtype, shape and contiguity are checked here."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dtype:
        raise TypeError(f"{name}: expected a {dtype} CUDA tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def npad(n: int) -> int:
    return (n + BLOCK - 1) // BLOCK * BLOCK


# ----------------------------------------------------------------------------------
# the C-ABI calls (same names, argument marshalling only)
# ----------------------------------------------------------------------------------
def qattn_quant_qk(q, k, q8, q_scale, k8, k_scale, k_mean, stream=None) -> None:
    _need(q, torch.bfloat16, "q")
    _need(k, torch.bfloat16, "k")
    B, Nq, H, D = q.shape
    Nk = k.shape[1]
    if k.shape[0] != B or k.shape[2] != H or k.shape[3] != D:
        raise ValueError("q and k must agree on B, H, D")
    _buf(q8, torch.int8, (B, H, npad(Nq), D), "q8")
    _buf(q_scale, torch.float32, (B, H, npad(Nq) // BLOCK), "q_scale")
    _buf(k8, torch.int8, (B, H, npad(Nk), D), "k8")
    _buf(k_scale, torch.float32, (B, H, npad(Nk) // BLOCK), "k_scale")
    _buf(k_mean, torch.float32, (B, H, D), "k_mean")
    _check(_lib.qattn_quant_qk(_ptr(q), _I64x3(*q.stride()[:3]), _ptr(k), _I64x3(*k.stride()[:3]), B, H, Nq, Nk, D,
                               _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(k_mean), _stream(stream)),
           "qattn_quant_qk")


def qattn_quant_v(v, v8t, v_scale, vbf=None, stream=None) -> None:
    _need(v, torch.bfloat16, "v")
    B, Nk, H, D = v.shape
    _buf(v8t, torch.uint8, (B, H, D, npad(Nk)), "v8t")
    _buf(v_scale, torch.float32, (B, H, D), "v_scale")
    if vbf is not None:
        _buf(vbf, torch.bfloat16, (B, H, D, npad(Nk)), "vbf")
    _check(_lib.qattn_quant_v(_ptr(v), _I64x3(*v.stride()[:3]), B, H, Nk, D, _ptr(v8t), _ptr(v_scale),
                              None if vbf is None else _ptr(vbf), _stream(stream)), "qattn_quant_v")


def qattn_prep(q, k, v, q8, q_scale, k8, k_scale, k_mean, v8t, v_scale, vbf=None, stream=None) -> None:
    _need(q, torch.bfloat16, "q")
    _need(k, torch.bfloat16, "k")
    _need(v, torch.bfloat16, "v")
    B, Nq, H, D = q.shape
    Nk = k.shape[1]
    if k.shape[0] != B or k.shape[2] != H or k.shape[3] != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q, k and v must agree on B, H, D (and k, v on N)")
    _buf(q8, torch.int8, (B, H, npad(Nq), D), "q8")
    _buf(q_scale, torch.float32, (B, H, npad(Nq) // BLOCK), "q_scale")
    _buf(k8, torch.int8, (B, H, npad(Nk), D), "k8")
    _buf(k_scale, torch.float32, (B, H, npad(Nk) // BLOCK), "k_scale")
    _buf(k_mean, torch.float32, (B, H, D), "k_mean")
    if v8t is None and vbf is None:
        raise ValueError("qattn_prep: v8t and vbf cannot both be None")
    if v8t is not None:
        _buf(v8t, torch.uint8, (B, H, D, npad(Nk)), "v8t")
    _buf(v_scale, torch.float32, (B, H, D), "v_scale")
    if vbf is not None:
        _buf(vbf, torch.bfloat16, (B, H, D, npad(Nk)), "vbf")
    _check(_lib.qattn_prep(_ptr(q), _I64x3(*q.stride()[:3]), _ptr(k), _I64x3(*k.stride()[:3]), _ptr(v),
                           _I64x3(*v.stride()[:3]), B, H, Nq, Nk, D, _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale),
                           _ptr(k_mean), _ptr(v8t), _ptr(v_scale), _ptr(vbf), _stream(stream)), "qattn_prep")


def qattn_fwd(q8, q_scale, k8, k_scale, vbf, v_scale, Nq: int, Nk: int, out, scale_log2: float = 0.0,
              causal: bool = False, stream=None) -> None:
    B, H, _, D = q8.shape
    _buf(q8, torch.int8, (B, H, npad(Nq), D), "q8")
    _buf(q_scale, torch.float32, (B, H, npad(Nq) // BLOCK), "q_scale")
    _buf(k8, torch.int8, (B, H, npad(Nk), D), "k8")
    _buf(k_scale, torch.float32, (B, H, npad(Nk) // BLOCK), "k_scale")
    _buf(vbf, torch.bfloat16, (B, H, D, npad(Nk)), "vbf")
    _buf(v_scale, torch.float32, (B, H, D), "v_scale")
    if not out.is_cuda or tuple(out.shape) != (B, Nq, H, D) or out.stride(3) != 1:
        raise ValueError(f"out: expected a CUDA [B, Nq, H, D] = {(B, Nq, H, D)} view with unit channel stride")
    od = QATTN_OUT_BF16 if out.dtype == torch.bfloat16 else QATTN_OUT_F32 if out.dtype == torch.float32 else -1
    _check(_lib.qattn_fwd(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(vbf), _ptr(v_scale), B, H, Nq, Nk,
                          D, float(scale_log2), 1 if causal else 0, _ptr(out), _I64x3(*out.stride()[:3]), od,
                          _stream(stream)), "qattn_fwd")


def qattn_fwd_i8kv_workspace_bytes(H: int, Nq: int, Nk: int, D: int, kv_splits: int) -> int:
    return int(_lib.qattn_fwd_i8kv_workspace_bytes(H, Nq, Nk, D, kv_splits))


def qattn_fwd_i8kv_kv_splits(H: int, Nq: int, Nk: int, pos0: int) -> int:
    return int(_lib.qattn_fwd_i8kv_kv_splits(H, Nq, Nk, pos0))


def qattn_fwd_i8kv(q, k_cache, k_tok_scale, v_cache, v_tok_scale, pos0: int, workspace, out,
                   scale_log2: float = 0.0, stream=None, kv_splits: int = 0) -> None:
    _need(q, torch.bfloat16, "q")
    Nq, H, D = q.shape
    Nk = k_cache.shape[1]
    _buf(k_cache, torch.int8, (H, Nk, D), "k_cache")
    _buf(k_tok_scale, torch.float32, (H, Nk), "k_tok_scale")
    _buf(v_cache, torch.int8, (H, Nk, D), "v_cache")
    _buf(v_tok_scale, torch.float32, (H, Nk), "v_tok_scale")
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace: expected a contiguous CUDA tensor")
    if not out.is_cuda or tuple(out.shape) != (Nq, H, D) or out.stride(2) != 1:
        raise ValueError(f"out: expected a CUDA [Nq, H, D] = {(Nq, H, D)} view with unit channel stride")
    od = QATTN_OUT_BF16 if out.dtype == torch.bfloat16 else QATTN_OUT_F32 if out.dtype == torch.float32 else -1
    _check(_lib.qattn_fwd_i8kv(_ptr(q), _I64x2(*q.stride()[:2]), _ptr(k_cache), _ptr(k_tok_scale), _ptr(v_cache),
                               _ptr(v_tok_scale), H, Nq, Nk, D, int(pos0), float(scale_log2), int(kv_splits),
                               _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(out), _I64x2(*out.stride()[:2]), od,
                               _stream(stream)), "qattn_fwd_i8kv")


def qattn_fwd_i8kv_noalloc(q, k_cache, k_tok_scale, v_cache, v_tok_scale, pos0: int, out, scale_log2: float = 0.0,
                           stream=None, kv_splits: int = 0) -> None:
    """qattn_fwd_i8kv with the library's static per-GPU workspace (allocates nothing)."""
    _need(q, torch.bfloat16, "q")
    Nq, H, D = q.shape
    Nk = k_cache.shape[1]
    _buf(k_cache, torch.int8, (H, Nk, D), "k_cache")
    _buf(k_tok_scale, torch.float32, (H, Nk), "k_tok_scale")
    _buf(v_cache, torch.int8, (H, Nk, D), "v_cache")
    _buf(v_tok_scale, torch.float32, (H, Nk), "v_tok_scale")
    if not out.is_cuda or tuple(out.shape) != (Nq, H, D) or out.stride(2) != 1:
        raise ValueError(f"out: expected a CUDA [Nq, H, D] = {(Nq, H, D)} view with unit channel stride")
    od = QATTN_OUT_BF16 if out.dtype == torch.bfloat16 else QATTN_OUT_F32 if out.dtype == torch.float32 else -1
    _check(_lib.qattn_fwd_i8kv_noalloc(_ptr(q), _I64x2(*q.stride()[:2]), _ptr(k_cache), _ptr(k_tok_scale),
                                       _ptr(v_cache), _ptr(v_tok_scale), H, Nq, Nk, D, int(pos0), float(scale_log2),
                                       int(kv_splits), _ptr(out), _I64x2(*out.stride()[:2]), od, _stream(stream)),
           "qattn_fwd_i8kv_noalloc")


def qattn_kv_append_i8(x, cache, tok_scale, pos: int, stream=None) -> None:
    """x: bf16 [Nnew, H, D] view; cache: int8 [H, Nmax, D]; tok_scale: f32 [H, Nmax]."""
    _need(x, torch.bfloat16, "x")
    Nnew, H, D = x.shape
    if cache.dim() != 3:
        raise ValueError("cache: expected [H, Nmax, D]")
    Nmax = cache.shape[1]
    _buf(cache, torch.int8, (H, Nmax, D), "cache")
    _buf(tok_scale, torch.float32, (H, Nmax), "tok_scale")
    _check(_lib.qattn_kv_append_i8(_ptr(x), _I64x2(*x.stride()[:2]), Nnew, H, D, _ptr(cache), _ptr(tok_scale), Nmax,
                                   int(pos), _stream(stream)), "qattn_kv_append_i8")


def qattn_selftest_p8_codes(u, codes, saturating: bool = False, stream=None) -> None:
    """Self-test hook (not part of the attention interface): the FP8 code of P' the
    fused kernel's softmax forms for each exponent argument u."""
    _need(u, torch.float32, "u")
    _buf(u, torch.float32, (u.numel(),), "u")
    _buf(codes, torch.uint8, (u.numel(),), "codes")
    _check(_lib.qattn_selftest_p8_codes(_ptr(u), _ptr(codes), u.numel(), 1 if saturating else 0, _stream(stream)),
           "qattn_selftest_p8_codes")


# ----------------------------------------------------------------------------------
# allocation helpers (torch owns the memory; the library allocates nothing)
# ----------------------------------------------------------------------------------
def _alloc_on(stream):
    """Allocations for a call on `stream` are made on that stream, so that the caching
    allocator does not hand their memory to other work before the call's kernels ran."""
    if stream is None or not isinstance(stream, torch.cuda.Stream):
        return _contextlib.nullcontext()
    return torch.cuda.stream(stream)


def alloc_qk(B: int, H: int, Nq: int, Nk: int, D: int, device="cuda"):
    kw = dict(device=device)
    return dict(
        q8=torch.empty((B, H, npad(Nq), D), dtype=torch.int8, **kw),
        q_scale=torch.empty((B, H, npad(Nq) // BLOCK), dtype=torch.float32, **kw),
        k8=torch.empty((B, H, npad(Nk), D), dtype=torch.int8, **kw),
        k_scale=torch.empty((B, H, npad(Nk) // BLOCK), dtype=torch.float32, **kw),
        k_mean=torch.empty((B, H, D), dtype=torch.float32, **kw),
    )


def alloc_v(B: int, H: int, Nk: int, D: int, device="cuda", codes: bool = True):
    """v_scale and the loop's V operand vbf, and with codes=True the e4m3 codes v8t."""
    t = dict(v_scale=torch.empty((B, H, D), dtype=torch.float32, device=device),
             vbf=torch.empty((B, H, D, npad(Nk)), dtype=torch.bfloat16, device=device))
    if codes:
        t["v8t"] = torch.empty((B, H, D, npad(Nk)), dtype=torch.uint8, device=device)
    return t


def alloc_prep(B: int, H: int, Nq: int, Nk: int, D: int, device="cuda", codes: bool = False):
    """Every buffer qattn_prep writes for a later qattn_fwd (the V codes only with codes=True)."""
    return {**alloc_qk(B, H, Nq, Nk, D, device), **alloc_v(B, H, Nk, D, device, codes)}


def prep_into(q, k, v, t: dict, stream=None) -> None:
    """qattn_prep into the buffers of alloc_prep."""
    qattn_prep(q, k, v, t["q8"], t["q_scale"], t["k8"], t["k_scale"], t["k_mean"], t.get("v8t"), t["v_scale"],
               t["vbf"], stream)


def fwd_from(t: dict, Nq: int, Nk: int, out, scale_log2: float = 0.0, causal: bool = False, stream=None) -> None:
    """qattn_fwd on the buffers of alloc_prep."""
    qattn_fwd(t["q8"], t["q_scale"], t["k8"], t["k_scale"], t["vbf"], t["v_scale"], Nq, Nk, out, scale_log2, causal,
              stream)


def quant_qk(q, k, stream=None):
    B, Nq, H, D = q.shape
    with _alloc_on(stream):
        t = alloc_qk(B, H, Nq, k.shape[1], D, q.device)
    qattn_quant_qk(q, k, t["q8"], t["q_scale"], t["k8"], t["k_scale"], t["k_mean"], stream)
    return t


def quant_v(v, stream=None):
    B, Nk, H, D = v.shape
    with _alloc_on(stream):
        t = alloc_v(B, H, Nk, D, v.device)
    qattn_quant_v(v, t["v8t"], t["v_scale"], t["vbf"], stream)
    return t


def prep(q, k, v, stream=None, codes: bool = True):
    """Steps 1-2 through the fused preparation; returns the intermediates of quant_qk and
    quant_v (the V codes v8t only with codes=True)."""
    B, Nq, H, D = q.shape
    with _alloc_on(stream):
        t = alloc_prep(B, H, Nq, k.shape[1], D, q.device, codes)
    prep_into(q, k, v, t, stream)
    return t


def attention(q, k, v, causal: bool = False, scale_log2: float = 0.0, out_dtype=torch.bfloat16, stream=None):
    """Steps 1-5 on bf16 [B, N, H, D] views (fused preparation, then the fused loop);
    returns (out [B, Nq, H, D], intermediates)."""
    B, Nq, H, D = q.shape
    qk = prep(q, k, v, stream)
    with _alloc_on(stream):
        out = torch.empty((B, Nq, H, D), dtype=out_dtype, device=q.device)
    fwd_from(qk, Nq, k.shape[1], out, scale_log2, causal, stream)
    return out, qk


def attention_i8kv(q, k_cache, k_tok_scale, v_cache, v_tok_scale, pos0: int, scale_log2: float = 0.0,
                   out_dtype=torch.bfloat16, stream=None, kv_splits: int = 0):
    """kv_splits = 0: the library's rule (qattn_fwd_i8kv_kv_splits)."""
    Nq, H, D = q.shape
    Nk = k_cache.shape[1]
    S = kv_splits if kv_splits > 0 else qattn_fwd_i8kv_kv_splits(H, Nq, Nk, pos0)
    with _alloc_on(stream):
        ws = torch.empty(qattn_fwd_i8kv_workspace_bytes(H, Nq, Nk, D, S), dtype=torch.uint8, device=q.device)
        out = torch.empty((Nq, H, D), dtype=out_dtype, device=q.device)
    qattn_fwd_i8kv(q, k_cache, k_tok_scale, v_cache, v_tok_scale, pos0, ws, out, scale_log2, stream, kv_splits=S)
    return out, ws


__all__ = [n for n in dir() if n.startswith("qattn_")] + ["attention", "attention_i8kv", "prep", "prep_into", "fwd_from",
                                                           "quant_qk", "quant_v", "alloc_qk", "alloc_v", "alloc_prep",
                                                           "QattnError", "LIB_PATH", "PV_INSTRUCTION", "V_OPERAND_BYTES"]
