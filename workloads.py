"""Seeded synthetic workloads for the quantized attention forward.

This module only draws inputs.  It holds none of the method's arithmetic and is the
one module that both the HIP path's tests and the CPU oracle read inputs from.

Recipe (every tensor is independent and reproducible):
  * ``numpy.random.default_rng([seed, tensor_id])`` draws fp32 values, which are rounded
    to bf16 (round to nearest even on the bit pattern);
  * tensor ids: 0 = Q, 1 = K, 2 = V, 3 = per-(b, h, channel) K offset ~ U[-2, 2] added
    to K in fp32 before the bf16 rounding, 4 = prefill queries, 5 = K-cache source,
    6 = V-cache source;
  * Q, K, V ~ N(0, 1); dense tensors are laid out [B, N, H, D] (token-major BSHD);
  * KV caches: a bf16 N(0, 1) source [H, Nk, D] is stored as int8 with one fp32 scale
    per (head, token): scale = absmax / 127 and code = rint(x / scale).  This is input
    synthesis for the cache the prefill call consumes, not a step of the method.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

SEED_BASE = 1000


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "dense" or "i8kv"
    H: int
    D: int
    Nq: int
    Nk: int
    B: int = 1
    causal: bool = False
    pos0: int = 0  # first query position (i8kv)
    seed: int = SEED_BASE

    def ops(self) -> float:
        """Attention ops 4*Nq*Nk*D*H*B (visible pairs only when causal)."""
        return 4.0 * self.pairs() * self.D * self.H * self.B

    def pairs(self) -> int:
        if not self.causal:
            return self.Nq * self.Nk
        off = self.pos0 if self.kind == "i8kv" else self.Nk - self.Nq
        tot = 0
        for i in range(self.Nq):
            tot += max(0, min(self.Nk, i + off + 1))
        return tot


TINY = Workload("tiny_b1_h2_n256_d64", "dense", H=2, D=64, Nq=256, Nk=256, seed=SEED_BASE + 1)
DENSE4096 = Workload("dense_b1_h16_n4096_d128", "dense", H=16, D=128, Nq=4096, Nk=4096, seed=SEED_BASE + 2)
PREFILL32K = Workload("prefill_i8kv_h32_d128_q1024_ctx32768", "i8kv", H=32, D=128, Nq=1024, Nk=32768, causal=True,
                      pos0=31744, seed=SEED_BASE + 3)
PREFILL64K = Workload("prefill_i8kv_h32_d128_q512_ctx65536", "i8kv", H=32, D=128, Nq=512, Nk=65536, causal=True,
                      pos0=65024, seed=SEED_BASE + 4)
VIDEO37810 = Workload("video_dit_b1_h24_n37810_d128", "dense", H=24, D=128, Nq=37810, Nk=37810, seed=SEED_BASE + 5)
# the longer video baseline the pages name ("74K tokens"; count taken literally, ragged last tile)
VIDEO74000 = Workload("video_dit_b1_h24_n74000_d128", "dense", H=24, D=128, Nq=74000, Nk=74000, seed=SEED_BASE + 6)
# causal dense self-attention at the video size (ops counted on the visible pairs)
CAUSAL37810 = Workload("causal_b1_h24_n37810_d128", "dense", H=24, D=128, Nq=37810, Nk=37810, causal=True,
                       seed=SEED_BASE + 7)

ALL = [TINY, DENSE4096, PREFILL32K, PREFILL64K, VIDEO37810, VIDEO74000, CAUSAL37810]
BY_NAME = {w.name: w for w in ALL}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, tid: int) -> np.random.Generator:
    return np.random.default_rng([seed, tid])


def normal_bf16(seed: int, tid: int, shape) -> np.ndarray:
    return bf16_bits(_rng(seed, tid).standard_normal(shape, dtype=np.float32))


def dense_inputs(w: Workload, k_offset: bool = True):
    """Q, K, V bf16 bits [B, N, H, D]; K carries a per-(b, h, channel) offset ~ U[-2, 2]."""
    B, H, D = w.B, w.H, w.D
    q = normal_bf16(w.seed, 0, (B, w.Nq, H, D))
    kf = _rng(w.seed, 1).standard_normal((B, w.Nk, H, D), dtype=np.float32)
    if k_offset:
        off = _rng(w.seed, 3).uniform(-2.0, 2.0, size=(B, 1, H, D)).astype(np.float32)
        kf += off
    k = bf16_bits(kf)
    del kf
    v = normal_bf16(w.seed, 2, (B, w.Nk, H, D))
    return q, k, v


def int8_cache(seed: int, tid: int, H: int, Nk: int, D: int):
    """An int8 cache [H, Nk, D] with fp32 per-(head, token) scales [H, Nk] from a bf16 N(0,1) source."""
    src = bf16_to_f32(normal_bf16(seed, tid, (H, Nk, D)))
    amax = np.abs(src).max(axis=2)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = np.clip(np.rint(src / safe[:, :, None]), -127, 127).astype(np.int8)
    return codes, scale


def i8kv_inputs(w: Workload):
    """q bf16 bits [Nq, H, D]; k_cache, v_cache int8 [H, Nk, D]; per-token scales [H, Nk]."""
    q = normal_bf16(w.seed, 4, (w.Nq, w.H, w.D))
    kc, ks = int8_cache(w.seed, 5, w.H, w.Nk, w.D)
    vc, vs = int8_cache(w.seed, 6, w.H, w.Nk, w.D)
    return q, kc, ks, vc, vs


def sha256(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
