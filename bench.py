"""Benchmark of the quantized attention forward on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  dense workloads:   qattn_prep (fused preparation of Q, K, V) -> qattn_fwd
  prefill workloads: qattn_fwd_i8kv (q quantization, cache V requantization, fused loop)
The printed JSON line reports whole-step throughput as attention TOPS
(4 * N_q * N_k * D * H per step, visible pairs only for causal workloads), the fused
kernel's own roofline (its launches timed with events on the stream it runs on) and the
CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_INT8_FP8_TOPS = 5000.0  # MI355X dense INT8 / FP8 MFMA (TOPS)
DEFAULT_WORKLOAD = W.VIDEO37810.name
KERNEL_SRC = os.path.join(ROOT, "quantized_attention_qattn_amd", "csrc", "attn_fwd.hip")

# HBM traffic of the fused kernel per launch, from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE passes over this script (KiB per dispatch), scaled by what the same counters
# read for a copy of known size (--calibrate-copy).  Keyed by the SHA-256 of the kernel
# source the counters were taken on: any other source reports traffic as null.
MEASURED_TRAFFIC = {
    "d5ae441991e8291c24eb618505d9cbd083d3499884b45470fccbc0c6457de2bb": {
        "workload": "video_dit_b1_h24_n37810_d128",
        "fetch_kib": 964938.0, "fetch_scale": 1048576.0 / 524309.0,  # 1 GiB copy read as 524309 KiB
        "write_kib": 233930.5, "write_scale": 1048576.0 / 1048576.0,
    },
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=[w.name for w in W.ALL])
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle wall time")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run one elementwise copy of MIB MiB (fp32) on the GPU: the reference dispatch "
                        "that scales the FETCH_SIZE / WRITE_SIZE counters")
    return p.parse_args()


def kernel_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def calibrate_copy(mib: int) -> None:
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads and writes mib MiB
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4}), flush=True)


def cpu_baseline(w: W.Workload, target_s: float):
    """The oracle as it stands, on a bounded sample: whole query blocks of a few heads."""
    import oracle

    oracle.build(force=False)
    workers = oracle.default_workers()
    rng = np.random.default_rng(0)
    if w.kind == "dense":
        q, k, v = W.dense_inputs(w)
        q8, qs, k8, ks, _ = oracle.quant_qk(q, k)
        v8t, vs = oracle.quant_v(v)
        del q, k, v
        lam = oracle.default_lambda(w.D)
        pos_off, per_tok, causal = w.Nk - w.Nq, False, w.causal
    else:
        q, kc, kts, vc, vts = W.i8kv_inputs(w)
        q8, qs = oracle.quant_i8_blocks(q[None])
        v8t, vs = oracle.requant_v_cache(vc, vts)
        k8, ks, v8t, vs = kc[None], kts[None], v8t[None], vs[None]
        lam = oracle.default_lambda(w.D)
        pos_off, per_tok, causal = w.pos0, True, True

    def run(nblk):
        blocks = rng.choice((w.Nq + 63) // 64, size=min(nblk, (w.Nq + 63) // 64), replace=False)
        rows = np.array([r for b in blocks for r in range(b * 64, min(w.Nq, b * 64 + 64))])
        heads = list(range(min(w.H, workers)))
        sel = (slice(None), heads)
        t0 = time.perf_counter()
        oracle.attn(q8[sel], qs[sel], k8[sel], ks[sel], v8t[sel], vs[sel], w.Nq, w.Nk, lam, causal=causal,
                    pos_off=pos_off, k_scale_per_token=per_tok, rows=rows, workers=workers)
        dt = time.perf_counter() - t0
        if causal:
            pairs = sum(max(0, min(w.Nk, r + pos_off + 1)) for r in rows)
        else:
            pairs = len(rows) * w.Nk
        return dt, 4.0 * pairs * w.D * len(heads), len(rows), len(heads)

    dt, ops, nrows, nheads = run(1)  # calibration
    nblk = max(1, int(target_s / max(dt, 1e-3)))
    dt, ops, nrows, nheads = run(nblk)
    return {
        "value": ops / dt / 1e12,
        "unit": "TOPS",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{nrows} query rows x {nheads} heads of {w.name} (fused loop only; the full workload is "
                  f"{w.Nq} rows x {w.H} heads), {dt:.1f} s on {workers} threads",
    }


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path shards by heads with no "
              f"communication, so multi-GPU figures are not produced by this benchmark.", file=sys.stderr)
        sys.exit(2)
    import torch

    import quantized_attention_qattn_amd as qa

    w = W.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def dev_bf16(u16):
        return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(dev).view(torch.bfloat16)

    if w.kind == "dense":
        q, k, v = W.dense_inputs(w)
        in_sha = W.sha256(q, k, v)
        dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
        del q, k, v
        t_qk = qa.alloc_qk(w.B, w.H, w.Nq, w.Nk, w.D, dev)
        t_v = qa.alloc_v(w.B, w.H, w.Nk, w.D, dev)
        out = torch.empty((w.B, w.Nq, w.H, w.D), dtype=torch.bfloat16, device=dev)
        ev_pairs = []

        def step(record):
            qa.qattn_prep(dq, dk, dv, t_qk["q8"], t_qk["q_scale"], t_qk["k8"], t_qk["k_scale"], t_qk["k_mean"],
                          t_v["v8t"], t_v["v_scale"], t_v["vbf"])
            if record:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            qa.qattn_fwd(t_qk["q8"], t_qk["q_scale"], t_qk["k8"], t_qk["k_scale"], t_v["vbf"], t_v["v_scale"], w.Nq,
                         w.Nk, out, 0.0, w.causal)
            if record:
                e1.record(stream)
                ev_pairs.append((e0, e1))
    else:
        q, kc, kts, vc, vts = W.i8kv_inputs(w)
        in_sha = W.sha256(q, kc, kts, vc, vts)
        dq = dev_bf16(q)
        dkc, dkts = torch.from_numpy(kc).to(dev), torch.from_numpy(kts).to(dev)
        dvc, dvts = torch.from_numpy(vc).to(dev), torch.from_numpy(vts).to(dev)
        kv_splits = qa.qattn_fwd_i8kv_kv_splits(w.H, w.Nq, w.Nk, w.pos0)  # the library's rule
        ws = torch.empty(qa.qattn_fwd_i8kv_workspace_bytes(w.H, w.Nq, w.Nk, w.D, kv_splits), dtype=torch.uint8,
                         device=dev)
        out = torch.empty((w.Nq, w.H, w.D), dtype=torch.bfloat16, device=dev)
        ev_pairs = []

        def step(record):
            if record:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            qa.qattn_fwd_i8kv(dq, dkc, dkts, dvc, dvts, w.pos0, ws, out)
            if record:
                e1.record(stream)
                ev_pairs.append((e0, e1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps
    ops = w.ops()
    value = ops / (ms_step * 1e-3) / 1e12
    kern_ms = float(np.median([a.elapsed_time(b) for a, b in ev_pairs]))
    achieved = ops / (kern_ms * 1e-3) / 1e12

    sha = kernel_sha()
    tr = MEASURED_TRAFFIC.get(sha)
    traffic = None
    if tr is not None and tr["workload"] == w.name:
        traffic = round((tr["fetch_kib"] * tr["fetch_scale"] + tr["write_kib"] * tr["write_scale"]) * 1024.0)
    rec = {
        "metric": "attention TOPS (4*N_q*N_k*D*H / step time) on one MI355X",
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 QK (int32 acc); fp8 e4m3 P and V, P.V products exact (fp32 acc)",
        "data": "synthetic (seeded N(0,1) bf16 inputs; see workloads.py)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N_q": w.Nq, "N_k": w.Nk, "D": w.D,
                   "causal": w.causal, "pos0": w.pos0 if w.kind == "i8kv" else None,
                   "kv_splits": kv_splits if w.kind == "i8kv" else 1,
                   "step": "prep + fwd" if w.kind == "dense" else "fwd_i8kv (incl. q quant, V requant)",
                   "input_sha256": in_sha},
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_kernel" if w.kind == "dense" else "fwd_i8kv call",
                     "achieved": round(achieved, 3), "peak": PEAK_INT8_FP8_TOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_INT8_FP8_TOPS, 4), "traffic": traffic,
                     "traffic_unit": "bytes per launch", "kernel_ms_median": round(kern_ms, 4),
                     "kernel_source_sha256": sha[:16]},
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
