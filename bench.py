"""Benchmark of the quantized attention forward on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  dense workloads:   qattn_prep (fused preparation of Q, K, V) -> qattn_fwd
  prefill workloads: qattn_fwd_i8kv (q quantization, cache V requantization, fused loop)
The printed JSON line reports whole-step throughput as attention TOPS
(4 * N_q * N_k * D * H per step, visible pairs only for causal workloads) over exactly
K timed steps, the fused kernel's own roofline (its launches timed with events on the
stream it runs on, p10/p50/p90 over at least 30 launches, against the nominal peak and
against the shader clock sampled while it runs), the preparation's HBM rate with a warm
and a cold cache, and the CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_INT8_FP8_TOPS = 5000.0  # MI355X dense INT8 / FP8 MFMA (TOPS) at 2.4 GHz
PEAK_BF16_TOPS = 2500.0      # MI355X dense bf16 MFMA
NOMINAL_SCLK_MHZ = 2400.0
PEAK_HBM_GBPS = 8000.0
DEFAULT_WORKLOAD = W.VIDEO37810.name
KERNEL_SRC = os.path.join(ROOT, "quantized_attention_qattn_amd", "csrc", "attn_fwd.hip")

# Counters of the fused kernel per launch, from rocprofv3 --pmc passes over this script:
# HBM traffic from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), scaled by what the same
# counters read for a copy of known size (--calibrate-copy), and SQ_INSTS_VALU (wave-level
# VALU instructions per dispatch).  Keyed by the SHA-256 of the kernel source the counters
# were taken on: any other source reports them as null.
MEASURED_COUNTERS = {
    "993dfbd5b29302dcea70aa0448fd86e61b65b9ddb91855a8689303e386a51830": {
        "workload": "video_dit_b1_h24_n37810_d128",
        "fetch_kib": 965030.9, "fetch_scale": 1048576.0 / 524309.0,  # 1 GiB copy read as 524309 KiB
        "write_kib": 230869.9, "write_scale": 1048576.0 / 1048576.0,
        "valu_insts": 3.85629e+09,
    },
}
# VALU budget per score element at the MFMA peak: a CU retires 8,192 INT8/FP8 MFMA ops per
# clock and a score costs 4 D of them (QK and PV), i.e. 16 scores per clock at D = 128,
# against 64 fp32 VALU lanes per clock: 4 lane-ops per score.  With P.V on the bf16 MFMA
# (4,096 ops per clock) a score costs 2 D / 8192 + 2 D / 4096 clocks: 6 lane-ops.
VALU_LANES_PER_CU_CLK = 64
MFMA_OPS_PER_CU_CLK = {"int8_fp8": 8192, "bf16": 4096}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=[w.name for w in W.ALL])
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle wall time")
    p.add_argument("--clock-seconds", type=float, default=2.0,
                   help="length of the fused-kernel run during which the shader clock is sampled (0: none)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run one elementwise copy of MIB MiB (fp32) on the GPU: the reference dispatch "
                        "that scales the FETCH_SIZE / WRITE_SIZE counters")
    return p.parse_args()


def kernel_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def pct(xs) -> dict:
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 4), "p50": round(float(np.percentile(a, 50)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "n": int(a.size)}


def calibrate_copy(mib: int) -> None:
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads and writes mib MiB
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4}), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_operands(w: W.Workload):
    import oracle

    if w.kind == "dense":
        q, k, v = W.dense_inputs(w)
        q8, qs, k8, ks, _ = oracle.quant_qk(q, k)
        v8t, vs = oracle.quant_v(v)
        return dict(ops=(q8, qs, k8, ks, v8t, vs), pos_off=w.Nk - w.Nq, per_tok=False, causal=w.causal, splits=1)
    q, kc, kts, vc, vts = W.i8kv_inputs(w)
    q8, qs = oracle.quant_i8_blocks(q[None])
    v8t, vs = oracle.requant_v_cache(vc, vts)
    wgs = w.H * ((w.Nq + 255) // 256)  # the library's key-range rule (qattn_fwd_i8kv_kv_splits)
    T = (min(w.Nk, w.pos0 + w.Nq) + 63) // 64
    S = max(1, min((256 + wgs - 1) // wgs, T // 16, 64))
    return dict(ops=(q8, qs, kc[None], kts[None], v8t[None], vs[None]), pos_off=w.pos0, per_tok=True, causal=True,
                splits=S)


def _oracle_rate(w: W.Workload, o: dict, nblk: int, workers: int, rng, nheads: int | None = None):
    """Oracle wall time on nblk whole 64-row query blocks of nheads (default min(H, workers)) heads."""
    import oracle

    blocks = rng.choice((w.Nq + 63) // 64, size=min(nblk, (w.Nq + 63) // 64), replace=False)
    rows = np.array([r for b in sorted(blocks) for r in range(b * 64, min(w.Nq, b * 64 + 64))])
    heads = list(range(min(w.H, nheads or max(1, workers))))
    sel = (slice(None), heads)
    q8, qs, k8, ks, v8t, vs = o["ops"]
    t0 = time.perf_counter()
    oracle.attn(q8[sel], qs[sel], k8[sel], ks[sel], v8t[sel], vs[sel], w.Nq, w.Nk, oracle.default_lambda(w.D),
                causal=o["causal"], pos_off=o["pos_off"], k_scale_per_token=o["per_tok"], rows=rows, workers=workers,
                kv_splits=o["splits"])
    dt = time.perf_counter() - t0
    off = o["pos_off"]
    pairs = sum(max(0, min(w.Nk, r + off + 1)) for r in rows) if o["causal"] else len(rows) * w.Nk
    return dt, 4.0 * pairs * w.D * len(heads), len(rows), len(heads)


def cpu_baseline(w: W.Workload, target_s: float):
    """The oracle as it stands, on a bounded sample: whole query blocks of a few heads, on
    the host's cores (at most 16 threads), plus one-thread figures for the two small
    workloads."""
    import oracle

    oracle.build(force=False)
    workers = oracle.default_workers()
    rng = np.random.default_rng(0)
    o = _oracle_operands(w)
    dt, ops, nrows, nheads = _oracle_rate(w, o, 1, workers, rng)  # calibration
    nblk = max(1, int(target_s / max(dt, 1e-3)))
    dt, ops, nrows, nheads = _oracle_rate(w, o, nblk, workers, rng)
    one_core = {}
    # one thread: the whole tiny workload, and about two seconds of the 4,096-token one
    so = _oracle_operands(W.TINY)
    d1, o1, r1, h1 = _oracle_rate(W.TINY, so, 4, 1, rng, nheads=W.TINY.H)
    one_core[W.TINY.name] = {"value": o1 / d1 / 1e12, "unit": "TOPS", "sample": f"{r1} rows x {h1} heads (all)",
                             "seconds": round(d1, 3)}
    so = _oracle_operands(W.DENSE4096)
    d1, o1, r1, h1 = _oracle_rate(W.DENSE4096, so, 1, 1, rng)
    d1, o1, r1, h1 = _oracle_rate(W.DENSE4096, so, max(1, int(2.0 / max(d1, 1e-3))), 1, rng)
    one_core[W.DENSE4096.name] = {"value": o1 / d1 / 1e12, "unit": "TOPS", "sample": f"{r1} rows x {h1} head",
                                  "seconds": round(d1, 2)}
    return {
        "value": ops / dt / 1e12,
        "unit": "TOPS",
        "cores": workers,
        "host_cores": os.cpu_count(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{nrows} query rows x {nheads} heads of {w.name} (fused loop only; the full workload is "
                  f"{w.Nq} rows x {w.H} heads), {dt:.1f} s on {workers} threads",
        "one_core": one_core,
    }


class ClockSampler:
    """Samples the GPU shader clock with amd-smi in a child process started before this
    process touches the GPU; samples() returns the clock readings (MHz) taken inside a
    time window (None when the tool is missing or prints nothing usable)."""

    CHILD = r"""
import json, subprocess, sys, time
out, stop = sys.argv[1], sys.argv[2]
import os
while not os.path.exists(stop):
    t = time.time()
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True, text=True, timeout=5)
        line = json.dumps({"t": t, "out": r.stdout})
    except Exception as e:
        line = json.dumps({"t": t, "err": str(e)})
    with open(out, "a") as f:
        f.write(line + "\n")
    time.sleep(0.05)
"""

    def __init__(self):
        import tempfile

        self.dir = tempfile.mkdtemp(prefix="qattn_sclk_")
        self.out, self.stop = os.path.join(self.dir, "samples.jsonl"), os.path.join(self.dir, "stop")
        try:
            self.proc = subprocess.Popen([sys.executable, "-c", self.CHILD, self.out, self.stop],
                                         stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        except OSError:
            self.proc = None

    @staticmethod
    def _clock(text: str):
        try:
            d = json.loads(text)
        except ValueError:
            return None
        found = []

        def walk(x, key=""):
            if isinstance(x, dict):
                for k2, v2 in x.items():
                    walk(v2, f"{key}/{k2}")
            elif isinstance(x, list):
                for i, v2 in enumerate(x):
                    walk(v2, f"{key}/{i}")
            elif "/gfx" in key.lower() and key.lower().endswith("/clk/value"):
                # the current clock of one XCD ("gfx_<i>"), not its min_clk / max_clk limits
                try:
                    found.append(float(x if not isinstance(x, str) else x.split()[0]))
                except (TypeError, ValueError):
                    pass

        walk(d)
        return float(np.mean(found)) if found else None  # mean over the XCDs

    def samples(self, t0: float, t1: float):
        vals = []
        try:
            with open(self.out) as f:
                for line in f:
                    r = json.loads(line)
                    if t0 <= r["t"] <= t1 and "out" in r:
                        v = self._clock(r["out"])
                        if v:
                            vals.append(v)
        except (OSError, ValueError):
            return None
        return vals or None

    def close(self):
        open(self.stop, "w").close()
        if self.proc is not None:
            try:
                self.proc.wait(timeout=10)
            except subprocess.TimeoutExpired:
                self.proc.kill()


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path shards by heads with no "
              f"communication, so multi-GPU figures are not produced by this benchmark.", file=sys.stderr)
        sys.exit(2)
    # The clock sampler is a child process started before this one touches the GPU.  Under
    # a profiler (whose preloaded library initializes the GPU before this script runs) no
    # child is started: a GPU-initialized process must not exec another program.
    profiled = any(k.startswith("ROCPROF") for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", "")
    sampler = ClockSampler() if args.clock_seconds > 0 and not profiled else None
    try:
        run(args, sampler)
    finally:
        if sampler is not None:
            sampler.close()


def run(args, sampler):
    import torch

    import quantized_attention_qattn_amd as qa

    w = W.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def dev_bf16(u16):
        return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(dev).view(torch.bfloat16)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    prep_fn = None
    if w.kind == "dense":
        q, k, v = W.dense_inputs(w)
        in_sha = W.sha256(q, k, v)
        dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
        del q, k, v
        t = qa.alloc_prep(w.B, w.H, w.Nq, w.Nk, w.D, dev)
        out = torch.empty((w.B, w.Nq, w.H, w.D), dtype=torch.bfloat16, device=dev)

        def prep_fn():
            qa.prep_into(dq, dk, dv, t)

        def fwd_fn():
            qa.fwd_from(t, w.Nq, w.Nk, out, 0.0, w.causal)

        # algorithmic bytes of steps 1-2: read Q, K, V once (2 B per element each), write the
        # Q and K codes (1 B each), the loop's V operand (V_OPERAND_BYTES) and the scales
        prep_bytes = float(w.B * w.H * w.D * (w.Nq * 3 + w.Nk * 3 + w.Nk * (2 + qa.V_OPERAND_BYTES)))
        prep_bytes += sum(x.numel() * x.element_size() for n, x in t.items() if n.endswith("scale") or n == "k_mean")
        kernel_name, steps_desc = "attn_fwd_kernel", "prep + fwd"
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

        def fwd_fn():
            qa.qattn_fwd_i8kv(dq, dkc, dkts, dvc, dvts, w.pos0, ws, out)

        kernel_name, steps_desc = "fwd_i8kv call", "fwd_i8kv (incl. q quant, V requant)"

    def step():
        if prep_fn is not None:
            prep_fn()
        fwd_fn()

    # ---- the timed region: exactly K steps, synchronized on both sides ----
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    marks = [ev() for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    ops = w.ops()
    value = ops / (ms_step * 1e-3) / 1e12

    # ---- the fused kernel alone: >= 30 launches, each bracketed by events on its stream ----
    nk = max(30, args.steps)
    pairs = [(ev(), ev()) for _ in range(nk)]
    for a, b in pairs:
        a.record(stream)
        fwd_fn()
        b.record(stream)
    torch.cuda.synchronize()
    kern = [a.elapsed_time(b) for a, b in pairs]
    kern_p = pct(kern)
    achieved = ops / (kern_p["p50"] * 1e-3) / 1e12

    # ---- shader clock sampled by the child over a run of fused-kernel launches ----
    clocks = None
    if sampler is not None:
        tw0 = time.time()
        while time.time() < tw0 + args.clock_seconds:
            for _ in range(8):
                fwd_fn()
            torch.cuda.synchronize()
        clocks = sampler.samples(tw0 + 0.2, time.time())
    sclk = float(np.mean(clocks)) if clocks else None

    # ---- the preparation's HBM rate, warm (back to back) and cold (after a 1 GiB write) ----
    quant = None
    if prep_fn is not None:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        warm, cold = [], []
        for cold_run in (False, True):
            for _ in range(nk):
                if cold_run:
                    flush.fill_(1.0)
                a, b = ev(), ev()
                a.record(stream)
                prep_fn()
                b.record(stream)
                torch.cuda.synchronize()
                (cold if cold_run else warm).append(a.elapsed_time(b))
        del flush
        pw, pc = pct(warm), pct(cold)
        quant = {"kernel": "qattn_prep", "algorithmic_bytes": int(prep_bytes), "bound": "hbm", "peak": PEAK_HBM_GBPS,
                 "unit": "GB/s", "warm_ms": pw, "cold_ms": pc,
                 "warm_gbps": round(prep_bytes / (pw["p50"] * 1e-3) / 1e9, 1),
                 "cold_gbps": round(prep_bytes / (pc["p50"] * 1e-3) / 1e9, 1)}

    sha = kernel_sha()
    tr = MEASURED_COUNTERS.get(sha)
    if tr is not None and tr["workload"] != w.name:
        tr = None
    traffic = None
    if tr is not None:
        traffic = round((tr["fetch_kib"] * tr["fetch_scale"] + tr["write_kib"] * tr["write_scale"]) * 1024.0)
    roof = {"bound": "mfma", "kernel": kernel_name, "achieved": round(achieved, 3), "peak": PEAK_INT8_FP8_TOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_INT8_FP8_TOPS, 4), "traffic": traffic,
            "traffic_unit": "bytes per launch", "kernel_ms": kern_p, "kernel_source_sha256": sha[:16],
            "sclk_mhz_measured": None if sclk is None else round(sclk, 1),
            "sclk_samples": 0 if not clocks else len(clocks),
            "frac_at_measured_sclk": None if sclk is None else
            round(achieved / (PEAK_INT8_FP8_TOPS * sclk / NOMINAL_SCLK_MHZ), 4)}
    pv_bf16 = qa.PV_INSTRUCTION.endswith("bf16")
    if pv_bf16:
        # the instructions actually issued: half the ops on INT8 MFMA (5.0 POPS), half on bf16 MFMA (2.5)
        mix = 1.0 / (0.5 / PEAK_INT8_FP8_TOPS + 0.5 / PEAK_BF16_TOPS)
        roof["peak_of_issued_mix"] = round(mix, 1)
        roof["frac_of_issued_mix"] = round(achieved / mix, 4)
    # secondary roofline: VALU lane-operations per score element (SQ_INSTS_VALU x 64 lanes
    # over the scores the metric counts) against the per-score VALU budget at the MFMA peak
    valu = None
    if tr is not None and "valu_insts" in tr:
        scores = ops / (4.0 * w.D)
        per_score = tr["valu_insts"] * 64 / scores
        clk_int8 = 4.0 * w.D / MFMA_OPS_PER_CU_CLK["int8_fp8"]
        clk_mix = 2.0 * w.D / MFMA_OPS_PER_CU_CLK["int8_fp8"] + 2.0 * w.D / MFMA_OPS_PER_CU_CLK["bf16"]
        valu = {"counter": "SQ_INSTS_VALU", "lane_ops_per_score": round(per_score, 3),
                "budget_at_int8_fp8_peak": round(VALU_LANES_PER_CU_CLK * clk_int8, 3),
                "budget_at_issued_mix": round(VALU_LANES_PER_CU_CLK * (clk_mix if pv_bf16 else clk_int8), 3),
                "frac_of_peak_allowed_at_full_valu_rate": round(min(1.0, VALU_LANES_PER_CU_CLK * clk_int8 / per_score), 4)}
    roof["valu"] = valu
    rec = {
        "metric": "attention TOPS (4*N_q*N_k*D*H / step time) on one MI355X",
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms": pct(step_ms),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"int8 QK (v_mfma_i32_32x32x32_i8, int32 acc); fp8 e4m3 P and V, P.V on {qa.PV_INSTRUCTION} "
                 f"(fp32 acc)",
        "data": "synthetic (seeded N(0,1) bf16 inputs; see workloads.py)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N_q": w.Nq, "N_k": w.Nk, "D": w.D,
                   "causal": w.causal, "pos0": w.pos0 if w.kind == "i8kv" else None,
                   "kv_splits": kv_splits if w.kind == "i8kv" else 1, "step": steps_desc, "input_sha256": in_sha},
        "roofline": roof,
        "quantizer": quant,
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
