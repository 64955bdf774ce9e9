"""Throughput of the fused varlen attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of ``varlen_attn_fwd`` (one kernel launch: scheduler,
Q/K/V staging, QK^T, masking, online softmax, PV and epilogue) over one
batch of seeded synthetic bf16 inputs already resident in HBM.  The default
workload is the ViT full-attention batch (8 images, lengths drawn from
{576, 1024, 2304, 4096} with seed 2, 16 heads, d = 80, non-causal).

Prints one JSON line.  ``value`` is algorithmic TFLOP/s over the timed
steps (FLOPs = heads * visible (query, key) pairs * 2 * (d_qk + d_v); no
padding or skipped-tile work is counted).  ``roofline`` compares the kernel's
average duration, measured with HIP events on the launch stream, against the
MI355X dense bf16 MFMA peak (2.5 PFLOP/s).  ``cpu_baseline`` times the fp64
numpy oracle on a bounded sample of the same workload on the host cores.

Other modes (for the rocprofv3 summaries under profiles/):
    python bench.py --copy-calibration     a plain 1 GiB device copy, to scale
                                            FETCH_SIZE / WRITE_SIZE counters
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of MI355X bf16 MFMA peak, ViT d=80 and MLA 192/128"
PEAK_BF16_TFLOPS = 2500.0
DEFAULT_WORKLOAD = "vit_full_d80"
KERNEL_SOURCES = [
    os.path.join(ROOT, "varlen_attention_forward_amd", "csrc", "varlen_attn_fwd.hip"),
    os.path.join(ROOT, "varlen_attention_forward_amd", "csrc", "tile_schedule.h"),
]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def visible_pairs(seqlens_q, seqlens_k, causal, window) -> int:
    """Visible (query, key) pairs per head (closed forms per segment)."""
    wl, wr = window
    total = 0
    for lq, lk in zip(seqlens_q, seqlens_k):
        if lq <= 0 or lk <= 0:
            continue
        if not causal and wl < 0 and wr < 0:
            total += lq * lk
            continue
        off = lk - lq
        for i in range(lq):
            p = i + off
            lo = max(0, p - wl) if wl >= 0 else 0
            hi = lk - 1
            if causal:
                hi = min(hi, p)
            elif wr >= 0:
                hi = min(hi, p + wr)
            total += max(0, hi - lo + 1)
    return total


def algorithmic_flops(w) -> float:
    pairs = visible_pairs(w.seqlens_q, w.seqlens_k, w.causal, w.window)
    return float(w.num_heads) * pairs * 2.0 * (w.head_dim_qk + w.head_dim_v)


def algorithmic_bytes(w) -> float:
    """Read Q, K, V once; write O (bf16) and LSE (fp32, when returned)."""
    h = w.num_heads
    b = 2.0 * h * (w.total_q * w.head_dim_qk + w.total_k * (w.head_dim_qk + w.head_dim_v) + w.total_q * w.head_dim_v)
    if w.return_lse:
        b += 4.0 * h * w.total_q
    return b


def load_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return float(t["hbm_bytes_per_launch"])


def cpu_baseline(w, inp, budget_s: float = 12.0) -> dict:
    """Time the fp64 oracle on whole heads of the workload until ``budget_s``."""
    import numpy as np
    import torch
    from oracle import attention_fwd

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = os.cpu_count() or 1
    q = inp.q.to(torch.float32).numpy()
    k = inp.k.to(torch.float32).numpy()
    v = inp.v.to(torch.float32).numpy()
    cu_q, cu_k = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
    wl, wr = w.window
    per_head = algorithmic_flops(w) / w.num_heads
    t0 = time.perf_counter()
    done = 0
    rows = None
    if w.name == "vit_long65536_d128":
        rows = np.arange(0, w.total_q, 64)  # 1/64 of the rows: every row costs the same
    for h in range(w.num_heads):
        attention_fwd(q, k, v, cu_q, cu_k, w.scale, w.causal, wl, wr, rows=rows, heads=[h])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    frac_rows = 1.0 if rows is None else len(rows) / w.total_q
    flops = per_head * done * frac_rows
    sample = "%d of %d heads, %s rows, fp64 numpy oracle" % (
        done, w.num_heads, "all" if rows is None else "every 64th of the")
    return {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": sample,
        "seconds": round(el, 3),
    }


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5) -> None:
    import torch

    x = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rotate", type=int, default=0,
                    help="input copies to cycle through (0 = 3 when the inputs fit the 256 MB MALL, else 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr, flush=True)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0

    import torch
    import varlen_attention_forward_amd as va
    from varlen_attention_forward_amd import workloads

    if args.workload not in workloads.WORKLOADS:
        print("unknown workload %r; choose from %s" % (args.workload, list(workloads.WORKLOADS)), file=sys.stderr)
        return 2
    w = workloads.WORKLOADS[args.workload]
    print("bench: workload %s, building inputs" % w.name, file=sys.stderr, flush=True)
    cpu_inp = workloads.workload_inputs(w)
    in_bytes = algorithmic_bytes(w)
    rotate = args.rotate or (3 if in_bytes < 256e6 else 1)
    dev = "cuda:0"
    copies = []
    for _ in range(rotate):
        d = cpu_inp.to(dev)
        out = torch.empty((w.total_q, w.num_heads, w.head_dim_v), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.num_heads, w.total_q), dtype=torch.float32, device=dev) if w.return_lse else None
        copies.append((d, out, lse))

    def step(i):
        d, out, lse = copies[i % rotate]
        va.varlen_attn_fwd(d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, d.max_seqlen_q, d.max_seqlen_k,
                           softmax_scale=d.softmax_scale, causal=d.causal, window_size=d.window,
                           out=out, return_lse=lse is not None, lse=lse)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_s = (t1 - t0) / args.steps
    kernel_s = ev0.elapsed_time(ev1) / 1e3 / args.steps

    flops = algorithmic_flops(w)
    achieved = flops / kernel_s / 1e12
    plan = va.plan(w.head_dim_qk, w.head_dim_v, w.batch, w.num_heads, w.max_seqlen_q, w.max_seqlen_k, w.causal)
    result = {
        "metric": METRIC,
        "value": round(flops / wall_s / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16)",
        "config": {
            "workload": w.name,
            "description": w.description,
            "segments": w.batch,
            "tokens": w.total_q,
            "heads": w.num_heads,
            "head_dim_qk": w.head_dim_qk,
            "head_dim_v": w.head_dim_v,
            "causal": w.causal,
            "gflop_per_step": round(flops / 1e9, 3),
            "block_m": plan["block_m"],
            "block_n": plan["block_n"],
            "grid": plan["grid"],
            "input_copies": rotate,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": plan["kernel"],
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "kernel_ms": round(kernel_s * 1e3, 4),
            "traffic": load_traffic(w.name),
            "algorithmic_bytes": in_bytes,
        },
    }
    if not args.no_cpu_baseline:
        print("bench: timing the oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, cpu_inp)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
