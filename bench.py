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
MI355X dense bf16 MFMA peak (2.5 PFLOP/s) for workloads above the ridge
(312.5 flop per algorithmic byte), else against the 8 TB/s HBM peak with
achieved = algorithmic bytes / duration in GB/s.  ``cpu_baseline`` times the fp64
numpy oracle on a bounded sample of the same workload on the host cores.

Other modes (for the summaries under profiles/):
    python bench.py --copy-calibration     a plain 1 GiB device copy, to scale
                                            FETCH_SIZE / WRITE_SIZE counters
    python bench.py --report [--workload W]  every workload (or W): 10 rounds of
                                            5 warm-up + 20 timed launches (best and
                                            median), the same launches replayed from
                                            a HIP graph, the host-inclusive eager rate
                                            and the shader clock seen meanwhile; then
                                            the merge of two MLA-shaped partials (GB/s)
    python bench.py --pages                the same protocol over the shapes of the
                                            SGLang PR #41344 speed tables (16 heads,
                                            d 64/72/80, non-causal, no LSE)
"""
from __future__ import annotations

import argparse
import hashlib
import struct
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of MI355X bf16 MFMA peak, ViT d=80 and MLA 192/128"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0  # dense e4m3 MFMA, the roofline of the fp8 workloads
PEAK_HBM_GBS = 8000.0
RIDGE_FLOP_PER_BYTE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # 312.5
DEFAULT_WORKLOAD = "vit_full_d80"
def _elf_sections(data: bytes, base: int = 0) -> dict:
    """Section name -> (file offset, size) of the little-endian ELF64 image at data[base:]."""
    if data[base:base + 4] != b"\x7fELF" or data[base + 4] != 2 or data[base + 5] != 1:
        raise ValueError("not a little-endian ELF64 image")
    shoff, = struct.unpack_from("<Q", data, base + 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, base + 0x3A)
    hdrs = [struct.unpack_from("<IIQQQQ", data, base + shoff + i * shentsize) for i in range(shnum)]
    strtab = base + hdrs[shstrndx][4]
    out = {}
    for name_off, _typ, _flags, _addr, off, size in hdrs:
        end = data.index(b"\0", strtab + name_off)
        out[data[strtab + name_off:end].decode()] = (base + off, size)
    return out


def kernel_code_hash(lib_path: str = None) -> str:
    """First 16 hex digits of the sha256 of the library's gfx950 machine code: the
    .text and .rodata sections of every gfx950 code object in the clang offload
    bundles of its .hip_fatbin section, in order.  Comments, host code and
    symbol tables do not enter it, so a traffic record stays valid exactly as
    long as the kernels it was taken on are the ones that run."""
    if lib_path is None:
        from varlen_attention_forward_amd import _binding
        lib_path = _binding.LIB_PATH
    with open(lib_path, "rb") as f:
        data = f.read()
    off, size = _elf_sections(data)[".hip_fatbin"]
    fat = data[off:off + size]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    h = hashlib.sha256()
    n_code = 0
    pos = fat.find(magic)
    while pos >= 0:
        entries, = struct.unpack_from("<Q", fat, pos + len(magic))
        q = pos + len(magic) + 8
        for _ in range(entries):
            eoff, esize, tlen = struct.unpack_from("<QQQ", fat, q)
            triple = fat[q + 24:q + 24 + tlen].decode()
            q += 24 + tlen
            if triple.endswith("gfx950") and esize > 0:
                secs = _elf_sections(fat, pos + eoff)
                for name in (".text", ".rodata"):
                    so, sz = secs[name]
                    h.update(fat[so:so + sz])
                n_code += 1
        pos = fat.find(magic, pos + 1)
    if n_code == 0:
        raise ValueError("no gfx950 code object in %s" % lib_path)
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
    """Read Q, K, V once (2 bytes an element, 1 for e4m3); write O (bf16) and
    LSE (fp32, when returned)."""
    h, hk = w.num_heads, w.heads_k
    eb = 1.0 if w.dtype == "e4m3" else 2.0
    b = eb * (h * w.total_q * w.head_dim_qk + hk * w.total_k * (w.head_dim_qk + w.head_dim_v))
    b += 2.0 * h * w.total_q * w.head_dim_v
    if w.return_lse:
        b += 4.0 * h * w.total_q
    return b


def load_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernels' machine code changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_code_sha") != kernel_code_hash():
        return None
    return float(t["hbm_bytes_per_launch"])


def host_info() -> dict:
    """The host's core counts and CPU model, as the oracle baseline reports them."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - not Linux
        affinity = os.cpu_count() or 1
    return {"cpu_count": os.cpu_count(), "affinity": affinity, "cpu_model": model}


# Oracle tasks run in forked worker processes that inherit these arrays.
_ORACLE_ARGS = {}


def _limit_blas_threads():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass


def _oracle_task(task):
    """One (segment, head, block of query rows) of the workload through the
    oracle, on that segment and head alone."""
    import numpy as np

    a = _ORACLE_ARGS
    b, h, r0, r1, _ = task
    cu_q, cu_k, group = a["cu_q"], a["cu_k"], a["group"]
    q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
    hk = h // group
    sl_q, sl_k = slice(q0, q1), slice(k0, k1)
    rows = np.arange(r0, r1)
    if a["fp8"]:
        from oracle import attention_fwd_fp8

        one = lambda x: x[b:b + 1, hk:hk + 1]
        attention_fwd_fp8(a["q"][sl_q, h:h + 1], a["k"][sl_k, hk:hk + 1], a["v"][sl_k, hk:hk + 1], [0, q1 - q0],
                          [0, k1 - k0], a["scale"], a["causal"], a["wl"], a["wr"], rows=rows,
                          q_descale=one(a["q_descale"]), k_descale=one(a["k_descale"]),
                          v_descale=one(a["v_descale"]))
    else:
        from oracle import attention_fwd

        attention_fwd(a["q"][sl_q, h:h + 1], a["k"][sl_k, hk:hk + 1], a["v"][sl_k, hk:hk + 1], [0, q1 - q0],
                      [0, k1 - k0], a["scale"], a["causal"], a["wl"], a["wr"], rows=rows)
    return task


def cpu_baseline(w, inp, budget_s: float = 12.0, row_block: int = 512) -> dict:
    """The fp64 oracle timed on the host cores: one task per (segment, head,
    block of ``row_block`` query rows), in a seeded random order, on a pool
    of forked worker processes (one per core of this process's affinity,
    at most 16), each with one BLAS thread.  Tasks run until ``budget_s`` of
    wall time has passed; the rate is the algorithmic FLOPs of the completed
    tasks over that time.  Must run before the GPU is initialised (the
    workers are forks of this process)."""
    import multiprocessing

    import numpy as np
    import torch

    fp8 = w.dtype == "e4m3"
    if fp8:
        u8 = lambda t: t.view(torch.uint8).numpy()
        arrays = dict(q=u8(inp.q), k=u8(inp.k), v=u8(inp.v), q_descale=inp.q_descale.numpy(),
                      k_descale=inp.k_descale.numpy(), v_descale=inp.v_descale.numpy())
    else:
        f = lambda t: t.to(torch.float32).numpy()
        arrays = dict(q=f(inp.q), k=f(inp.k), v=f(inp.v))
    cu_q, cu_k = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
    wl, wr = w.window
    _ORACLE_ARGS.clear()
    _ORACLE_ARGS.update(arrays, cu_q=cu_q, cu_k=cu_k, group=w.num_heads // w.heads_k, scale=w.scale,
                        causal=w.causal, wl=wl, wr=wr, fp8=fp8)
    flop_per_pair = 2.0 * (w.head_dim_qk + w.head_dim_v)
    tasks = []
    for b in range(w.batch):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for r0 in range(0, lq, row_block):
            r1 = min(r0 + row_block, lq)
            pairs = _pairs_in_rows(lq, lk, r0, r1, w.causal, w.window)
            for h in range(w.num_heads):
                tasks.append((b, h, r0, r1, pairs * flop_per_pair))
    order = np.random.default_rng(0).permutation(len(tasks))
    tasks = [tasks[i] for i in order]
    info = host_info()
    workers = max(1, min(info["affinity"], 16))
    ctx = multiprocessing.get_context("fork")
    done_flops, done = 0.0, 0
    pool = ctx.Pool(workers, initializer=_limit_blas_threads)
    try:
        t0 = time.perf_counter()
        for task in pool.imap_unordered(_oracle_task, tasks, chunksize=1):
            done_flops += task[4]
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
    finally:
        pool.terminate()
        pool.join()
        _ORACLE_ARGS.clear()
    total = sum(t[4] for t in tasks)
    return {
        "value": done_flops / el / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": "%d of %d (segment, head, %d-row block) tasks in seeded random order, %.1f%% of the "
                  "workload's FLOPs, fp64 numpy oracle%s, %d worker processes x 1 BLAS thread" % (
                      done, len(tasks), row_block, 100.0 * done_flops / total,
                      " on dequantised e4m3" if fp8 else "", workers),
        "seconds": round(el, 3),
        "cpu_count": info["cpu_count"],
        "affinity": info["affinity"],
        "cpu_model": info["cpu_model"],
    }


def _pairs_in_rows(lq, lk, r0, r1, causal, window) -> int:
    """Visible (query, key) pairs of query rows [r0, r1) of one segment."""
    if lq <= 0 or lk <= 0:
        return 0
    wl, wr = window
    if not causal and wl < 0 and wr < 0:
        return (r1 - r0) * lk
    total = 0
    off = lk - lq
    for i in range(r0, r1):
        p = i + off
        lo = max(0, p - wl) if wl >= 0 else 0
        hi = lk - 1
        if causal:
            hi = min(hi, p)
        elif wr >= 0:
            hi = min(hi, p + wr)
        total += max(0, hi - lo + 1)
    return total


def device_inputs(w, cpu_inp, rotate: int = 0):
    """Input/output copies on cuda:0: three when the inputs fit the 256 MB
    last-level cache (so the timed reads come from HBM), else one."""
    import torch

    rotate = rotate or (3 if algorithmic_bytes(w) < 256e6 else 1)
    copies = []
    for _ in range(rotate):
        d = cpu_inp.to("cuda:0")
        out = torch.empty((w.total_q, w.num_heads, w.head_dim_v), dtype=torch.bfloat16, device="cuda:0")
        lse = torch.empty((w.num_heads, w.total_q), dtype=torch.float32, device="cuda:0") if w.return_lse else None
        copies.append((d, out, lse))
    return copies


def launch(copies, i, num_splits=1, max_seqlen_q=None):
    """One call on input copy i; ``max_seqlen_q`` overrides the bound (a
    looser one selects the unpacked launch, for comparison)."""
    import dataclasses

    import varlen_attention_forward_amd as va
    from varlen_attention_forward_amd import workloads

    d, out, lse = copies[i % len(copies)]
    if max_seqlen_q is not None:
        d = dataclasses.replace(d, max_seqlen_q=max_seqlen_q)
    if isinstance(d, workloads.Fp8Inputs):
        va.varlen_attn_fwd_fp8(d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, d.max_seqlen_q, d.max_seqlen_k,
                               softmax_scale=d.softmax_scale, causal=d.causal, window_size=d.window,
                               q_descale=d.q_descale, k_descale=d.k_descale, v_descale=d.v_descale,
                               out=out, return_lse=lse is not None, lse=lse, num_splits=num_splits)
    else:
        va.varlen_attn_fwd(d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, d.max_seqlen_q, d.max_seqlen_k,
                           softmax_scale=d.softmax_scale, causal=d.causal, window_size=d.window,
                           out=out, return_lse=lse is not None, lse=lse, num_splits=num_splits)


def peak_tflops(w) -> float:
    return PEAK_FP8_TFLOPS if w.dtype == "e4m3" else PEAK_BF16_TFLOPS


class ClockSampler:
    """Samples the shader clock (MHz) and board power (W) of cuda:0 in a
    background thread: the starred (current) level of the amdgpu driver's
    pp_dpm_sclk and its hwmon power1_input, for the PCI device that backs
    cuda:0 (power1_cap gives the board's power limit).  Read from sysfs, not
    through rocm-smi: no child process, so nothing is exec'd from a process
    that holds the GPU."""

    def __init__(self, period_s: float = 0.25):
        import threading

        self.samples, self.times = [], []  # shader clock (MHz) and when it was read
        self.power, self.power_times = [], []
        self.period_s = period_s
        dev = self._find()
        self._path = None if dev is None else os.path.join(dev, "pp_dpm_sclk")
        self._power_path, self.power_cap_w = self._hwmon(dev)
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _find():
        import glob

        import torch

        try:
            pr = torch.cuda.get_device_properties(0)
            want = "%04x:%02x:%02x." % (pr.pci_domain_id, pr.pci_bus_id, pr.pci_device_id)
        except Exception:
            return None
        for d in sorted(glob.glob("/sys/class/drm/card*/device")):
            if os.path.basename(os.path.realpath(d)).lower().startswith(want):
                return d
        return None

    @staticmethod
    def _hwmon(dev):
        import glob

        if dev is None:
            return None, None
        for h in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))):
            inp = os.path.join(h, "power1_input")
            if os.path.exists(inp):
                try:
                    with open(os.path.join(h, "power1_cap")) as fh:
                        cap = round(int(fh.read().strip()) / 1e6, 1)
                except (OSError, ValueError):
                    cap = None
                return inp, cap
        return None, None

    def _read(self):
        import re

        clk = pw = None
        try:
            if self._path is not None:
                with open(self._path) as fh:
                    m = re.search(r"(\d+)\s*mhz\s*\*", fh.read(), re.IGNORECASE)
                    clk = int(m.group(1)) if m else None
            if self._power_path is not None:
                with open(self._power_path) as fh:
                    pw = int(fh.read().strip()) / 1e6
        except (OSError, ValueError):
            pass
        return clk, pw

    def _run(self):
        while not self._stop.is_set():
            clk, pw = self._read()
            now = time.perf_counter()
            if clk is not None:
                self.samples.append(clk)
                self.times.append(now)
            if pw is not None:
                self.power.append(pw)
                self.power_times.append(now)
            self._stop.wait(self.period_s)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=15)

    def median(self, since=None):
        """Median of the samples read at or after perf_counter time `since`."""
        v = sorted(x for x, t in zip(self.samples, self.times) if since is None or t >= since)
        return v[len(v) // 2] if v else None

    def power_median(self, since=None):
        v = sorted(x for x, t in zip(self.power, self.power_times) if since is None or t >= since)
        return round(v[len(v) // 2], 1) if v else None

    def count(self, since=None):
        return sum(1 for t in self.times if since is None or t >= since)


def protocol_report(names, rounds: int = 10, warmup: int = 5, timed: int = 20, registry=None) -> None:
    """Per workload: best and median of `rounds` rounds of `timed` launches
    (HIP events on the launch stream, `warmup` untimed launches before each),
    the same `timed` launches captured once in a HIP graph and replayed
    `rounds` times (every replay's outputs checked bit-equal to eager ones),
    and the eager rate with host time included."""
    import statistics

    import torch
    from varlen_attention_forward_amd import workloads

    rows = []
    for name in names:
        w = (registry or workloads.WORKLOADS)[name]
        print("report: %s" % name, file=sys.stderr, flush=True)
        copies = device_inputs(w, workloads.workload_inputs(w))
        flops, nbytes = algorithmic_flops(w), algorithmic_bytes(w)
        stream = torch.cuda.current_stream()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        eager_ms, wall_ms = [], []
        ns = w.num_splits
        with ClockSampler(period_s=0.02) as clk:
            for _ in range(rounds):
                for i in range(warmup):
                    launch(copies, i, ns)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                ev0.record(stream)
                for i in range(timed):
                    launch(copies, i, ns)
                ev1.record(stream)
                torch.cuda.synchronize()
                wall_ms.append((time.perf_counter() - t0) * 1e3 / timed)
                eager_ms.append(ev0.elapsed_time(ev1) / timed)
        # eager reference outputs of every copy
        for i in range(len(copies)):
            launch(copies, i, ns)
        torch.cuda.synchronize()
        ref = [(o.clone(), None if l is None else l.clone()) for _, o, l in copies]
        graph = torch.cuda.CUDAGraph()
        for _, o, l in copies:  # replays must rewrite these
            o.zero_()
            if l is not None:
                l.zero_()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for i in range(timed):
                launch(copies, i, ns)
        graph_ms = []
        for _ in range(rounds):
            for _, o, _l in copies:
                o.zero_()
            torch.cuda.synchronize()
            ev0.record(stream)
            graph.replay()
            ev1.record(stream)
            torch.cuda.synchronize()
            graph_ms.append(ev0.elapsed_time(ev1) / timed)
            for (_, o, l), (ro, rl) in zip(copies, ref):
                if not torch.equal(o, ro) or (l is not None and not torch.equal(l, rl)):
                    raise RuntimeError("%s: graph replay differs from the eager result" % name)
        del graph
        unpacked = None
        pl = __import__("varlen_attention_forward_amd").plan(
            w.head_dim_qk, w.head_dim_v, w.batch, w.num_heads, w.max_seqlen_q, w.max_seqlen_k, w.causal,
            fp8=w.dtype == "e4m3", num_heads_k=w.heads_k)
        # the same call unpacked on the four-wave kernel, for comparison: a looser
        # max_seqlen_q (257, or 4096 where 257 still leaves a launch small
        # enough for the short kernel's key split)
        unpacked_q = None
        if pl["pack_mode"] != 0 or pl["kernel"] == "attn_fwd_short":
            for mq in (257, 4096, 16384):
                p2 = __import__("varlen_attention_forward_amd").plan(
                    w.head_dim_qk, w.head_dim_v, w.batch, w.num_heads, mq, w.max_seqlen_k, w.causal,
                    num_heads_k=w.heads_k)
                if p2["kernel"] == "attn_fwd_wide" and p2["pack_mode"] == 0:
                    unpacked_q = mq
                    break
        if unpacked_q is not None:
            times = []
            for _ in range(rounds):
                for i in range(warmup):
                    launch(copies, i, ns, unpacked_q)
                torch.cuda.synchronize()
                ev0.record(stream)
                for i in range(timed):
                    launch(copies, i, ns, unpacked_q)
                ev1.record(stream)
                torch.cuda.synchronize()
                times.append(ev0.elapsed_time(ev1) / timed)
            unpacked = min(times)
        unsplit = None
        if ns != 1:  # the same call without split-KV, for comparison
            times = []
            for _ in range(rounds):
                for i in range(warmup):
                    launch(copies, i, 1)
                torch.cuda.synchronize()
                ev0.record(stream)
                for i in range(timed):
                    launch(copies, i, 1)
                ev1.record(stream)
                torch.cuda.synchronize()
                times.append(ev0.elapsed_time(ev1) / timed)
            unsplit = min(times)
        best, med = min(eager_ms), statistics.median(eager_ms)
        row = {
            "workload": name,
            "kernel_ms_best": round(best, 4),
            "kernel_ms_median": round(med, 4),
            "tflops_best": round(flops / best / 1e9, 2),
            "tflops_median": round(flops / med / 1e9, 2),
            "frac_of_bf16_peak_best": round(flops / best / 1e9 / PEAK_BF16_TFLOPS, 4),
            "dtype": w.dtype,
            "frac_of_own_peak_best": round(flops / best / 1e9 / peak_tflops(w), 4),
            "gbs_best": round(nbytes / best / 1e6, 1),
            "graph_ms_best": round(min(graph_ms), 4),
            "graph_ms_median": round(statistics.median(graph_ms), 4),
            "eager_wall_ms_median": round(statistics.median(wall_ms), 4),
            "sclk_mhz_median": clk.median(),
            "sclk_samples": len(clk.samples),
            "board_power_w_median": clk.power_median(),
            "input_copies": len(copies),
        }
        if unpacked is not None:
            row["pack_mode"] = pl["pack_mode"]
            row["kernel"] = pl["kernel"]
            row["key_split"] = pl["key_split"]
            row["unpacked_max_seqlen_q"] = unpacked_q
            row["unpacked_kernel_ms_best"] = round(unpacked, 4)
            row["unpacked_tflops_best"] = round(flops / unpacked / 1e9, 2)
        if unsplit is not None:
            va_mod = __import__("varlen_attention_forward_amd")
            row["num_splits"] = va_mod.auto_num_splits(w.head_dim_qk, w.head_dim_v, w.batch, w.num_heads,
                                                       w.max_seqlen_q, w.max_seqlen_k, num_heads_k=w.heads_k,
                                                       fp8=w.dtype == "e4m3") if ns == 0 else ns
            row["unsplit_kernel_ms_best"] = round(unsplit, 4)
            row["unsplit_tflops_best"] = round(flops / unsplit / 1e9, 2)
        rows.append(row)
        print(json.dumps(row), flush=True)
    print("| workload | kernel ms best / median | TFLOP/s best / median | % of its dtype's peak | GB/s "
          "| graph ms best / median | eager wall ms | sclk MHz | board W |", flush=True)
    print("|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print("| %s | %.4f / %.4f | %.1f / %.1f | %.1f%% (%s) | %.0f | %.4f / %.4f | %.4f | %s | %s |" % (
            r["workload"], r["kernel_ms_best"], r["kernel_ms_median"], r["tflops_best"], r["tflops_median"],
            100 * r["frac_of_own_peak_best"], r["dtype"], r["gbs_best"], r["graph_ms_best"], r["graph_ms_median"],
            r["eager_wall_ms_median"], r["sclk_mhz_median"], r["board_power_w_median"]), flush=True)


MERGE_SHAPE = (16384, 128, 128)  # rows, heads, d_v: the MLA prefill batch's output


def merge_report(rounds: int = 10, warmup: int = 5, timed: int = 20) -> dict:
    """varlen_attn_merge of two partial results shaped like the MLA batch's
    output (three input/output copies cycled, so every read comes from HBM):
    best and median kernel time over `rounds` rounds, and GB/s of its
    algorithmic bytes (two bf16 outputs and two fp32 LSEs read, one of each
    written) against the 8 TB/s HBM peak."""
    import statistics

    import torch
    import varlen_attention_forward_amd as va

    rows, heads, dim = MERGE_SHAPE
    g = torch.Generator(device="cuda:0").manual_seed(7)
    copies = []
    for _ in range(3):
        oa = torch.randn((rows, heads, dim), generator=g, device="cuda:0").to(torch.bfloat16)
        ob = torch.randn((rows, heads, dim), generator=g, device="cuda:0").to(torch.bfloat16)
        la = torch.randn((heads, rows), generator=g, device="cuda:0") * 4
        lb = torch.randn((heads, rows), generator=g, device="cuda:0") * 4
        copies.append((oa, la, ob, lb, torch.empty_like(oa), torch.empty_like(la)))
    nbytes = 3 * rows * heads * dim * 2 + 3 * rows * heads * 4
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(rounds):
        for i in range(warmup):
            oa, la, ob, lb, o, l = copies[i % 3]
            va.varlen_attn_merge(oa, la, ob, lb, out=o, lse=l)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(timed):
            oa, la, ob, lb, o, l = copies[i % 3]
            va.varlen_attn_merge(oa, la, ob, lb, out=o, lse=l)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms.append(ev0.elapsed_time(ev1) / timed)
    best, med = min(ms), statistics.median(ms)
    return {"kernel": "merge_states", "shape": "%d rows x %d heads x d %d" % MERGE_SHAPE,
            "kernel_ms_best": round(best, 4), "kernel_ms_median": round(med, 4),
            "gbs_best": round(nbytes / best / 1e6, 1), "gbs_median": round(nbytes / med / 1e6, 1),
            "frac_of_hbm_peak_best": round(nbytes / best / 1e6 / PEAK_HBM_GBS, 4), "bytes": nbytes}


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5) -> None:
    import torch

    x = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


# The secondary configuration the metric names (MLA prefill); timed in the
# default run beside the ViT batch, which gives ``value``.
SECONDARY_WORKLOADS = ("mla_causal_192_128",)
# Warm-up continues past --warmup launches until this much wall time has
# passed: from idle the shader clock takes tens of milliseconds to ramp up.
MIN_WARMUP_S = 0.3


def time_workload(w, copies, steps: int, warmup: int, min_warmup_s: float = MIN_WARMUP_S) -> dict:
    """``warmup`` untimed launches (more until ``min_warmup_s`` of wall time
    has passed), then exactly ``steps`` launches between HIP events on the
    launch stream, the shader clock sampled meanwhile."""
    import torch

    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with ClockSampler(period_s=0.02) as clk:
        t0 = time.perf_counter()
        n_warm = 0
        while n_warm < warmup or time.perf_counter() - t0 < min_warmup_s:
            launch(copies, n_warm, w.num_splits)
            n_warm += 1
            if n_warm % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        warm_s = time.perf_counter() - t0
        t0 = time.perf_counter()
        since = t0 - 0.15  # the clock and power of the last 150 ms of warm-up and the timed steps
        ev0.record(stream)
        for i in range(steps):
            launch(copies, i, w.num_splits)
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    return {"wall_s": (t1 - t0) / steps, "kernel_s": ev0.elapsed_time(ev1) / 1e3 / steps,
            "warmup_launches": n_warm, "warmup_s": warm_s, "sclk_mhz_median": clk.median(since),
            "sclk_samples": clk.count(since), "board_power_w_median": clk.power_median(since),
            "power_cap_w": clk.power_cap_w}


def result_fields(w, t: dict, steps: int, warmup: int, rotate: int) -> dict:
    """The bench-contract fields of one workload from its timing."""
    import varlen_attention_forward_amd as va

    flops, in_bytes = algorithmic_flops(w), algorithmic_bytes(w)
    wall_s, kernel_s = t["wall_s"], t["kernel_s"]
    mfma_bound = flops / in_bytes >= RIDGE_FLOP_PER_BYTE
    if mfma_bound:
        achieved, peak, r_unit = flops / kernel_s / 1e12, peak_tflops(w), "TFLOP/s"
    else:
        achieved, peak, r_unit = in_bytes / kernel_s / 1e9, PEAK_HBM_GBS, "GB/s"
    plan = va.plan(w.head_dim_qk, w.head_dim_v, w.batch, w.num_heads, w.max_seqlen_q, w.max_seqlen_k, w.causal,
                   fp8=w.dtype == "e4m3", num_heads_k=w.heads_k)
    return {
        "value": round(flops / wall_s / 1e12, 2),
        "unit": "TFLOP/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall_s * 1e3, 4),
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) %s)" % ("bf16" if w.dtype == "bf16" else
                                                  "quantised to e4m3 with per-(segment, head) descales"),
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
            "bound": "mfma" if mfma_bound else "hbm",
            "kernel": plan["kernel"],
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": r_unit,
            "frac": round(achieved / peak, 4),
            "tflops_kernel": round(flops / kernel_s / 1e12, 2),
            "kernel_ms": round(kernel_s * 1e3, 4),
            "traffic": load_traffic(w.name),
            "algorithmic_bytes": in_bytes,
        },
        "clock": {
            "sclk_mhz_median": t["sclk_mhz_median"],
            "sclk_samples": t["sclk_samples"],
            "board_power_w_median": t["board_power_w_median"],
            "power_cap_w": t["power_cap_w"],
            "warmup_launches": t["warmup_launches"],
            "warmup_ms": round(t["warmup_s"] * 1e3, 1),
        },
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rotate", type=int, default=0,
                    help="input copies to cycle through (0 = 3 when the inputs fit the 256 MB MALL, else 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="time only --workload (by default the MLA prefill is timed beside the ViT batch)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--report", action="store_true",
                    help="timing protocol over every workload (or --workload if given explicitly)")
    ap.add_argument("--pages", action="store_true",
                    help="the same protocol over the shapes of the SGLang PR #41344 speed tables")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr, flush=True)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.pages:
        from varlen_attention_forward_amd import workloads

        protocol_report(list(workloads.PAGE_SHAPES), registry=workloads.PAGE_SHAPES)
        return 0
    if args.report:
        from varlen_attention_forward_amd import workloads

        explicit = any(a == "--workload" or a.startswith("--workload=") for a in sys.argv[1:])
        protocol_report([args.workload] if explicit else list(workloads.WORKLOADS))
        if not explicit:
            print(json.dumps(merge_report()), flush=True)
        return 0

    from varlen_attention_forward_amd import workloads

    if args.workload not in workloads.WORKLOADS:
        print("unknown workload %r; choose from %s" % (args.workload, list(workloads.WORKLOADS)), file=sys.stderr)
        return 2
    names = [args.workload]
    if args.workload == DEFAULT_WORKLOAD and not args.no_secondary:
        names += list(SECONDARY_WORKLOADS)

    # Inputs on the host, then the oracle baselines, all before the GPU is
    # touched (the oracle's worker processes are forks of this one).
    cpu_inputs, baselines = {}, {}
    for name in names:
        print("bench: workload %s, building inputs" % name, file=sys.stderr, flush=True)
        cpu_inputs[name] = workloads.workload_inputs(workloads.WORKLOADS[name])
    if not args.no_cpu_baseline:
        for name in names:
            print("bench: timing the oracle on the host (%s)" % name, file=sys.stderr, flush=True)
            baselines[name] = cpu_baseline(workloads.WORKLOADS[name], cpu_inputs[name])

    import torch

    results = {}
    for name in names:
        w = workloads.WORKLOADS[name]
        copies = device_inputs(w, cpu_inputs.pop(name), args.rotate)
        print("bench: timing %d steps of %s" % (args.steps, name), file=sys.stderr, flush=True)
        t = time_workload(w, copies, args.steps, args.warmup)
        results[name] = result_fields(w, t, args.steps, args.warmup, len(copies))
        if name in baselines:
            results[name]["cpu_baseline"] = baselines[name]
        del copies
        torch.cuda.empty_cache()

    main_r = results[names[0]]
    result = {
        "metric": METRIC,
        "value": main_r["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_r["dtype"],
        "data": main_r["data"],
        "config": main_r["config"],
        "roofline": main_r["roofline"],
        "clock": main_r["clock"],
    }
    if "cpu_baseline" in main_r:
        result["cpu_baseline"] = main_r["cpu_baseline"]
    others = [dict(results[n], vs_baseline=None) for n in names[1:]]
    if others:
        result["other_configs"] = others
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
