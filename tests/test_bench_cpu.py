"""Host-side logic of bench.py: FLOP and byte counts, the roofline choice and
the single-GPU guard.  No GPU needed."""
import json
import os
import struct
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from varlen_attention_forward_amd import workloads  # noqa: E402


def _brute_pairs(lq, lk, causal, wl, wr):
    i = np.arange(lq)[:, None] + (lk - lq)
    j = np.arange(lk)[None, :]
    vis = np.ones((lq, lk), dtype=bool)
    if causal:
        vis &= j <= i
    if wl >= 0:
        vis &= j >= i - wl
    if wr >= 0:
        vis &= j <= i + wr
    return int(vis.sum())


@pytest.mark.parametrize("lq,lk", [(0, 5), (5, 0), (1, 1), (7, 7), (5, 9), (9, 5), (33, 64)])
@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (3, 0)),
                                           (True, (4, -1)), (False, (0, 2))])
def test_visible_pairs_brute_force(lq, lk, causal, window):
    want = _brute_pairs(lq, lk, causal, *window)
    assert bench.visible_pairs([lq], [lk], causal, window) == want


@pytest.mark.parametrize("name,gflop", [
    ("tiny_varlen_d64", 0.2852), ("vit_full_d80", 320.82), ("vit_window256_d80", 12.08),
    ("vit_long65536_d128", 35184.4), ("mla_causal_192_128", 2749.45), ("mla_context_chunk_tp8", 85.899),
    ("vit_window64_d80", 14.680), ("vit_long65536_d128_fp8", 35184.4), ("mla_causal_192_128_fp8", 2749.45),
    ("gqa_chunk64_d128", 135.325),
])
def test_algorithmic_flops(name, gflop):
    """H x visible pairs x 2 (d_qk + d_v), against the figures worked out by hand
    for each configuration (causal: L (L + 1) / 2 pairs per segment)."""
    w = workloads.WORKLOADS[name]
    assert bench.algorithmic_flops(w) / 1e9 == pytest.approx(gflop, rel=2e-4)


def test_roofline_bound_follows_the_ridge():
    """Workloads below 312.5 flop per algorithmic byte are reported against HBM."""
    bounds = {n: bench.algorithmic_flops(w) / bench.algorithmic_bytes(w) >= bench.RIDGE_FLOP_PER_BYTE
              for n, w in workloads.WORKLOADS.items()}
    assert bounds == {"tiny_varlen_d64": False, "vit_full_d80": True, "vit_window256_d80": False,
                      "vit_window64_d80": False,
                      "vit_long65536_d128": True, "mla_causal_192_128": True, "mla_context_chunk_tp8": True,
                      "vit_long65536_d128_fp8": True, "mla_causal_192_128_fp8": True, "gqa_chunk64_d128": True}


def test_fp8_workloads_read_one_byte_per_input_element():
    """The e4m3 twins of the long-image and MLA workloads read half the input
    bytes (O is bf16 in both) and are priced against the 5 PFLOP/s fp8 peak."""
    for name in ("vit_long65536_d128", "mla_causal_192_128"):
        w, w8 = workloads.WORKLOADS[name], workloads.WORKLOADS[name + "_fp8"]
        h = w.num_heads
        inputs = h * (w.total_q * w.head_dim_qk + w.total_k * (w.head_dim_qk + w.head_dim_v))
        assert bench.algorithmic_bytes(w) - bench.algorithmic_bytes(w8) == pytest.approx(inputs)
        assert bench.peak_tflops(w8) == 5000.0 and bench.peak_tflops(w) == 2500.0


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_grouped_kv_workload_counts_kv_heads_once():
    """K and V are read once per KV head (4 here), Q and O once per query head."""
    w = workloads.WORKLOADS["gqa_chunk64_d128"]
    q_o = 2 * 32 * 4096 * (128 + 128)
    kv = 2 * 4 * (64 * 2048) * (128 + 128)
    assert bench.algorithmic_bytes(w) == pytest.approx(q_o + kv + 4 * 32 * 4096)


@pytest.mark.parametrize("lq,lk", [(1, 1), (7, 7), (600, 600), (300, 1000), (1000, 300)])
@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (100, 30)),
                                           (True, (64, -1))])
def test_oracle_task_pairs_add_up(lq, lk, causal, window):
    """The oracle baseline prices each (segment, head, row block) task by the
    visible pairs of its rows; over the blocks of a segment they add up to
    the segment's pairs."""
    total = sum(bench._pairs_in_rows(lq, lk, r0, min(r0 + 256, lq), causal, window) for r0 in range(0, lq, 256))
    assert total == bench.visible_pairs([lq], [lk], causal, window) == _brute_pairs(lq, lk, causal, *window)


def test_host_info_reports_core_counts():
    info = bench.host_info()
    assert info["cpu_count"] >= 1 and 1 <= info["affinity"] <= info["cpu_count"]


def test_kernel_code_hash_reads_the_built_machine_code(tmp_path):
    """Traffic records are keyed by a hash of the library's gfx950 machine
    code (.text and .rodata of each code object in the offload bundles): the
    built library yields one, the same on every read, and a record carrying
    another hash is treated as stale."""
    from varlen_attention_forward_amd import _binding
    h = bench.kernel_code_hash(_binding.LIB_PATH)
    assert len(h) == 16 and int(h, 16) >= 0
    assert bench.kernel_code_hash(_binding.LIB_PATH) == h
    # a copy whose machine code differs in one byte of .text hashes differently
    data = bytearray(open(_binding.LIB_PATH, "rb").read())
    off, size = bench._elf_sections(bytes(data))[".hip_fatbin"]
    fat = bytes(data[off:off + size])
    pos = fat.find(b"__CLANG_OFFLOAD_BUNDLE__")
    n, = struct.unpack_from("<Q", fat, pos + 24)
    q = pos + 32
    for _ in range(n):
        eoff, esize, tlen = struct.unpack_from("<QQQ", fat, q)
        triple = fat[q + 24:q + 24 + tlen].decode()
        q += 24 + tlen
        if triple.endswith("gfx950") and esize > 0:
            text_off, _ = bench._elf_sections(fat, pos + eoff)[".text"]
            data[off + text_off] ^= 0xFF
            break
    mod = tmp_path / "mod.so"
    mod.write_bytes(bytes(data))
    assert bench.kernel_code_hash(str(mod)) != h


def test_stale_traffic_record_reads_as_null(tmp_path, monkeypatch):
    """load_traffic returns the record's bytes only while its hash matches."""
    rec = {"kernel_code_sha": "0" * 16, "hbm_bytes_per_launch": 123}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic_x.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_code_hash", lambda lib_path=None: "0" * 16)
    assert bench.load_traffic("x") == 123.0
    monkeypatch.setattr(bench, "kernel_code_hash", lambda lib_path=None: "1" * 16)
    assert bench.load_traffic("x") is None
