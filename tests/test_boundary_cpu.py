"""Host-side tests of the C interface (no GPU needed).

* the built library loads and exports every function include/varlen_attn.h
  declares;
* argument validation returns the documented status codes before any HIP
  call (only failing or no-launch cases are used here, so nothing is ever
  launched with the placeholder pointers);
* the kernel's tile schedule (the same __host__ __device__ function the
  kernel runs, exported as varlen_attn_tile_range) equals brute force over
  the oracle's visibility mask: the visited key tiles are exactly those with
  at least one visible (row, key) pair, and the unmasked ones exactly those
  whose every pair is visible.
"""
import ctypes
import os
import random
import re

import numpy as np

import pytest

import varlen_attention_forward_amd as pkg
from varlen_attention_forward_amd import _binding as B
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "varlen_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(varlen_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert sorted(pkg.EXPORTED_SYMBOLS) == declared
    lib = ctypes.CDLL(pkg.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(-8, 1):
        s = pkg.status_string(code)
        assert isinstance(s, str) and s != "unknown status"
    assert pkg.status_string(12345) == "unknown status"
    assert pkg.status_string(B.VA_ERR_HEADDIM).startswith("unsupported")


# ---------------------------------------------------------------------------
# validation (placeholder pointers; every call below must fail or return
# before launching)
# ---------------------------------------------------------------------------
FAKE = 0x100000  # 16-byte aligned, never dereferenced


def _t(rows=10, heads=2, dim=64, row_stride=None, head_stride=None, data=FAKE):
    hs = dim if head_stride is None else head_stride
    rs = heads * dim if row_stride is None else row_stride
    return B.VaTensor(data, rows, heads, dim, rs, hs)


def _call(q=None, k=None, v=None, out=None, cu_q=FAKE, cu_k=FAKE, batch=1, mq=10, mk=10,
          scale=0.125, causal=0, wl=-1, wr=-1, lse=0):
    q = q if q is not None else _t()
    k = k if k is not None else _t()
    v = v if v is not None else _t()
    out = out if out is not None else _t()
    return B.raw_fwd(q, k, v, cu_q, cu_k, batch, mq, mk, scale, causal, wl, wr, out, lse, 0)


def _lib_call_null(which):
    lib = pkg.library()
    t = _t()
    args = [ctypes.byref(t)] * 3
    args[which] = None
    return lib.varlen_attn_fwd(*args, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 1, 10, 10,
                               ctypes.c_float(0.125), 0, -1, -1, ctypes.byref(t), None, None)


@pytest.mark.parametrize("which", [0, 1, 2])
def test_null_descriptor(which):
    assert _lib_call_null(which) == B.VA_ERR_NULL


def test_null_out_descriptor():
    lib = pkg.library()
    t = _t()
    st = lib.varlen_attn_fwd(ctypes.byref(t), ctypes.byref(t), ctypes.byref(t), ctypes.c_void_p(FAKE),
                             ctypes.c_void_p(FAKE), 1, 10, 10, ctypes.c_float(0.125), 0, -1, -1, None, None, None)
    assert st == B.VA_ERR_NULL


def test_null_data_and_cu_seqlens():
    assert _call(q=_t(data=0)) == B.VA_ERR_NULL
    assert _call(k=_t(data=0)) == B.VA_ERR_NULL
    assert _call(out=_t(data=0)) == B.VA_ERR_NULL
    assert _call(cu_q=0) == B.VA_ERR_NULL
    assert _call(cu_k=0) == B.VA_ERR_NULL


@pytest.mark.parametrize("dims", [(32, 32), (96, 96), (256, 256), (192, 192), (128, 64), (80, 64), (0, 0)])
def test_unsupported_head_dims(dims):
    dqk, dv = dims
    st = _call(q=_t(dim=dqk), k=_t(dim=dqk), v=_t(dim=dv), out=_t(dim=dv))
    assert st == B.VA_ERR_HEADDIM


def test_shape_mismatches():
    # grouped KV heads: q heads a multiple of the k/v heads, k and v alike
    assert _call(q=_t(heads=3), out=_t(heads=3)) == B.VA_ERR_SHAPE  # 3 query heads over 2 KV heads
    assert _call(k=_t(heads=1, dim=64)) == B.VA_ERR_SHAPE           # k and v head counts differ
    assert _call(k=_t(heads=0), v=_t(heads=0)) == B.VA_ERR_SHAPE
    assert _call(out=_t(heads=1)) == B.VA_ERR_SHAPE
    assert _call(v=_t(rows=11)) == B.VA_ERR_SHAPE
    assert _call(out=_t(rows=9)) == B.VA_ERR_SHAPE
    assert _call(k=_t(dim=80)) == B.VA_ERR_SHAPE
    assert _call(out=_t(dim=128)) == B.VA_ERR_SHAPE
    assert _call(q=_t(heads=0)) == B.VA_ERR_SHAPE
    assert _call(q=_t(rows=-1), out=_t(rows=-1)) == B.VA_ERR_SHAPE


def test_strides_and_alignment():
    assert _call(q=_t(row_stride=0)) == B.VA_ERR_STRIDE
    assert _call(v=_t(head_stride=-64)) == B.VA_ERR_STRIDE
    assert _call(k=_t(row_stride=132)) == B.VA_ERR_ALIGN  # not a multiple of 8 elements
    assert _call(out=_t(head_stride=68)) == B.VA_ERR_ALIGN
    assert _call(q=_t(data=FAKE + 8)) == B.VA_ERR_ALIGN
    assert _call(lse=FAKE + 2) == B.VA_ERR_ALIGN


def test_scalar_arguments():
    assert _call(scale=0.0) == B.VA_ERR_ARG
    assert _call(scale=-0.1) == B.VA_ERR_ARG
    assert _call(scale=float("nan")) == B.VA_ERR_ARG
    assert _call(scale=float("inf")) == B.VA_ERR_ARG
    assert _call(causal=2) == B.VA_ERR_ARG
    assert _call(wl=-2) == B.VA_ERR_ARG
    assert _call(wr=-5) == B.VA_ERR_ARG
    assert _call(batch=-1) == B.VA_ERR_ARG
    assert _call(mq=-1) == B.VA_ERR_ARG
    assert _call(mk=-1) == B.VA_ERR_ARG


def test_empty_work_returns_ok_without_launch():
    # batch == 0, max_seqlen_q == 0 and total_q == 0 are valid no-ops.
    assert _call(batch=0) == B.VA_OK
    assert _call(mq=0) == B.VA_OK
    assert _call(q=_t(rows=0, data=0), out=_t(rows=0, data=0)) == B.VA_OK
    assert _call(batch=0, cu_q=0, cu_k=0) == B.VA_OK


def test_plan():
    p = pkg.plan(80, 80, 8, 16, 4096, 4096)
    assert p["block_n"] in (32, 64) and p["threads"] in (256, 512)
    assert p["kernel"] == "attn_fwd_wide" and p["block_m"] == 256 and p["threads"] == 256
    # one launch shape for every head dim and segment length
    short = pkg.plan(80, 80, 36, 16, 256, 256)
    assert short["kernel"] == "attn_fwd_wide" and short["block_m"] == 256 and short["threads"] == 256
    assert pkg.plan(64, 64, 16, 16, 257, 257)["kernel"] == "attn_fwd_wide"
    assert pkg.plan(128, 128, 1, 16, 4096, 4096)["kernel"] == "attn_fwd_wide"
    # 64-row blocks that fit one round of two workgroups a CU on each XCD
    # (2 x 8 (segment, head) groups x 5 blocks = 80 <= 8 x 64):
    # the short-segment kernel, a workgroup's four waves splitting each block's keys
    ks = pkg.plan(64, 64, 1, 16, 257, 257)
    assert (ks["kernel"], ks["block_m"], ks["threads"], ks["key_split"]) == ("attn_fwd_short", 64, 256, 4)
    assert ks["grid"] == ks["units"] == 8 * 2 * 5  # 16 heads pad to 2 x 8 groups, 5 blocks of 64
    assert pkg.plan(128, 128, 1, 16, 257, 257)["key_split"] == 1  # head dims > 80: four-wave kernel
    assert p["key_split"] == 1 and short["key_split"] == 1
    # 8 x 16 (segment, head) groups, already a multiple of the 8 XCDs
    assert p["grid"] == 8 * 16 * -(-4096 // p["block_m"])
    # 3 x 5 = 15 groups pad to 16
    assert pkg.plan(128, 128, 3, 5, 4096, 4096)["grid"] == 16 * -(-4096 // p["block_m"])
    with pytest.raises(ValueError):
        pkg.plan(96, 96, 1, 1, 10, 10)


def test_abi_struct_layouts_match_binding(tmp_path):
    """The structs of include/varlen_attn.h as a C compiler lays them out
    (offset and size of every field the binding declares, and each struct's
    size) are the ctypes structures the binding passes across the C ABI."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"va_tensor": B.VaTensor, "va_plan": B.VaPlan}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "varlen_attn.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append('  printf("%s - %%zu %%zu\\n", (size_t)0, sizeof(%s));' % (cname, cname))
        for field, _ in cls._fields_:
            lines.append('  printf("%s %s %%zu %%zu\\n", offsetof(%s, %s), sizeof(((%s*)0)->%s));'
                         % (cname, field, cname, field, cname, field))
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    include = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([cc, "-std=c99", "-I", include, str(src), "-o", str(exe)], check=True)
    got = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    for line in filter(None, got):
        cname, field, off, size = line.split()
        cls = structs[cname]
        if field == "-":
            assert int(size) == ctypes.sizeof(cls), cname
        else:
            desc = getattr(cls, field)
            assert (int(off), int(size)) == (desc.offset, desc.size), (cname, field)


def test_python_binding_rejects_cpu_tensors():
    import torch

    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises((TypeError, ValueError)):
        pkg.varlen_attn_fwd(q, q, q, cu, cu, 4, 4)


# ---------------------------------------------------------------------------
# tile schedule vs brute force
# ---------------------------------------------------------------------------


def _brute(Lq, Lk, r0, r1, causal, wl, wr, bn):
    m = oracle.visible_mask(Lq, Lk, causal, wl, wr)[r0:r1]
    ntiles = max(1, -(-max(Lk, 1) // bn)) + 1
    visited, full = set(), set()
    for t in range(ntiles):
        block = np.zeros((r1 - r0, bn), dtype=bool)
        lo, hi = t * bn, min((t + 1) * bn, Lk)
        if hi > lo:
            block[:, : hi - lo] = m[:, lo:hi]
        if block.any():
            visited.add(t)
            if block.all():
                full.add(t)
    return visited, full


def _kernel_sets(Lq, Lk, r0, r1, causal, wl, wr, bn):
    kb, ke, fb, fe = pkg.tile_range(Lq, Lk, r0, r1, causal, wl, wr, bn)
    return set(range(kb, ke)), set(range(fb, fe))


def test_tile_range_exhaustive_small():
    bn = 4
    count = 0
    for Lq in range(1, 10):
        for Lk in range(0, 11):
            for causal in (0, 1):
                for wl in (-1, 0, 1, 2, 5):
                    for wr in (-1, 0, 1, 3):
                        for r0 in range(0, Lq, 3):
                            for r1 in (min(r0 + 3, Lq), min(r0 + 5, Lq), Lq):
                                if r1 <= r0:
                                    continue
                                got = _kernel_sets(Lq, Lk, r0, r1, causal, wl, wr, bn)
                                want = _brute(Lq, Lk, r0, r1, causal, wl, wr, bn)
                                assert got == want, (Lq, Lk, r0, r1, causal, wl, wr, got, want)
                                count += 1
    assert count > 10000


@pytest.mark.parametrize("seed", range(4))
def test_tile_range_random_kernel_shapes(seed):
    """Kernel-sized tiles (64 keys, 128-row blocks) on random lengths and masks."""
    rng = np.random.default_rng(seed)
    for _ in range(150):
        Lq = int(rng.integers(1, 700))
        Lk = int(rng.integers(0, 700))
        causal = int(rng.integers(0, 2))
        wl = int(rng.choice([-1, 0, 1, 63, 64, 65, 200]))
        wr = int(rng.choice([-1, 0, 1, 63, 64, 100]))
        bm = 128
        for r0 in range(0, Lq, bm):
            r1 = min(r0 + bm, Lq)
            got = _kernel_sets(Lq, Lk, r0, r1, causal, wl, wr, 64)
            want = _brute(Lq, Lk, r0, r1, causal, wl, wr, 64)
            assert got == want, (Lq, Lk, r0, r1, causal, wl, wr)


def test_tile_range_config_shapes():
    # MLA causal 4096: q-tile t of 128 rows visits tiles 0 .. 2t+1 and masks
    # exactly the two diagonal tiles.
    for t in range(32):
        kb, ke, fb, fe = pkg.tile_range(4096, 4096, 128 * t, 128 * (t + 1), 1, -1, -1, 64)
        assert (kb, ke) == (0, 2 * t + 2)
        assert (fb, fe) == (0, 2 * t)
    # full attention on 576 keys: 9 tiles, all unmasked
    assert pkg.tile_range(576, 576, 0, 128, 0, -1, -1, 64) == (0, 9, 0, 9)
    # 100 keys: the partial second tile is masked
    assert pkg.tile_range(100, 100, 0, 100, 0, -1, -1, 64) == (0, 2, 0, 1)


def test_tile_range_rejects_bad_arguments():
    with pytest.raises(ValueError):
        pkg.tile_range(10, 10, 5, 5, 0, -1, -1, 64)
    with pytest.raises(ValueError):
        pkg.tile_range(10, 10, 0, 11, 0, -1, -1, 64)
    with pytest.raises(ValueError):
        pkg.tile_range(10, 10, 0, 10, 0, -1, -1, 0)


# ---------------------------------------------------------------------------
# workgroup -> (segment, head, q-tile) mapping
# ---------------------------------------------------------------------------
def _ragged(seed, batch, lo, hi):
    rng = random.Random(seed)
    return [rng.randint(lo, hi) for _ in range(batch)]


def _head_group_shift(d_qk, d_v, heads, heads_k=None, in_bytes=2):
    """Adjacent heads dealt together: the fewest 2^s heads whose rows of Q,
    K, V (in_bytes per element) and O (bf16) fill whole 128-byte lines."""
    if heads_k is not None and heads_k != heads:
        return 0
    for s_ in range(4):
        hg = 1 << s_
        if heads % hg:
            break
        if (hg * d_qk * in_bytes) % 128 == 0 and (hg * d_v * in_bytes) % 128 == 0 and (hg * d_v * 2) % 128 == 0:
            return s_
    return 0


@pytest.mark.parametrize("batch,heads", [(700, 16), (5, 3), (33, 8), (1, 1)])
def test_short_kernel_workgroups_cover_units(batch, heads):
    """The short-segment kernel's workgroups hold four one-wave units:
    workgroup w's wave v takes unit ((w >> 3) * 4 + v) * 8 + (w & 7).  Over
    the plan's grid every unit below va_plan.units is taken exactly once, on
    the XCD (w % 8) its dealing intends (unit % 8), and no workgroup is
    launched whose waves all fall past the units."""
    p = pkg.plan(80, 80, batch, heads, 64, 64)
    assert p["kernel"] == "attn_fwd_short" and p["threads"] == 256
    taken = {}
    for w in range(p["grid"]):
        us = [((w >> 3) * 4 + v) * 8 + (w & 7) for v in range(4)]
        assert any(u < p["units"] for u in us)
        for u in us:
            if u < p["units"]:
                assert u not in taken and u % 8 == w % 8
                taken[u] = w
    assert sorted(taken) == list(range(p["units"]))


def _short_head_group_shift(d_qk, d_v, heads, batch):
    """The one-wave short-segment kernel deals more heads together: all of a
    segment's heads (up to 16) while every XCD still gets at least 8 (segment,
    head group) groups, and never fewer than _head_group_shift."""
    s_ = _head_group_shift(d_qk, d_v, heads)
    while s_ < 4 and heads % (2 << s_) == 0 and batch * (heads >> (s_ + 1)) >= 64:
        s_ += 1
    return s_


def _expect_pairs(dq, dv, batch, heads, max_q, max_k, heads_k=None):
    """Whether a causal launch of the four-wave kernel pairs q-tiles: head dims
    that run one workgroup per CU (d_qk > 80), several q-tiles, unpacked, at
    least two rounds of unpaired units on each XCD (padded grid / 8 over its 32
    CUs) and pairs that fill at least 15/16 of their last round."""
    p0 = pkg.plan(dq, dv, batch, heads, max_q, max_k, 0, num_heads_k=heads_k or heads)
    n_qt = -(-max_q // p0["block_m"])
    if dq <= 80 or n_qt < 2 or p0["segments_per_block"] != 1 or p0["pack_mode"] != 0:
        return False
    solo = p0["units"] // 8
    pairs = solo // n_qt * ((n_qt + 1) // 2)
    return solo >= 64 and 16 * pairs >= 15 * 32 * -(-pairs // 32)


@pytest.mark.parametrize("lq,lk,heads,causal,dims", [
    ([4096] * 8, [4096] * 8, 16, 0, (80, 80)),            # alike: packing order
    ([256] * 36, [256] * 36, 16, 0, (80, 80)),
    ([65536], [65536], 16, 0, (128, 128)),
    ([1, 1], [1, 1], 1, 0, (72, 72)),                     # short: one wave per segment and head
    ([64] * 9, [80] * 9, 3, 1, (64, 64)),
    ([64] * 700, None, 16, 0, (80, 80)),                  # 64-token windows: all 16 heads together
    ([64] * 20, None, 16, 0, (80, 80)),                   # 20 windows: heads stay in fours (eights: < 8 groups an XCD)
    ([64] * 9, [80] * 9, 3, 1, (128, 128)),               # four 64-query segments per workgroup
    ([100, 3, 128, 0, 77], [500, 3, 9, 0, 77], 5, 0, (192, 128)),  # two per workgroup
    ([576, 1024, 2304, 4096, 1024, 576, 4096, 2304], None, 16, 0, (80, 80)),  # ragged: longest first
    ([700, 0, 300, 1], [700, 5, 0, 1], 5, 1, (64, 64)),
    ([3000, 100, 2000, 4096], None, 128, 1, (192, 128)),
    (_ragged(1, 64, 0, 900), None, 3, 0, (128, 128)),     # 64 segments: still longest first
    (_ragged(2, 65, 1, 900), None, 3, 1, (64, 64)),       # 65 segments: packing order
    ([500, 500, 500], [500, 900, 500], 7, 1, (80, 80)),   # ties broken by packing order
])
def test_work_unit_covers_every_tile_once(lq, lk, heads, causal, dims):
    lk = lq if lk is None else lk
    batch, max_q = len(lq), max(lq)
    p = pkg.plan(dims[0], dims[1], batch, heads, max_q, max(lk), causal)
    short = p["kernel"] == "attn_fwd_short"  # one wave per (segment, head, 64 rows)
    # small launches of longer segments: four waves on one 64-row block
    ksplit = p["key_split"] == 4
    assert ksplit == (dims[0] <= 80 and max_q > 64 and 8 * -(-batch * heads // 8) * -(-max_q // 64) <= 512)
    # head groups only where every segment is one q-tile (or packed)
    hs = ((_short_head_group_shift(dims[0], dims[1], heads, batch) if short
           else _head_group_shift(dims[0], dims[1], heads)) if max_q <= p["block_m"] else 0)
    bm = p["block_m"]
    pack = p["segments_per_block"]
    assert short == ((max_q <= 64 or ksplit) and dims[0] <= 80)
    assert pack == (1 if short else 4 if max_q <= 64 else 2 if max_q <= 128 else 1)
    assert (bm, p["threads"]) == (64, 256) if short else (256, 256)
    # one-wave units, four to a workgroup, for the short-segment kernel
    assert p["units"] % 8 == 0
    assert p["grid"] == ((p["units"] // 8 + 3) // 4 * 8 if short and not ksplit else p["units"])
    if pack > 1:
        # short segments: block owns segments [b, b + pack) of one head, q-tile 0
        seen = {}
        for blk in range(p["units"]):
            b, h, qt = pkg.work_unit(blk, heads, dims[0], dims[1], lq, lk, causal)
            if b < 0:
                continue
            assert qt == 0 and b % pack == 0
            for s_ in range(b, min(b + pack, batch)):
                assert (s_, h) not in seen
                seen[(s_, h)] = blk
            assert (b // pack * (heads >> hs) + (h >> hs)) % 8 == blk % 8
        assert set(seen) == {(b, h) for b in range(batch) for h in range(heads)}
        return
    n_qt = -(-max_q // bm)
    longest_first = batch <= 64 and len(set(zip(lq, lk))) > 1
    # causal launches of the one-workgroup-per-CU head dims: a unit runs
    # q-tile qt and then n_b - 1 - qt, so every unit has n_b + 1 key tiles
    pair = p["pair_q_tiles"] == 1
    assert pair == (bool(causal) and _expect_pairs(dims[0], dims[1], batch, heads, max_q, max(lk)))
    n_units_qt = (n_qt + 1) // 2 if pair else n_qt
    # tiles each segment must get: its own q-tiles when dealt longest first,
    # else the same number for every segment (tiles past its end exit early)
    want = {(b, h, qt) for b in range(batch) for h in range(heads)
            for qt in range(-(-lq[b] // bm) if longest_first else n_qt)}
    rank = sorted(range(batch), key=lambda i: (-lk[i], i))
    rank = {b: r for r, b in enumerate(rank)}
    seen = {}
    order = [[] for _ in range(8)]  # per XCD, owners in dispatch order
    valid = 0
    for blk in range(p["units"]):
        b, h, qt = pkg.work_unit(blk, heads, dims[0], dims[1], lq, lk, causal)
        if b < 0:
            assert h == -1 and qt == -1
            continue
        valid += 1
        tiles = [qt]
        if pair:
            nb = -(-lq[b] // bm)
            assert 2 * qt >= nb - 1  # the later tile of the two is reported
            tiles += [nb - 1 - qt] if nb - 1 - qt != qt else []
        for t in tiles:
            key = (b, h, t)
            assert key in want, key
            assert key not in seen, (blk, key, seen.get(key))
            seen[key] = blk
        order[blk % 8].append((blk >> 3, b))
        # (segment, head group) groups are dealt round-robin over the 8 XCDs
        # (block % 8); a group's 2^hs heads run on one XCD
        g = (rank[b] if longest_first else b) * (heads >> hs) + (h >> hs)
        assert g % 8 == blk % 8
    assert set(seen) == want
    if longest_first:
        # each XCD starts the segments in order of decreasing key length, up
        # to the order inside aligned quads of its dispatch index
        for owners in order:
            quads = {}
            for k, b in owners:
                quads.setdefault(k // 4, []).append(lk[b])
            ks = sorted(quads)
            assert all(min(quads[a]) >= max(quads[c]) for a, c in zip(ks, ks[1:]))
    else:
        assert p["units"] - valid < (8 * n_units_qt) << hs
    if causal and not pair:
        # within a group, one of the four q-tiles with the most keys is
        # dispatched first
        first = {}
        for (b, h, qt), blk in seen.items():
            if (b, h) not in first or blk < first[(b, h)][0]:
                first[(b, h)] = (blk, qt)
        for (b, h), (_, qt) in first.items():
            assert qt >= (-(-lq[b] // bm) if longest_first else n_qt) - 4


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads,heads_k,lq", [(64, 8, [4096, 4096]), (32, 4, [700, 900, 33]), (12, 1, [300]),
                                              (16, 16, [1000, 2000]), (24, 8, [513] * 3)])
def test_work_unit_grouped_kv_heads(heads, heads_k, lq, causal):
    """With grouped KV heads every (segment, query head, q-tile) is still owned
    once (causal: q-tiles in pairs qt, n_b - 1 - qt), and when the KV heads
    are a multiple of 8 the query heads of one KV head all run on one XCD
    (block % 8), sharing its L2."""
    p = pkg.plan(128, 128, len(lq), heads, max(lq), max(lq), int(causal))
    bm = p["block_m"]
    longest_first = len(set(lq)) > 1
    n_qt = -(-max(lq) // bm)
    assert p["pair_q_tiles"] == int(causal and _expect_pairs(128, 128, len(lq), heads, max(lq), max(lq), heads_k))
    want = {(b, h, qt) for b in range(len(lq)) for h in range(heads)
            for qt in range(-(-lq[b] // bm) if longest_first else n_qt)}
    seen, xcd_of = set(), {}
    for blk in range(p["grid"]):
        b, h, qt = pkg.work_unit(blk, heads, 128, 128, lq, lq, causal, num_heads_k=heads_k)
        if b < 0:
            continue
        tiles = [qt]
        if p["pair_q_tiles"] and 2 * qt > -(-lq[b] // bm) - 1:
            tiles.append(-(-lq[b] // bm) - 1 - qt)
        for t in tiles:
            assert (b, h, t) not in seen
            seen.add((b, h, t))
        xcd_of.setdefault((b, h // (heads // heads_k)), set()).add(blk % 8)
    assert seen == want
    if heads_k % 8 == 0:
        assert all(len(x) == 1 for x in xcd_of.values())
    with pytest.raises(ValueError):
        pkg.work_unit(0, heads, 128, 128, lq, lq, False, num_heads_k=heads_k + 1 if heads % (heads_k + 1) else 0)


@pytest.mark.parametrize("batch,heads,max_q,causal", [(4, 128, 4096, 1), (1, 16, 65536, 0), (3, 5, 700, 1)])
def test_work_unit_snake_balances_engines(batch, heads, max_q, causal):
    """The k-th workgroup of an XCD goes to shader engine (k + c) % 4; over
    every aligned run of 8 dispatch slots the four engines get equal key
    counts (each q-tile's keys, causal: (qt + 1) x 256, a pair of q-tiles
    qt and n_b - 1 - qt together: (n_b + 1) x 256)."""
    p = pkg.plan(192, 128, batch, heads, max_q, max_q, causal)
    n_b = -(-max_q // p["block_m"])
    cost = {}
    for blk in range(p["grid"]):
        b, h, qt = pkg.work_unit(blk, heads, 192, 128, [max_q] * batch, [max_q] * batch, causal)
        if b >= 0:
            cost[blk] = (qt + 1) if causal else 1
            if p["pair_q_tiles"] and 2 * qt > n_b - 1:  # and then q-tile n_b - 1 - qt
                cost[blk] += n_b - qt
    n_qt = -(-max_q // p["block_m"])
    if p["pair_q_tiles"]:
        # pairs of q-tiles: every unit but a middle one has n_b + 1 key tiles
        assert causal and all(c == n_b + 1 for c in cost.values() if c != (n_b + 1) // 2)
        n_qt = (n_qt + 1) // 2
    per_xcd = p["grid"] // 8
    for x in range(8):
        for k0 in range(0, per_xcd - per_xcd % 8, 8):
            eng = [0] * 4
            for k in range(k0, k0 + 8):
                eng[k % 4] += cost.get(8 * k + x, 0)
            if n_qt % 4 == 0 and all(8 * k + x in cost for k in range(k0, k0 + 8)):
                assert len(set(eng)) == 1, (x, k0, eng)


def test_work_unit_rejects_out_of_grid():
    p = pkg.plan(64, 64, 2, 3, 100, 100)
    with pytest.raises(ValueError):
        pkg.work_unit(p["grid"], 3, 64, 64, [100, 100], [100, 100])
    with pytest.raises(ValueError):
        pkg.work_unit(-1, 3, 64, 64, [100, 100], [100, 100])
    with pytest.raises(ValueError):
        pkg.work_unit(0, 3, 96, 96, [100, 100], [100, 100])
    with pytest.raises(ValueError):
        pkg.work_unit(0, 3, 64, 64, [100, -1], [100, 100])
    with pytest.raises(ValueError):
        pkg.work_unit(0, 3, 64, 64, [0, 0], [100, 100])

# ---------------------------------------------------------------------------
# varlen_attn_merge validation (placeholder pointers; no call below launches)
# ---------------------------------------------------------------------------
def _merge(a=None, b=None, out=None, lse_a=FAKE, lse_b=FAKE, lse=FAKE):
    a = a if a is not None else _t()
    b = b if b is not None else _t()
    out = out if out is not None else _t()
    lib = pkg.library()
    return lib.varlen_attn_merge(ctypes.byref(a), ctypes.c_void_p(lse_a), ctypes.byref(b), ctypes.c_void_p(lse_b),
                                 ctypes.byref(out), ctypes.c_void_p(lse), ctypes.c_void_p(0))


def test_splitkv_workspace_bytes():
    f = pkg.splitkv_workspace_bytes
    assert f(100, 3, 64, 1) == 0 and f(100, 3, 64, 0) == 0 and f(0, 3, 64, 4) == 0
    o = 4 * 100 * 3 * 64 * 4
    assert f(100, 3, 64, 4) == -(-o // 256) * 256 + 4 * 3 * 100 * 4
    o = 7 * 33 * 5 * 80 * 4
    assert f(33, 5, 80, 7) == -(-o // 256) * 256 + 7 * 5 * 33 * 4


def _split_call(num_splits, ws=FAKE, nbytes=1 << 30):
    t = _t()
    return B.raw_fwd_splitkv(t, t, t, FAKE, FAKE, 1, 10, 10, 0.125, 0, -1, -1, t, 0, num_splits, ws, nbytes, 0)


def test_splitkv_rejects_bad_arguments():
    assert _split_call(0) == B.VA_ERR_ARG
    assert _split_call(129) == B.VA_ERR_ARG
    assert _split_call(4, ws=0) == B.VA_ERR_NULL
    assert _split_call(4, ws=FAKE + 16) == B.VA_ERR_ALIGN
    assert _split_call(4, nbytes=pkg.splitkv_workspace_bytes(10, 2, 64, 4) - 1) == B.VA_ERR_ARG
    # the plain checks run first
    t = _t()
    assert B.raw_fwd_splitkv(t, _t(dim=80), t, FAKE, FAKE, 1, 10, 10, 0.125, 0, -1, -1, t, 0, 4, FAKE, 1 << 30,
                             0) == B.VA_ERR_SHAPE


def test_noalloc_validation_before_any_device_call():
    """The allocation-free split-KV entry point runs the plain checks, then
    rejects partials larger than its scratch array (VA_ERR_SCRATCH), all
    before any HIP call; one split needs no scratch."""
    assert pkg.scratch_bytes() == 64 << 20
    t = _t()
    call = lambda q, out, splits, batch=1: B.raw_fwd_splitkv_noalloc(
        q, t, t, FAKE, FAKE, batch, 10, 10, 0.125, 0, -1, -1, out, 0, splits, 0)
    assert call(t, t, 0) == B.VA_ERR_ARG
    assert call(t, t, 129) == B.VA_ERR_ARG
    assert call(_t(dim=80), t, 4) == B.VA_ERR_SHAPE
    big_q = _t(rows=1 << 16, heads=2, dim=64)
    big_o = _t(rows=1 << 16, heads=2, dim=64)
    assert pkg.splitkv_workspace_bytes(1 << 16, 2, 64, 2) > pkg.scratch_bytes()
    assert call(big_q, big_o, 2) == B.VA_ERR_SCRATCH
    assert call(big_q, big_o, 2, batch=0) == B.VA_OK  # nothing to launch


def test_auto_num_splits():
    n = pkg.auto_num_splits(128, 128, 1, 16, 512, 32768)
    assert 1 <= n <= 128
    assert pkg.auto_num_splits(128, 128, 0, 16, 512, 32768) == 1
    assert 1 <= pkg.auto_num_splits(128, 128, 1, 32, 64, 32768, num_heads_k=4) <= 128
    assert 1 <= pkg.auto_num_splits(192, 128, 1, 16, 512, 32768, fp8=True) <= 128
    with pytest.raises(ValueError):
        pkg.auto_num_splits(96, 96, 1, 16, 512, 32768)
    with pytest.raises(ValueError):
        pkg.auto_num_splits(80, 80, 1, 16, 512, 32768, fp8=True)  # no fp8 kernel at d 80
    with pytest.raises(ValueError):
        pkg.auto_num_splits(128, 128, 1, 16, 512, 32768, num_heads_k=3)  # 16 heads over 3 KV heads


def test_merge_rejects_bad_arguments():
    lib = pkg.library()
    t = _t()
    assert lib.varlen_attn_merge(None, FAKE, ctypes.byref(t), FAKE, ctypes.byref(t), FAKE, None) == B.VA_ERR_NULL
    assert _merge(lse_a=0) == B.VA_ERR_NULL
    assert _merge(lse_b=0) == B.VA_ERR_NULL
    assert _merge(b=_t(rows=9)) == B.VA_ERR_SHAPE
    assert _merge(out=_t(heads=3)) == B.VA_ERR_SHAPE
    assert _merge(b=_t(dim=80)) == B.VA_ERR_SHAPE
    assert _merge(a=_t(dim=4), b=_t(dim=4), out=_t(dim=4)) == B.VA_ERR_SHAPE     # below 8
    assert _merge(a=_t(dim=12), b=_t(dim=12), out=_t(dim=12)) == B.VA_ERR_SHAPE  # not a multiple of 8
    assert _merge(a=_t(dim=264), b=_t(dim=264), out=_t(dim=264)) == B.VA_ERR_SHAPE
    assert _merge(a=_t(row_stride=0)) == B.VA_ERR_STRIDE
    assert _merge(out=_t(head_stride=-64)) == B.VA_ERR_STRIDE
    assert _merge(b=_t(row_stride=132)) == B.VA_ERR_ALIGN
    assert _merge(out=_t(data=FAKE + 8)) == B.VA_ERR_ALIGN
    assert _merge(a=_t(data=0)) == B.VA_ERR_NULL
    assert _merge(lse=FAKE + 2) == B.VA_ERR_ALIGN


def test_merge_of_no_rows_launches_nothing():
    z = _t(rows=0, data=0)
    assert _merge(a=z, b=z, out=z, lse_a=0, lse_b=0, lse=0) == B.VA_OK


# ---------------------------------------------------------------------------
# fp8 entry point: validation only (every call fails or returns before launching)
# ---------------------------------------------------------------------------
def _call_fp8(q=None, k=None, v=None, out=None, dq=0, dk=0, dv=0, out_scale=0, batch=1, mq=10, mk=10,
              splits=1, ws=0, ws_bytes=0, lse=0):
    q = q if q is not None else _t(dim=128, row_stride=256, head_stride=128)
    k = k if k is not None else _t(dim=128, row_stride=256, head_stride=128)
    v = v if v is not None else _t(dim=128, row_stride=256, head_stride=128)
    out = out if out is not None else _t(dim=128, row_stride=256, head_stride=128)
    return B.raw_fwd_fp8(q, k, v, dq, dk, dv, FAKE, FAKE, batch, mq, mk, 0.1, 0, -1, -1, out, out_scale, lse,
                         splits, ws, ws_bytes, 0)


def test_fp8_head_dims():
    # (64,64), (128,128), (192,128) only: the fp8 MFMA takes 64 head dims at a time
    for d in (72, 80):
        t = _t(dim=d, row_stride=2 * d, head_stride=d)
        assert _call_fp8(q=t, k=t, v=t, out=t) == B.VA_ERR_HEADDIM


def test_fp8_alignment_is_in_bytes():
    # one byte per element: strides must be multiples of 16 elements (bf16 output: 8)
    assert _call_fp8(q=_t(dim=128, row_stride=264, head_stride=128)) == B.VA_ERR_ALIGN
    assert _call_fp8(k=_t(dim=128, row_stride=256, head_stride=136)) == B.VA_ERR_ALIGN
    assert _call_fp8(dq=FAKE + 2) == B.VA_ERR_ALIGN
    assert _call_fp8(dv=FAKE + 1) == B.VA_ERR_ALIGN
    assert _call_fp8(out_scale=FAKE + 3) == B.VA_ERR_ALIGN


def test_fp8_scalar_arguments():
    assert _call_fp8(splits=0) == B.VA_ERR_ARG
    assert _call_fp8(splits=129) == B.VA_ERR_ARG
    assert _call_fp8(out_scale=FAKE, splits=2) == B.VA_ERR_NULL  # e4m3 output with splits: needs a workspace
    assert _call_fp8(splits=2, ws=0) == B.VA_ERR_NULL
    assert _call_fp8(splits=2, ws=FAKE + 16, ws_bytes=1 << 30) == B.VA_ERR_ALIGN
    assert _call_fp8(splits=2, ws=FAKE, ws_bytes=16) == B.VA_ERR_ARG


def test_fp8_empty_work_returns_ok_without_launch():
    assert _call_fp8(batch=0) == B.VA_OK
    assert _call_fp8(mq=0) == B.VA_OK


@pytest.mark.parametrize("heads,heads_k,lq,pack", [
    (32, 4, [64, 1, 0, 50, 64], 4),      # group 8, <= 64 queries: four query heads a workgroup
    (16, 4, [33, 64], 4),                # group 4
    (12, 3, [100, 128, 65], 2),          # group 4, <= 128 queries: two query heads, two waves each
    (16, 8, [128, 7], 2),                # group 2
])
def test_work_unit_head_packing(heads, heads_k, lq, pack):
    """Grouped KV heads with short segments: a workgroup takes `pack` query
    heads of one KV head over one segment (FA4's pack_gqa), every (segment,
    query head) owned once, and a KV head's groups stay on one XCD when the
    KV heads are a multiple of 8 (here: by construction of the dealing)."""
    p = pkg.plan(128, 128, len(lq), heads, max(lq), max(lq), 0, num_heads_k=heads_k)
    assert p["segments_per_block"] == pack and p["pack_mode"] == 2
    grp = heads // heads_k
    seen = set()
    for blk in range(p["grid"]):
        b, h, qt = pkg.work_unit(blk, heads, 128, 128, lq, lq, False, num_heads_k=heads_k)
        if b < 0:
            continue
        assert qt == 0 and h % pack == 0 and h // grp == (h + pack - 1) // grp
        for x in range(h, h + pack):
            assert (b, x) not in seen
            seen.add((b, x))
    assert seen == {(b, h) for b in range(len(lq)) for h in range(heads)}


@pytest.mark.parametrize("heads,heads_k,max_q,mode", [
    (32, 4, 64, 2), (32, 4, 65, 2), (32, 4, 129, 0),   # head packing up to 128 queries, then none
    (6, 3, 64, 1),                                     # group 2 is not a multiple of 4: segments
    (6, 3, 100, 2),                                    # but of 2
    (8, 8, 64, 1), (9, 3, 64, 1),                      # no grouping / group 3: segments
])
def test_pack_mode_choice(heads, heads_k, max_q, mode):
    """bf16 segments of at most 64 queries that would be packed by segment
    take the one-wave short-segment kernel instead (no packing, pack_mode 0)
    where the head dims have it (<= 80); fp8 and d 128 keep the packing."""
    short = mode == 1 and max_q <= 64
    # unpacked and too small for the CUs (5 x heads units of 256 rows < 256):
    # four waves split each 64-row block's keys on the short-segment kernel
    ksplit = mode in (0, 1) and max_q > 64 and 8 * -(-5 * heads // 8) * -(-max_q // 64) <= 512
    p = pkg.plan(64, 64, 5, heads, max_q, max_q, 0, num_heads_k=heads_k)
    assert p["pack_mode"] == (0 if short else mode)
    assert p["kernel"] == ("attn_fwd_short" if short or ksplit else "attn_fwd_wide")
    assert p["key_split"] == (4 if ksplit else 1)
    assert pkg.plan(128, 128, 5, heads, max_q, max_q, 0, num_heads_k=heads_k)["pack_mode"] == mode
    assert pkg.plan(64, 64, 5, heads, max_q, max_q, 0, fp8=True, num_heads_k=heads_k)["pack_mode"] == mode


def _call_quant(out=None, out_scale=FAKE, lse=0, batch=1):
    lib = pkg.library()
    t = _t()
    out = out if out is not None else _t(row_stride=128, head_stride=64)
    return lib.varlen_attn_fwd_quant_out(ctypes.byref(t), ctypes.byref(t), ctypes.byref(t), ctypes.c_void_p(FAKE),
                                         ctypes.c_void_p(FAKE), batch, 10, 10, ctypes.c_float(0.125), 0, -1, -1,
                                         ctypes.byref(out), ctypes.c_void_p(out_scale), ctypes.c_void_p(lse), None)


def test_quant_out_validation():
    assert _call_quant(out_scale=0) == B.VA_ERR_NULL
    assert _call_quant(out_scale=FAKE + 2) == B.VA_ERR_ALIGN
    # the e4m3 output's strides count bytes and are written 8 bytes at a
    # time: multiples of 8 pass (a contiguous d_v 72 head), others do not
    assert _call_quant(out=_t(row_stride=132, head_stride=64)) == B.VA_ERR_ALIGN
    assert _call_quant(out=_t(row_stride=128, head_stride=68)) == B.VA_ERR_ALIGN
    assert _call_quant(out=_t(data=FAKE + 4)) == B.VA_ERR_ALIGN
    # (batch 0: every check runs, nothing is launched)
    assert _call_quant(out=_t(row_stride=144, head_stride=72, data=FAKE + 8), batch=0) == B.VA_OK
    assert _call_quant(out=_t(row_stride=144, head_stride=72, data=FAKE + 4), batch=0) == B.VA_ERR_ALIGN


@pytest.mark.parametrize("dims,lds_kib", [((64, 64), 55), ((128, 128), 103), ((192, 128), 127)])
def test_plan_fp8(dims, lds_kib):
    """The fp8 kernel: 256-row workgroups of 4 waves, 64-key tiles (one fp8
    PV MFMA takes 64 keys), six LDS stages of K (plus a pad chunk a row) and
    V bytes; the grid is the bf16 kernel's (same work units), save where the
    bf16 kernel pairs causal q-tiles (not here: 48 pairs an XCD would fill
    3/4 of their second round); the fp8 kernel never does."""
    p8 = pkg.plan(dims[0], dims[1], 3, 16, 4096, 4096, 1, fp8=True)
    p16 = pkg.plan(dims[0], dims[1], 3, 16, 4096, 4096, 1)
    assert p8["kernel"] == "attn_fwd_fp8" and p8["block_n"] == 64 and p8["block_m"] == 256
    assert p16["pair_q_tiles"] == _expect_pairs(dims[0], dims[1], 3, 16, 4096, 4096) and p8["pair_q_tiles"] == 0
    assert p8["threads"] == 256 and p8["grid"] == p16["grid"] * (2 if p16["pair_q_tiles"] else 1)
    assert p8["lds_bytes"] // 1024 == lds_kib and p8["lds_bytes"] <= 160 * 1024
    with pytest.raises(ValueError):
        pkg.plan(80, 80, 1, 16, 64, 64, 0, fp8=True)  # d 80 has no fp8 instantiation


def _fastdiv(d):
    """The multiplier and shift the kernel's FastDiv uses (tile_schedule.h)."""
    s = 0
    while (1 << s) < d:
        s += 1
    m = ((1 << (32 + s)) + d - 1) // d
    return m - (1 << 32), s


@pytest.mark.parametrize("d", list(range(1, 300)) + [511, 512, 513, 1000, 4095, 4096, 65535, 65536, 65537,
                                                         (1 << 20) + 3, (1 << 30) + 1, (1 << 31) - 1])
def test_fastdiv_is_exact(d):
    """floor(n / d) = (umulhi(n, mul) + n) >> shift for every numerator the
    kernel divides (0 <= n < 2^31): checked at the divisor's multiples and
    their neighbours, the top of the range and random numerators."""
    mul, s = _fastdiv(d)
    assert 0 <= mul < (1 << 32)
    rng = random.Random(d)
    ns = {0, 1, (1 << 31) - 1, (1 << 31) - 2}
    for q in list(range(0, 70)) + [((1 << 31) - 1) // d - i for i in range(3)] + [rng.randrange(0, (1 << 31) // d)
                                                                                  for _ in range(50)]:
        for r in (-1, 0, 1, d - 1):
            n = q * d + r
            if 0 <= n < (1 << 31):
                ns.add(n)
    ns.update(rng.randrange(0, 1 << 31) for _ in range(200))
    for n in ns:
        t = (n * mul) >> 32
        assert t + n < (1 << 32)
        assert (t + n) >> s == n // d, (n, d)


def test_dynamic_split_counts_validation():
    """Per-segment split counts: a misaligned counts pointer is refused by
    the split-KV entry points, and the device count helper checks its
    arguments before launching anything (batch 0 launches nothing)."""
    t = _t()
    assert B.raw_fwd_splitkv(t, t, t, FAKE, FAKE, 1, 10, 10, 0.125, 0, -1, -1, t, 0, 4, FAKE, 1 << 30, 0,
                             splits_dyn_ptr=FAKE + 2) == B.VA_ERR_ALIGN
    lib = pkg.library()
    counts = lambda cu, batch, mx, kps, out: lib.varlen_attn_splitkv_counts(
        ctypes.c_void_p(cu), batch, mx, kps, ctypes.c_void_p(out), None)
    assert counts(FAKE, -1, 4, 512, FAKE) == B.VA_ERR_ARG
    assert counts(FAKE, 3, 0, 512, FAKE) == B.VA_ERR_ARG
    assert counts(FAKE, 3, 129, 512, FAKE) == B.VA_ERR_ARG
    assert counts(FAKE, 3, 4, 0, FAKE) == B.VA_ERR_ARG
    assert counts(0, 3, 4, 512, FAKE) == B.VA_ERR_NULL
    assert counts(FAKE, 3, 4, 512, 0) == B.VA_ERR_NULL
    assert counts(FAKE + 2, 3, 4, 512, FAKE) == B.VA_ERR_ALIGN
    assert counts(FAKE, 3, 4, 512, FAKE + 1) == B.VA_ERR_ALIGN
    assert counts(0, 0, 4, 512, 0) == B.VA_OK
