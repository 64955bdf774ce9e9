"""GPU parity of the fp8 e4m3 path (``varlen_attn_fwd_fp8``) against the fp64
oracle on the dequantised inputs (marked ``gpu``).

Tolerance, derived from the kernel's arithmetic.  The scores come from exact
e4m3 products accumulated by the fp8 MFMA (at less than fp32 precision, see
ds below) and the LSE from the fp32 sum of the unrounded probabilities, so
|dLSE| <= 1e-3 + ds per row.  O differs
from the exact result by the e4m3 rounding of each probability before the
PV product: a normal p is off by at most 2^-4 p (half an ulp of a 3-bit
mantissa), a subnormal one by at most 2^-10, both measured against the row's
true maximum (the running max a tile was scaled by never exceeds it).  So,
per output element d of a row with probabilities p_j = exp(s_j - max) over
its visible keys, l = sum p_j and dequantised values v_jd:

    |dO_d| <= (2^-4 sum_j p_j |v_jd| + 2^-10 sum_j |v_jd|) / l
              + 2^-8 |O_d|           (bf16 rounding of O, with margin)
              + 1e-3 sum_j p_j |v_jd| / l + 1e-5   (fp32 arithmetic)
              + 2 ds (sum_j p_j |v_jd| / l + |O_d|)

checked element by element, where ds bounds the error of every score of the
row: the fp8 MFMA accumulates its 64 products with less than fp32 precision,
taken as ds = 2^-15 scale max_j sum_i |q_i k_ji| over the row's visible keys
(``test_fp8_score_error_single_key`` pins that constant: with one key the
LSE is the score itself, so its error is the dot product's); a score error ds moves each p (and l) by a
factor within e^(+-ds).  For the same reason |dLSE| <= 1e-3 + ds per row
(the LSE moves by at most the largest score error).  With an e4m3 output the decoded code times
out_scale may in addition be off by half an e4m3 ulp of O / out_scale.

A call without an LSE runs the same arithmetic (the fp32 row sum is kept):
its O is bit-identical to the call that returns one.

Integer-exact checks: descales None equal descales of ones bit for bit, and
halving softmax_scale while doubling every q descale gives the same bits (an
exact power-of-two change of the fp32 score scale).
"""
import zlib

import numpy as np
import pytest
import torch

import varlen_attention_forward_amd as va
from varlen_attention_forward_amd import workloads
from helpers import f64
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_LSE = 1e-3
DIMS = [(64, 64), (128, 128), (192, 128)]
LEN_SETS = {
    "ragged": ([1, 63, 64, 65, 127, 128, 129, 255, 256, 257], None),
    "q_lt_k": ([1, 40, 64, 100, 129], [70, 64, 200, 100, 300]),
    "empty_segments": ([0, 37, 0, 190, 5], [0, 0, 50, 190, 0]),
}
MODES = {
    "full": (False, (-1, -1)),
    "causal": (True, (-1, -1)),
    "window": (False, (40, 17)),
    "causal_window": (True, (70, -1)),
}


def u8(t):
    return t.detach().cpu().view(torch.uint8).numpy()


def make(lens_q, lens_k, dims, seed, mode="full", heads=4, heads_k=None, std=1.0):
    causal, window = MODES[mode]
    return workloads.make_fp8_inputs(lens_q, lens_k if lens_k is not None else lens_q, heads, dims[0], dims[1],
                                     seed, causal=causal, window=window, num_heads_k=heads_k, std=std)


def run_fp8(inp, out_scale=None, num_splits=1, return_lse=True, descales=True, scale=None, q_descale=None):
    d = inp.to(DEV)
    lse = None
    if return_lse:
        lse = torch.full((inp.q.shape[1], inp.q.shape[0]), float("nan"), dtype=torch.float32, device=DEV)
    os_t = None if out_scale is None else torch.tensor([out_scale], dtype=torch.float32, device=DEV)
    qd = d.q_descale if q_descale is None else q_descale.to(DEV)
    res = va.varlen_attn_fwd_fp8(
        d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, inp.max_seqlen_q, inp.max_seqlen_k,
        softmax_scale=inp.softmax_scale if scale is None else scale, causal=inp.causal, window_size=inp.window,
        q_descale=qd if descales else None, k_descale=d.k_descale if descales else None,
        v_descale=d.v_descale if descales else None, out_scale=os_t, return_lse=return_lse, lse=lse,
        num_splits=num_splits,
    )
    torch.cuda.synchronize()
    return res if return_lse else (res, None)


def oracle_fp8(inp, rows=None, heads=None):
    wl, wr = inp.window
    return oracle.attention_fwd_fp8(
        u8(inp.q), u8(inp.k), u8(inp.v), inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist(), inp.softmax_scale,
        causal=inp.causal, window_left=wl, window_right=wr, q_descale=inp.q_descale.numpy(),
        k_descale=inp.k_descale.numpy(), v_descale=inp.v_descale.numpy(), rows=rows, heads=heads,
    )


def o_tolerance(inp, rows=None, heads=None, want_ds=False):
    """The per-element bound of the module docstring, NaN off the requested rows."""
    H, H_kv = inp.q.shape[1], inp.k.shape[1]
    grp = H // H_kv
    cq, ck = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
    qc, kc, vc = u8(inp.q), u8(inp.k), u8(inp.v)
    qdesc = np.repeat(inp.q_descale.numpy(), grp, axis=1)
    head_list = list(range(H)) if heads is None else list(heads)
    # dequantised per head (whole-tensor float64 copies would not fit at full sizes)
    qd = {h: oracle.dequantize(qc, cq, qdesc, heads=[h])[:, 0, :] for h in head_list}
    kd = {hk: oracle.dequantize(kc, ck, inp.k_descale.numpy(), heads=[hk])[:, 0, :]
          for hk in {h // grp for h in head_list}}
    vd = {hk: oracle.dequantize(vc, ck, inp.v_descale.numpy(), heads=[hk])[:, 0, :] for hk in kd}
    scale = float(np.float32(inp.softmax_scale))
    wl, wr = inp.window
    tol = np.full((inp.q.shape[0], H, inp.v.shape[2]), np.nan)
    dsr = np.full((H, inp.q.shape[0]), np.nan)  # score error bound per (head, row)
    want = None
    if rows is not None:
        want = np.zeros(inp.q.shape[0], dtype=bool)
        want[np.asarray(rows)] = True
    for b in range(len(cq) - 1):
        Lq, Lk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        idx = np.arange(Lq)
        if want is not None:
            idx = idx[want[cq[b]:cq[b + 1]]]
        if len(idx) == 0:
            continue
        lo, hi = oracle.visible_interval(idx, Lq, Lk, inp.causal, wl, wr)
        j = np.arange(Lk)[None, :]
        vis = (j >= lo[:, None]) & (j <= hi[:, None])
        for h in head_list:
            hk = h // grp
            s = scale * (qd[h][cq[b] + idx, :] @ kd[hk][ck[b]:ck[b + 1], :].T)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1) if Lk else np.full(len(idx), -np.inf)
            ok = np.isfinite(m)
            p = np.exp(s - np.where(ok, m, 0.0)[:, None])
            l = np.where(ok, p.sum(axis=1), 1.0)[:, None]
            av = np.abs(vd[hk][ck[b]:ck[b + 1], :])
            a = (p @ av) / l
            o = np.abs(p @ vd[hk][ck[b]:ck[b + 1], :]) / l
            c = (vis.astype(np.float64) @ av) / l
            absdot = scale * (np.abs(qd[h][cq[b] + idx, :]) @ np.abs(kd[hk][ck[b]:ck[b + 1], :]).T)
            ds = 2.0 ** -15 * np.where(vis, absdot, 0.0).max(axis=1) if Lk else np.zeros(len(idx))
            dsr[h, cq[b] + idx] = ds
            tol[cq[b] + idx, h, :] = (2.0 ** -4 * a + 2.0 ** -10 * c + 2.0 ** -8 * o + 1e-3 * a + 1e-5
                                      + 2.0 * ds[:, None] * (a + o))
    if want_ds:
        return tol, dsr
    return tol


def assert_fp8_parity(inp, out, lse, rows=None, heads=None, what=""):
    ref_o, ref_lse = oracle_fp8(inp, rows=rows, heads=heads)
    tol, dsr = o_tolerance(inp, rows=rows, heads=heads, want_ds=True)
    o = f64(out)
    sel = ~np.isnan(ref_o)
    assert np.all(np.isfinite(tol[sel])), "%s: the bound is not finite where it is checked" % what
    assert np.all(np.isfinite(o[sel])), "%s: non-finite output" % what
    err = np.abs(o - ref_o)
    bad = sel & (err > tol)
    assert not bad.any(), "%s: %d elements over the bound, worst excess %.3e (err %.3e)" % (
        what, int(bad.sum()), float(np.max((err - tol)[bad])), float(np.max(err[bad])))
    worst = float(np.max(err[sel])) if sel.any() else 0.0
    if lse is not None:
        l = f64(lse)
        lsel = ~np.isnan(ref_lse)
        neg = lsel & (ref_lse == -np.inf)
        assert np.array_equal(l[lsel] == -np.inf, neg[lsel]), "%s: -inf LSE rows differ" % what
        fin = lsel & ~neg
        assert np.all(np.isfinite(dsr[fin])), "%s: score-error bound not finite" % what
        with np.errstate(invalid="ignore"):  # -inf - -inf off the checked rows
            excess = (np.abs(l - ref_lse) - (TOL_LSE + dsr))[fin]
        assert not (excess > 0).any(), "%s: LSE over 1e-3 + ds by up to %.3e" % (what, float(np.max(excess)))
    return worst


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("lens", list(LEN_SETS))
def test_fp8_small_parity(dims, mode, lens):
    lq, lk = LEN_SETS[lens]
    inp = make(lq, lk, dims, seed=zlib.crc32(("%s %s %s" % (dims, mode, lens)).encode()) % 10000, mode=mode)
    out, lse = run_fp8(inp)
    assert out.dtype == torch.bfloat16
    assert_fp8_parity(inp, out, lse, what="%s %s %s" % (dims, mode, lens))
    out2, _ = run_fp8(inp, return_lse=False)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", ["causal", "causal_window"])
@pytest.mark.parametrize("order", ["longest_first", "packing_order"])
def test_fp8_causal_multi_tile_segments(dims, mode, order):
    """Causal segments of many q-tiles (odd and even counts, one-tile and
    empty segments, a ragged last tile, Lq != Lk), dealt longest first and in
    packing order; the e4m3 kernel runs one q-tile a workgroup."""
    if order == "longest_first":
        lq = [1029, 512, 40, 700, 513, 1280, 1, 0]
        lk = [1029, 600, 333, 901, 513, 1280, 1, 0]
    else:
        rng = np.random.default_rng(dims[0] + 1)
        lq = [int(x) for x in rng.integers(0, 1100, 70)]
        lq[0], lq[1], lq[2] = 1100, 256, 257
        lk = [x if i % 4 else x + int(rng.integers(0, 200)) for i, x in enumerate(lq)]
    assert va.plan(dims[0], dims[1], len(lq), 2, max(lq), max(lk), 1, fp8=True)["pair_q_tiles"] == 0
    inp = make(lq, lk, dims, seed=zlib.crc32(("multi %s %s %s" % (dims, mode, order)).encode()) % 10000,
               mode=mode, heads=2)
    out, lse = run_fp8(inp)
    assert_fp8_parity(inp, out, lse, what="multi %s %s %s" % (dims, mode, order))


@pytest.mark.parametrize("dims", [(128, 128), (192, 128)], ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("heads,heads_k", [(8, 1), (8, 2), (6, 3)])
@pytest.mark.parametrize("mode", ["full", "causal"])
def test_fp8_grouped_kv_heads(dims, heads, heads_k, mode):
    inp = make([100, 300, 17], [260, 300, 80], dims, seed=heads * 7 + heads_k, mode=mode, heads=heads,
               heads_k=heads_k)
    out, lse = run_fp8(inp)
    assert_fp8_parity(inp, out, lse, what="gqa %s %d/%d %s" % (dims, heads, heads_k, mode))


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("lens", ["le64", "le128"])
@pytest.mark.parametrize("mode", ["full", "causal"])
def test_fp8_packed_short_segments(dims, lens, mode):
    g = np.random.default_rng(len(lens) + dims[0])
    hi = 64 if lens == "le64" else 128
    lq = g.integers(0, hi + 1, 23).tolist()
    if mode == "causal":
        lk = [x + int(g.integers(0, 30)) for x in lq]
    else:
        lk = [int(g.integers(0, 200)) for _ in lq]
    inp = make(lq, lk, dims, seed=hi + dims[0], mode=mode, heads=4)
    assert va.plan(dims[0], dims[1], len(lq), 4, max(lq), max(lk), fp8=True)["segments_per_block"] > 1
    out, lse = run_fp8(inp)
    assert_fp8_parity(inp, out, lse, what="packed %s %s %s" % (dims, lens, mode))
    out2, _ = run_fp8(inp, return_lse=False)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("splits", [2, 5])
@pytest.mark.parametrize("mode", ["full", "causal"])
def test_fp8_split_kv(dims, splits, mode):
    inp = make([64, 300, 1], [2000, 900, 700], dims, seed=splits * 13 + dims[0], mode=mode, heads=4)
    out, lse = run_fp8(inp, num_splits=splits)
    assert_fp8_parity(inp, out, lse, what="split %s %d %s" % (dims, splits, mode))


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", ["full", "causal"])
def test_fp8_output_quantisation(dims, mode):
    inp = make([64, 129, 255], None, dims, seed=dims[0] + 3, mode=mode, heads=4)
    ref_o, _ = oracle_fp8(inp)
    s = float(np.float32(np.nanmax(np.abs(ref_o)) / 200.0))
    out, lse = run_fp8(inp, out_scale=s)
    assert out.dtype == torch.float8_e4m3fn
    got = oracle.e4m3_decode(u8(out)) * s
    tol = o_tolerance(inp)
    y = np.abs(ref_o) / s + tol / s
    half_ulp = s * np.maximum(2.0 ** -4 * y, 2.0 ** -10)
    sel = ~np.isnan(ref_o)
    err = np.abs(got - ref_o)
    assert not (sel & (err > tol + half_ulp)).any(), "max excess %.3e" % float(np.max((err - tol - half_ulp)[sel]))
    # the LSE does not depend on the output format
    _, lse2 = run_fp8(inp)
    assert torch.equal(lse, lse2)


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
def test_fp8_output_quantisation_with_split_kv(dims):
    """With split-KV the combine kernel writes the e4m3 codes: within the
    parity bound plus half an e4m3 ulp of the oracle.  (Not compared code for
    code with the unsplit call: each split rounds its probabilities to e4m3
    relative to its own running max, so the two O differ by that rounding,
    inside the bound, not by fp32 rounding alone.)  The LSE matches the
    unsplit call's."""
    inp = make([64, 300, 1], [2000, 900, 700], dims, seed=dims[0] + 9, mode="causal")
    ref_o, _ = oracle_fp8(inp)
    s = float(np.float32(np.nanmax(np.abs(ref_o)) / 200.0))
    out, lse = run_fp8(inp, out_scale=s, num_splits=3)
    got = oracle.e4m3_decode(u8(out)) * s
    tol = o_tolerance(inp)
    half_ulp = s * np.maximum(2.0 ** -4 * (np.abs(ref_o) + tol) / s, 2.0 ** -10)
    sel = ~np.isnan(ref_o)
    assert not (sel & (np.abs(got - ref_o) > tol + half_ulp)).any()
    _, lse1 = run_fp8(inp, out_scale=s)
    np.testing.assert_allclose(f64(lse), f64(lse1), rtol=0, atol=5e-5)


def test_fp8_descales_none_are_ones_bit_exact():
    inp = make([100, 257], [300, 257], (128, 128), seed=21, mode="causal")
    ones = dataclass_with_unit_descales(inp)
    a, la = run_fp8(inp, descales=False)
    b, lb = run_fp8(ones)
    assert torch.equal(a, b) and torch.equal(la, lb)


def dataclass_with_unit_descales(inp):
    import dataclasses

    one = torch.ones_like(inp.q_descale)
    return dataclasses.replace(inp, q_descale=one, k_descale=one.clone(), v_descale=one.clone())


@pytest.mark.parametrize("dims", [(128, 128), (192, 128)], ids=lambda d: "d%d_%d" % d)
def test_fp8_power_of_two_rescale_is_bit_exact(dims):
    inp = make([77, 300], [200, 300], dims, seed=22, mode="causal")
    a, la = run_fp8(inp)
    b, lb = run_fp8(inp, scale=inp.softmax_scale / 2, q_descale=inp.q_descale * 2)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_fp8_rows_outside_segments_untouched():
    inp = make([0, 50, 0, 70], [10, 50, 0, 90], (128, 128), seed=23)
    d = inp.to(DEV)
    total = inp.q.shape[0]
    out = torch.full((total + 5, 4, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    cu_q = torch.tensor([2, 2, 52, 52, 122], dtype=torch.int32, device=DEV)  # rows 0, 1 belong to no segment
    q = torch.zeros((total + 5, 4, 128), dtype=torch.float8_e4m3fn, device=DEV)
    q[2:2 + total] = d.q
    va.varlen_attn_fwd_fp8(q, d.k, d.v, cu_q, d.cu_seqlens_k, inp.max_seqlen_q, inp.max_seqlen_k,
                           q_descale=d.q_descale, k_descale=d.k_descale, v_descale=d.v_descale, out=out)
    torch.cuda.synchronize()
    assert bool((out[:2] == 7.0).all()) and bool((out[2 + total:] == 7.0).all())


def test_fp8_empty_and_zero_key_segments():
    inp = make([0, 5, 3], [0, 0, 9], (64, 64), seed=24)
    out, lse = run_fp8(inp)
    assert bool((out[:5] == 0).all())
    assert bool(torch.isinf(lse[:, :5]).all())
    assert_fp8_parity(inp, out, lse, what="zero keys")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["vit_long65536_d128_fp8", "mla_causal_192_128_fp8"])
def test_fp8_workload_sampled(name):
    """Full-size fp8 workloads in the launch bench.py times, checked on sampled
    rows (each segment's first and last rows and random ones) of three heads."""
    w = workloads.WORKLOADS[name]
    inp = workloads.workload_inputs(w)
    out, lse = run_fp8(inp, return_lse=w.return_lse)
    cq = inp.cu_seqlens_q.tolist()
    g = np.random.default_rng(7)
    rows = set(g.integers(0, w.total_q, 40).tolist())
    for b in range(len(cq) - 1):
        if cq[b + 1] > cq[b]:
            rows |= {cq[b], cq[b + 1] - 1, (cq[b] + cq[b + 1]) // 2}
    rows = np.array(sorted(rows))
    heads = [0, w.num_heads // 2 + 1, w.num_heads - 1]
    assert_fp8_parity(inp, out, lse, rows=rows, heads=heads, what=name)


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("heads,heads_k,hi", [(32, 4, 64), (12, 3, 128)])
@pytest.mark.parametrize("mode", ["full", "causal"])
def test_fp8_packed_query_heads(dims, heads, heads_k, hi, mode):
    import dataclasses

    g = np.random.default_rng(heads + hi + dims[0])
    lq = g.integers(0, hi + 1, 9).tolist()
    lq[0] = hi
    lk = [x + int(g.integers(0, 300)) for x in lq]
    inp = make(lq, lk, dims, seed=heads * 3 + hi, mode=mode, heads=heads, heads_k=heads_k)
    assert va.plan(dims[0], dims[1], len(lq), heads, hi, max(lk), fp8=True, num_heads_k=heads_k)["pack_mode"] == 2
    out, lse = run_fp8(inp)
    assert_fp8_parity(inp, out, lse, what="fp8 packed heads %s %d/%d %d %s" % (dims, heads, heads_k, hi, mode))
    out2, lse2 = run_fp8(dataclasses.replace(inp, max_seqlen_q=257))
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("splits", [1, 3])
def test_fp8_hip_graph_replay_matches_eager(splits):
    """The fp8 call (with split-KV: two kernels, workspace allocated before
    capture) replays from a HIP graph bit-equal to the eager call, three times
    with eager work in between."""
    inp = make([300, 77, 1029], [300, 500, 1029], (128, 128), seed=25, mode="causal", heads=2)
    d = inp.to(DEV)
    nbytes = va.splitkv_workspace_bytes(inp.q.shape[0], 2, 128, splits)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)

    def call(out, lse):
        st = va.raw_fwd_fp8(
            va._binding._desc(d.q, "q", torch.float8_e4m3fn), va._binding._desc(d.k, "k", torch.float8_e4m3fn),
            va._binding._desc(d.v, "v", torch.float8_e4m3fn), d.q_descale.data_ptr(), d.k_descale.data_ptr(),
            d.v_descale.data_ptr(), d.cu_seqlens_q.data_ptr(), d.cu_seqlens_k.data_ptr(), 3, d.max_seqlen_q,
            d.max_seqlen_k, d.softmax_scale, 1, -1, -1, va._binding._desc(out, "out"), 0, lse.data_ptr(), splits,
            ws.data_ptr() if splits > 1 else 0, nbytes, torch.cuda.current_stream().cuda_stream)
        assert st == 0

    shape_o, shape_l = (d.q.shape[0], 2, 128), (2, d.q.shape[0])
    out_e = torch.empty(shape_o, dtype=torch.bfloat16, device=DEV)
    lse_e = torch.empty(shape_l, dtype=torch.float32, device=DEV)
    call(out_e, lse_e)
    out_g = torch.zeros(shape_o, dtype=torch.bfloat16, device=DEV)
    lse_g = torch.zeros(shape_l, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out_g, lse_g)
    for _ in range(3):
        out_g.zero_()
        lse_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e)
        call(torch.empty_like(out_e), torch.empty_like(lse_e))
        torch.cuda.synchronize()
    assert_fp8_parity(inp, out_g, lse_g, what="fp8 graph replay")


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", ["full", "causal"])
@pytest.mark.parametrize("std", [3.0, 6.0])
def test_fp8_peaked_scores(dims, mode, std):
    """Q and K of std 3 and 6 (before quantisation): the running max moves by
    more than the rescale threshold on many tiles, so the slow path runs
    repeatedly, and many probabilities fall into the e4m3 subnormal range or
    to zero; O stays within the element-wise bound and the LSE within
    1e-3 + ds of the module docstring (ds reaches the 1e-3 range here); the
    call without an LSE gives the same O bit for bit."""
    inp = make([700, 129, 1000], [900, 129, 1000], dims, seed=int(std) * 11 + dims[0], mode=mode, std=std)
    out, lse = run_fp8(inp)
    assert_fp8_parity(inp, out, lse, what="peaked %s %s std %g" % (dims, mode, std))
    out2, _ = run_fp8(inp, return_lse=False)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("std", [1.0, 3.0])
def test_fp8_score_error_single_key(dims, std):
    """Pins the score-error constant ds of the module docstring.  With one
    key per segment every row's only probability is exp2(s c - fp32(s c)),
    1 up to fp32 rounding, so its LSE is the fp32 image of its score
    scale * q_descale * k_descale * (q . k) and the LSE error is the error
    of the fp8 MFMA's dot product plus a few fp32 roundings.  Over 16
    segments of 257 queries (so the unpacked kernel runs) x 4 heads, at
    input std 1 and 3, |dLSE| <= 2^-15 scale sum_i |q_i k_i| + 2^-21 |s|
    + 1e-6 on every row."""
    n_seg, lq = 16, 257
    inp = make([lq] * n_seg, [1] * n_seg, dims, seed=int(std) * 7 + dims[0], heads=4, std=std)
    _, lse = run_fp8(inp)
    l = f64(lse)
    cq = inp.cu_seqlens_q.tolist()
    ck = inp.cu_seqlens_k.tolist()
    qd = oracle.dequantize(u8(inp.q), cq, inp.q_descale.numpy())  # [T, H, d]
    kd = oracle.dequantize(u8(inp.k), ck, inp.k_descale.numpy())  # [n_seg, H, d]
    seg = np.repeat(np.arange(n_seg), lq)
    scale = float(np.float32(inp.softmax_scale))
    prod = qd * kd[seg]  # [T, H, d]
    s = scale * prod.sum(axis=2).T  # [H, T]
    absdot = scale * np.abs(prod).sum(axis=2).T
    err = np.abs(l - s)
    bound = 2.0 ** -15 * absdot + 2.0 ** -21 * np.abs(s) + 1e-6
    ratio = float(np.max((err - 2.0 ** -21 * np.abs(s)) / absdot))
    print("fp8 %s std %g: max |dLSE| %.3e, max (|dLSE| - fp32 rounding) / (scale sum|q k|) %.3e (2^-15 = %.3e)" % (
        dims, std, float(err.max()), ratio, 2.0 ** -15))
    assert np.all(err <= bound), "score error above 2^-15 scale sum|q k| by up to %.3e" % float(np.max(err - bound))


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
def test_fp8_split_kv_dynamic_counts(dims):
    """fp8 inputs with per-segment split counts (explicit and the library's)
    against the oracle, within the element-wise bound."""
    inp = make([1, 64, 300, 17], [3000, 64, 1200, 900], dims, seed=dims[0] + 77, mode="causal")
    d = inp.to(DEV)
    for counts in ([3, 1, 0, 9], "auto"):
        dyn = counts if isinstance(counts, str) else torch.tensor(counts, dtype=torch.int32, device=DEV)
        out, lse = va.varlen_attn_fwd_fp8(
            d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, inp.max_seqlen_q, inp.max_seqlen_k, causal=True,
            q_descale=d.q_descale, k_descale=d.k_descale, v_descale=d.v_descale, return_lse=True, num_splits=6,
            num_splits_dynamic=dyn)
        torch.cuda.synchronize()
        assert_fp8_parity(inp, out, lse, what="fp8 dyn %s %s" % (dims, counts))
