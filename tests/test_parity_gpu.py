"""GPU parity of the HIP path against the fp64 oracle (marked ``gpu``).

Tolerances: max |O_gpu - O_oracle| <= 2e-2 and max |LSE_gpu - LSE_oracle|
<= 1e-3 for bf16 inputs, with -inf LSE exactly where the oracle has it.
Mask indexing and tile skipping are checked bit-exactly by probes whose
results are integers:

* zero-Q count probe: with Q = 0 every visible score is 0, so each p is 1
  and the row sum is the integer |J_i|; exp(LSE) must round to |J_i|.
* integer-score probe: scale 1, q = (1, 256, 0, ...), k_j = (j mod 256,
  j div 256, 0, ...) makes s_j = j exactly in bf16 x bf16 -> fp32, so
  LSE = j_max + ln sum_{t<n} e^-t and j_max must round to max J_i.

All calls go through the C interface via the ctypes binding.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import varlen_attention_forward_amd as va
from varlen_attention_forward_amd import workloads
from helpers import f64, f32, oracle_on
import oracle

pytestmark = pytest.mark.gpu

TOL_O = 2e-2
TOL_LSE = 1e-3
DEV = "cuda:0"
DIMS = [(64, 64), (72, 72), (80, 80), (128, 128), (192, 128)]


def guarded(t: torch.Tensor, rows: int = 256) -> torch.Tensor:
    """Copy ``t`` to the GPU with ``rows`` NaN rows after its last row."""
    buf = torch.full((t.shape[0] + rows,) + tuple(t.shape[1:]), float("nan"), dtype=t.dtype, device=DEV)
    buf[: t.shape[0]].copy_(t)
    return buf[: t.shape[0]]


def run_gpu(inp, out=None, lse_fill=None, return_lse=True, v=None):
    q, k = guarded(inp.q), guarded(inp.k)
    v = guarded(inp.v) if v is None else v
    cu_q, cu_k = inp.cu_seqlens_q.to(DEV), inp.cu_seqlens_k.to(DEV)
    lse = None
    if return_lse:
        lse = torch.full((inp.q.shape[1], inp.q.shape[0]), float("nan") if lse_fill is None else lse_fill,
                         dtype=torch.float32, device=DEV)
    res = va.varlen_attn_fwd(
        q, k, v, cu_q, cu_k, inp.max_seqlen_q, inp.max_seqlen_k,
        softmax_scale=inp.softmax_scale, causal=inp.causal, window_size=inp.window,
        out=out, return_lse=return_lse, lse=lse,
    )
    torch.cuda.synchronize()
    return res if return_lse else (res, None)


def assert_parity(out, lse, ref_o, ref_lse, rows=None, what=""):
    o = f64(out)
    if rows is not None:
        o, ref_o = o[rows], ref_o[rows]
    assert np.all(np.isfinite(o)), "%s: non-finite output" % what
    err_o = float(np.max(np.abs(o - ref_o))) if o.size else 0.0
    assert err_o <= TOL_O, "%s: max|dO| = %.3e" % (what, err_o)
    if lse is not None:
        l = f64(lse)
        if rows is not None:
            l, ref_lse = l[:, rows], ref_lse[:, rows]
        neg = ref_lse == -np.inf
        assert np.array_equal(l == -np.inf, neg), "%s: -inf LSE rows differ" % what
        fin = ~neg
        err_l = float(np.max(np.abs(l[fin] - ref_lse[fin]))) if fin.any() else 0.0
        assert err_l <= TOL_LSE, "%s: max|dLSE| = %.3e" % (what, err_l)
        return err_o, err_l
    return err_o, None


# ---------------------------------------------------------------------------
# small full-oracle parity over head dims, masks and ragged lengths
# ---------------------------------------------------------------------------
LEN_SETS = {
    "ragged": ([1, 63, 64, 65, 127, 128, 129, 255, 256, 257], None),
    "q_lt_k": ([1, 40, 64, 100, 129], [70, 64, 200, 100, 300]),
    "q_gt_k": ([64, 130, 300], [10, 129, 65]),
    "empty_segments": ([0, 37, 0, 190, 5], [0, 0, 50, 190, 0]),
}
MODES = {
    "full": (False, (-1, -1)),
    "causal": (True, (-1, -1)),
    "window": (False, (40, 17)),
    "causal_window": (True, (70, -1)),
    "left_only": (False, (0, -1)),
}


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("lens", list(LEN_SETS))
def test_small_parity(dims, mode, lens):
    d_qk, d_v = dims
    causal, window = MODES[mode]
    lq, lk = LEN_SETS[lens]
    lk = lq if lk is None else lk
    heads = 3 if d_qk < 192 else 2
    seed = zlib.crc32(repr((dims, mode, lens)).encode()) % 1000
    inp = workloads.make_inputs(lq, lk, heads, d_qk, d_v, seed=seed, causal=causal, window=window)
    out, lse = run_gpu(inp)
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out, lse, ref_o, ref_lse, what="%s/%s/%s" % (dims, mode, lens))


@pytest.mark.parametrize("dims", [(64, 64), (72, 72), (80, 80)], ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", ["full", "causal", "window", "causal_window"])
def test_multi_block_segments(dims, mode):
    """Segments spanning several 256-row query blocks, with a ragged last
    block, one of exactly two blocks and one of two blocks and a row, a short
    one and Lq != Lk."""
    d_qk, d_v = dims
    causal, window = MODES[mode]
    lq = [1029, 512, 40, 700, 513]
    lk = [1029, 512, 333, 901, 513]
    seed = zlib.crc32(repr(("multi", dims, mode)).encode()) % 1000
    inp = workloads.make_inputs(lq, lk, 2, d_qk, d_v, seed=seed, causal=causal, window=window)
    out, lse = run_gpu(inp)
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out, lse, ref_o, ref_lse, what="multi/%s/%s" % (dims, mode))


@pytest.mark.parametrize("dims", [(128, 128), (192, 128)], ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", ["causal", "causal_window"])
@pytest.mark.parametrize("order", ["longest_first", "packing_order"])
def test_causal_q_tile_pairs(dims, mode, order):
    """Causal launches at d_qk 128/192 run q-tiles n_b - 1 - t and t of a
    segment in one workgroup where the pairs fill their rounds: odd and even
    q-tile counts (the middle tile of an odd count runs alone), one-tile
    segments, a ragged last tile, Lq != Lk, dealt longest first (few segments)
    and in packing order (more than 64)."""
    d_qk, d_v = dims
    causal, window = MODES[mode]
    # shapes whose pairs fill their rounds: 8 x 8 groups of 4 pairs, 128 x 2 of 2
    if order == "longest_first":
        lq = [1029, 512, 40, 700, 513, 2048, 1, 0]
        lk = [1029, 600, 333, 901, 513, 2048, 1, 0]
        heads = 8
    else:
        rng = np.random.default_rng(d_qk)
        lq = [int(x) for x in rng.integers(0, 769, 128)]
        lq[0], lq[1], lq[2] = 768, 256, 257
        lk = [x if i % 4 else x + int(rng.integers(0, 200)) for i, x in enumerate(lq)]
        heads = 2
    assert va.plan(d_qk, d_v, len(lq), heads, max(lq), max(lk), 1)["pair_q_tiles"] == 1
    seed = zlib.crc32(repr(("pairs", dims, mode, order)).encode()) % 1000
    inp = workloads.make_inputs(lq, lk, heads, d_qk, d_v, seed=seed, causal=causal, window=window)
    out, lse = run_gpu(inp)
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out, lse, ref_o, ref_lse, what="pairs/%s/%s/%s" % (dims, mode, order))


@pytest.mark.parametrize("batch", [2, 64, 90])
@pytest.mark.parametrize("dims,causal", [((64, 64), False), ((128, 128), True), ((80, 80), False)],
                         ids=lambda x: str(x))
def test_many_ragged_segments(batch, dims, causal):
    """Ragged batches dealt longest first (up to 64 segments, including empty
    ones and equal lengths) and in packing order (more than 64)."""
    d_qk, d_v = dims
    rng = np.random.default_rng(batch * 7 + d_qk)
    lq = [int(x) for x in rng.integers(0, 400, batch)]
    lq[0], lq[-1] = 300, 300
    lk = [x if i % 5 else int(rng.integers(0, 600)) for i, x in enumerate(lq)]
    inp = workloads.make_inputs(lq, lk, 2, d_qk, d_v, seed=batch, causal=causal)
    out, lse = run_gpu(inp)
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out, lse, ref_o, ref_lse, what="many/%d/%s/%s" % (batch, dims, causal))


@pytest.mark.parametrize("dims,lens,causal", [
    ((128, 128), [300, 77], False),
    ((64, 64), [700, 77, 1100], False),   # several 256-row blocks
    ((80, 80), [700, 77, 1100], True),
])
@pytest.mark.parametrize("with_lse", [True, False])
def test_large_scores_and_tiny_scale(dims, lens, causal, with_lse):
    """Peaked softmax (Q, K with std 4: scores of std ~16, so the running max
    moves by far more than the rescale threshold on many tiles, taking the
    rescale path over and over) and a tiny scale.  V keeps unit scale: a bf16
    output of magnitude >= 4 alone rounds by up to 1.6e-2."""
    for std, scale in ((4.0, None), (1.0, 1e-3), (2.0, 0.5)):
        inp = workloads.make_inputs(lens, lens, 2, dims[0], dims[1], seed=11, std=std, softmax_scale=scale,
                                    causal=causal)
        out, lse = run_gpu(inp, return_lse=with_lse)
        ref_o, ref_lse = oracle_on(inp)
        assert_parity(out, lse, ref_o, ref_lse if with_lse else None,
                      what="%s std=%s scale=%s lse=%s" % (dims, std, scale, with_lse))


# ---------------------------------------------------------------------------
# exact probes of mask indexing and tile skipping
# ---------------------------------------------------------------------------
def _visible_counts(inp):
    wl, wr = inp.window
    cu_q, cu_k = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
    n = np.full(inp.q.shape[0], -1, dtype=np.int64)
    jmax = np.full(inp.q.shape[0], -1, dtype=np.int64)
    for b in range(len(cu_q) - 1):
        Lq, Lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        lo, hi = oracle.visible_interval(np.arange(Lq), Lq, Lk, inp.causal, wl, wr)
        n[cu_q[b]: cu_q[b + 1]] = np.maximum(hi - lo + 1, 0)
        jmax[cu_q[b]: cu_q[b + 1]] = hi
    return n, jmax


PROBE_CASES = [
    ("square_causal", [64, 256, 577, 1000], None, True, (-1, -1)),
    ("chunked_prefill", [100, 64, 257], [612, 64, 300], True, (-1, -1)),
    ("q_gt_k_causal", [300, 129], [100, 1], True, (-1, -1)),
    ("band", [700, 256], [700, 256], False, (100, 63)),
    ("causal_window", [1000], [1000], True, (127, -1)),
    ("look_ahead", [333], [400], False, (0, 129)),
    ("full_ragged", [1, 65, 129, 1023], None, False, (-1, -1)),
]


@pytest.mark.parametrize("case", PROBE_CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("dims", [(64, 64), (80, 80), (192, 128)], ids=lambda d: "d%d_%d" % d)
def test_zero_q_count_probe(case, dims):
    name, lq, lk, causal, window = case
    lk = lq if lk is None else lk
    inp = workloads.make_inputs(lq, lk, 2, dims[0], dims[1], seed=3, causal=causal, window=window)
    inp.q.zero_()
    out, lse = run_gpu(inp)
    n, _ = _visible_counts(inp)
    l = f64(lse)
    for h in range(2):
        got = np.where(l[h] == -np.inf, 0, np.rint(np.exp(np.where(l[h] == -np.inf, 0, l[h]))))
        assert np.array_equal(got.astype(np.int64), n), "%s head %d: visible counts differ" % (name, h)
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out, lse, ref_o, ref_lse, what=name)


@pytest.mark.parametrize("case", PROBE_CASES, ids=lambda c: c[0])
def test_integer_score_probe(case):
    name, lq, lk, causal, window = case
    lk = lq if lk is None else lk
    inp = workloads.make_inputs(lq, lk, 1, 64, 64, seed=4, causal=causal, window=window, softmax_scale=1.0)
    inp.q.zero_()
    inp.q[:, :, 0] = 1.0
    inp.q[:, :, 1] = 256.0
    inp.k.zero_()
    cu_k = inp.cu_seqlens_k.tolist()
    for b in range(len(cu_k) - 1):
        j = torch.arange(cu_k[b + 1] - cu_k[b])
        inp.k[cu_k[b]: cu_k[b + 1], 0, 0] = (j % 256).to(torch.bfloat16)
        inp.k[cu_k[b]: cu_k[b + 1], 0, 1] = (j // 256).to(torch.bfloat16)
    out, lse = run_gpu(inp)
    n, jmax = _visible_counts(inp)
    l = f64(lse)[0]
    has = n > 0
    assert np.all(l[~has] == -np.inf)
    tail = np.log((1 - np.exp(-n[has].astype(np.float64))) / (1 - math.exp(-1)))
    got = np.rint(l[has] - tail).astype(np.int64)
    assert np.array_equal(got, jmax[has]), "%s: last visible key differs" % name


def test_single_key_is_exact():
    """Lk = 1: p = exp2(0) = 1 exactly, so O = V[0] bit for bit (also causal row 0)."""
    for causal in (False, True):
        # bottom-right causal: with one key only a segment's last row sees it
        lq = [1, 1, 1] if causal else [5, 70, 1]
        inp = workloads.make_inputs(lq, [1, 1, 1], 4, 128, 128, seed=5, causal=causal)
        out, lse = run_gpu(inp)
        cu_q, cu_k = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
        for b in range(len(cu_q) - 1):
            rows = slice(cu_q[b], cu_q[b + 1])
            expect = inp.v[cu_k[b]].to(DEV).unsqueeze(0).expand(cu_q[b + 1] - cu_q[b], -1, -1)
            assert torch.equal(out[rows], expect)
        ref_o, ref_lse = oracle_on(inp)
        assert_parity(out, lse, ref_o, ref_lse, what="single key")


def test_constant_v():
    inp = workloads.make_inputs([500, 64], [500, 64], 2, 80, 80, seed=6, causal=True)
    c = torch.randn((2, 80), generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    inp.v[:] = c
    out, _ = run_gpu(inp)
    err = (out.float().cpu() - c.float()).abs().max().item()
    assert err <= TOL_O


def test_key_permutation_invariance():
    inp = workloads.make_inputs([300], [517], 2, 128, 128, seed=7)
    out1, lse1 = run_gpu(inp)
    perm = torch.randperm(517, generator=torch.Generator().manual_seed(1))
    inp2 = workloads.Inputs(**{**inp.__dict__, "k": inp.k[perm].contiguous(), "v": inp.v[perm].contiguous()})
    out2, lse2 = run_gpu(inp2)
    assert (out1.float() - out2.float()).abs().max().item() <= TOL_O
    assert (lse1 - lse2).abs().max().item() <= TOL_LSE


# ---------------------------------------------------------------------------
# bit-exact invariances: packing, heads, repeat runs, strides
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_packing_invariance_bit_exact(causal):
    lq, lk = [77, 300, 129, 512], [90, 300, 129, 600]
    inp = workloads.make_inputs(lq, lk, 4, 80, 80, seed=8, causal=causal)
    out, lse = run_gpu(inp)
    cu_q, cu_k = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
    for b in range(4):
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        one = workloads.Inputs(
            q=inp.q[qs].clone(), k=inp.k[ks].clone(), v=inp.v[ks].clone(),
            cu_seqlens_q=workloads.cu_seqlens([lq[b]]), cu_seqlens_k=workloads.cu_seqlens([lk[b]]),
            max_seqlen_q=lq[b], max_seqlen_k=lk[b], softmax_scale=inp.softmax_scale,
            causal=causal, window=(-1, -1),
        )
        o1, l1 = run_gpu(one)
        assert torch.equal(out[qs], o1), "segment %d output depends on packing" % b
        assert torch.equal(lse[:, qs], l1), "segment %d LSE depends on packing" % b


def test_determinism_and_head_permutation():
    inp = workloads.make_inputs([1000, 333], [1000, 333], 6, 128, 128, seed=9, causal=True)
    o1, l1 = run_gpu(inp)
    o2, l2 = run_gpu(inp)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    perm = torch.tensor([3, 0, 5, 1, 4, 2])
    inp2 = workloads.Inputs(**{**inp.__dict__, "q": inp.q[:, perm].contiguous(), "k": inp.k[:, perm].contiguous(),
                               "v": inp.v[:, perm].contiguous()})
    o3, l3 = run_gpu(inp2)
    assert torch.equal(o3, o1[:, perm.to(DEV)]) and torch.equal(l3, l1[perm.to(DEV)])


def test_strided_mla_v_and_strided_out():
    """V as a view into the interleaved [T, H, nope + v] buffer (MLA layout), and
    a caller-provided strided out; results equal the contiguous call bit for bit."""
    inp = workloads.make_inputs([257, 1000], [257, 1000], 4, 192, 128, seed=10, causal=True)
    o_ref, l_ref = run_gpu(inp)
    T = inp.k.shape[0]
    kv = torch.full((T, 4, 128 + 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    kv[:, :, 128:] = inp.v.to(DEV)
    v_view = kv[:, :, 128:]
    assert v_view.stride() == (4 * 256, 256, 1)
    big = torch.full((inp.q.shape[0], 4, 256), 7.0, dtype=torch.bfloat16, device=DEV)
    out_view = big[:, :, 64:192]
    o2, l2 = run_gpu(inp, out=out_view, v=v_view)
    assert torch.equal(o2, o_ref) and torch.equal(l2, l_ref)
    assert torch.all(big[:, :, :64] == 7.0) and torch.all(big[:, :, 192:] == 7.0)


def test_rows_outside_segments_untouched():
    inp = workloads.make_inputs([10, 200], [10, 200], 2, 64, 64, seed=12)
    # cu_seqlens cover only the first 150 of 210 rows
    inp = workloads.Inputs(**{**inp.__dict__, "cu_seqlens_q": torch.tensor([0, 10, 150], dtype=torch.int32),
                              "cu_seqlens_k": torch.tensor([0, 10, 150], dtype=torch.int32),
                              "max_seqlen_q": 140, "max_seqlen_k": 140})
    sentinel = torch.full((210, 2, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    out, lse = run_gpu(inp, out=sentinel, lse_fill=5.0)
    assert torch.all(out[150:] == 3.0)
    assert torch.all(lse[:, 150:] == 5.0)
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out, lse, ref_o, ref_lse, rows=np.arange(150), what="partial cover")


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", ["full", "causal", "window"])
def test_no_lse_row_sum_over_bf16(dims, mode):
    """Without an LSE, d_v 72/80 take the row sum over the bf16
    probabilities (a ones column in the padded V tile): O must still match
    the oracle, on multi-block segments with ragged tails and rows that see
    no key, and stay within the tolerance of the LSE call's O.  The other
    head dims run the same fp32 row sum with or without an LSE, so there the
    two calls' O agree bit for bit."""
    causal, window = MODES[mode]
    lq = [1029, 700, 40, 513] if dims[0] < 192 else [600, 40, 257]
    lk = [1029, 901, 0, 513] if dims[0] < 192 else [700, 0, 257]
    seed = zlib.crc32(repr(("nolse", dims, mode)).encode()) % 1000
    inp = workloads.make_inputs(lq, lk, 2, dims[0], dims[1], seed=seed, causal=causal, window=window)
    out, _ = run_gpu(inp, return_lse=False)
    ref_o, _ = oracle_on(inp)
    assert_parity(out, None, ref_o, None, what="nolse/%s/%s" % (dims, mode))
    with_lse, _ = run_gpu(inp)
    if dims[1] in (72, 80):
        assert float((out.float() - with_lse.float()).abs().max()) <= TOL_O
    else:
        assert torch.equal(out, with_lse)


@pytest.mark.parametrize("dims", [(64, 64), (80, 80), (128, 128), (192, 128)], ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("heads,heads_k", [(8, 1), (8, 2), (6, 3), (16, 8)])
@pytest.mark.parametrize("mode", ["full", "causal", "window"])
def test_grouped_kv_heads(dims, heads, heads_k, mode):
    """Grouped KV heads (query head h reads KV head h // (H / H_kv)) against
    the oracle, on ragged multi-block segments with q < k and q > k, with
    and without an LSE; and a call with each KV head repeated to H heads
    (plain multi-head attention) gives the same O and LSE bit for bit."""
    causal, window = MODES[mode]
    lq, lk = [300, 1, 530, 64], [300, 90, 530, 40]
    seed = zlib.crc32(repr(("gqa", dims, heads, heads_k, mode)).encode()) % 1000
    inp = workloads.make_inputs(lq, lk, heads, dims[0], dims[1], seed=seed, causal=causal, window=window,
                                num_heads_k=heads_k)
    out, lse = run_gpu(inp)
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out, lse, ref_o, ref_lse, what="gqa/%s/%d/%d/%s" % (dims, heads, heads_k, mode))
    rep = heads // heads_k
    mha = workloads.Inputs(**{**inp.__dict__, "k": inp.k.repeat_interleave(rep, dim=1).contiguous(),
                              "v": inp.v.repeat_interleave(rep, dim=1).contiguous()})
    out2, lse2 = run_gpu(mha)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    out3, _ = run_gpu(inp, return_lse=False)
    assert_parity(out3, None, ref_o, None, what="gqa-nolse")


def run_gpu_split(inp, num_splits, out=None, lse_fill=None, return_lse=True):
    q, k, v = guarded(inp.q), guarded(inp.k), guarded(inp.v)
    cu_q, cu_k = inp.cu_seqlens_q.to(DEV), inp.cu_seqlens_k.to(DEV)
    lse = None
    if return_lse:
        lse = torch.full((inp.q.shape[1], inp.q.shape[0]), float("nan") if lse_fill is None else lse_fill,
                         dtype=torch.float32, device=DEV)
    res = va.varlen_attn_fwd(q, k, v, cu_q, cu_k, inp.max_seqlen_q, inp.max_seqlen_k,
                             softmax_scale=inp.softmax_scale, causal=inp.causal, window_size=inp.window,
                             out=out, return_lse=return_lse, lse=lse, num_splits=num_splits)
    torch.cuda.synchronize()
    return res if return_lse else (res, None)


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", ["full", "causal", "window", "causal_window"])
@pytest.mark.parametrize("splits", [2, 3, 8])
def test_split_kv(dims, mode, splits):
    """Split-KV: each unit's key tiles in `splits` runs, combined at the end,
    against the oracle on ragged segments (q < k chunked-prefill shapes,
    q > k, a segment with no keys, runs shorter than a tile and empty runs),
    with and without an LSE; rows outside every segment stay untouched."""
    causal, window = MODES[mode]
    lq, lk = [1, 300, 77, 530, 9], [700, 300, 0, 900, 2]
    seed = zlib.crc32(repr(("split", dims, mode, splits)).encode()) % 1000
    inp = workloads.make_inputs(lq, lk, 2, dims[0], dims[1], seed=seed, causal=causal, window=window)
    sentinel = torch.full((inp.q.shape[0] + 40, 2, dims[1]), 3.0, dtype=torch.bfloat16, device=DEV)
    out, lse = run_gpu_split(inp, splits, out=sentinel[: inp.q.shape[0]])
    assert torch.all(sentinel[inp.q.shape[0]:] == 3.0)
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out, lse, ref_o, ref_lse, what="split%d/%s/%s" % (splits, dims, mode))
    out2, _ = run_gpu_split(inp, splits, return_lse=False)
    assert_parity(out2, None, ref_o, None, what="split%d-nolse" % splits)


def test_split_kv_one_split_is_the_plain_call():
    inp = workloads.make_inputs([300, 77], [500, 77], 3, 128, 128, seed=40, causal=True)
    a, la = run_gpu(inp)
    b, lb = run_gpu_split(inp, 1)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_split_kv_rows_outside_segments_untouched():
    inp = workloads.make_inputs([10, 140], [10, 140], 2, 64, 64, seed=13)
    inp = workloads.Inputs(**{**inp.__dict__, "q": torch.cat([inp.q, inp.q[:60]]),
                              "cu_seqlens_q": torch.tensor([0, 10, 150], dtype=torch.int32)})
    sentinel = torch.full((210, 2, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    out, lse = run_gpu_split(inp, 4, out=sentinel, lse_fill=5.0)
    assert torch.all(out[150:] == 3.0) and torch.all(lse[:, 150:] == 5.0)
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out, lse, ref_o, ref_lse, rows=np.arange(150), what="split partial cover")


def test_split_kv_auto_count_and_grouped_heads():
    """The library's split count on a short-query, long-key call (8 heads
    over 2 KV heads) is > 1, and the result matches the oracle."""
    inp = workloads.make_inputs([200, 64], [6000, 3000], 8, 128, 128, seed=41, causal=True, num_heads_k=2)
    n = va.auto_num_splits(128, 128, 2, 8, 200, 6000)
    assert 1 < n <= 128
    out, lse = run_gpu_split(inp, 0)
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out, lse, ref_o, ref_lse, what="split auto (%d)" % n)


@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", ["full", "causal", "window", "left_only"])
@pytest.mark.parametrize("lens", ["le64", "le128", "le128_small", "q_lt_k"])
def test_packed_short_segments(dims, mode, lens):
    """Short segments share workgroups (four per workgroup when every segment
    has at most 64 queries, two when at most 128), each wave or pair of waves
    on its own segment whose keys start anywhere inside the workgroup's key
    tiles; at most 64 queries with head dims <= 80 take the one-wave
    short-segment kernel instead, and at most 128 queries on a launch too
    small for the CUs (3 heads) the same kernel with its waves splitting each
    64-row block's keys.  Against the oracle with ragged lengths, empty
    segments, a partial last group and q < k, with and without an LSE; rows
    outside every segment stay untouched."""
    causal, window = MODES[mode]
    lq, lk, heads = {
        "le64": ([1, 64, 0, 37, 64, 5, 63, 2, 50], None, 3),
        "le128": ([128, 1, 65, 100, 0, 127, 3], None, 80),  # 1120 64-row blocks: packed two a workgroup
        "le128_small": ([128, 1, 65, 100, 0, 127, 3], None, 3),
        "q_lt_k": ([40, 64, 1, 17, 64], [300, 64, 90, 0, 77], 3),
    }[lens]
    lk = lq if lk is None else lk
    seed = zlib.crc32(repr(("packed", dims, mode, lens)).encode()) % 1000
    inp = workloads.make_inputs(lq, lk, heads, dims[0], dims[1], seed=seed, causal=causal, window=window)
    pl = va.plan(dims[0], dims[1], len(lq), heads, max(lq), max(lk), causal)
    blocks = 8 * -(-len(lq) * heads // 8) * -(-max(lq) // 64)
    ks = 4 if dims[0] <= 80 and max(lq) > 64 and blocks <= 512 else 1
    short = (max(lq) <= 64 or ks > 1) and dims[0] <= 80
    assert pl["kernel"] == ("attn_fwd_short" if short else "attn_fwd_wide")
    assert pl["key_split"] == ks
    assert pl["segments_per_block"] == (1 if short else 4 if max(lq) <= 64 else 2)
    sentinel = torch.full((inp.q.shape[0] + 30, heads, dims[1]), 3.0, dtype=torch.bfloat16, device=DEV)
    out, lse = run_gpu(inp, out=sentinel[: inp.q.shape[0]])
    assert torch.all(sentinel[inp.q.shape[0]:] == 3.0)
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out, lse, ref_o, ref_lse, what="packed/%s/%s/%s" % (dims, mode, lens))
    out2, _ = run_gpu(inp, return_lse=False)
    assert_parity(out2, None, ref_o, None, what="packed-nolse")


SHORT_LENS = {
    "le64": ([1, 64, 0, 37, 64, 5, 63, 2, 50], None),
    "q_lt_k": ([40, 64, 1, 17, 64], [300, 64, 90, 0, 77]),
    "q_gt_k": ([64, 33, 50], [10, 1, 49]),
    "windows": ([64] * 24, None),
}


@pytest.mark.parametrize("dims", [(64, 64), (72, 72), (80, 80)], ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("lens", list(SHORT_LENS))
def test_short_kernel_bit_equal_to_unpacked(dims, mode, lens):
    """Segments of at most 64 queries (head dims <= 80) run one wave per
    (segment, head) on the short-segment kernel, whose arithmetic per key
    tile is the four-wave kernel's: O and LSE are bit-identical to the
    four-wave kernel's unpacked launch of the same call (max_seqlen_q passed
    as 4096: enough 256-row units that the launch is not split by keys), with
    the fp32 row sum (LSE returned) and the ones-column sum (no LSE), and
    with e4m3 output; and within the oracle's tolerance.  Eight heads, so
    d 72 and 80 deal heads in groups (8 and 4)."""
    causal, window = MODES[mode]
    lq, lk = SHORT_LENS[lens]
    lk = lq if lk is None else lk
    heads = 8
    seed = zlib.crc32(repr(("short", dims, mode, lens)).encode()) % 1000
    inp = workloads.make_inputs(lq, lk, heads, dims[0], dims[1], seed=seed, causal=causal, window=window)
    assert va.plan(dims[0], dims[1], len(lq), heads, max(lq), max(lk), causal)["kernel"] == "attn_fwd_short"
    assert va.plan(dims[0], dims[1], len(lq), heads, 4096, max(lk), causal)["kernel"] == "attn_fwd_wide"
    d = inp.to(DEV)

    def call(max_q, return_lse, out_scale=None):
        res = va.varlen_attn_fwd(d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, max_q, inp.max_seqlen_k,
                                 softmax_scale=inp.softmax_scale, causal=causal, window_size=window,
                                 return_lse=return_lse, out_scale=out_scale)
        torch.cuda.synchronize()
        return res if return_lse else (res, None)

    out, lse = call(inp.max_seqlen_q, True)
    out_w, lse_w = call(4096, True)
    assert torch.equal(out, out_w) and torch.equal(lse, lse_w)
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out, lse, ref_o, ref_lse, what="short/%s/%s/%s" % (dims, mode, lens))
    out, _ = call(inp.max_seqlen_q, False)
    out_w, _ = call(4096, False)
    assert torch.equal(out, out_w)
    assert_parity(out, None, ref_o, None, what="short-nolse")
    sc = torch.tensor([0.01], dtype=torch.float32, device=DEV)
    out, _ = call(inp.max_seqlen_q, False, sc)
    out_w, _ = call(4096, False, sc)
    assert torch.equal(out.view(torch.uint8), out_w.view(torch.uint8))


KEY_SPLIT_LENS = {
    "one_257": ([257], None, 16),
    "one_1024": ([1024], None, 16),
    "tiny_64_256": ([64, 256], None, 16),
    "ragged": ([300, 1, 700, 129, 0, 65], [300, 40, 900, 129, 7, 0], 3),
    "q_lt_k": ([130, 200], [2000, 333], 16),
}


@pytest.mark.parametrize("dims", [(64, 64), (72, 72), (80, 80)], ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("lens", list(KEY_SPLIT_LENS))
def test_key_split_small_launches(dims, mode, lens):
    """Launches of segments longer than 64 queries whose 64-row blocks fit one
    round run the short-segment kernel with a workgroup's four waves on one
    block, each over a quarter of its key tiles, merged through LDS: against the oracle with the LSE, without it (d 72 / 80: the
    ones-column row sum) and with e4m3 output, and against the four-wave
    kernel (max_seqlen_q passed as 8192) within the same tolerance.  Empty
    segments, a segment without keys, key ranges shorter than four tiles
    (waves with nothing to do) and masks that leave a wave's rows no key."""
    causal, window = MODES[mode]
    lq, lk, heads = KEY_SPLIT_LENS[lens]
    lk = lq if lk is None else lk
    p = va.plan(dims[0], dims[1], len(lq), heads, max(lq), max(lk), causal)
    assert (p["kernel"], p["key_split"]) == ("attn_fwd_short", 4)
    seed = zlib.crc32(repr(("ksplit", dims, mode, lens)).encode()) % 1000
    inp = workloads.make_inputs(lq, lk, heads, dims[0], dims[1], seed=seed, causal=causal, window=window)
    d = inp.to(DEV)

    def call(max_q, return_lse, out_scale=None):
        res = va.varlen_attn_fwd(d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, max_q, inp.max_seqlen_k,
                                 softmax_scale=inp.softmax_scale, causal=causal, window_size=window,
                                 return_lse=return_lse, out_scale=out_scale)
        torch.cuda.synchronize()
        return res if return_lse else (res, None)

    ref_o, ref_lse = oracle_on(inp)
    out, lse = call(inp.max_seqlen_q, True)
    assert_parity(out, lse, ref_o, ref_lse, what="ksplit/%s/%s/%s" % (dims, mode, lens))
    assert va.plan(dims[0], dims[1], len(lq), heads, 8192, max(lk), causal)["key_split"] == 1
    out_w, lse_w = call(8192, True)
    assert_parity(out_w, lse_w, ref_o, ref_lse, what="wide/%s/%s/%s" % (dims, mode, lens))
    out, _ = call(inp.max_seqlen_q, False)
    assert_parity(out, None, ref_o, None, what="ksplit-nolse")
    sc = torch.tensor([0.01], dtype=torch.float32, device=DEV)
    # e4m3 codes of O / 0.01, decoded: within the O tolerance of the oracle
    # clipped to the e4m3 range (+-448 x 0.01, where the output saturates)
    # plus half an e4m3 step of |O| (2^-4 relative; 2^-10 x 0.01 below the
    # normal range), for both kernels
    ref_c = np.clip(ref_o, -4.48, 4.48)
    for max_q in (inp.max_seqlen_q, 8192):
        out8, _ = call(max_q, False, sc)
        o8 = f64(out8.view(torch.float8_e4m3fn).float()) * 0.01
        err = np.abs(o8 - ref_c) - (TOL_O + 2.0 ** -4 * (np.abs(ref_c) + TOL_O) + 2.0 ** -10 * 0.01)
        assert np.all(err <= 0), "e4m3 O, max_seqlen_q %d: %.3e over" % (max_q, err.max())


@pytest.mark.parametrize("key_split", [1, 4])
def test_short_kernel_strided_views(key_split):
    """The short-segment kernel on views: Q and K with a padded head stride,
    V inside an interleaved [T, H, 2 x d] buffer, O written into a strided
    view whose padding stays untouched; bit-identical to the contiguous
    call.  One wave a segment (at most 64 queries), and the key split of a
    small launch of longer segments."""
    lq = [64, 17, 0, 64, 1, 50, 64, 33] if key_split == 1 else [300, 17, 0, 700, 1, 129]
    inp = workloads.make_inputs(lq, lq, 4, 80, 80, seed=77, causal=False, window=(20, 5))
    p = va.plan(80, 80, len(lq), 4, max(lq), max(lq), False)
    assert (p["kernel"], p["key_split"]) == ("attn_fwd_short", key_split)
    o_ref, l_ref = run_gpu(inp)
    T = inp.q.shape[0]

    def padded(t, width):
        buf = torch.full((T, 4, width), float("nan"), dtype=torch.bfloat16, device=DEV)
        buf[:, :, width - 80:] = t.to(DEV)
        return buf[:, :, width - 80:]

    q_view, k_view, v_view = padded(inp.q, 96), padded(inp.k, 128), padded(inp.v, 160)
    assert q_view.stride() == (4 * 96, 96, 1) and v_view.stride() == (4 * 160, 160, 1)
    big = torch.full((T, 4, 112), 7.0, dtype=torch.bfloat16, device=DEV)
    out_view = big[:, :, 16:96]
    lse = torch.full((4, T), float("nan"), dtype=torch.float32, device=DEV)
    va.varlen_attn_fwd(q_view, k_view, v_view, inp.cu_seqlens_q.to(DEV), inp.cu_seqlens_k.to(DEV),
                       inp.max_seqlen_q, inp.max_seqlen_k, softmax_scale=inp.softmax_scale,
                       window_size=inp.window, out=out_view, return_lse=True, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out_view, o_ref) and torch.equal(lse, l_ref)
    assert torch.all(big[:, :, :16] == 7.0) and torch.all(big[:, :, 96:] == 7.0)


def test_short_kernel_beyond_2gib():
    """64-bit addressing in the short-segment kernel: 36000 windows of 64
    tokens, 8 heads, d 64, so Q, K, V and O each span 2.36 GB and the last
    windows start past 2^31 bytes.  Sampled windows (first, middle, last
    three) against the oracle run on just those windows."""
    B, L, H, D = 36000, 64, 8, 64
    assert B * L * H * D * 2 > 2 ** 31
    g = torch.Generator(device=DEV).manual_seed(2025)
    q = torch.randn((B * L, H, D), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B * L, H, D), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B * L, H, D), generator=g, device=DEV).to(torch.bfloat16)
    cu = torch.arange(0, (B + 1) * L, L, dtype=torch.int32, device=DEV)
    assert va.plan(D, D, B, H, L, L, False)["kernel"] == "attn_fwd_short"
    out, lse = va.varlen_attn_fwd(q, k, v, cu, cu, L, L, return_lse=True)
    torch.cuda.synchronize()
    from oracle import attention_fwd

    for b in (0, B // 2, B - 3, B - 2, B - 1):
        sl = slice(b * L, (b + 1) * L)
        ref_o, ref_lse = attention_fwd(f32(q[sl]), f32(k[sl]), f32(v[sl]), [0, L], [0, L], D ** -0.5)
        assert_parity(out[sl], lse[:, sl].contiguous(), ref_o, ref_lse, what="window %d" % b)
    del q, k, v, out, lse
    torch.cuda.empty_cache()


def test_packed_short_segments_with_split_kv_and_grouped_heads():
    inp = workloads.make_inputs([64, 30, 64, 1, 64], [2000, 30, 700, 5, 64], 8, 128, 128, seed=42, causal=True,
                                num_heads_k=2)
    ref_o, ref_lse = oracle_on(inp)
    for splits in (1, 4):
        out, lse = run_gpu_split(inp, splits)
        assert_parity(out, lse, ref_o, ref_lse, what="packed split %d" % splits)


GRAPH_CASES = {
    "wide_d128_causal": (([300, 77, 1029], [300, 500, 1029], 2, 128, 128), dict(seed=21, causal=True), 1),
    "short_d80_windows": (([64, 17, 64, 40, 0, 64] * 4, [64, 17, 64, 40, 0, 64] * 4, 4, 80, 80), dict(seed=22), 1),
    "split4_192_128": (([256, 64], [5000, 3000], 2, 192, 128), dict(seed=23, causal=True), 4),
    "key_split_d64": (([1024, 300], [1024, 700], 4, 64, 64), dict(seed=24, causal=True), 1),
}


@pytest.mark.parametrize("case", list(GRAPH_CASES))
def test_hip_graph_replay_matches_eager(case):
    """The call enqueues its kernel launches and nothing else (one kernel, or
    with split-KV the kernel and the combine, the workspace taken from the
    graph's memory pool), so it can be captured in a HIP graph: three
    replays, with eager calls between them, reproduce the eager O and LSE bit
    for bit (outputs cleared outside the graph first), for the four-wave
    kernel, the one-wave short-segment kernel, its key split on a small
    launch and a split-KV call."""
    args, kw, splits = GRAPH_CASES[case]
    inp = workloads.make_inputs(*args, **kw)
    d = inp.to(DEV)
    heads, dv = args[2], args[4]

    def call(out, lse):
        va.varlen_attn_fwd(d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, d.max_seqlen_q, d.max_seqlen_k,
                           softmax_scale=d.softmax_scale, causal=d.causal, out=out, return_lse=True, lse=lse,
                           num_splits=splits)

    shape_o, shape_l = (d.q.shape[0], heads, dv), (heads, d.q.shape[0])
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
        call(torch.empty_like(out_e), torch.empty_like(lse_e))  # eager work between replays
        torch.cuda.synchronize()
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out_g, lse_g, ref_o, ref_lse, what="graph replay")


def test_empty_batch_and_zero_keys():
    inp = workloads.make_inputs([5, 6], [0, 0], 2, 64, 64, seed=14)
    out, lse = run_gpu(inp)
    assert torch.all(out == 0) and torch.all(lse == -float("inf"))
    e = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    cu = torch.zeros(1, dtype=torch.int32, device=DEV)
    assert va.varlen_attn_fwd(e, e, e, cu, cu, 0, 0).shape == (0, 2, 64)


def test_tensors_beyond_2gib():
    """64-bit addressing: 2100 segments of 1024 tokens, 8 heads, d 64, so Q,
    K, V and O each span 2.2 GB and the last segments start past 2^31 bytes
    (and past 2^31 elements of O in total).  Inputs are drawn on the GPU
    from a seeded generator; sampled segments (first, middle and the last
    three) are checked against the oracle run on just those segments."""
    B, L, H, D = 2100, 1024, 8, 64
    assert B * L * H * D * 2 > 2 ** 31
    g = torch.Generator(device=DEV).manual_seed(2024)
    q = torch.randn((B * L, H, D), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B * L, H, D), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B * L, H, D), generator=g, device=DEV).to(torch.bfloat16)
    cu = torch.arange(0, (B + 1) * L, L, dtype=torch.int32, device=DEV)
    out, lse = va.varlen_attn_fwd(q, k, v, cu, cu, L, L, causal=True, return_lse=True)
    torch.cuda.synchronize()
    from oracle import attention_fwd

    for b in (0, B // 2, B - 3, B - 2, B - 1):
        sl = slice(b * L, (b + 1) * L)
        ref_o, ref_lse = attention_fwd(f32(q[sl]), f32(k[sl]), f32(v[sl]), [0, L], [0, L], D ** -0.5,
                                       causal=True)
        assert_parity(out[sl], lse[:, sl].contiguous(), ref_o, ref_lse, what="segment %d" % b)
    del q, k, v, out, lse
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# the named workloads at full size (sampled rows where the oracle is slow)
# ---------------------------------------------------------------------------
def _sample_rows(inp, n_random, seed=0):
    """Rows 0, 1, L - 2, L - 1 of every segment, the rows on both sides of
    every query-block boundary (b * block_m - 1, b * block_m,
    b * block_m + 1 for every block b), and ``n_random`` seeded random rows."""
    bm = va.plan(inp.q.shape[2], inp.v.shape[2], len(inp.cu_seqlens_q) - 1, inp.q.shape[1],
                 inp.max_seqlen_q, inp.max_seqlen_k, inp.causal)["block_m"]
    cu = inp.cu_seqlens_q.tolist()
    rows = set()
    for b in range(len(cu) - 1):
        L = cu[b + 1] - cu[b]
        cand = [0, 1, L - 2, L - 1]
        for t in range(1, (L + bm - 1) // bm):
            cand += [t * bm - 1, t * bm, t * bm + 1]
        rows.update(cu[b] + r for r in cand if 0 <= r < L)
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, cu[-1], n_random).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["tiny_varlen_d64", "vit_window256_d80", "vit_window64_d80", "mla_context_chunk_tp8"])
def test_workload_full_oracle(name):
    w = workloads.WORKLOADS[name]
    inp = workloads.workload_inputs(w)
    if w.num_splits != 1:
        out, lse = run_gpu_split(inp, w.num_splits, return_lse=w.return_lse)
    else:
        out, lse = run_gpu(inp, return_lse=w.return_lse)
    ref_o, ref_lse = oracle_on(inp)
    e = assert_parity(out, lse, ref_o, ref_lse, what=name)
    print("%s: max|dO| %.3e max|dLSE| %s" % (name, e[0], e[1]))


@pytest.mark.parametrize("name,n_random,heads", [
    ("vit_full_d80", 384, None),
    ("vit_long65536_d128", 1024, None),
    ("mla_causal_192_128", 128, None),
    ("gqa_chunk64_d128", 256, None),
    ("page_1x32768_d72", 256, None),   # shapes of the pages' speed tables
    ("page_64x1024_d64", 256, None),
])
def test_workload_sampled(name, n_random, heads):
    w = workloads.WORKLOADS[name] if name in workloads.WORKLOADS else workloads.PAGE_SHAPES[name]
    inp = workloads.workload_inputs(w)
    out, lse = run_gpu(inp, return_lse=w.return_lse)
    rows = _sample_rows(inp, n_random)
    ref_o, ref_lse = oracle_on(inp, rows=rows, heads=heads)
    e = assert_parity(out, lse, ref_o, ref_lse, rows=rows, what=name)
    print("%s: %d rows, max|dO| %.3e max|dLSE| %s" % (name, len(rows), e[0], e[1]))


# ---------------------------------------------------------------------------
# grouped KV heads with short segments: a workgroup takes several query heads
# of one KV head (pack_mode 2)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("heads,heads_k,lens", [
    (16, 4, "le64"), (32, 4, "le64"), (12, 3, "le128"), (16, 8, "le128"),
])
@pytest.mark.parametrize("mode", ["full", "causal", "window"])
def test_packed_query_heads(dims, heads, heads_k, lens, mode):
    g = np.random.default_rng(heads * 31 + heads_k + dims[0])
    hi = 64 if lens == "le64" else 128
    lq = g.integers(0, hi + 1, 11).tolist()
    lq[0] = hi
    lk = [x + int(g.integers(0, 300)) for x in lq]
    causal, window = MODES[mode]
    inp = workloads.make_inputs(lq, lk, heads, dims[0], dims[1], seed=hi + heads, causal=causal, window=window,
                                num_heads_k=heads_k)
    assert va.plan(dims[0], dims[1], len(lq), heads, hi, max(lk), causal, num_heads_k=heads_k)["pack_mode"] == 2
    out, lse = run_gpu(inp)
    ref_o, ref_lse = oracle_on(inp)
    assert_parity(out, lse, ref_o, ref_lse, what="packed heads %s %d/%d %s %s" % (dims, heads, heads_k, lens, mode))
    # the same call with a looser max_seqlen_q runs unpacked on the four-wave
    # kernel (4096: enough 256-row units that the launch is not split by
    # keys): same rows, same tiles, same bits
    import dataclasses
    assert va.plan(dims[0], dims[1], len(lq), heads, 4096, max(lk), causal, num_heads_k=heads_k)["key_split"] == 1
    out2, lse2 = run_gpu(dataclasses.replace(inp, max_seqlen_q=4096))
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


# ---------------------------------------------------------------------------
# bf16 inputs, e4m3 output under a static per-tensor scale
# (varlen_attn_fwd_quant_out)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dims", DIMS, ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", ["full", "causal", "window"])
@pytest.mark.parametrize("with_lse", [True, False])
def test_quantised_output(dims, mode, with_lse):
    """O before rounding is within the bf16 path's 2e-2 of the oracle; the
    e4m3 rounding adds at most half an ulp of O / s (2^-4 relative, 2^-10
    absolute below the normal range): |decode(code) s - O_ref| <= 2e-2 +
    s max(2^-4 (|O_ref| + 2e-2) / s, 2^-10).  The LSE is the bf16 call's."""
    lq, lk = LEN_SETS["ragged"]
    causal, window = MODES[mode]
    inp = workloads.make_inputs(lq, lq, 4, dims[0], dims[1], seed=dims[0] + len(mode), causal=causal, window=window)
    ref_o, ref_lse = oracle_on(inp)
    s = float(np.float32(np.nanmax(np.abs(ref_o)) / 100.0))
    d = inp.to(DEV)
    sc = torch.tensor([s], dtype=torch.float32, device=DEV)
    # one byte an element: d_v 72 needs heads padded to 80 bytes (16-byte strides)
    dvp = -(-dims[1] // 16) * 16
    out_buf = torch.empty((inp.q.shape[0], 4, dvp), dtype=torch.float8_e4m3fn, device=DEV)
    res = va.varlen_attn_fwd(d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, inp.max_seqlen_q, inp.max_seqlen_k,
                             softmax_scale=inp.softmax_scale, causal=causal, window_size=window,
                             return_lse=with_lse, out_scale=sc, out=out_buf[:, :, :dims[1]])
    out, lse = res if with_lse else (res, None)
    torch.cuda.synchronize()
    assert out.dtype == torch.float8_e4m3fn
    got = oracle.e4m3_decode(out.cpu().contiguous().view(torch.uint8).numpy()) * s
    tol = 2e-2 + s * np.maximum(2.0 ** -4 * (np.abs(ref_o) + 2e-2) / s, 2.0 ** -10)
    err = np.abs(got - ref_o)
    assert np.all(err <= tol), "max excess %.3e" % float(np.max(err - tol))
    ref_out, ref_l = run_gpu(inp, return_lse=with_lse)
    if with_lse:
        assert torch.equal(lse, ref_l)
    # the codes are the RNE e4m3 codes of the bf16 call's O / s wherever that
    # O (bf16-rounded) is not within a bf16 ulp of a rounding boundary: check
    # the decoded values agree within one e4m3 ulp everywhere
    y = f64(ref_out) / s
    ulp = np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(got / s - np.clip(y, -448, 448)) <= ulp)


def test_quantised_output_default_allocation_d72():
    """d_v 72 with out=None: the binding allocates a contiguous [T, H, 72]
    e4m3 tensor (72-byte heads, which the 8-byte rule for e4m3 outputs
    accepts); its codes equal those written into a head-padded buffer."""
    lq = [300, 77, 129]
    inp = workloads.make_inputs(lq, lq, 4, 72, 72, seed=72, causal=True)
    d = inp.to(DEV)
    sc = torch.tensor([0.01], dtype=torch.float32, device=DEV)
    args = (d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, inp.max_seqlen_q, inp.max_seqlen_k)
    out = va.varlen_attn_fwd(*args, causal=True, out_scale=sc)
    buf = torch.empty((inp.q.shape[0], 4, 80), dtype=torch.float8_e4m3fn, device=DEV)
    out2 = va.varlen_attn_fwd(*args, causal=True, out_scale=sc, out=buf[:, :, :72])
    torch.cuda.synchronize()
    assert out.shape == (inp.q.shape[0], 4, 72) and out.is_contiguous()
    assert torch.equal(out.view(torch.uint8), out2.view(torch.uint8))
    ref_o, _ = oracle_on(inp)
    got = oracle.e4m3_decode(out.cpu().view(torch.uint8).numpy()) * 0.01
    tol = 2e-2 + 0.01 * np.maximum(2.0 ** -4 * (np.abs(ref_o) + 2e-2) / 0.01, 2.0 ** -10)
    assert np.all(np.abs(got - ref_o) <= tol)


def _host_counts(lk, max_splits, keys_per_split):
    return [min(max(-(-x // keys_per_split), 1), max_splits) for x in lk]


def test_splitkv_counts_kernel():
    """varlen_attn_splitkv_counts against the formula it documents."""
    lk = [0, 1, 511, 512, 513, 4096, 70000, 33, 100000]
    cu = workloads.cu_seqlens(lk).to(DEV)
    for mx, kps in ((8, 512), (128, 512), (3, 1000), (1, 512)):
        got = va.splitkv_counts(cu, mx, kps).cpu().tolist()
        assert got == _host_counts(lk, mx, kps), (mx, kps, got)


@pytest.mark.parametrize("dims", [(64, 64), (80, 80), (192, 128)], ids=lambda d: "d%d_%d" % d)
@pytest.mark.parametrize("mode", ["full", "causal", "window"])
def test_split_kv_dynamic_counts(dims, mode):
    """Per-segment split counts (num_splits_dynamic): explicit counts with
    zero, one, more than num_splits and in between, and the library's own
    ("auto"), on segments of very different key lengths (short queries
    that the plain launch would pack several to a workgroup, and long
    ones), against the oracle; counts all equal to num_splits give the
    static split call bit for bit."""
    causal, window = MODES[mode]
    lq, lk = [1, 64, 17, 300, 40], [3000, 64, 900, 1200, 0]
    S = 6
    seed = zlib.crc32(repr(("dyn", dims, mode)).encode()) % 1000
    inp = workloads.make_inputs(lq, lk, 3, dims[0], dims[1], seed=seed, causal=causal, window=window)
    ref_o, ref_lse = oracle_on(inp)
    d = inp.to(DEV)
    args = (d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, inp.max_seqlen_q, inp.max_seqlen_k)
    kw = dict(softmax_scale=inp.softmax_scale, causal=causal, window_size=window, return_lse=True, num_splits=S)
    for counts in ([0, 1, 9, 3, 2], [S] * 5, "auto"):
        dyn = counts if isinstance(counts, str) else torch.tensor(counts, dtype=torch.int32, device=DEV)
        out, lse = va.varlen_attn_fwd(*args, num_splits_dynamic=dyn, **kw)
        torch.cuda.synchronize()
        assert_parity(out, lse, ref_o, ref_lse, what="dyn %s %s %s" % (dims, mode, counts))
        if counts == [S] * 5:
            o2, l2 = va.varlen_attn_fwd(*args, **kw)
            torch.cuda.synchronize()
            assert torch.equal(out, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("dims", [(80, 80), (128, 128)], ids=lambda d: "d%d_%d" % d)
def test_split_kv_dynamic_counts_short_queries(dims):
    """Every segment at most 64 queries, so the plain launch would pack four
    segments to a workgroup; with per-segment counts each workgroup holds one
    segment.  Against the oracle, causal (bottom-right, q < k)."""
    lq, lk = [64, 1, 30, 64, 7, 64], [2000, 64, 700, 5000, 7, 64]
    inp = workloads.make_inputs(lq, lk, 4, dims[0], dims[1], seed=dims[0] + 5, causal=True)
    ref_o, ref_lse = oracle_on(inp)
    d = inp.to(DEV)
    for counts in ([4, 1, 2, 8, 1, 1], "auto"):
        dyn = counts if isinstance(counts, str) else torch.tensor(counts, dtype=torch.int32, device=DEV)
        out, lse = va.varlen_attn_fwd(d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, 64, 5000, causal=True,
                                      return_lse=True, num_splits=8, num_splits_dynamic=dyn)
        torch.cuda.synchronize()
        assert_parity(out, lse, ref_o, ref_lse, what="dyn short %s %s" % (dims, counts))


def test_concurrent_streams_bit_equal():
    """Calls on different HIP streams at once share nothing: a short-segment
    (one-wave kernel) call, a causal d 128 call, a split-KV 192/128 call
    with its own workspace and a merge, each launched three times on its own
    stream (default priority) and interleaved, give outputs bit-equal to the
    same calls run one after another on the default stream."""
    short = [64, 17, 64, 40] * 6
    cases = [
        workloads.make_inputs(short, short, 8, 80, 80, seed=501),
        workloads.make_inputs([700, 300, 1029], [700, 300, 1029], 4, 128, 128, seed=502, causal=True),
        workloads.make_inputs([256, 64], [5000, 3000], 4, 192, 128, seed=503, causal=True),
    ]
    dev = [c.to(DEV) for c in cases]
    splits = [1, 1, 4]

    def call(i, out, lse):
        d = dev[i]
        return va.varlen_attn_fwd(d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, d.max_seqlen_q, d.max_seqlen_k,
                                  softmax_scale=d.softmax_scale, causal=d.causal, window_size=d.window,
                                  out=out, return_lse=True, lse=lse, num_splits=splits[i])

    def buffers(i):
        d = dev[i]
        out = torch.full((d.q.shape[0], d.q.shape[1], d.v.shape[2]), 7.0, dtype=torch.bfloat16, device=DEV)
        lse = torch.full((d.q.shape[1], d.q.shape[0]), 7.0, dtype=torch.float32, device=DEV)
        return out, lse

    ref = []
    for i in range(len(cases)):
        out, lse = buffers(i)
        call(i, out, lse)
        ref.append((out, lse))
    # the merge of case 2 with itself: O unchanged, LSE + ln 2
    m_ref = va.varlen_attn_merge(ref[2][0], ref[2][1], ref[2][0], ref[2][1])
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in range(len(cases) + 1)]
    bufs = [[buffers(i) for _ in range(3)] for i in range(len(cases))]
    merged = []
    torch.cuda.synchronize()
    for rep in range(3):
        for i, s in enumerate(streams[:-1]):
            with torch.cuda.stream(s):
                call(i, *bufs[i][rep])
        with torch.cuda.stream(streams[-1]):
            merged.append(va.varlen_attn_merge(ref[2][0], ref[2][1], ref[2][0], ref[2][1]))
    torch.cuda.synchronize()
    for i in range(len(cases)):
        for rep in range(3):
            out, lse = bufs[i][rep]
            assert torch.equal(out, ref[i][0]) and torch.equal(lse, ref[i][1]), (i, rep)
    for o, l in merged:
        assert torch.equal(o, m_ref[0]) and torch.equal(l, m_ref[1])
