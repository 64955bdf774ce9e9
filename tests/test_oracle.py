"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: hand-enumerated
mask sets (tests/golden/mask_cases.json), closed forms stated for this
method (single key, zero Q, constant V, key permutation), an exactly
summable geometric case, and a library routine for the special case of an
explicit boolean mask (torch's scaled_dot_product_attention and logsumexp in
float64).  The last group plants plausible mistakes in the oracle and checks
that one of these pins fails for each.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oracle_mod
from varlen_attention_forward_amd import workloads
from helpers import f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _mask_cases():
    with open(os.path.join(GOLDEN, "mask_cases.json")) as f:
        return json.load(f)["cases"]


def _run(q, k, v, cu_q, cu_k, scale, causal=False, wl=-1, wr=-1):
    return oracle.attention_fwd(q, k, v, cu_q, cu_k, scale, causal, wl, wr)


# --------------------------------------------------------------------------
# mask reading: hand-enumerated sets
# --------------------------------------------------------------------------


def check_mask_fixture():
    for c in _mask_cases():
        m = oracle.visible_mask(c["Lq"], c["Lk"], c["causal"], *c["window"])
        got = [sorted(np.nonzero(row)[0].tolist()) for row in m]
        assert got == c["visible"], (c, got)


def test_mask_fixture():
    check_mask_fixture()


def test_mask_fixture_through_attention():
    """The attention itself (not just the mask helper) honours the sets:
    with Q = 0 every visible score is 0, so O = mean of visible V rows and
    LSE = ln |J_i| (closed form for zero queries)."""
    rng = np.random.default_rng(0)
    for c in _mask_cases():
        Lq, Lk = c["Lq"], c["Lk"]
        q = np.zeros((Lq, 1, 8))
        k = rng.standard_normal((Lk, 1, 8))
        v = rng.standard_normal((Lk, 1, 4))
        o, lse = _run(q, k, v, [0, Lq], [0, Lk], 0.5, c["causal"], *c["window"])
        for i, vis in enumerate(c["visible"]):
            if vis:
                np.testing.assert_allclose(o[i, 0], v[vis, 0].mean(axis=0), rtol=0, atol=1e-13)
                assert abs(lse[0, i] - math.log(len(vis))) < 1e-13
            else:
                assert np.all(o[i, 0] == 0.0) and lse[0, i] == -np.inf


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------


def check_single_key(seed=1):
    """Lk = 1: O = V[0] and LSE = scale * q.k for every query row."""
    rng = np.random.default_rng(seed)
    for d_qk, d_v in [(64, 64), (80, 80), (192, 128)]:
        q = rng.standard_normal((5, 3, d_qk))
        k = rng.standard_normal((1, 3, d_qk))
        v = rng.standard_normal((1, 3, d_v))
        scale = 0.37
        o, lse = _run(q, k, v, [0, 5], [0, 1], scale)
        s32 = float(np.float32(scale))
        for h in range(3):
            for i in range(5):
                dot = math.fsum(q[i, h, c] * k[0, h, c] for c in range(d_qk))
                assert abs(lse[h, i] - s32 * dot) < 1e-12 * max(1.0, abs(s32 * dot))
                np.testing.assert_allclose(o[i, h], v[0, h], rtol=0, atol=1e-14)


def test_single_key():
    check_single_key()


def check_zero_q():
    """Q = 0: every score is 0, so O = mean(V) and LSE = ln n."""
    rng = np.random.default_rng(2)
    n = 37
    q = np.zeros((11, 2, 64))
    k = rng.standard_normal((n, 2, 64))
    v = rng.standard_normal((n, 2, 64))
    o, lse = _run(q, k, v, [0, 11], [0, n], 0.125)
    for h in range(2):
        np.testing.assert_allclose(o[:, h], np.broadcast_to(v[:, h].mean(0), (11, 64)), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[h], math.log(n), rtol=0, atol=1e-13)


def test_zero_q():
    check_zero_q()


def check_constant_v():
    """V rows all equal c: O = c whatever the weights."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((9, 2, 80)) * 3
    k = rng.standard_normal((13, 2, 80)) * 3
    c = rng.standard_normal((2, 80))
    v = np.broadcast_to(c, (13, 2, 80)).copy()
    o, _ = _run(q, k, v, [0, 9], [0, 13], 80 ** -0.5, causal=True)
    for h in range(2):
        np.testing.assert_allclose(o[:, h], np.broadcast_to(c[h], (9, 80)), rtol=1e-13, atol=1e-13)


def test_constant_v():
    check_constant_v()


def test_key_permutation_invariance():
    """Non-causal: permuting keys together with their values changes nothing."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((7, 2, 64))
    k = rng.standard_normal((19, 2, 64))
    v = rng.standard_normal((19, 2, 64))
    perm = rng.permutation(19)
    o1, l1 = _run(q, k, v, [0, 7], [0, 19], 0.125)
    o2, l2 = _run(q, k[perm], v[perm], [0, 7], [0, 19], 0.125)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)


def check_geometric():
    """Integer scores s_j = j (scale 1, q = e_0, k_j = j e_0) with one-hot V rows:
    O_i[j] = e^j / S and LSE = ln S with S = (e^n - 1) / (e - 1)."""
    n = 12
    q = np.zeros((1, 1, 16))
    q[0, 0, 0] = 1.0
    k = np.zeros((n, 1, 16))
    k[:, 0, 0] = np.arange(n)
    v = np.zeros((n, 1, 16))
    v[np.arange(n), 0, np.arange(n)] = 1.0
    o, lse = _run(q, k, v, [0, 1], [0, n], 1.0)
    S = (math.e ** n - 1) / (math.e - 1)
    assert abs(lse[0, 0] - math.log(S)) < 1e-12
    for j in range(n):
        assert abs(o[0, 0, j] - math.e ** j / S) < 1e-14
    # causal, Lq = Lk = n: row i sees keys 0..i
    qq = np.repeat(q, n, axis=0)
    o, lse = _run(qq, k, v, [0, n], [0, n], 1.0, causal=True)
    for i in range(n):
        Si = (math.e ** (i + 1) - 1) / (math.e - 1)
        assert abs(lse[0, i] - math.log(Si)) < 1e-12
        assert abs(o[i, 0, i] - math.e ** i / Si) < 1e-14
        assert np.all(o[i, 0, i + 1 :] == 0.0)


def test_geometric_case():
    check_geometric()


def test_scale_is_rounded_to_fp32():
    """The oracle uses float32(scale), the value the C interface carries."""
    q = np.ones((1, 1, 8))
    k = np.ones((1, 1, 8))
    v = np.ones((1, 1, 8))
    _, lse = _run(q, k, v, [0, 1], [0, 1], 0.1)
    assert lse[0, 0] == float(np.float32(0.1)) * 8.0


def test_segments_are_independent():
    """Packing: a segment's result equals the result of running it alone."""
    inp = workloads.make_inputs([5, 17, 0, 9], [7, 17, 3, 9], 2, 64, 64, seed=5, causal=True)
    q, k, v = f64(inp.q), f64(inp.k), f64(inp.v)
    cu_q, cu_k = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
    o, lse = _run(q, k, v, cu_q, cu_k, inp.softmax_scale, True)
    for b in range(4):
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        o1, l1 = _run(q[qs], k[ks], v[ks], [0, cu_q[b + 1] - cu_q[b]], [0, cu_k[b + 1] - cu_k[b]], inp.softmax_scale, True)
        assert np.array_equal(o[qs], o1) and np.array_equal(lse[:, qs], l1)


# --------------------------------------------------------------------------
# library routine on the special case of an explicit mask
# --------------------------------------------------------------------------


def _distance_mask(Lq, Lk, causal, wl, wr):
    """Brute-force (i, j) enumeration of the reading, phrased with positions:
    query i is at position Lk - Lq + i on the key axis."""
    m = np.zeros((Lq, Lk), dtype=bool)
    for i in range(Lq):
        pos = Lk - Lq + i
        for j in range(Lk):
            ok = True
            if causal and j > pos:
                ok = False
            if wl >= 0 and pos - j > wl:
                ok = False
            if (not causal) and wr >= 0 and j - pos > wr:
                ok = False
            m[i, j] = ok
    return m


def test_interval_mask_matches_brute_force():
    for Lq in range(0, 7):
        for Lk in range(0, 7):
            for causal in (False, True):
                for wl in range(-1, 4):
                    for wr in range(-1, 4):
                        a = oracle.visible_mask(Lq, Lk, causal, wl, wr)
                        b = _distance_mask(Lq, Lk, causal, wl, wr)
                        assert np.array_equal(a, b), (Lq, Lk, causal, wl, wr)


DIMS = [(64, 64), (72, 72), (80, 80), (128, 128), (192, 128)]


@pytest.mark.parametrize("dims", DIMS)
@pytest.mark.parametrize("mode", ["none", "causal", "window", "causal_window"])
def test_against_sdpa(dims, mode):
    d_qk, d_v = dims
    causal = mode.startswith("causal")
    wl, wr = (-1, -1)
    if mode == "window":
        wl, wr = 5, 3
    if mode == "causal_window":
        wl, wr = 6, -1
    seqlens_q = [1, 23, 40, 64]
    seqlens_k = [1, 31, 40, 50]
    inp = workloads.make_inputs(seqlens_q, seqlens_k, 3, d_qk, d_v, seed=7 + d_qk, causal=causal, window=(wl, wr))
    q, k, v = f64(inp.q), f64(inp.k), f64(inp.v)
    cu_q, cu_k = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
    o, lse = _run(q, k, v, cu_q, cu_k, inp.softmax_scale, causal, wl, wr)
    scale = float(np.float32(inp.softmax_scale))
    for b in range(len(seqlens_q)):
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        Lq, Lk = seqlens_q[b], seqlens_k[b]
        m = torch.from_numpy(_distance_mask(Lq, Lk, causal, wl, wr))
        tq = torch.from_numpy(q[qs]).transpose(0, 1)  # [H, Lq, d]
        tk = torch.from_numpy(k[ks]).transpose(0, 1)
        tv = torch.from_numpy(v[ks]).transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale)
        scores = torch.matmul(tq, tk.transpose(1, 2).contiguous()) * scale
        scores = scores.masked_fill(~m, float("-inf"))
        ref_lse = torch.logsumexp(scores, dim=-1)  # [H, Lq]
        rows = m.any(dim=1).numpy()
        got = o[qs].transpose(1, 0, 2)  # [H, Lq, d_v]
        np.testing.assert_allclose(got[:, rows], ref.numpy()[:, rows], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[:, qs][:, rows], ref_lse.numpy()[:, rows], rtol=1e-12, atol=1e-12)
        assert np.all(got[:, ~rows] == 0.0)
        assert np.all(lse[:, qs][:, ~rows] == -np.inf)


@pytest.mark.parametrize("heads,heads_k", [(6, 1), (6, 2), (8, 4), (4, 4)])
def test_grouped_kv_heads_against_sdpa(heads, heads_k):
    """Grouped KV heads: query head h uses KV head h // (H // H_kv).  Pinned
    to torch's scaled_dot_product_attention with enable_gqa (float64), which
    repeats each KV head over consecutive query heads."""
    seqlens_q, seqlens_k = [5, 33, 17], [9, 33, 40]
    inp = workloads.make_inputs(seqlens_q, seqlens_k, heads, 64, 64, seed=31 + heads_k, causal=True,
                                num_heads_k=heads_k)
    q, k, v = f64(inp.q), f64(inp.k), f64(inp.v)
    assert k.shape[1] == heads_k and v.shape[1] == heads_k
    cu_q, cu_k = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
    o, lse = _run(q, k, v, cu_q, cu_k, inp.softmax_scale, True)
    scale = float(np.float32(inp.softmax_scale))
    for b in range(len(seqlens_q)):
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        m = torch.from_numpy(_distance_mask(seqlens_q[b], seqlens_k[b], True, -1, -1))
        tq = torch.from_numpy(q[qs]).transpose(0, 1)
        tk = torch.from_numpy(k[ks]).transpose(0, 1)
        tv = torch.from_numpy(v[ks]).transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale,
                                                               enable_gqa=True)
        rows = m.any(dim=1).numpy()
        got = o[qs].transpose(1, 0, 2)
        np.testing.assert_allclose(got[:, rows], ref.numpy()[:, rows], rtol=1e-10, atol=1e-12)


def test_planted_interleaved_kv_grouping_is_caught(monkeypatch):
    """Reading KV head h % H_kv (interleaved grouping) instead of
    h // (H // H_kv) must fail the grouped-heads pin."""
    orig = oracle_mod.attention_fwd

    def interleaved(q, k, v, *a, **kw):
        hk = k.shape[1]
        if hk == q.shape[1]:
            return orig(q, k, v, *a, **kw)
        rep = q.shape[1] // hk
        # tile (not repeat) the KV heads: query head h then reads h % H_kv
        return orig(q, np.tile(k, (1, rep, 1)), np.tile(v, (1, rep, 1)), *a, **kw)

    monkeypatch.setattr(oracle, "attention_fwd", interleaved)
    assert _fails(lambda: test_grouped_kv_heads_against_sdpa(6, 2))


def test_rows_subset_matches_full():
    inp = workloads.make_inputs([100, 37], [120, 37], 4, 64, 64, seed=9, causal=True)
    q, k, v = f64(inp.q), f64(inp.k), f64(inp.v)
    cu_q, cu_k = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
    o, lse = _run(q, k, v, cu_q, cu_k, inp.softmax_scale, True)
    rows = np.array([0, 5, 99, 100, 136])
    o2, l2 = oracle.attention_fwd(q, k, v, cu_q, cu_k, inp.softmax_scale, True, rows=rows, heads=[1, 3])
    assert np.array_equal(o2[rows][:, [1, 3]], o[rows][:, [1, 3]])
    assert np.array_equal(l2[[1, 3]][:, rows], lse[[1, 3]][:, rows])
    assert np.isnan(o2[1]).all() and np.isnan(o2[rows][:, 0]).all()


def test_visible_pairs_closed_forms():
    # non-causal: Lq * Lk; causal square: L (L + 1) / 2
    assert oracle.visible_pairs([0, 64, 320], [0, 64, 320], False, -1, -1) == 64 * 64 + 256 * 256
    assert oracle.visible_pairs([0, 4096], [0, 4096], True, -1, -1) == 4096 * 4097 // 2


# --------------------------------------------------------------------------
# planted mistakes: each must make at least one pin above fail
# --------------------------------------------------------------------------


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_top_left_causal_is_caught(monkeypatch):
    orig = oracle_mod.visible_interval

    def top_left(i, Lq, Lk, causal, wl, wr):
        # plausible mistake: align the causal diagonal at the top-left corner
        return orig(i, Lk, Lk, causal, wl, wr)

    monkeypatch.setattr(oracle_mod, "visible_interval", top_left)
    assert _fails(check_mask_fixture)


def test_planted_log2_lse_is_caught(monkeypatch):
    real_log = np.log

    class _NP:
        def __getattr__(self, name):
            return getattr(np, name)

        @staticmethod
        def log(x):
            return real_log(x) / real_log(2.0)  # mistake: base-2 LSE

    monkeypatch.setattr(oracle_mod, "np", _NP())
    assert _fails(check_zero_q)


def test_planted_missing_scale_is_caught(monkeypatch):
    orig = oracle_mod._segment_head
    monkeypatch.setattr(oracle_mod, "_segment_head", lambda qs, ks, vs, scale, mask: orig(qs, ks, vs, 1.0, mask))
    assert _fails(check_single_key)


def test_planted_max_normalisation_is_caught(monkeypatch):
    def bad(qs, ks, vs, scale, mask):
        s = np.where(mask, scale * (qs @ ks.T), -np.inf)
        m = s.max(axis=1)
        w = np.exp(s - m[:, None])
        return w @ vs, m  # mistake: no division by the softmax sum

    monkeypatch.setattr(oracle_mod, "_segment_head", bad)
    assert _fails(check_constant_v)


def test_planted_transposed_probabilities_are_caught(monkeypatch):
    orig = oracle_mod._segment_head

    def bad(qs, ks, vs, scale, mask):
        o, l = orig(qs, ks, vs, scale, mask)
        return o[::-1].copy(), l  # mistake: rows of O assigned to the wrong queries

    monkeypatch.setattr(oracle_mod, "_segment_head", bad)
    assert _fails(check_geometric)
