"""Pins for the oracle's merge of two attention results (CPU only).

The merge is tied to the attention definition, not to its own formula:
attention of every query over two disjoint parts of its keys, merged, must
equal attention over all the keys (with parts that may be empty, Lq != Lk,
and a causal prefill split into its context and its new tokens).  Exact
identities (an empty part, order of merging) and planted mistakes follow.
"""
import numpy as np
import pytest

import oracle
from oracle import merge as merge_mod


def _bf16_exact(rng, shape):
    # values on the bf16 grid, like the GPU inputs
    x = rng.standard_normal(shape).astype(np.float32)
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def _split_keys(k, v, cu_k, cuts):
    """Keys of segment b split at cuts[b] into parts [0, cut) and [cut, Lk)."""
    ka, va, kb, vb, la, lb = [], [], [], [], [], []
    for b, cut in enumerate(cuts):
        k0, k1 = cu_k[b], cu_k[b + 1]
        ka.append(k[k0:k0 + cut]), va.append(v[k0:k0 + cut]), la.append(cut)
        kb.append(k[k0 + cut:k1]), vb.append(v[k0 + cut:k1]), lb.append(k1 - k0 - cut)
    return (np.concatenate(ka), np.concatenate(va), _cu(la)), (np.concatenate(kb), np.concatenate(vb), _cu(lb))


def check_split_keys(seed=0, d=64, heads=3):
    rng = np.random.default_rng(seed)
    lq, lk = [5, 1, 9, 4, 7], [6, 3, 9, 0, 12]
    cuts = [0, 3, 4, 0, 12]  # empty first part, empty second part, both, Lq != Lk
    q = _bf16_exact(rng, (sum(lq), heads, d))
    k = _bf16_exact(rng, (sum(lk), heads, d))
    v = _bf16_exact(rng, (sum(lk), heads, d))
    cu_q, cu_k = _cu(lq), _cu(lk)
    scale = d ** -0.5
    want_o, want_l = oracle.attention_fwd(q, k, v, cu_q, cu_k, scale)
    (ka, va, cka), (kb, vb, ckb) = _split_keys(k, v, cu_k, cuts)
    oa, la = oracle.attention_fwd(q, ka, va, cu_q, cka, scale)
    ob, lb = oracle.attention_fwd(q, kb, vb, cu_q, ckb, scale)
    got_o, got_l = oracle.merge_states(oa, la, ob, lb)
    assert np.array_equal(got_l == -np.inf, want_l == -np.inf)
    fin = want_l != -np.inf
    assert np.max(np.abs(got_l[fin] - want_l[fin])) < 1e-12
    assert np.max(np.abs(got_o - want_o)) < 1e-12


def check_chunked_prefill(seed=1, d=80, heads=2):
    """Causal prefill of Lq new tokens after Lc context tokens = the context
    part (non-causal, Lq x Lc) merged with the new-token part (causal,
    Lq x Lq): the bottom-right causal reading over all Lc + Lq keys."""
    rng = np.random.default_rng(seed)
    lc, ln = [13, 0, 5], [7, 6, 1]
    q = _bf16_exact(rng, (sum(ln), heads, d))
    kc, vc = _bf16_exact(rng, (sum(lc), heads, d)), _bf16_exact(rng, (sum(lc), heads, d))
    kn, vn = _bf16_exact(rng, (sum(ln), heads, d)), _bf16_exact(rng, (sum(ln), heads, d))
    scale = d ** -0.5
    cu_q, cu_c = _cu(ln), _cu(lc)
    oc, lsec = oracle.attention_fwd(q, kc, vc, cu_q, cu_c, scale, causal=False)
    on, lsen = oracle.attention_fwd(q, kn, vn, cu_q, cu_q, scale, causal=True)
    got_o, got_l = oracle.merge_states(oc, lsec, on, lsen)
    # all keys of segment b: its context, then its new tokens
    kall, vall, lall = [], [], []
    for b in range(len(ln)):
        kall += [kc[cu_c[b]:cu_c[b + 1]], kn[cu_q[b]:cu_q[b + 1]]]
        vall += [vc[cu_c[b]:cu_c[b + 1]], vn[cu_q[b]:cu_q[b + 1]]]
        lall.append(lc[b] + ln[b])
    want_o, want_l = oracle.attention_fwd(q, np.concatenate(kall), np.concatenate(vall), cu_q, _cu(lall), scale,
                                          causal=True)
    assert np.max(np.abs(got_l - want_l)) < 1e-12
    assert np.max(np.abs(got_o - want_o)) < 1e-12


def test_merge_of_key_parts_is_attention_over_all_keys():
    check_split_keys()


def test_merge_of_context_and_new_tokens_is_causal_prefill():
    check_chunked_prefill()


def test_empty_part_is_the_identity():
    rng = np.random.default_rng(3)
    oa = rng.standard_normal((6, 2, 16))
    la = rng.standard_normal((2, 6))
    la[1, 2] = -np.inf
    oa[2, 1] = 0.0
    ob = np.full_like(oa, np.nan)  # never read: its LSE says it saw no key
    lb = np.full_like(la, -np.inf)
    o, lse = oracle.merge_states(oa, la, ob, lb)
    assert np.array_equal(o, oa) and np.array_equal(lse, la)
    o, lse = oracle.merge_states(ob, lb, oa, la)
    assert np.array_equal(o, oa) and np.array_equal(lse, la)


def test_merge_order_does_not_matter():
    rng = np.random.default_rng(4)
    parts = [(rng.standard_normal((5, 3, 8)), rng.standard_normal((3, 5)) * 4) for _ in range(3)]
    parts[1][1][0, 0] = -np.inf
    ab = oracle.merge_states(*parts[0], *parts[1])
    ba = oracle.merge_states(*parts[1], *parts[0])
    abc = oracle.merge_states(*ab, *parts[2])
    a_bc = oracle.merge_states(*parts[0], *oracle.merge_states(*parts[1], *parts[2]))
    for x, y in ((ab, ba), (abc, a_bc)):
        assert np.max(np.abs(x[0] - y[0])) < 1e-12 and np.max(np.abs(x[1] - y[1])) < 1e-12


# --------------------------------------------------------------------------
# planted mistakes in the merge: each must fail a pin above
# --------------------------------------------------------------------------


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_base2_merge_is_caught(monkeypatch):
    class _NP:
        def __getattr__(self, name):
            return getattr(np, name)

        @staticmethod
        def logaddexp(a, b):
            return np.logaddexp2(a, b)  # mistake: base-2 log-sum

    monkeypatch.setattr(merge_mod, "np", _NP())
    assert _fails(check_split_keys)


def test_planted_unnormalised_weights_are_caught(monkeypatch):
    class _NP:
        def __getattr__(self, name):
            return getattr(np, name)

        @staticmethod
        def exp(x):
            return np.exp(x) * 0.5 + 0.25  # mistake: weights that do not sum to one

    monkeypatch.setattr(merge_mod, "np", _NP())
    assert _fails(check_chunked_prefill)


def test_planted_swapped_parts_are_caught(monkeypatch):
    orig = merge_mod.merge_states

    def swapped(out_a, lse_a, out_b, lse_b):
        return orig(out_b, lse_a, out_a, lse_b)  # mistake: each weight on the other part's output

    monkeypatch.setattr(oracle, "merge_states", swapped)
    assert _fails(check_split_keys)
