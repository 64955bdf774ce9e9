"""GPU parity of varlen_attn_merge against the fp64 oracle (marked ``gpu``).

* random partial states (bf16 outputs, fp32 LSEs with -inf rows in either
  part or both) against the oracle's merge of the same values;
* merging in place (output = an input) and a strided output;
* split-KV and chunked prefill composed from varlen_attn_fwd calls over key
  parts and merges, against the oracle's attention over all the keys
  (O <= 2e-2, LSE <= 1e-3, -inf rows exactly).

All calls go through the C interface via the ctypes binding.
"""
import numpy as np
import pytest
import torch

import varlen_attention_forward_amd as va
from varlen_attention_forward_amd import workloads
from helpers import f64, f32
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O = 2e-2
TOL_LSE = 1e-3


def _random_states(rows, heads, dim, seed):
    g = torch.Generator().manual_seed(seed)
    oa = torch.randn((rows, heads, dim), generator=g).to(torch.bfloat16)
    ob = torch.randn((rows, heads, dim), generator=g).to(torch.bfloat16)
    la = torch.randn((heads, rows), generator=g) * 6
    lb = torch.randn((heads, rows), generator=g) * 6
    la[0, :7] = -float("inf")  # part a saw no key
    lb[0, 5:11] = -float("inf")  # part b saw no key (rows 5, 6: neither)
    oa[:7, 0] = float("nan")  # never read behind a -inf LSE
    ob[5:11, 0] = float("nan")
    return oa.to(DEV), la.to(DEV), ob.to(DEV), lb.to(DEV)


def _check(out, lse, want_o, want_l, what):
    o, l = f64(out), f64(lse)
    assert np.all(np.isfinite(o)), what
    assert np.max(np.abs(o - want_o)) <= TOL_O, what
    assert np.array_equal(l == -np.inf, want_l == -np.inf), what
    fin = want_l != -np.inf
    assert np.max(np.abs(l[fin] - want_l[fin])) <= TOL_LSE, what


@pytest.mark.parametrize("dim", [64, 72, 80, 128])
def test_merge_random_states(dim):
    oa, la, ob, lb = _random_states(1000, 3, dim, seed=dim)
    out, lse = va.varlen_attn_merge(oa, la, ob, lb)
    torch.cuda.synchronize()
    want_o, want_l = oracle.merge_states(f64(oa), f64(la), f64(ob), f64(lb))
    _check(out, lse, want_o, want_l, "merge d=%d" % dim)
    # rows 5, 6 of head 0 saw no key in either part
    assert torch.all(out[5:7, 0] == 0) and torch.all(lse[0, 5:7] == -float("inf"))
    # the merge is exact up to one rounding of O to bf16 and fp32 exp/log
    fin = want_l != -np.inf
    assert np.max(np.abs(f64(lse)[fin] - want_l[fin])) <= 1e-5


def test_merge_in_place_and_strided_out():
    oa, la, ob, lb = _random_states(333, 4, 128, seed=5)
    ref_o, ref_l = va.varlen_attn_merge(oa, la, ob, lb)
    big = torch.zeros((333, 4, 160), dtype=torch.bfloat16, device=DEV)
    strided = big[:, :, 16:144]  # row stride 640, head stride 160
    va.varlen_attn_merge(oa, la, ob, lb, out=strided, return_lse=False)
    a2, l2 = oa.clone(), la.clone()
    va.varlen_attn_merge(a2, l2, ob, lb, out=a2, lse=l2)  # in place over part a
    torch.cuda.synchronize()
    assert torch.equal(strided, ref_o) and torch.all(big[:, :, :16] == 0) and torch.all(big[:, :, 144:] == 0)
    assert torch.equal(a2, ref_o) and torch.equal(l2, ref_l)


def _fwd(q, k, v, cu_q, cu_k, lens_q, lens_k, scale, causal):
    out, lse = va.varlen_attn_fwd(q, k, v, cu_q, cu_k, max(lens_q), max(lens_k), softmax_scale=scale,
                                  causal=causal, return_lse=True)
    return out, lse


def _cu(lens):
    return workloads.cu_seqlens(lens).to(DEV)


@pytest.mark.parametrize("dims", [(128, 128), (80, 80), (64, 64)], ids=lambda d: "d%d" % d[0])
def test_split_kv_by_merge(dims):
    """Keys of every segment split at a cut (empty first or second parts, a
    multi-tile part, Lq != Lk): fwd over each part, merged, equals attention
    over all keys."""
    d_qk, d_v = dims
    lq, lk = [300, 17, 513, 64], [700, 333, 513, 0]
    cuts = [0, 333, 200, 0]
    inp = workloads.make_inputs(lq, lk, 2, d_qk, d_v, seed=31)
    q, k, v = inp.q.to(DEV), inp.k.to(DEV), inp.v.to(DEV)
    cu_q = inp.cu_seqlens_q.to(DEV)
    cuk = inp.cu_seqlens_k.tolist()
    parts = []
    for first in (True, False):
        ks, vs, lens = [], [], []
        for b, cut in enumerate(cuts):
            k0, k1 = cuk[b], cuk[b + 1]
            lo, hi = (k0, k0 + cut) if first else (k0 + cut, k1)
            ks.append(k[lo:hi]), vs.append(v[lo:hi]), lens.append(hi - lo)
        parts.append(_fwd(q, torch.cat(ks).contiguous(), torch.cat(vs).contiguous(), cu_q, _cu(lens), lq,
                          [max(1, x) for x in lens], inp.softmax_scale, False))
    out, lse = va.varlen_attn_merge(parts[0][0], parts[0][1], parts[1][0], parts[1][1])
    torch.cuda.synchronize()
    want_o, want_l = oracle.attention_fwd(f32(inp.q), f32(inp.k), f32(inp.v), inp.cu_seqlens_q.tolist(), cuk,
                                          inp.softmax_scale)
    _check(out, lse, want_o, want_l, "split-kv %s" % (dims,))


def test_chunked_prefill_by_merge():
    """A causal prefill of new tokens after a context read separately: the
    context part (non-causal) merged with the new-token part (causal) equals
    causal attention over context + new keys (bottom-right alignment), at the
    MLA head dims with LSE."""
    ln, lc = [257, 100, 64], [1000, 0, 333]
    heads, d_qk, d_v = 4, 192, 128
    g = torch.Generator().manual_seed(41)
    q = torch.randn((sum(ln), heads, d_qk), generator=g).to(torch.bfloat16)
    kc = torch.randn((sum(lc), heads, d_qk), generator=g).to(torch.bfloat16)
    vc = torch.randn((sum(lc), heads, d_v), generator=g).to(torch.bfloat16)
    kn = torch.randn((sum(ln), heads, d_qk), generator=g).to(torch.bfloat16)
    vn = torch.randn((sum(ln), heads, d_v), generator=g).to(torch.bfloat16)
    scale = d_qk ** -0.5
    qd = q.to(DEV)
    ctx = _fwd(qd, kc.to(DEV), vc.to(DEV), _cu(ln), _cu(lc), ln, [max(1, x) for x in lc], scale, False)
    new = _fwd(qd, kn.to(DEV), vn.to(DEV), _cu(ln), _cu(ln), ln, ln, scale, True)
    out, lse = va.varlen_attn_merge(ctx[0], ctx[1], new[0], new[1])
    torch.cuda.synchronize()
    cu_l, cu_n = workloads.cu_seqlens(lc).tolist(), workloads.cu_seqlens(ln).tolist()
    kall, vall = [], []
    for b in range(len(ln)):
        kall += [kc[cu_l[b]:cu_l[b + 1]], kn[cu_n[b]:cu_n[b + 1]]]
        vall += [vc[cu_l[b]:cu_l[b + 1]], vn[cu_n[b]:cu_n[b + 1]]]
    want_o, want_l = oracle.attention_fwd(f32(q), f32(torch.cat(kall)), f32(torch.cat(vall)), cu_n,
                                          workloads.cu_seqlens([a + b for a, b in zip(lc, ln)]).tolist(), scale,
                                          causal=True)
    _check(out, lse, want_o, want_l, "chunked prefill")
