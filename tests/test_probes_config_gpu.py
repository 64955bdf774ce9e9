"""Bit-exact probes of mask indexing and tile skipping at the full shapes of
the named workloads (marked ``gpu``).

Every expected result below is a closed form in integers, so all rows and
all heads are checked at full size, in the launch configuration that
bench.py times, without the fp64 oracle (only its visible-interval rule,
pinned by ``tests/test_oracle.py``, gives the expected key ranges):

* count probe (LSE returned): Q = 0 makes every visible score 0, so every
  probability is exactly 1 and the row sum is the integer n_i = |J_i|:
  round(exp(LSE)) must equal n_i, and a row with no visible key must get
  LSE = -inf and O = 0.  O is then the mean of V over J_i, checked against
  fp64 prefix sums of V within the 2e-2 tolerance.
* last-key probe (LSE returned): softmax scale 1, q = (1, 256, 65536, 0,
  ...) and k_j = (j mod 256, (j div 256) mod 256, j div 65536, 0, ...) with
  j the key's global index make s_j = j exactly (bf16 integers below 256
  and powers of two, products and sums exact in fp32), so
  LSE = j_max + ln sum_{t<n} e^-t: rounding LSE minus that tail recovers
  the last visible key of every row.
* key-bit probes (the workload's own LSE choice, i.e. the kernel
  instantiation bench.py times, which for the ViT workloads returns no
  LSE): the same K, V_jc = bit c of j for c < 17, and q = +(1, 256, 65536,
  0, ...) or its negative.  The largest (smallest) visible index then carries
  at least 1 / sum_t e^-t > 0.63 of the row's softmax weight and every
  other key together less than 0.37, so O_c > 1/2 exactly when bit c of
  that key is set: O alone gives the last and the first visible key of
  every row.

Keys are numbered globally, so reading past a segment's keys into a
neighbouring segment's (or into the padding after the last one) changes
the recovered key.  Inputs are built on the GPU (integers, bit patterns and
a seeded normal V).
"""
import math

import numpy as np
import pytest
import torch

import varlen_attention_forward_amd as va
from varlen_attention_forward_amd import workloads
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O = 2e-2
NBITS = 17  # key indices below 2^17 in every workload

CONFIG_WORKLOADS = [
    "tiny_varlen_d64",
    "vit_full_d80",
    "vit_window256_d80",
    "vit_window64_d80",
    "vit_long65536_d128",
    "mla_causal_192_128",
    "gqa_chunk64_d128",
]


def intervals(w):
    """Per global query row: the visible key count and the first and last
    visible key as global indices (-1 where none)."""
    n = np.zeros(w.total_q, dtype=np.int64)
    lo_g = np.full(w.total_q, -1, dtype=np.int64)
    hi_g = np.full(w.total_q, -1, dtype=np.int64)
    q0 = k0 = 0
    wl, wr = w.window
    for lq, lk in zip(w.seqlens_q, w.seqlens_k):
        lo, hi = oracle.visible_interval(np.arange(lq), lq, lk, w.causal, wl, wr)
        cnt = np.maximum(hi - lo + 1, 0)
        n[q0:q0 + lq] = cnt
        lo_g[q0:q0 + lq] = np.where(cnt > 0, k0 + lo, -1)
        hi_g[q0:q0 + lq] = np.where(cnt > 0, k0 + hi, -1)
        q0 += lq
        k0 += lk
    return n, lo_g, hi_g


class Probe:
    """Device tensors shared by the probes of one workload."""

    def __init__(self, w):
        assert w.total_k <= 2 ** NBITS and w.head_dim_v >= NBITS
        self.w = w
        T_q, T_k, H, H_kv = w.total_q, w.total_k, w.num_heads, w.heads_k
        self.cu_q = workloads.cu_seqlens(w.seqlens_q).to(DEV)
        self.cu_k = workloads.cu_seqlens(w.seqlens_k).to(DEV)
        j = torch.arange(T_k, device=DEV)
        self.k = torch.zeros((T_k, H_kv, w.head_dim_qk), dtype=torch.bfloat16, device=DEV)
        self.k[:, :, 0] = (j % 256).to(torch.bfloat16)[:, None]
        self.k[:, :, 1] = ((j // 256) % 256).to(torch.bfloat16)[:, None]
        self.k[:, :, 2] = (j // 65536).to(torch.bfloat16)[:, None]
        self.v_bits = torch.zeros((T_k, H_kv, w.head_dim_v), dtype=torch.bfloat16, device=DEV)
        for c in range(NBITS):
            self.v_bits[:, :, c] = ((j >> c) & 1).to(torch.bfloat16)[:, None]
        g = torch.Generator(device=DEV).manual_seed(w.seed)
        self.v_rand = torch.randn((T_k, H_kv, w.head_dim_v), generator=g, device=DEV).to(torch.bfloat16)
        self.q = torch.zeros((T_q, H, w.head_dim_qk), dtype=torch.bfloat16, device=DEV)

    def set_q(self, sign):
        """Q = 0 (sign 0) or sign * (1, 256, 65536, 0, ...) on every row and head."""
        self.q.zero_()
        if sign:
            self.q[:, :, 0] = float(sign)
            self.q[:, :, 1] = float(256 * sign)
            self.q[:, :, 2] = float(65536 * sign)

    def run(self, v, scale, return_lse):
        w = self.w
        res = va.varlen_attn_fwd(self.q, self.k, v, self.cu_q, self.cu_k, w.max_seqlen_q, w.max_seqlen_k,
                                 softmax_scale=scale, causal=w.causal, window_size=w.window,
                                 return_lse=return_lse)
        torch.cuda.synchronize()
        return res if return_lse else (res, None)


def decode_bits(out):
    """The key index whose bits O[..., :NBITS] hold (O_c > 1/2 <=> bit c set)."""
    bits = (out[:, :, :NBITS].float() > 0.5).to(torch.int64).cpu()
    return (bits << torch.arange(NBITS)).sum(dim=2).numpy()  # [T_q, H]


@pytest.fixture(scope="module", params=CONFIG_WORKLOADS)
def probe(request):
    p = Probe(workloads.WORKLOADS[request.param])
    yield p
    del p
    torch.cuda.empty_cache()


def test_count_probe(probe):
    w = probe.w
    n, lo_g, hi_g = intervals(w)
    probe.set_q(0)
    out, lse = probe.run(probe.v_rand, w.scale, True)
    l = lse.double().cpu().numpy()  # [H, T_q]
    empty = n == 0
    assert np.all(l[:, empty] == -np.inf), "%s: rows without keys must get LSE -inf" % w.name
    got = np.rint(np.exp(np.where(np.isfinite(l), l, 0.0))).astype(np.int64)
    bad = (got != n[None, :]) & ~empty[None, :]
    assert not bad.any(), "%s: visible counts differ at %d (head, row) pairs, first %s" % (
        w.name, int(bad.sum()), np.argwhere(bad)[:3].tolist())
    # O = mean of V over the visible keys, from fp64 prefix sums per segment
    grp = w.num_heads // w.heads_k
    q0 = k0 = 0
    worst = 0.0
    for lq, lk in zip(w.seqlens_q, w.seqlens_k):
        if lq == 0:
            k0 += lk
            continue
        rows = slice(q0, q0 + lq)
        o = out[rows].double()
        cnt = torch.from_numpy(n[rows]).to(DEV)
        if lk == 0:
            assert torch.all(o == 0)
        else:
            csum = torch.cat([torch.zeros((1,) + tuple(probe.v_rand.shape[1:]), dtype=torch.float64, device=DEV),
                              torch.cumsum(probe.v_rand[k0:k0 + lk].double(), dim=0)])
            lo = torch.from_numpy(np.maximum(lo_g[rows] - k0, 0)).to(DEV)
            hi = torch.from_numpy(np.maximum(hi_g[rows] - k0, -1)).to(DEV)
            mean = (csum[hi + 1] - csum[lo]) / torch.clamp(cnt, min=1).double()[:, None, None]
            mean = mean.repeat_interleave(grp, dim=1)  # query head h reads KV head h // grp
            mean[cnt == 0] = 0.0
            err = float((o - mean).abs().max())
            worst = max(worst, err)
            assert err <= TOL_O, "%s: max|dO| %.3e" % (w.name, err)
        q0 += lq
        k0 += lk
    print("%s count probe: %d rows x %d heads exact, max|dO| %.3e" % (w.name, w.total_q, w.num_heads, worst))


def test_last_key_probe(probe):
    w = probe.w
    n, _, hi_g = intervals(w)
    probe.set_q(1)
    _, lse = probe.run(probe.v_rand, 1.0, True)
    l = lse.double().cpu().numpy()
    has = n > 0
    assert np.all(l[:, ~has] == -np.inf)
    tail = np.log((1.0 - np.exp(-n[has].astype(np.float64))) / (1.0 - math.exp(-1.0)))
    got = np.rint(l[:, has] - tail[None, :]).astype(np.int64)
    bad = got != hi_g[has][None, :]
    assert not bad.any(), "%s: last visible key differs at %d (head, row) pairs" % (w.name, int(bad.sum()))


@pytest.mark.parametrize("end", ["last", "first"])
def test_key_bit_probe(probe, end):
    w = probe.w
    n, lo_g, hi_g = intervals(w)
    probe.set_q(1 if end == "last" else -1)
    out, _ = probe.run(probe.v_bits, 1.0, w.return_lse)
    has = n > 0
    assert torch.all(out[torch.from_numpy(~has).to(DEV)] == 0), "%s: rows without keys must get O = 0" % w.name
    got = decode_bits(out)[has]  # [rows, H]
    want = (hi_g if end == "last" else lo_g)[has][:, None]
    bad = got != want
    assert not bad.any(), "%s: %s visible key differs at %d (row, head) pairs, first %s" % (
        w.name, end, int(bad.sum()), np.argwhere(bad)[:3].tolist())
