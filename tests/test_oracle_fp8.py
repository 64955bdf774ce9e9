"""Pins for the fp8 part of the oracle (CPU only).

The e4m3 decoder and encoder are tied to the format's definition (fixed
points of the OCP E4M3 encoding) and to a library routine (torch's
float8_e4m3fn conversions, for every code and for ties and random values).
The attention on fp8 inputs is tied to closed forms (a uniform q descale is
a change of softmax scale, a uniform v descale scales O and leaves the LSE),
to a brute-force loop over (segment, head) on tiny inputs with per-(segment,
KV head) descales and grouped heads, and a planted mistake (the KV heads'
descales swapped) must fail that loop.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as fp8_mod
from varlen_attention_forward_amd import workloads


def _torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_decode_matches_torch_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got, ref = oracle.e4m3_decode(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


@pytest.mark.parametrize(
    "code,value",
    [
        (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0),
        (0x3C, 1.5), (0x3F, 1.875), (0x40, 2.0), (0x77, 240.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0),
    ],
)
def test_decode_format_points(code, value):
    # sign, 4-bit exponent with bias 7, 3-bit mantissa; exponent 0 subnormal m/8 * 2^-6
    assert oracle.e4m3_decode([code])[0] == value


def test_decode_nan_and_signed_zero():
    v = oracle.e4m3_decode([0x7F, 0xFF, 0x80])
    assert np.isnan(v[0]) and np.isnan(v[1])
    assert v[2] == 0.0 and np.signbit(v[2])


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_ties_go_to_even():
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448
    mids = (vals[1:] + vals[:-1]) / 2  # exact in float32 and float64
    got = oracle.e4m3_encode(mids)
    assert np.all(got % 2 == 0)  # the even neighbour
    assert np.array_equal(got, _torch_encode(mids))
    assert np.array_equal(oracle.e4m3_encode(-mids), _torch_encode(-mids))


def test_encode_matches_torch_on_random_values():
    g = np.random.default_rng(3)
    x = (g.standard_normal(20000) * np.exp2(g.integers(-14, 9, 20000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    assert np.array_equal(oracle.e4m3_encode(x.astype(np.float64)), _torch_encode(x))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.e4m3_encode([449.0])
    with pytest.raises(ValueError):
        oracle.e4m3_encode([float("nan")])


def test_quantize_output_matches_torch_clamp_and_convert():
    g = np.random.default_rng(4)
    o = g.standard_normal((64, 3, 8)) * 40
    scale = 0.0625
    got = oracle.quantize_output(o, scale)
    y = np.clip(o / scale, -448, 448).astype(np.float32)  # exact: scale is a power of two
    assert np.array_equal(got, _torch_encode(y))


# --------------------------------------------------------------------------
# attention on fp8 inputs
# --------------------------------------------------------------------------


def _fp8_case(seed=11, seqlens=((5, 7), (0, 3), (6, 6)), H=4, H_kv=2, d=8, dv=8):
    lq = [a for a, _ in seqlens]
    lk = [b for _, b in seqlens]
    inp = workloads.make_fp8_inputs(lq, lk, H, d, dv, seed, num_heads_k=H_kv)
    u8 = lambda t: t.view(torch.uint8).numpy()
    return inp, u8(inp.q), u8(inp.k), u8(inp.v)


def test_unit_descales_reduce_to_the_bf16_oracle_on_decoded_inputs():
    inp, q, k, v = _fp8_case()
    o1, l1 = oracle.attention_fwd_fp8(q, k, v, inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist(), 0.3)
    o2, l2 = oracle.attention_fwd(oracle.e4m3_decode(q), oracle.e4m3_decode(k), oracle.e4m3_decode(v),
                                  inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist(), 0.3)
    assert np.array_equal(np.isnan(o1), np.isnan(o2))
    np.testing.assert_allclose(np.nan_to_num(o1), np.nan_to_num(o2), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(np.nan_to_num(l1, neginf=0), np.nan_to_num(l2, neginf=0), rtol=1e-13, atol=1e-13)


def test_uniform_q_descale_is_a_softmax_scale():
    # scores scale * (c q) . k = (c scale) q . k
    inp, q, k, v = _fp8_case(seed=12)
    B, Hk = len(inp.cu_seqlens_q) - 1, 2
    c = 0.5  # a power of two: both sides see the same fp32 scale
    cq, ck = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
    o1, l1 = oracle.attention_fwd_fp8(q, k, v, cq, ck, 0.25, q_descale=np.full((B, Hk), c))
    o2, l2 = oracle.attention_fwd_fp8(q, k, v, cq, ck, 0.25 * c)
    np.testing.assert_allclose(np.nan_to_num(o1), np.nan_to_num(o2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.nan_to_num(l1, neginf=0), np.nan_to_num(l2, neginf=0), rtol=1e-12, atol=1e-12)


def test_uniform_v_descale_scales_o_only():
    inp, q, k, v = _fp8_case(seed=13)
    B, Hk = len(inp.cu_seqlens_q) - 1, 2
    cq, ck = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
    o1, l1 = oracle.attention_fwd_fp8(q, k, v, cq, ck, 0.3, v_descale=np.full((B, Hk), 3.0))
    o2, l2 = oracle.attention_fwd_fp8(q, k, v, cq, ck, 0.3)
    np.testing.assert_allclose(np.nan_to_num(o1), 3.0 * np.nan_to_num(o2), rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.nan_to_num(l1, neginf=0), np.nan_to_num(l2, neginf=0))


def _brute(q, k, v, cq, ck, scale, dq, dk, dv, H, H_kv, causal=False):
    """Loop over (segment, query head, row, key) with per-(segment, KV head) descales."""
    dec = oracle.e4m3_decode
    grp = H // H_kv
    out = np.full((q.shape[0], H, v.shape[2]), np.nan)
    lse = np.full((H, q.shape[0]), np.nan)
    sc = float(np.float32(scale))
    for b in range(len(cq) - 1):
        Lq, Lk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        for h in range(H):
            hk = h // grp
            for i in range(Lq):
                p = i + Lk - Lq
                keys = [j for j in range(Lk) if (not causal or j <= p)]
                t = cq[b] + i
                if not keys:
                    out[t, h, :] = 0.0
                    lse[h, t] = -math.inf
                    continue
                qi = dec(q[t, h]) * dq[b][hk]
                s = [sc * float(np.dot(qi, dec(k[ck[b] + j, hk]) * dk[b][hk])) for j in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                den = sum(w)
                acc = sum(wj * dec(v[ck[b] + j, hk]) * dv[b][hk] for wj, j in zip(w, keys))
                out[t, h, :] = acc / den
                lse[h, t] = m + math.log(den)
    return out, lse


@pytest.mark.parametrize("causal", [False, True])
def test_per_segment_kv_head_descales_against_brute_force(causal):
    inp, q, k, v = _fp8_case(seed=14)
    H, H_kv = 4, 2
    cq, ck = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
    g = np.random.default_rng(5)
    # the inputs' own descales (O(1) decoded values), spread per (segment, KV head)
    dq, dk, dv = ((d.numpy() * g.uniform(0.5, 2.0, (3, H_kv))).astype(np.float32)
                  for d in (inp.q_descale, inp.k_descale, inp.v_descale))
    o1, l1 = oracle.attention_fwd_fp8(q, k, v, cq, ck, 0.3, causal=causal, q_descale=dq, k_descale=dk, v_descale=dv)
    o2, l2 = _brute(q, k, v, cq, ck, 0.3, dq.astype(np.float64), dk.astype(np.float64), dv.astype(np.float64),
                    H, H_kv, causal)
    np.testing.assert_allclose(np.nan_to_num(o1), np.nan_to_num(o2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.nan_to_num(l1, neginf=-1e300), np.nan_to_num(l2, neginf=-1e300), rtol=1e-12)


def test_planted_query_head_descale_index_is_caught(monkeypatch):
    inp, q, k, v = _fp8_case(seed=15)
    H, H_kv = 4, 2
    cq, ck = inp.cu_seqlens_q.tolist(), inp.cu_seqlens_k.tolist()
    g = np.random.default_rng(6)
    dq = (inp.q_descale.numpy() * g.uniform(0.5, 2.0, (3, H_kv))).astype(np.float32)
    dk = inp.k_descale.numpy()
    ref, _ = _brute(q, k, v, cq, ck, 0.3, dq.astype(np.float64), dk.astype(np.float64), np.ones((3, H_kv)),
                    H, H_kv)

    def wrong_descale(d, batch, heads_k):  # the mistake: the KV heads' entries swapped
        d = np.ones((batch, heads_k)) if d is None else np.asarray(d, dtype=np.float32).astype(np.float64)
        return d.reshape(batch, heads_k)[:, ::-1]

    monkeypatch.setattr(fp8_mod, "_descale", wrong_descale)
    bad, _ = oracle.attention_fwd_fp8(q, k, v, cq, ck, 0.3, q_descale=dq, k_descale=dk)
    assert not np.allclose(np.nan_to_num(bad), np.nan_to_num(ref), rtol=1e-6, atol=1e-6)


def test_fp8_input_generator_codes_are_finite_and_descales_positive():
    inp = workloads.make_fp8_inputs([40, 0, 70], [33, 5, 70], 4, 64, 64, seed=3, num_heads_k=2)
    for t in (inp.q, inp.k, inp.v):
        assert t.dtype == torch.float8_e4m3fn
        assert not torch.isnan(t.to(torch.float32)).any()
    for d in (inp.q_descale, inp.k_descale, inp.v_descale):
        assert d.shape == (3, 2) and d.dtype == torch.float32 and bool((d > 0).all())
