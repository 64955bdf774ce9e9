"""fp8 e4m3 inputs with descales, and the e4m3 output quantisation: fp64 oracle.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the HIP library
shares nothing with it.

Passages followed:

* SGLang PR #41344, "Accuracy Tests": fp8 e4m3 with descales is one of the
  FA4 configurations run there.  The pages give no formula; the plainest
  reading, used here, is that the descales undo the quantisation of the
  inputs: the attention of ``decode(Q) * q_descale``, ``decode(K) *
  k_descale``, ``decode(V) * v_descale`` with the usual scale and masks.
  The descales are one fp32 per (segment, KV head) (a reading: the pages do
  not give their shape; a per-tensor scale is the case of equal entries);
  query head h uses the entry of its KV head h // (H // H_kv).
* vLLM MLA prefill docs page, ``supports_quant_output`` (``kFp8StaticTensorSym``)
  and the ``output_scale`` argument of ``_flash_attn_varlen_diff_headdims``:
  the output may leave as fp8 under one static per-tensor symmetric scale.
  Read as: code = round_to_nearest_even(clamp(O / out_scale, -448, 448)).

The e4m3 format is the OCP 8-bit floating-point E4M3 encoding (the one
gfx950's fp8 instructions and ``torch.float8_e4m3fn`` use): a sign bit, four
exponent bits with bias 7 and three mantissa bits; exponent field 0 encodes
subnormals m / 8 * 2^-6; the code S.1111.111 is NaN; there are no
infinities, so the largest finite value is 1.75 * 2^8 = 448.

Pins: ``tests/test_oracle_fp8.py``.
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np

from .attention import attention_fwd

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Values of e4m3 codes (uint8 array-like) as float64; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = sign * (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, subnormal, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def _positive_table() -> Tuple[np.ndarray, np.ndarray]:
    codes = np.arange(0x7F, dtype=np.uint8)  # 0x00 .. 0x7E: every finite non-negative code
    return codes, e4m3_decode(codes)


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code of each finite value in [-448, 448], ties to the
    even code (even mantissa); the sign of zero and of values that round to
    zero is kept.  Values outside the range raise."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode takes finite values in [-448, 448]; clamp first")
    codes, vals = _positive_table()
    a = np.abs(x)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    out = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    return np.where(np.signbit(x), out | 0x80, out).astype(np.uint8)


def quantize_output(o, out_scale: float) -> np.ndarray:
    """e4m3 codes of clamp(O / out_scale, -448, 448) (see module docstring)."""
    y = np.asarray(o, dtype=np.float64) / float(np.float32(out_scale))
    return e4m3_encode(np.clip(y, -E4M3_MAX, E4M3_MAX))


def _descale(d, batch: int, heads_k: int) -> np.ndarray:
    if d is None:
        return np.ones((batch, heads_k))
    d = np.asarray(d, dtype=np.float32).astype(np.float64).reshape(batch, heads_k)
    return d


def dequantize(codes, cu_seqlens: Iterable[int], descale, heads: Optional[Iterable[int]] = None) -> np.ndarray:
    """decode(codes) * descale[b, hk] for the rows of segment b and head hk,
    float64 [total, H', d] over the requested heads (default all); rows
    outside every segment are NaN."""
    c = np.asarray(codes, dtype=np.uint8)
    cu = [int(x) for x in cu_seqlens]
    total, H, d = c.shape
    hl = list(range(H)) if heads is None else [int(h) for h in heads]
    ds = _descale(descale, len(cu) - 1, H)
    out = np.full((total, len(hl), d), np.nan)
    for b in range(len(cu) - 1):
        r0, r1 = cu[b], cu[b + 1]
        for i, h in enumerate(hl):
            out[r0:r1, i, :] = e4m3_decode(c[r0:r1, h, :]) * ds[b, h]
    return out


def attention_fwd_fp8(
    q_codes,
    k_codes,
    v_codes,
    cu_seqlens_q: Iterable[int],
    cu_seqlens_k: Iterable[int],
    softmax_scale: float,
    causal: bool = False,
    window_left: int = -1,
    window_right: int = -1,
    q_descale=None,
    k_descale=None,
    v_descale=None,
    rows: Optional[np.ndarray] = None,
    heads: Optional[Iterable[int]] = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 attention of the dequantised fp8 inputs (module docstring).

    ``*_codes`` are uint8 arrays [total, heads, d] of e4m3 codes (Q with H
    heads, K/V with H_kv); descales are [batch, H_kv] (None: ones).  Returns
    ``(out [total_q, H, d_v], lse [H, total_q])`` like ``attention_fwd``,
    NaN outside the requested rows and heads.
    """
    qc = np.asarray(q_codes, dtype=np.uint8)
    kc = np.asarray(k_codes, dtype=np.uint8)
    vc = np.asarray(v_codes, dtype=np.uint8)
    cu_q = [int(x) for x in cu_seqlens_q]
    cu_k = [int(x) for x in cu_seqlens_k]
    batch = len(cu_q) - 1
    total_q, H, _ = qc.shape
    H_kv = kc.shape[1]
    assert H % H_kv == 0
    group = H // H_kv
    dq, dk, dv = _descale(q_descale, batch, H_kv), _descale(k_descale, batch, H_kv), _descale(v_descale, batch, H_kv)
    head_list = list(range(H)) if heads is None else [int(h) for h in heads]
    out = np.full((total_q, H, vc.shape[2]), np.nan)
    lse = np.full((H, total_q), np.nan)
    for h in head_list:
        hk = h // group
        # The query head's rows take its KV head's q descale, segment by segment.
        qh = np.full((total_q, 1, qc.shape[2]), np.nan)
        for b in range(batch):
            qh[cu_q[b]:cu_q[b + 1], 0, :] = e4m3_decode(qc[cu_q[b]:cu_q[b + 1], h, :]) * dq[b, hk]
        kh = dequantize(kc, cu_k, dk, heads=[hk])
        vh = dequantize(vc, cu_k, dv, heads=[hk])
        o, l = attention_fwd(qh, kh, vh, cu_q, cu_k, softmax_scale, causal=causal, window_left=window_left,
                             window_right=window_right, rows=rows)
        out[:, h, :] = o[:, 0, :]
        lse[h, :] = l[0, :]
    return out, lse
