"""Plain fp64 CPU oracle for the variable-length attention forward pass.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never calls it and shares no code with it: no kernels, headers, helpers or
tables.  It takes plain numpy arrays, so it does not even need torch.

What it computes is the plain definition of softmax attention over packed
segments, evaluated directly, row by row, in float64:

    for each segment b and head h, for each query row i of the segment:
        J_i   = the keys row i may see (see ``visible_interval``)
        s_j   = scale * <q_i, k_j>                      for j in J_i
        O_i   = sum_j exp(s_j) v_j / sum_j exp(s_j)
        LSE_i = ln sum_j exp(s_j)                       (natural log)

with O_i = 0 and LSE_i = -inf when J_i is empty.  Passages followed:

* The formula O = softmax(scale * Q K^T [+ mask]) V with a per-row
  log-sum-exp is the fused forward that FA4's ``flash_attn_varlen_func``
  computes; the pages never print it, they describe the call:
  vLLM docs page "vllm.v1.attention.backends.mla.prefill.flash_attn",
  FlashAttnPrefillBackend (``_flash_attn_varlen_diff_headdims``,
  ``run_prefill_new_tokens``, ``run_prefill_context_chunk``).
* The LSE is what lets partial results be merged (same page,
  FA4SplitKVCombineKernel and the ``merge_attn_states`` remark), so it is the
  log of the full softmax denominator including the scale.
* The default scale is qk_head_dim^-0.5 (same page, FA4MLAPrefillKernel
  ``dispatch``); the caller's fp32 value is used here exactly as the GPU
  receives it.
* Packed layout: Q [total_q, H, d_qk], K [total_k, H, d_qk],
  V [total_k, H, d_v], segments given by ``cu_seqlens`` prefix offsets
  (same page, ``dispatch``: q/k/v shapes and ``cu_seqlens_*_shape``).
  LSE is stored [H, total_q] (same page, FA4SplitKVCombineKernel ``kernel``:
  the lse tensor is allocated (num_heads, total_q) and viewed transposed);
  O is token-major [total_q, H, d_v] (FlashAttnPrefillBackend: the output is
  normalised to token-major for ``merge_attn_states``).

Readings where the pages are silent:

* Causal alignment when Lq != Lk is bottom-right: query row i sits at key
  position p = i + (Lk - Lq) and sees keys j <= p.  The SGLang PR #41344
  "Accuracy Tests" section lists chunked prefill (q < k) among the causal
  cases; only this alignment lets the new (last) queries see the whole
  context.
* ``window_size = (left, right)``: key j is visible when
  p - left <= j <= p + right, -1 meaning unbounded on that side; causal
  caps the right side at p (the vLLM MLA prefill page, FA4MLAPrefillKernel
  ``_is_valid_warmup_shape_probe``, notes that sliding-window prefill is
  always causal, so the two combine).
* Rows with no visible key give O = 0 and LSE = -inf.
* Grouped KV heads (GQA): the SGLang PR #41344 "Accuracy Tests" section
  lists GQA among the cases FA4 runs but does not spell the grouping out.
  Read the usual way: with H query heads and H_kv KV heads (H a multiple of
  H_kv), query head h attends with KV head h // (H // H_kv), so consecutive
  query heads share a KV head.

Rows of the output that belong to no segment are left as NaN here (the GPU
leaves them untouched).  This module has pins in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Tuple

import numpy as np


def visible_interval(i, Lq: int, Lk: int, causal: bool, window_left: int, window_right: int):
    """Inclusive key interval ``[lo, hi]`` visible to query row(s) ``i``.

    ``i`` may be an int or an integer numpy array of row indices local to a
    segment of ``Lq`` queries and ``Lk`` keys.  ``lo > hi`` means the row sees
    no key.  Bottom-right aligned (see module docstring).
    """
    i = np.asarray(i, dtype=np.int64)
    p = i + (Lk - Lq)
    lo = np.zeros_like(p)
    hi = np.full_like(p, Lk - 1)
    if window_left >= 0:
        lo = np.maximum(lo, p - window_left)
    if causal:
        hi = np.minimum(hi, p)
    elif window_right >= 0:
        hi = np.minimum(hi, p + window_right)
    return lo, hi


def visible_mask(Lq: int, Lk: int, causal: bool, window_left: int, window_right: int) -> np.ndarray:
    """Boolean ``[Lq, Lk]`` matrix, True where query i may see key j."""
    lo, hi = visible_interval(np.arange(Lq), Lq, Lk, causal, window_left, window_right)
    j = np.arange(Lk)[None, :]
    return (j >= lo[:, None]) & (j <= hi[:, None])


def _segment_head(qs, ks, vs, scale, mask):
    """Attention of one head of one segment for the requested rows.

    ``qs`` [n, d_qk], ``ks`` [Lk, d_qk], ``vs`` [Lk, d_v], ``mask`` [n, Lk].
    Returns (O [n, d_v], LSE [n]) in float64.
    """
    s = scale * (qs @ ks.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] > 0 else np.full(s.shape[0], -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 on hidden keys
    l = w.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = (w @ vs) / l[:, None]
        lse = m_safe + np.log(l)
    o[empty] = 0.0
    lse[empty] = -np.inf
    return o, lse


def attention_fwd(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    cu_seqlens_q: Iterable[int],
    cu_seqlens_k: Iterable[int],
    softmax_scale: float,
    causal: bool = False,
    window_left: int = -1,
    window_right: int = -1,
    rows: Optional[np.ndarray] = None,
    heads: Optional[Iterable[int]] = None,
    row_block: int = 1024,
) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 attention forward over packed segments.

    ``q``/``k``/``v`` are float arrays shaped [total, H, d] (bf16 inputs
    upcast exactly); ``k`` and ``v`` may have fewer heads H_kv, H a multiple
    of H_kv (grouped KV heads, see the module docstring).
    ``softmax_scale`` is rounded to float32 first, since
    that is the value the GPU receives through its C interface.
    ``rows`` restricts the computation to the given global query rows and
    ``heads`` to the given heads; everything else stays NaN.

    Returns ``(out [total_q, H, d_v], lse [H, total_q])`` as float64.
    """
    # Inputs may be float32 (an exact image of bf16); each slice is upcast to
    # float64 where it is used, so large inputs are never copied whole.
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    cu_q = [int(x) for x in cu_seqlens_q]
    cu_k = [int(x) for x in cu_seqlens_k]
    assert len(cu_q) == len(cu_k)
    total_q, H, _ = q.shape
    d_v = v.shape[2]
    H_kv = k.shape[1]
    assert v.shape[1] == H_kv and H_kv > 0 and H % H_kv == 0, "H must be a multiple of the KV heads"
    group = H // H_kv
    scale = float(np.float32(softmax_scale))
    head_list = list(range(H)) if heads is None else [int(h) for h in heads]

    out = np.full((total_q, H, d_v), np.nan)
    lse = np.full((H, total_q), np.nan)
    want = None
    if rows is not None:
        want = np.zeros(total_q, dtype=bool)
        want[np.asarray(rows, dtype=np.int64)] = True

    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        Lq, Lk = q1 - q0, k1 - k0
        if Lq <= 0:
            continue
        local = np.arange(Lq)
        if want is not None:
            local = local[want[q0:q1]]
        for start in range(0, len(local), row_block):
            idx = local[start : start + row_block]
            lo, hi = visible_interval(idx, Lq, Lk, causal, window_left, window_right)
            j = np.arange(Lk)[None, :]
            mask = (j >= lo[:, None]) & (j <= hi[:, None])
            for h in head_list:
                o, l = _segment_head(
                    q[q0 + idx, h, :].astype(np.float64),
                    k[k0:k1, h // group, :].astype(np.float64),
                    v[k0:k1, h // group, :].astype(np.float64),
                    scale,
                    mask,
                )
                out[q0 + idx, h, :] = o
                lse[h, q0 + idx] = l
    return out, lse


def visible_pairs(cu_seqlens_q, cu_seqlens_k, causal: bool, window_left: int, window_right: int) -> int:
    """Number of visible (query, key) pairs per head, summed over segments."""
    cu_q = [int(x) for x in cu_seqlens_q]
    cu_k = [int(x) for x in cu_seqlens_k]
    total = 0
    for b in range(len(cu_q) - 1):
        Lq, Lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        if Lq <= 0 or Lk <= 0:
            continue
        lo, hi = visible_interval(np.arange(Lq), Lq, Lk, causal, window_left, window_right)
        total += int(np.maximum(hi - lo + 1, 0).sum())
    return total


LN2 = math.log(2.0)
