"""Plain fp64 CPU oracle for merging two attention results.

TEST INFRASTRUCTURE: imported only by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg; the HIP library shares nothing with
it.

Attention of a query over the union of two disjoint key sets A and B follows
from the two partial results, because a normalised partial output is
O_x = sum_{j in x} e^{s_j} v_j / e^{L_x} with L_x = ln sum_{j in x} e^{s_j}:

    L = ln(e^{L_A} + e^{L_B}),    O = e^{L_A - L} O_A + e^{L_B - L} O_B.

A part that saw no key (L = -inf) contributes nothing; with both empty the
row keeps O = 0 and L = -inf, as the forward writes for such a row.  This is
the combine a prefill that reads its context in chunks applies to the
token-major partials of its calls (vLLM docs page
"vllm.v1.attention.backends.mla.prefill.flash_attn", FlashAttnPrefillBackend:
``run_prefill_context_chunk`` and the merge_attn_states remark in
``_flash_attn_varlen_diff_headdims``), and the one a split-KV forward ends
with (same page, FA4SplitKVCombineKernel).  Pins: ``tests/test_oracle.py``.
"""
from __future__ import annotations

import numpy as np


def merge_states(out_a, lse_a, out_b, lse_b):
    """Merge two partial results.

    ``out_*`` [rows, H, d] and ``lse_*`` [H, rows] (natural log), any float
    type; computed in float64.  Returns ``(out [rows, H, d], lse [H, rows])``.
    """
    oa = np.asarray(out_a, dtype=np.float64)
    ob = np.asarray(out_b, dtype=np.float64)
    la = np.asarray(lse_a, dtype=np.float64).T  # [rows, H]
    lb = np.asarray(lse_b, dtype=np.float64).T
    lse = np.logaddexp(la, lb)  # -inf only when both are -inf
    empty = lse == -np.inf
    safe = np.where(empty, 0.0, lse)
    wa = np.where(la == -np.inf, 0.0, np.exp(la - safe))
    wb = np.where(lb == -np.inf, 0.0, np.exp(lb - safe))
    # a part with no weight is not read (its output rows may hold anything)
    ta = np.where(wa[:, :, None] > 0, wa[:, :, None] * np.nan_to_num(oa), 0.0)
    tb = np.where(wb[:, :, None] > 0, wb[:, :, None] * np.nan_to_num(ob), 0.0)
    out = ta + tb
    out[empty] = 0.0
    return out, lse.T.copy()
