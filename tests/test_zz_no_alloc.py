"""The allocation-free split-KV entry point (varlen_attn_fwd_splitkv_noalloc,
partials in the library's per-GPU scratch array) against the workspace entry
point (varlen_attn_fwd_splitkv) through the C interface: two calls in a row,
the second smaller, each bit-equal to the workspace call (same kernels, same
split count), and the smaller one within the 2e-2 / 1e-3 tolerance of the
fp64 oracle."""
import numpy as np
import pytest
import torch

import varlen_attention_forward_amd as va
from varlen_attention_forward_amd import workloads
from helpers import f64, oracle_on

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CALLS = [
    # 512 new queries over a 16384-key context chunk and a second segment,
    # 16 heads, MLA dims, 8 splits: 37 MB of partials
    ([512, 100], [16384, 3000], 16, (192, 128), False, 8),
    # then a smaller call on the same scratch: fewer rows, other dims
    ([64, 200, 1], [700, 900, 5], 4, (128, 128), True, 4),
]


def test_noalloc_matches_workspace_entry_point():
    assert va.scratch_bytes() == 64 << 20
    for i, (lq, lk, heads, dims, causal, splits) in enumerate(CALLS):
        inp = workloads.make_inputs(lq, lk, heads, dims[0], dims[1], seed=90 + i, causal=causal)
        need = va.splitkv_workspace_bytes(inp.q.shape[0], heads, dims[1], splits)
        assert 0 < need <= va.scratch_bytes()
        d = inp.to(DEV)
        args = (d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, inp.max_seqlen_q, inp.max_seqlen_k)
        out_ws, lse_ws = va.varlen_attn_fwd(*args, causal=causal, return_lse=True, num_splits=splits)
        out = torch.full_like(out_ws, float("nan"))
        lse = torch.full_like(lse_ws, float("nan"))
        res = va.varlen_attn_fwd_noalloc(*args, out=out, lse=lse, num_splits=splits, causal=causal)
        assert res[0] is out and res[1] is lse
        out_nolse = torch.full_like(out_ws, float("nan"))
        va.varlen_attn_fwd_noalloc(*args, out=out_nolse, num_splits=splits, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(out, out_ws) and torch.equal(lse, lse_ws), "call %d differs from the workspace call" % i
        ref_nolse = va.varlen_attn_fwd(*args, causal=causal, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out_nolse, ref_nolse)
        if i == 1:
            ref_o, ref_lse = oracle_on(inp)
            assert float(np.max(np.abs(f64(out) - ref_o))) <= 2e-2
            got_l = f64(lse)
            assert np.array_equal(got_l == -np.inf, ref_lse == -np.inf)
            fin = np.isfinite(ref_lse)
            assert float(np.max(np.abs(got_l[fin] - ref_lse[fin]))) <= 1e-3


def test_noalloc_rejects_more_than_its_scratch():
    """Partials above the scratch size: a clear error, nothing launched."""
    inp = workloads.make_inputs([2048], [2048], 64, 128, 128, seed=3)
    d = inp.to(DEV)
    need = va.splitkv_workspace_bytes(2048, 64, 128, 2)
    assert need > va.scratch_bytes()
    out = torch.zeros((2048, 64, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="VA_ERR_SCRATCH"):
        va.varlen_attn_fwd_noalloc(d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_k, 2048, 2048, out=out,
                                   num_splits=2)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
