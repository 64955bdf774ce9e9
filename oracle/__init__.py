"""fp64 CPU oracle for the varlen attention forward pass.

TEST INFRASTRUCTURE: imported only by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``.  The HIP library neither
imports nor links anything here.
"""
from .attention import attention_fwd, visible_interval, visible_mask, visible_pairs
from .fp8 import attention_fwd_fp8, dequantize, e4m3_decode, e4m3_encode, quantize_output
from .merge import merge_states

__all__ = [
    "attention_fwd",
    "attention_fwd_fp8",
    "dequantize",
    "e4m3_decode",
    "e4m3_encode",
    "merge_states",
    "quantize_output",
    "visible_interval",
    "visible_mask",
    "visible_pairs",
]
