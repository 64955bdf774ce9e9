"""fp64 CPU oracle for the varlen attention forward pass.

TEST INFRASTRUCTURE: imported only by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``.  The HIP library neither
imports nor links anything here.
"""
from .attention import attention_fwd, visible_interval, visible_mask, visible_pairs
from .merge import merge_states

__all__ = ["attention_fwd", "merge_states", "visible_interval", "visible_mask", "visible_pairs"]
