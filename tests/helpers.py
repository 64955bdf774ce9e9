"""Small shared helpers for the tests (no attention arithmetic here)."""
import numpy as np
import torch


def f64(x: torch.Tensor) -> np.ndarray:
    """Exact upcast of a bf16/fp32 tensor (any device) to a float64 numpy array."""
    return x.detach().to("cpu", torch.float64).numpy()


def f32(x: torch.Tensor) -> np.ndarray:
    """Exact image of a bf16 tensor as a float32 numpy array (half the memory of f64)."""
    return x.detach().to("cpu", torch.float32).numpy()


def oracle_on(inp, rows=None, heads=None):
    """Run the fp64 oracle on a ``workloads.Inputs`` (CPU or GPU tensors)."""
    from oracle import attention_fwd

    wl, wr = inp.window
    return attention_fwd(
        f32(inp.q),
        f32(inp.k),
        f32(inp.v),
        inp.cu_seqlens_q.cpu().tolist(),
        inp.cu_seqlens_k.cpu().tolist(),
        inp.softmax_scale,
        causal=inp.causal,
        window_left=wl,
        window_right=wr,
        rows=rows,
        heads=heads,
    )
