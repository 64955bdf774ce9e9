"""ctypes binding of ``libvarlen_attn.so`` (see include/varlen_attn.h).

Argument marshalling only: every step of the attention runs in the HIP
library.  There is no fallback: if the library is missing, calls raise.
PyTorch supplies device memory and the current stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

VA_OK = 0
VA_ERR_NULL = -1
VA_ERR_SHAPE = -2
VA_ERR_HEADDIM = -3
VA_ERR_STRIDE = -4
VA_ERR_ALIGN = -5
VA_ERR_ARG = -6
VA_ERR_LAUNCH = -7
VA_ERR_SCRATCH = -8

STATUS_NAMES = {
    VA_OK: "VA_OK",
    VA_ERR_NULL: "VA_ERR_NULL",
    VA_ERR_SHAPE: "VA_ERR_SHAPE",
    VA_ERR_HEADDIM: "VA_ERR_HEADDIM",
    VA_ERR_STRIDE: "VA_ERR_STRIDE",
    VA_ERR_ALIGN: "VA_ERR_ALIGN",
    VA_ERR_ARG: "VA_ERR_ARG",
    VA_ERR_LAUNCH: "VA_ERR_LAUNCH",
    VA_ERR_SCRATCH: "VA_ERR_SCRATCH",
}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvarlen_attn.so")

# Every symbol include/varlen_attn.h declares.
EXPORTED_SYMBOLS = (
    "varlen_attn_fwd",
    "varlen_attn_status_string",
    "varlen_attn_tile_range",
    "varlen_attn_plan",
    "varlen_attn_work_unit",
    "varlen_attn_merge",
    "varlen_attn_fwd_splitkv",
    "varlen_attn_splitkv_workspace_bytes",
    "varlen_attn_num_splits",
    "varlen_attn_fwd_fp8",
    "varlen_attn_plan_fp8",
    "varlen_attn_fwd_quant_out",
    "varlen_attn_fwd_splitkv_noalloc",
    "varlen_attn_scratch_bytes",
    "varlen_attn_splitkv_counts",
)


class VaTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("heads", ctypes.c_int32),
        ("dim", ctypes.c_int32),
        ("row_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64),
    ]


class VaPlan(ctypes.Structure):
    _fields_ = [
        ("block_m", ctypes.c_int32),
        ("block_n", ctypes.c_int32),
        ("threads", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32),
        ("grid", ctypes.c_int64),
        ("kernel", ctypes.c_char_p),
        ("segments_per_block", ctypes.c_int32),
        ("pack_mode", ctypes.c_int32),
        ("units", ctypes.c_int64),
        ("pair_q_tiles", ctypes.c_int32),
        ("key_split", ctypes.c_int32),
    ]


class VarlenAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (%d): %s" % (STATUS_NAMES.get(status, "?"), status, message))
        self.status = status


_lib = None


def library() -> ctypes.CDLL:
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libvarlen_attn.so is missing at %s; build it with "
            "`python -m varlen_attention_forward_amd.build`" % LIB_PATH
        )
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.varlen_attn_fwd.restype = ctypes.c_int
    lib.varlen_attn_fwd.argtypes = [
        P(VaTensor), P(VaTensor), P(VaTensor),
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        P(VaTensor), ctypes.c_void_p, ctypes.c_void_p,
    ]
    lib.varlen_attn_fwd_splitkv.restype = ctypes.c_int
    lib.varlen_attn_fwd_splitkv.argtypes = lib.varlen_attn_fwd.argtypes[:-1] + [
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.varlen_attn_splitkv_counts.restype = ctypes.c_int
    lib.varlen_attn_splitkv_counts.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_void_p, ctypes.c_void_p]
    lib.varlen_attn_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.varlen_attn_fwd_splitkv_noalloc.argtypes = lib.varlen_attn_fwd.argtypes[:-1] + [
        ctypes.c_int32, ctypes.c_void_p]
    lib.varlen_attn_scratch_bytes.restype = ctypes.c_size_t
    lib.varlen_attn_scratch_bytes.argtypes = []
    lib.varlen_attn_fwd_fp8.restype = ctypes.c_int
    lib.varlen_attn_fwd_fp8.argtypes = [
        P(VaTensor), P(VaTensor), P(VaTensor),
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, P(VaTensor),
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_size_t, ctypes.c_void_p,
    ]
    lib.varlen_attn_fwd_quant_out.restype = ctypes.c_int
    lib.varlen_attn_fwd_quant_out.argtypes = lib.varlen_attn_fwd.argtypes[:13] + [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.varlen_attn_splitkv_workspace_bytes.restype = ctypes.c_size_t
    lib.varlen_attn_splitkv_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                        ctypes.c_int32]
    lib.varlen_attn_num_splits.restype = ctypes.c_int
    lib.varlen_attn_num_splits.argtypes = [ctypes.c_int32] * 8 + [P(ctypes.c_int32)]
    lib.varlen_attn_merge.restype = ctypes.c_int
    lib.varlen_attn_merge.argtypes = [P(VaTensor), ctypes.c_void_p, P(VaTensor), ctypes.c_void_p,
                                      P(VaTensor), ctypes.c_void_p, ctypes.c_void_p]
    lib.varlen_attn_status_string.restype = ctypes.c_char_p
    lib.varlen_attn_status_string.argtypes = [ctypes.c_int]
    lib.varlen_attn_tile_range.restype = ctypes.c_int
    lib.varlen_attn_tile_range.argtypes = [ctypes.c_int32] * 8 + [P(ctypes.c_int32)] * 4
    lib.varlen_attn_work_unit.restype = ctypes.c_int
    lib.varlen_attn_work_unit.argtypes = ([ctypes.c_int64] + [ctypes.c_int32] * 5 + [P(ctypes.c_int32)] * 2
                                          + [ctypes.c_int32] + [P(ctypes.c_int32)] * 3)
    lib.varlen_attn_plan.restype = ctypes.c_int
    lib.varlen_attn_plan.argtypes = [ctypes.c_int32] * 8 + [P(VaPlan)]
    lib.varlen_attn_plan_fp8.restype = ctypes.c_int
    lib.varlen_attn_plan_fp8.argtypes = [ctypes.c_int32] * 8 + [P(VaPlan)]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return library().varlen_attn_status_string(int(status)).decode()


def _raise_for(status: int) -> None:
    if status == VA_OK:
        return
    msg = status_string(status)
    if status == VA_ERR_LAUNCH:
        raise VarlenAttnError(status, msg)
    err = VarlenAttnError(status, msg)
    raise ValueError(str(err)) from err


def tile_range(seqlen_q, seqlen_k, row_begin, row_end, causal, window_left, window_right, block_n):
    """The kernel's key-tile schedule for one block of query rows (host call)."""
    out = [ctypes.c_int32() for _ in range(4)]
    st = library().varlen_attn_tile_range(
        seqlen_q, seqlen_k, row_begin, row_end, int(causal), window_left, window_right, block_n,
        *[ctypes.byref(o) for o in out],
    )
    _raise_for(st)
    return tuple(o.value for o in out)


def work_unit(block, num_heads, head_dim_qk, head_dim_v, seqlens_q, seqlens_k, causal=False, num_heads_k=None):
    """(segment, head, q_tile) the kernel's workgroup ``block`` owns; -1s for padding.

    ``seqlens_q`` / ``seqlens_k`` are the per-segment lengths (host ints);
    ``num_heads_k`` the KV heads (default ``num_heads``).
    """
    num_heads_k = num_heads if num_heads_k is None else num_heads_k
    lq, lk = list(seqlens_q), list(seqlens_k)
    if len(lq) != len(lk):
        raise ValueError("seqlens_q and seqlens_k must have one entry per segment")
    arr = ctypes.c_int32 * max(1, len(lq))
    out = [ctypes.c_int32() for _ in range(3)]
    st = library().varlen_attn_work_unit(block, len(lq), num_heads, num_heads_k, head_dim_qk, head_dim_v,
                                         arr(*lq), arr(*lk),
                                         int(causal), *[ctypes.byref(o) for o in out])
    _raise_for(st)
    return tuple(o.value for o in out)


def plan(head_dim_qk, head_dim_v, batch, num_heads, max_seqlen_q, max_seqlen_k, causal=False,
         fp8: bool = False, num_heads_k=None) -> dict:
    """Launch shape the library would use (host call, no GPU needed); ``fp8``
    for ``varlen_attn_fwd_fp8``'s kernel; ``num_heads_k`` defaults to
    ``num_heads``."""
    pl = VaPlan()
    fn = library().varlen_attn_plan_fp8 if fp8 else library().varlen_attn_plan
    hk = num_heads if num_heads_k is None else num_heads_k
    st = fn(head_dim_qk, head_dim_v, batch, num_heads, hk, max_seqlen_q, max_seqlen_k, int(causal), ctypes.byref(pl))
    _raise_for(st)
    return {
        "block_m": pl.block_m,
        "block_n": pl.block_n,
        "threads": pl.threads,
        "lds_bytes": pl.lds_bytes,
        "grid": pl.grid,
        "kernel": pl.kernel.decode(),
        "segments_per_block": pl.segments_per_block,
        "pack_mode": pl.pack_mode,
        "units": pl.units,
        "pair_q_tiles": pl.pair_q_tiles,
        "key_split": pl.key_split,
    }


def raw_fwd(q: VaTensor, k: VaTensor, v: VaTensor, cu_q_ptr: int, cu_k_ptr: int, batch: int,
            max_seqlen_q: int, max_seqlen_k: int, softmax_scale: float, causal: int,
            window_left: int, window_right: int, out: VaTensor, lse_ptr: int, stream: int) -> int:
    """The C entry point with plain descriptors; returns the status code."""
    return library().varlen_attn_fwd(
        ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
        ctypes.c_void_p(cu_q_ptr), ctypes.c_void_p(cu_k_ptr), int(batch),
        int(max_seqlen_q), int(max_seqlen_k), float(softmax_scale),
        int(causal), int(window_left), int(window_right),
        ctypes.byref(out), ctypes.c_void_p(lse_ptr), ctypes.c_void_p(stream),
    )


def raw_fwd_splitkv(q: VaTensor, k: VaTensor, v: VaTensor, cu_q_ptr: int, cu_k_ptr: int, batch: int,
                    max_seqlen_q: int, max_seqlen_k: int, softmax_scale: float, causal: int,
                    window_left: int, window_right: int, out: VaTensor, lse_ptr: int, num_splits: int,
                    workspace_ptr: int, workspace_bytes: int, stream: int, splits_dyn_ptr: int = 0) -> int:
    """The split-KV C entry point with plain descriptors; returns the status code."""
    return library().varlen_attn_fwd_splitkv(
        ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
        ctypes.c_void_p(cu_q_ptr), ctypes.c_void_p(cu_k_ptr), int(batch),
        int(max_seqlen_q), int(max_seqlen_k), float(softmax_scale),
        int(causal), int(window_left), int(window_right),
        ctypes.byref(out), ctypes.c_void_p(lse_ptr), int(num_splits), ctypes.c_void_p(splits_dyn_ptr),
        ctypes.c_void_p(workspace_ptr), int(workspace_bytes), ctypes.c_void_p(stream),
    )


def splitkv_counts(cu_seqlens_k, max_splits: int, keys_per_split: int, out=None):
    """Per-segment split counts computed on the device from ``cu_seqlens_k``
    (varlen_attn_splitkv_counts): an int32 GPU tensor [batch]."""
    import torch

    batch = cu_seqlens_k.numel() - 1
    if out is None:
        out = torch.empty(max(batch, 0), dtype=torch.int32, device=cu_seqlens_k.device)
    st = library().varlen_attn_splitkv_counts(
        ctypes.c_void_p(cu_seqlens_k.data_ptr()), int(batch), int(max_splits), int(keys_per_split),
        ctypes.c_void_p(out.data_ptr() if batch > 0 else 0),
        ctypes.c_void_p(torch.cuda.current_stream(cu_seqlens_k.device).cuda_stream))
    _raise_for(st)
    return out


def raw_fwd_splitkv_noalloc(q: VaTensor, k: VaTensor, v: VaTensor, cu_q_ptr: int, cu_k_ptr: int, batch: int,
                            max_q: int, max_k: int, scale: float, causal: int, window_left: int,
                            window_right: int, out: VaTensor, lse_ptr: int, num_splits: int,
                            stream: int) -> int:
    return library().varlen_attn_fwd_splitkv_noalloc(
        ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
        ctypes.c_void_p(cu_q_ptr), ctypes.c_void_p(cu_k_ptr), int(batch),
        int(max_q), int(max_k), ctypes.c_float(scale), int(causal), int(window_left), int(window_right),
        ctypes.byref(out), ctypes.c_void_p(lse_ptr), int(num_splits), ctypes.c_void_p(stream))


def scratch_bytes() -> int:
    """Size of the per-GPU scratch array of the allocation-free entry point."""
    return int(library().varlen_attn_scratch_bytes())


def raw_fwd_fp8(q: VaTensor, k: VaTensor, v: VaTensor, q_descale_ptr: int, k_descale_ptr: int,
                v_descale_ptr: int, cu_q_ptr: int, cu_k_ptr: int, batch: int, max_seqlen_q: int,
                max_seqlen_k: int, softmax_scale: float, causal: int, window_left: int, window_right: int,
                out: VaTensor, out_scale_ptr: int, lse_ptr: int, num_splits: int, workspace_ptr: int,
                workspace_bytes: int, stream: int, splits_dyn_ptr: int = 0) -> int:
    """The fp8 C entry point with plain descriptors; returns the status code."""
    return library().varlen_attn_fwd_fp8(
        ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
        ctypes.c_void_p(q_descale_ptr), ctypes.c_void_p(k_descale_ptr), ctypes.c_void_p(v_descale_ptr),
        ctypes.c_void_p(cu_q_ptr), ctypes.c_void_p(cu_k_ptr), int(batch),
        int(max_seqlen_q), int(max_seqlen_k), float(softmax_scale),
        int(causal), int(window_left), int(window_right),
        ctypes.byref(out), ctypes.c_void_p(out_scale_ptr), ctypes.c_void_p(lse_ptr), int(num_splits),
        ctypes.c_void_p(splits_dyn_ptr), ctypes.c_void_p(workspace_ptr), int(workspace_bytes), ctypes.c_void_p(stream),
    )


def splitkv_workspace_bytes(total_q: int, num_heads: int, head_dim_v: int, num_splits: int) -> int:
    """Workspace bytes ``varlen_attn_fwd(..., num_splits=S)`` needs (host call)."""
    return int(library().varlen_attn_splitkv_workspace_bytes(total_q, num_heads, head_dim_v, num_splits))


def auto_num_splits(head_dim_qk: int, head_dim_v: int, batch: int, num_heads: int, max_seqlen_q: int,
                    max_seqlen_k: int, num_heads_k: int = None, fp8: bool = False) -> int:
    """The library's split count for these sizes (1: the units already fill
    the GPU), for the launch of ``varlen_attn_fwd`` (``fp8``: of
    ``varlen_attn_fwd_fp8``) with ``num_heads_k`` KV heads (None: num_heads)."""
    n = ctypes.c_int32()
    hk = num_heads if num_heads_k is None else num_heads_k
    st = library().varlen_attn_num_splits(head_dim_qk, head_dim_v, batch, num_heads, hk, max_seqlen_q,
                                          max_seqlen_k, int(bool(fp8)), ctypes.byref(n))
    _raise_for(st)
    return n.value


def _desc(t, name: str, dtype=None) -> VaTensor:
    import torch

    dtype = torch.bfloat16 if dtype is None else dtype
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU device" % name)
    if t.dim() != 3:
        raise ValueError("%s must be [tokens, heads, dim], got shape %s" % (name, tuple(t.shape)))
    if t.shape[2] > 1 and t.stride(2) != 1:
        raise ValueError("%s: the last dimension must be contiguous" % name)
    row_stride = t.stride(0) if t.shape[0] > 1 else t.shape[1] * t.stride(1)
    head_stride = t.stride(1) if t.shape[1] > 1 else t.shape[2]
    return VaTensor(t.data_ptr(), t.shape[0], t.shape[1], t.shape[2], row_stride, head_stride)


def varlen_attn_fwd(
    q,
    k,
    v,
    cu_seqlens_q,
    cu_seqlens_k,
    max_seqlen_q: int,
    max_seqlen_k: int,
    softmax_scale: Optional[float] = None,
    causal: bool = False,
    window_size: Tuple[int, int] = (-1, -1),
    out=None,
    return_lse: bool = False,
    lse=None,
    num_splits: int = 1,
    out_scale=None,
    num_splits_dynamic=None,
):
    """Fused varlen attention forward on the current HIP stream.

    ``q`` [total_q, H, d_qk], ``k`` [total_k, H_kv, d_qk], ``v`` [total_k, H_kv, d_v]
    in bf16 on the GPU (H a multiple of H_kv: query head h reads KV head
    h // (H // H_kv)); ``cu_seqlens_q/k`` int32 [batch + 1] on the GPU.
    Returns ``out`` [total_q, H, d_v] bf16, or ``(out, lse)`` with lse fp32
    [H, total_q] when ``return_lse``.  ``softmax_scale`` defaults to
    d_qk^-0.5.  ``window_size`` is ``(left, right)``, -1 for unbounded.
    ``num_splits`` splits every work unit's keys into that many runs (split-KV,
    combined at the end; the workspace is allocated here with torch); 0 lets
    the library choose (1 when the call already fills the GPU).
    ``num_splits_dynamic`` (with num_splits > 1): per-segment split counts,
    an int32 GPU tensor [batch], or ``"auto"`` to have the library compute
    them on the device from ``cu_seqlens_k`` (one split per 16 key tiles, at
    most num_splits); segment b's keys then take min(count_b, num_splits)
    runs.
    ``out_scale`` (a one-element fp32 GPU tensor) makes ``out`` e4m3 codes
    of O / out_scale (``torch.float8_e4m3fn``; no split-KV).
    """
    import torch

    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if not isinstance(cu, torch.Tensor) or cu.dtype != torch.int32 or not cu.is_cuda:
            raise TypeError("%s must be an int32 GPU tensor" % name)
        if cu.dim() != 1 or not cu.is_contiguous():
            raise ValueError("%s must be a contiguous 1-D tensor" % name)
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have batch + 1 entries")
    batch = cu_seqlens_q.numel() - 1
    total_q, H, d_qk = q.shape
    d_v = v.shape[2]
    if softmax_scale is None:
        softmax_scale = d_qk ** -0.5
    out_dtype = torch.bfloat16 if out_scale is None else torch.float8_e4m3fn
    if out is None:
        out = torch.empty((total_q, H, d_v), dtype=out_dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() or tuple(lse.shape) != (H, total_q):
            raise ValueError("lse must be a contiguous float32 GPU tensor of shape [H, total_q]")
    wl, wr = window_size
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if out_scale is not None:
        if num_splits != 1:
            raise ValueError("an e4m3 output (out_scale) takes no split-KV")
        st = library().varlen_attn_fwd_quant_out(
            ctypes.byref(_desc(q, "q")), ctypes.byref(_desc(k, "k")), ctypes.byref(_desc(v, "v")),
            ctypes.c_void_p(cu_seqlens_q.data_ptr()), ctypes.c_void_p(cu_seqlens_k.data_ptr()), batch,
            int(max_seqlen_q), int(max_seqlen_k), float(softmax_scale), int(bool(causal)), int(wl), int(wr),
            ctypes.byref(_desc(out, "out", torch.float8_e4m3fn)), ctypes.c_void_p(_f32_ptr(out_scale, "out_scale", 1)),
            ctypes.c_void_p(lse.data_ptr() if lse is not None else 0), ctypes.c_void_p(stream),
        )
        _raise_for(st)
        return (out, lse) if return_lse else out
    if num_splits == 0:
        num_splits = auto_num_splits(d_qk, d_v, batch, H, max_seqlen_q, max_seqlen_k, num_heads_k=k.shape[1])
    if num_splits == 1:
        st = raw_fwd(
            _desc(q, "q"), _desc(k, "k"), _desc(v, "v"),
            cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), batch,
            max_seqlen_q, max_seqlen_k, softmax_scale, int(bool(causal)), wl, wr,
            _desc(out, "out"), lse.data_ptr() if lse is not None else 0, stream,
        )
    else:
        nbytes = splitkv_workspace_bytes(total_q, H, d_v, num_splits)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        dyn = _split_counts(num_splits_dynamic, cu_seqlens_k, batch, num_splits,
                            plan(d_qk, d_v, batch, H, max_seqlen_q, max_seqlen_k, causal,
                                 num_heads_k=k.shape[1])["block_n"])
        st = raw_fwd_splitkv(
            _desc(q, "q"), _desc(k, "k"), _desc(v, "v"),
            cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), batch,
            max_seqlen_q, max_seqlen_k, softmax_scale, int(bool(causal)), wl, wr,
            _desc(out, "out"), lse.data_ptr() if lse is not None else 0, num_splits,
            ws.data_ptr(), nbytes, stream, splits_dyn_ptr=0 if dyn is None else dyn.data_ptr(),
        )
    _raise_for(st)
    if return_lse:
        return out, lse
    return out


def varlen_attn_fwd_noalloc(
    q,
    k,
    v,
    cu_seqlens_q,
    cu_seqlens_k,
    max_seqlen_q: int,
    max_seqlen_k: int,
    out,
    num_splits: int,
    lse=None,
    softmax_scale: Optional[float] = None,
    causal: bool = False,
    window_size: Tuple[int, int] = (-1, -1),
):
    """Split-KV forward that allocates nothing: the caller passes ``out``
    (bf16 [total_q, H, d_v]) and, to get the LSE, ``lse`` (fp32 [H,
    total_q]); the split partials live in the library's fixed per-GPU
    scratch array (``scratch_bytes()``), which calls that overlap on one GPU
    share.  ``num_splits`` as for ``varlen_attn_fwd`` but explicit (1 to
    128).  Returns ``out``, or ``(out, lse)`` when ``lse`` is given."""
    import torch

    batch = _check_cu(cu_seqlens_q, cu_seqlens_k)
    H, total_q, d_qk = q.shape[1], q.shape[0], q.shape[2]
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() or tuple(lse.shape) != (H, total_q):
            raise ValueError("lse must be a contiguous float32 GPU tensor of shape [H, total_q]")
    if softmax_scale is None:
        softmax_scale = d_qk ** -0.5
    wl, wr = window_size
    st = raw_fwd_splitkv_noalloc(
        _desc(q, "q"), _desc(k, "k"), _desc(v, "v"), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), batch,
        max_seqlen_q, max_seqlen_k, softmax_scale, int(bool(causal)), wl, wr, _desc(out, "out"),
        lse.data_ptr() if lse is not None else 0, num_splits, torch.cuda.current_stream(q.device).cuda_stream,
    )
    _raise_for(st)
    return out if lse is None else (out, lse)


def _split_counts(spec, cu_seqlens_k, batch: int, num_splits: int, block_n: int):
    """The per-segment split counts tensor for ``num_splits_dynamic``: None,
    the caller's int32 GPU tensor [batch] (checked), or ``"auto"``: computed
    on the device, one split per 16 key tiles of block_n keys."""
    import torch

    if spec is None:
        return None
    if isinstance(spec, str):
        if spec != "auto":
            raise ValueError("num_splits_dynamic must be None, 'auto' or an int32 GPU tensor")
        return splitkv_counts(cu_seqlens_k, num_splits, 16 * block_n)
    if (not isinstance(spec, torch.Tensor) or spec.dtype != torch.int32 or not spec.is_cuda
            or not spec.is_contiguous() or spec.numel() != batch):
        raise ValueError("num_splits_dynamic must be a contiguous int32 GPU tensor of batch entries")
    return spec


def _check_cu(cu_seqlens_q, cu_seqlens_k) -> int:
    import torch

    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if not isinstance(cu, torch.Tensor) or cu.dtype != torch.int32 or not cu.is_cuda:
            raise TypeError("%s must be an int32 GPU tensor" % name)
        if cu.dim() != 1 or not cu.is_contiguous():
            raise ValueError("%s must be a contiguous 1-D tensor" % name)
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have batch + 1 entries")
    return cu_seqlens_q.numel() - 1


def _f32_ptr(t, name: str, numel: int) -> int:
    import torch

    if t is None:
        return 0
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise TypeError("%s must be a contiguous float32 GPU tensor" % name)
    if t.numel() != numel:
        raise ValueError("%s must have %d elements, got %d" % (name, numel, t.numel()))
    return t.data_ptr()


def varlen_attn_fwd_fp8(
    q,
    k,
    v,
    cu_seqlens_q,
    cu_seqlens_k,
    max_seqlen_q: int,
    max_seqlen_k: int,
    softmax_scale: Optional[float] = None,
    causal: bool = False,
    window_size: Tuple[int, int] = (-1, -1),
    q_descale=None,
    k_descale=None,
    v_descale=None,
    out_scale=None,
    out=None,
    return_lse: bool = False,
    lse=None,
    num_splits: int = 1,
    num_splits_dynamic=None,
):
    """Varlen attention forward on fp8 e4m3 inputs, on the current HIP stream.

    ``q``/``k``/``v`` are ``torch.float8_e4m3fn`` tensors shaped as for
    ``varlen_attn_fwd``; ``q_descale``/``k_descale``/``v_descale`` fp32
    [batch, H_kv] GPU tensors (None: ones) multiply the decoded values of
    segment b and KV head hk.  ``out_scale`` (a one-element fp32 GPU tensor)
    makes ``out`` e4m3 codes of O / out_scale; else ``out`` is bf16.
    ``num_splits`` and ``num_splits_dynamic`` as for ``varlen_attn_fwd``.
    """
    import torch

    batch = _check_cu(cu_seqlens_q, cu_seqlens_k)
    total_q, H, d_qk = q.shape
    H_kv, d_v = v.shape[1], v.shape[2]
    if softmax_scale is None:
        softmax_scale = d_qk ** -0.5
    out_dtype = torch.float8_e4m3fn if out_scale is not None else torch.bfloat16
    if out is None:
        out = torch.empty((total_q, H, d_v), dtype=out_dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() or tuple(lse.shape) != (H, total_q):
            raise ValueError("lse must be a contiguous float32 GPU tensor of shape [H, total_q]")
    wl, wr = window_size
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if num_splits == 0:
        num_splits = auto_num_splits(d_qk, d_v, batch, H, max_seqlen_q, max_seqlen_k, num_heads_k=H_kv, fp8=True)
    nbytes, ws_ptr, dyn = 0, 0, None
    if num_splits > 1:
        nbytes = splitkv_workspace_bytes(total_q, H, d_v, num_splits)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        ws_ptr = ws.data_ptr()
        dyn = _split_counts(num_splits_dynamic, cu_seqlens_k, batch, num_splits,
                            plan(d_qk, d_v, batch, H, max_seqlen_q, max_seqlen_k, causal, fp8=True,
                                 num_heads_k=H_kv)["block_n"])
    f8 = torch.float8_e4m3fn
    st = raw_fwd_fp8(
        _desc(q, "q", f8), _desc(k, "k", f8), _desc(v, "v", f8),
        _f32_ptr(q_descale, "q_descale", batch * H_kv), _f32_ptr(k_descale, "k_descale", batch * H_kv),
        _f32_ptr(v_descale, "v_descale", batch * H_kv),
        cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), batch,
        max_seqlen_q, max_seqlen_k, softmax_scale, int(bool(causal)), wl, wr,
        _desc(out, "out", out_dtype), _f32_ptr(out_scale, "out_scale", 1),
        lse.data_ptr() if lse is not None else 0, num_splits, ws_ptr, nbytes, stream,
        splits_dyn_ptr=0 if dyn is None else dyn.data_ptr(),
    )
    _raise_for(st)
    if return_lse:
        return out, lse
    return out


def _lse_ptr(t, name: str, heads: int, rows: int) -> int:
    import torch

    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda:
        raise TypeError("%s must be a float32 GPU tensor" % name)
    if not t.is_contiguous() or tuple(t.shape) != (heads, rows):
        raise ValueError("%s must be contiguous of shape [H, rows] = %s" % (name, (heads, rows)))
    return t.data_ptr()


def varlen_attn_merge(out_a, lse_a, out_b, lse_b, out=None, lse=None, return_lse: bool = True):
    """Merge two attention results over disjoint key sets of the same queries.

    ``out_a``/``out_b`` bf16 [rows, H, d] and ``lse_a``/``lse_b`` fp32 [H, rows]
    (what ``varlen_attn_fwd(..., return_lse=True)`` returns for each part).
    Returns ``(out, lse)`` (``out`` alone when ``return_lse`` is False); ``out``
    and ``lse`` may be given, also as one of the inputs (merge in place).
    """
    import torch

    rows, heads, dim = out_a.shape
    if out is None:
        out = torch.empty_like(out_a)
    if return_lse and lse is None:
        lse = torch.empty((heads, rows), dtype=torch.float32, device=out_a.device)
    st = library().varlen_attn_merge(
        ctypes.byref(_desc(out_a, "out_a")), ctypes.c_void_p(_lse_ptr(lse_a, "lse_a", heads, rows)),
        ctypes.byref(_desc(out_b, "out_b")), ctypes.c_void_p(_lse_ptr(lse_b, "lse_b", heads, rows)),
        ctypes.byref(_desc(out, "out")),
        ctypes.c_void_p(_lse_ptr(lse, "lse", heads, rows) if lse is not None else 0),
        ctypes.c_void_p(torch.cuda.current_stream(out_a.device).cuda_stream),
    )
    _raise_for(st)
    return (out, lse) if return_lse else out
