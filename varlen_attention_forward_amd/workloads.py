"""Seeded synthetic inputs for the varlen attention forward pass.

This module only draws inputs: packed bf16 Q/K/V tensors and the
``cu_seqlens`` offsets that split them into segments.  It holds none of the
attention arithmetic, so both the fp64 oracle (under ``oracle/``) and the HIP
path can consume its tensors without sharing any compute code.

Shapes follow the workloads on the pages:

* ViT / multimodal-encoder attention: 16 heads, head dims 64/72/80/128,
  non-causal, full and windowed layouts, image token counts from the warmup
  candidate list {64, 256, 576, 1024, 2304, 4096, 9216, 16384, 36864, 65536}
  (vLLM PR "FA4 attention for ViT", section (2), kernel_warmup) and the ViT
  speed tables (SGLang PR #41344, "Speed Tests and Profiling").
* MLA prefill: causal, qk head dim 192 = 128 nope + 64 rope, v head dim 128,
  softmax scale 192^-0.5 (vLLM MLA prefill docs, FA4MLAPrefillKernel.dispatch
  and FlashAttnPrefillBackend.supports_mla_dimensions).

All values are standard normal draws rounded to bf16.  Generation always runs
on the CPU with a ``torch.Generator`` so that every machine sees bit-identical
inputs; callers move the tensors to the GPU themselves.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import torch

VIT_SEQLEN_CHOICES = (576, 1024, 2304, 4096)


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named synthetic configuration.

    ``seqlens_q``/``seqlens_k`` list the per-segment lengths in packing order.
    ``window`` is ``(left, right)`` with -1 meaning unbounded on that side.
    """

    name: str
    seed: int
    seqlens_q: tuple
    seqlens_k: tuple
    num_heads: int
    head_dim_qk: int
    head_dim_v: int
    causal: bool
    window: tuple = (-1, -1)
    return_lse: bool = True
    softmax_scale: Optional[float] = None
    description: str = ""
    num_splits: int = 1  # split-KV runs per work unit; 0: the library chooses
    dtype: str = "bf16"  # input element type: "bf16", or "e4m3" (fp8 with descales)
    num_heads_k: Optional[int] = None  # KV heads (grouped KV heads); None: num_heads

    @property
    def heads_k(self) -> int:
        return self.num_heads if self.num_heads_k is None else int(self.num_heads_k)

    @property
    def batch(self) -> int:
        return len(self.seqlens_q)

    @property
    def total_q(self) -> int:
        return int(sum(self.seqlens_q))

    @property
    def total_k(self) -> int:
        return int(sum(self.seqlens_k))

    @property
    def max_seqlen_q(self) -> int:
        return int(max(self.seqlens_q)) if self.seqlens_q else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(max(self.seqlens_k)) if self.seqlens_k else 0

    @property
    def scale(self) -> float:
        if self.softmax_scale is not None:
            return float(self.softmax_scale)
        return self.head_dim_qk ** -0.5


def _vit_full_seqlens(seed: int) -> tuple:
    g = torch.Generator().manual_seed(seed)
    idx = torch.randint(0, len(VIT_SEQLEN_CHOICES), (8,), generator=g)
    return tuple(VIT_SEQLEN_CHOICES[i] for i in idx.tolist())


def _named_workloads() -> dict:
    vit_full = _vit_full_seqlens(2)
    ws = [
        Workload(
            name="tiny_varlen_d64",
            seed=1,
            seqlens_q=(64, 256),
            seqlens_k=(64, 256),
            num_heads=16,
            head_dim_qk=64,
            head_dim_v=64,
            causal=False,
            description="2 packed segments [64, 256], 16 heads, d=64, non-causal",
        ),
        Workload(
            name="vit_full_d80",
            seed=2,
            seqlens_q=vit_full,
            seqlens_k=vit_full,
            num_heads=16,
            head_dim_qk=80,
            head_dim_v=80,
            causal=False,
            return_lse=False,  # the ViT call takes no LSE
            description="8 ViT images, lengths drawn from {576,1024,2304,4096} "
            "(seed 2), 16 heads, d=80, non-causal",
        ),
        Workload(
            name="vit_window256_d80",
            seed=3,
            seqlens_q=(256,) * 36,
            seqlens_k=(256,) * 36,
            num_heads=16,
            head_dim_qk=80,
            head_dim_v=80,
            causal=False,
            return_lse=False,  # the ViT call takes no LSE
            description="one 9216-token image as 36 block-diagonal windows of "
            "256 tokens, 16 heads, d=80",
        ),
        Workload(
            name="vit_window64_d80",
            seed=7,
            seqlens_q=(64,) * 700,
            seqlens_k=(64,) * 700,
            num_heads=16,
            head_dim_qk=80,
            head_dim_v=80,
            causal=False,
            return_lse=False,  # the ViT call takes no LSE
            description="windowed ViT layer with 64-token windows (a 4K image's ~700 windows of 8 x 8 "
            "merged patches), 16 heads, d=80, non-causal; one wave per window and head",
        ),
        Workload(
            name="vit_long65536_d128",
            seed=4,
            seqlens_q=(65536,),
            seqlens_k=(65536,),
            num_heads=16,
            head_dim_qk=128,
            head_dim_v=128,
            causal=False,
            return_lse=False,  # the ViT call takes no LSE
            description="one 65536-token image, 16 heads, d=128, non-causal",
        ),
        Workload(
            name="mla_causal_192_128",
            seed=5,
            seqlens_q=(4096,) * 4,
            seqlens_k=(4096,) * 4,
            num_heads=128,
            head_dim_qk=192,
            head_dim_v=128,
            causal=True,
            description="MLA-style causal prefill, 4 x 4096 tokens, 128 heads, "
            "qk dim 192 (128 nope + 64 rope), v dim 128, LSE returned",
        ),
        Workload(
            name="mla_context_chunk_tp8",
            seed=6,
            seqlens_q=(512,),
            seqlens_k=(16384,),
            num_heads=16,
            head_dim_qk=192,
            head_dim_v=128,
            causal=False,
            num_splits=0,
            description="MLA chunked-prefill context chunk at 16 heads per GPU (the MLA heads over 8 "
            "GPUs): 512 new tokens over a 16384-token context chunk, non-causal, qk dim 192, v dim "
            "128, LSE returned; split-KV with the library's split count",
        ),
        Workload(
            name="gqa_chunk64_d128",
            seed=8,
            seqlens_q=(64,) * 64,
            seqlens_k=(2048,) * 64,
            num_heads=32,
            head_dim_qk=128,
            head_dim_v=128,
            causal=True,
            num_heads_k=4,
            description="grouped KV heads with short queries: 64 segments of 64 new queries over 2048 keys "
            "each (causal, bottom-right), 32 query heads over 4 KV heads, d=128, LSE returned; four query "
            "heads of a KV head per workgroup",
        ),
        Workload(
            name="vit_long65536_d128_fp8",
            seed=4,
            seqlens_q=(65536,),
            seqlens_k=(65536,),
            num_heads=16,
            head_dim_qk=128,
            head_dim_v=128,
            causal=False,
            return_lse=False,
            dtype="e4m3",
            description="one 65536-token image, 16 heads, d=128, non-causal, fp8 e4m3 Q/K/V with "
            "per-(image, head) descales, bf16 out",
        ),
        Workload(
            name="mla_causal_192_128_fp8",
            seed=5,
            seqlens_q=(4096,) * 4,
            seqlens_k=(4096,) * 4,
            num_heads=128,
            head_dim_qk=192,
            head_dim_v=128,
            causal=True,
            dtype="e4m3",
            description="MLA-style causal prefill, 4 x 4096 tokens, 128 heads, qk dim 192, v dim 128, fp8 "
            "e4m3 Q/K/V with per-(segment, head) descales, bf16 out, LSE returned",
        ),
    ]
    return {w.name: w for w in ws}


WORKLOADS = _named_workloads()


def _page_shapes() -> dict:
    """The shapes of the speed tables on the SGLang PR #41344 page ("Speed
    Tests and Profiling": the tcgen05.ld.red on/off kernel times and the d=64
    ViT call timings): images of equal length, 16 heads, non-causal, no LSE.
    Timed by ``bench.py --pages`` beside the page's own figures (another GPU:
    context, not a target); the two rows whose segment lengths the page does
    not state (8 mixed-size images, a 32-frame video) are left out."""
    shapes = [(8, 4096, 80), (8, 4096, 72), (8, 4096, 64), (64, 1024, 80), (64, 1024, 64),
              (1, 32768, 80), (1, 32768, 72), (1, 32768, 64),
              (1, 256, 64), (1, 1024, 64), (4, 1024, 64), (16, 1024, 64), (1, 4096, 64), (4, 4096, 64),
              (1, 16384, 64)]
    ws = {}
    for n, L, d in shapes:
        name = "page_%dx%d_d%d" % (n, L, d)
        ws[name] = Workload(name=name, seed=7, seqlens_q=(L,) * n, seqlens_k=(L,) * n, num_heads=16,
                            head_dim_qk=d, head_dim_v=d, causal=False, return_lse=False,
                            description="%d image(s) x %d tokens, 16 heads, d=%d, non-causal, no LSE" % (n, L, d))
    return ws


PAGE_SHAPES = _page_shapes()
WORKLOAD_ORDER = (
    "tiny_varlen_d64",
    "vit_full_d80",
    "vit_window256_d80",
    "vit_window64_d80",
    "vit_long65536_d128",
    "mla_causal_192_128",
    "mla_context_chunk_tp8",
    "gqa_chunk64_d128",
    "vit_long65536_d128_fp8",
    "mla_causal_192_128_fp8",
)


def cu_seqlens(seqlens: Sequence[int]) -> torch.Tensor:
    """Exclusive prefix offsets ``[0, L0, L0+L1, ...]`` as int32 (CPU)."""
    out = [0]
    for n in seqlens:
        out.append(out[-1] + int(n))
    return torch.tensor(out, dtype=torch.int32)


@dataclasses.dataclass
class Inputs:
    q: torch.Tensor  # [total_q, H, d_qk] bf16
    k: torch.Tensor  # [total_k, H, d_qk] bf16
    v: torch.Tensor  # [total_k, H, d_v] bf16
    cu_seqlens_q: torch.Tensor  # [B+1] int32
    cu_seqlens_k: torch.Tensor  # [B+1] int32
    max_seqlen_q: int
    max_seqlen_k: int
    softmax_scale: float
    causal: bool
    window: tuple

    def to(self, device) -> "Inputs":
        return dataclasses.replace(
            self,
            q=self.q.to(device),
            k=self.k.to(device),
            v=self.v.to(device),
            cu_seqlens_q=self.cu_seqlens_q.to(device),
            cu_seqlens_k=self.cu_seqlens_k.to(device),
        )


def make_inputs(
    seqlens_q: Sequence[int],
    seqlens_k: Sequence[int],
    num_heads: int,
    head_dim_qk: int,
    head_dim_v: int,
    seed: int,
    causal: bool = False,
    window: tuple = (-1, -1),
    softmax_scale: Optional[float] = None,
    std: float = 1.0,
    v_std: float = 1.0,
    num_heads_k: Optional[int] = None,
) -> Inputs:
    """Draw Q, K ~ N(0, std^2) and V ~ N(0, v_std^2) in float32 (in that order)
    and round to bf16.  K and V get ``num_heads_k`` heads (default
    ``num_heads``)."""
    assert len(seqlens_q) == len(seqlens_k)
    hk = num_heads if num_heads_k is None else int(num_heads_k)
    g = torch.Generator().manual_seed(seed)
    tq, tk = int(sum(seqlens_q)), int(sum(seqlens_k))
    q = torch.randn((tq, num_heads, head_dim_qk), generator=g, dtype=torch.float32)
    k = torch.randn((tk, hk, head_dim_qk), generator=g, dtype=torch.float32)
    v = torch.randn((tk, hk, head_dim_v), generator=g, dtype=torch.float32)
    if std != 1.0:
        q, k = q * std, k * std
    if v_std != 1.0:
        v = v * v_std
    scale = head_dim_qk ** -0.5 if softmax_scale is None else float(softmax_scale)
    return Inputs(
        q=q.to(torch.bfloat16),
        k=k.to(torch.bfloat16),
        v=v.to(torch.bfloat16),
        cu_seqlens_q=cu_seqlens(seqlens_q),
        cu_seqlens_k=cu_seqlens(seqlens_k),
        max_seqlen_q=int(max(seqlens_q)) if len(seqlens_q) else 0,
        max_seqlen_k=int(max(seqlens_k)) if len(seqlens_k) else 0,
        softmax_scale=scale,
        causal=causal,
        window=tuple(window),
    )


@dataclasses.dataclass
class Fp8Inputs:
    """e4m3 codes (``torch.float8_e4m3fn``) with per-(segment, KV head) fp32
    descales [batch, H_kv]: decoded code * descale approximates the drawn
    value."""

    q: torch.Tensor  # [total_q, H, d_qk] e4m3
    k: torch.Tensor  # [total_k, H_kv, d_qk] e4m3
    v: torch.Tensor  # [total_k, H_kv, d_v] e4m3
    q_descale: torch.Tensor  # [batch, H_kv] fp32
    k_descale: torch.Tensor
    v_descale: torch.Tensor
    cu_seqlens_q: torch.Tensor
    cu_seqlens_k: torch.Tensor
    max_seqlen_q: int
    max_seqlen_k: int
    softmax_scale: float
    causal: bool
    window: tuple

    def to(self, device) -> "Fp8Inputs":
        mv = {f: getattr(self, f).to(device) for f in ("q", "k", "v", "q_descale", "k_descale", "v_descale",
                                                        "cu_seqlens_q", "cu_seqlens_k")}
        return dataclasses.replace(self, **mv)


def _quantize_blocks(x: torch.Tensor, cu: Sequence[int], heads_k: int):
    """Per (segment, KV head) block of ``x`` [rows, H, d]: descale = amax / 448
    (1 for an all-zero block), codes = e4m3(x / descale).  A query head's
    block is its KV head's group of query heads."""
    rows, H, d = x.shape
    grp = H // heads_k
    batch = len(cu) - 1
    desc = torch.ones((batch, heads_k), dtype=torch.float32)
    codes = torch.zeros((rows, H, d), dtype=torch.float8_e4m3fn)
    for b in range(batch):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        for hk in range(heads_k):
            blk = x[r0:r1, hk * grp:(hk + 1) * grp, :]
            amax = float(blk.abs().max()) if blk.numel() else 0.0
            ds = amax / 448.0 if amax > 0 else 1.0
            desc[b, hk] = ds
            codes[r0:r1, hk * grp:(hk + 1) * grp, :] = (blk / desc[b, hk]).clamp(-448, 448).to(torch.float8_e4m3fn)
    return codes, desc


def make_fp8_inputs(
    seqlens_q: Sequence[int],
    seqlens_k: Sequence[int],
    num_heads: int,
    head_dim_qk: int,
    head_dim_v: int,
    seed: int,
    causal: bool = False,
    window: tuple = (-1, -1),
    softmax_scale: Optional[float] = None,
    std: float = 1.0,
    num_heads_k: Optional[int] = None,
) -> Fp8Inputs:
    """The draws of ``make_inputs`` (same seed, same order, before the bf16
    rounding), quantised to e4m3 per (segment, KV head) block."""
    assert len(seqlens_q) == len(seqlens_k)
    hk = num_heads if num_heads_k is None else int(num_heads_k)
    g = torch.Generator().manual_seed(seed)
    tq, tk = int(sum(seqlens_q)), int(sum(seqlens_k))
    q = torch.randn((tq, num_heads, head_dim_qk), generator=g, dtype=torch.float32) * std
    k = torch.randn((tk, hk, head_dim_qk), generator=g, dtype=torch.float32) * std
    v = torch.randn((tk, hk, head_dim_v), generator=g, dtype=torch.float32)
    cq, ck = cu_seqlens(seqlens_q), cu_seqlens(seqlens_k)
    q8, qd = _quantize_blocks(q, cq.tolist(), hk)
    k8, kd = _quantize_blocks(k, ck.tolist(), hk)
    v8, vd = _quantize_blocks(v, ck.tolist(), hk)
    scale = head_dim_qk ** -0.5 if softmax_scale is None else float(softmax_scale)
    return Fp8Inputs(
        q=q8, k=k8, v=v8, q_descale=qd, k_descale=kd, v_descale=vd,
        cu_seqlens_q=cq, cu_seqlens_k=ck,
        max_seqlen_q=int(max(seqlens_q)) if len(seqlens_q) else 0,
        max_seqlen_k=int(max(seqlens_k)) if len(seqlens_k) else 0,
        softmax_scale=scale, causal=causal, window=tuple(window),
    )


def workload_inputs(w: Workload):
    """The seeded tensors of a named workload (the seed is part of ``w``):
    ``Inputs``, or ``Fp8Inputs`` for an e4m3 workload."""
    if w.dtype == "e4m3":
        return make_fp8_inputs(w.seqlens_q, w.seqlens_k, w.num_heads, w.head_dim_qk, w.head_dim_v, w.seed,
                               causal=w.causal, window=w.window, softmax_scale=w.softmax_scale,
                               num_heads_k=w.num_heads_k)
    if w.name == "vit_full_d80":
        # Keep the generator stream identical to drawing the lengths first and
        # then Q, K, V from the same generator.
        g = torch.Generator().manual_seed(w.seed)
        torch.randint(0, len(VIT_SEQLEN_CHOICES), (8,), generator=g)
        return _draw_with(g, w)
    g = torch.Generator().manual_seed(w.seed)
    return _draw_with(g, w)


def _draw_with(g: torch.Generator, w: Workload) -> Inputs:
    q = torch.randn((w.total_q, w.num_heads, w.head_dim_qk), generator=g, dtype=torch.float32)
    q = q.to(torch.bfloat16)
    k = torch.randn((w.total_k, w.heads_k, w.head_dim_qk), generator=g, dtype=torch.float32)
    k = k.to(torch.bfloat16)
    v = torch.randn((w.total_k, w.heads_k, w.head_dim_v), generator=g, dtype=torch.float32)
    v = v.to(torch.bfloat16)
    return Inputs(
        q=q,
        k=k,
        v=v,
        cu_seqlens_q=cu_seqlens(w.seqlens_q),
        cu_seqlens_k=cu_seqlens(w.seqlens_k),
        max_seqlen_q=w.max_seqlen_q,
        max_seqlen_k=w.max_seqlen_k,
        softmax_scale=w.scale,
        causal=w.causal,
        window=w.window,
    )


def random_seqlens(seed: int, batch: int, lo: int, hi: int) -> List[int]:
    """``batch`` lengths drawn uniformly from ``[lo, hi]`` (inclusive)."""
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, (batch,), generator=g).tolist()


def with_guard_rows(x: torch.Tensor, rows: int = 256, value: float = math.nan) -> torch.Tensor:
    """A view of ``x`` whose storage is followed by ``rows`` rows of ``value``.

    Used to check that no kernel reads past the last packed row: any such read
    pulls NaN into the result.
    """
    pad = torch.full((rows,) + tuple(x.shape[1:]), value, dtype=x.dtype, device=x.device)
    return torch.cat([x, pad], dim=0)[: x.shape[0]]
