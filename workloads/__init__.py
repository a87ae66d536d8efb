"""Seeded synthetic inputs for the Parallax attention operator.

This module is shared by the tests, the benchmark and the smoke check. It draws
random tensors and rounds them; it holds none of the operator's arithmetic.

Workloads (shapes of the pages' 0.6B- and 1.7B-parameter Qwen-3-style layers;
the pages give model sizes and the 4096 training context, the head layout
16 query / 8 key-value heads of width 128 is the task's):

  tiny       B=1, T=128, Hq=Hkv=2,  d=32,  fp32, P ~ N(0, 0.1^2/d), seed 0
  layer06    B=4, T=2048, Hq=16, Hkv=8, d=128, bf16, P ~ N(0, 0.02^2), seed 1
  layer17    B=2, T=8192, Hq=16, Hkv=8, d=128, bf16, K rows scaled to norm sqrt(d), seed 2
  train06    B=8, T=4096, Hq=16, Hkv=8, d=128, bf16, fwd+bwd with dO ~ N(0,1), seed 3
  decode     B=64 new queries, cache L=32768, Hq=16, Hkv=8, d=128, bf16, seed 4

Recipe: one ``torch.Generator`` seeded with the workload's seed draws, in this
order, Q, K, V, P and (for the backward) dO, each as float32 N(0,1) (P then
multiplied by its standard deviation).  For bf16 workloads each tensor is then
rounded to bfloat16 with round-to-nearest-even (torch's conversion).  For
``layer17`` each K row is scaled to Euclidean norm sqrt(d) in float32 before
rounding.  The probe-form forward takes a per-row probe rho like q: ``make_probe`` draws
it from a second generator seeded with seed + 1000, float32 N(0, (p_std *
sqrt(d))^2) (the spread u = P^T q has for these P and q), then rounds it the
same way.  Generation runs on whatever device is asked for; CPU and GPU
generators give different (but each deterministic) streams, so a test always
draws its inputs once and hands the same tensors to both sides.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen_q: int
    seqlen_k: int
    heads_q: int
    heads_kv: int
    head_dim: int
    dtype: str            # "f32" or "bf16": storage type of q, k, v, P, dO
    p_std: float          # standard deviation of the projector entries
    seed: int
    causal: bool = True
    window: int = 0
    k_row_norm: bool = False
    decode: bool = False  # one new query per sequence against a cache

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs the mask lets through, summed over batch and query heads."""
        return self.batch * self.heads_q * count_visible(
            self.seqlen_q, self.seqlen_k, self.causal, self.window)


def count_visible(Tq: int, Tk: int, causal: bool, window: int) -> int:
    """Visible pairs of a bottom-right aligned causal / windowed mask, by summing rows."""
    off = Tk - Tq
    total = 0
    for i in range(Tq):
        hi = min(Tk, i + off + 1) if causal else Tk
        lo = max(0, i + off - window + 1) if window > 0 else 0
        total += max(0, hi - lo)
    return total


WORKLOADS = {
    "tiny": Workload("tiny", 1, 128, 128, 2, 2, 32, "f32", 0.1 / math.sqrt(32), 0),
    "layer06": Workload("layer06", 4, 2048, 2048, 16, 8, 128, "bf16", 0.02, 1),
    "layer17": Workload("layer17", 2, 8192, 8192, 16, 8, 128, "bf16", 0.02, 2, k_row_norm=True),
    "train06": Workload("train06", 8, 4096, 4096, 16, 8, 128, "bf16", 0.02, 3),
    "decode": Workload("decode", 64, 1, 32768, 16, 8, 128, "bf16", 0.02, 4, decode=True),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller parity cases keep the recipe)."""
    return dataclasses.replace(w, **changes)


def make_inputs(w: Workload, device="cpu", with_dout: bool = False,
                seed: Optional[int] = None):
    """Draw q, k, v, P (and dO) for workload ``w`` on ``device``.

    Layouts: q [B, Tq, Hq, d] (decode: [B, Hq, d]), k and v [B, Tk, Hkv, d],
    P [Hq, d, d], dO like q.  Returned tensors have the workload's storage
    dtype (float32 or bfloat16).
    """
    g = torch.Generator(device=device)
    g.manual_seed(w.seed if seed is None else seed)
    B, Tq, Tk, Hq, Hkv, d = w.batch, w.seqlen_q, w.seqlen_k, w.heads_q, w.heads_kv, w.head_dim
    qshape = (B, Hq, d) if w.decode else (B, Tq, Hq, d)
    f32 = torch.float32
    q = torch.randn(qshape, generator=g, device=device, dtype=f32)
    k = torch.randn((B, Tk, Hkv, d), generator=g, device=device, dtype=f32)
    v = torch.randn((B, Tk, Hkv, d), generator=g, device=device, dtype=f32)
    P = torch.randn((Hq, d, d), generator=g, device=device, dtype=f32) * w.p_std
    dout = torch.randn(qshape, generator=g, device=device, dtype=f32) if with_dout else None
    if w.k_row_norm:
        k = k * (math.sqrt(d) / k.norm(dim=-1, keepdim=True))
    td = w.torch_dtype
    out = [t.to(td) for t in (q, k, v, P)]
    if with_dout:
        out.append(dout.to(td))
    return tuple(out)


def make_probe(w: Workload, device="cpu", seed: Optional[int] = None):
    """Draw the per-row probe rho [B, Tq, Hq, d] of the probe-form forward (storage dtype of ``w``)."""
    g = torch.Generator(device=device)
    g.manual_seed((w.seed if seed is None else seed) + 1000)
    shape = (w.batch, w.seqlen_q, w.heads_q, w.head_dim)
    rho = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * (w.p_std * math.sqrt(w.head_dim))
    return rho.to(w.torch_dtype)


def to_f64_numpy(t: torch.Tensor):
    """Exact upcast of a float32 / bfloat16 tensor to a float64 numpy array on the host."""
    return t.detach().to("cpu", torch.float64).numpy()
