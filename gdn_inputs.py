"""Seeded synthetic inputs for Gated DeltaNet chunked prefill.

This module only draws random tensors. It holds none of the method's
arithmetic, so both the GPU library and the CPU oracle may take their inputs
from it. Every draw happens on the CPU from a seeded torch.Generator, in a
fixed order, so the same seed always gives the same bytes.

Distributions (shared by all workloads):
  * q, k ~ N(0, 1) in fp32, L2-normalised over the key dimension per
    (batch, token, head), then cast to the input dtype (round to nearest even).
  * v ~ N(0, 1), cast to the input dtype.
  * beta = sigmoid(N(0, 1)), fp32.
  * g = -softplus(N(0, 1)) * 0.1 * s_h, fp32, where s_h is a per-head decay
    scale (1 unless the workload draws it uniformly in [0.01, 1]).
  * initial state ~ N(0, std) fp32 when the workload has one.
  * upstream gradients: dO ~ N(0, 1) in the input dtype, d(final state) ~ N(0, 0.1).

Draw order: per-head scales, q, k, v, beta logits, g logits, initial state,
dO, d(final state). Varlen sequence lengths come first, from their own
numpy generator, because they fix the token count.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "varlen_lengths"]


@dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe of one synthetic workload."""
    name: str
    B: int
    T: int                      # tokens per sequence (ignored when varlen)
    H: int
    K: int
    V: int
    dtype: torch.dtype
    chunk: int = 64
    head_scale_range: Optional[tuple] = None   # (lo, hi) uniform per-head decay scale
    init_std: Optional[float] = None           # None: zero initial state
    varlen_count: int = 0                      # >0: packed sequences via cu_seqlens
    varlen_range: tuple = (1024, 16384)
    varlen_total: int = 65536                  # target total, accepted within +-10%
    backward: bool = False
    cp: str = "auto"
    notes: str = ""


WORKLOADS = {
    # Tiny fp32 forward+backward case the oracle finishes instantly.
    "tiny": Workload("tiny", B=1, T=256, H=2, K=64, V=64, dtype=torch.float32,
                     backward=True),
    # Batch-1 agentic prefill on a small model: few heads, 32K tokens, mixed decay.
    "edge_prefill": Workload("edge_prefill", B=1, T=32768, H=16, K=128, V=128,
                             dtype=torch.bfloat16, head_scale_range=(0.01, 1.0),
                             init_std=0.1),
    # One tensor-parallel shard of a long prompt: 8 heads, 256K tokens.
    "tp8_long": Workload("tp8_long", B=1, T=262144, H=8, K=128, V=128,
                         dtype=torch.bfloat16),
    # Packed pretraining batch: 8 sequences of 1K-16K tokens, 32 heads.
    "varlen_packed": Workload("varlen_packed", B=1, T=0, H=32, K=128, V=128,
                              dtype=torch.bfloat16, varlen_count=8, cp="off"),
    # Training backward: 2 x 16K tokens, 16 heads.
    "backward": Workload("backward", B=2, T=16384, H=16, K=128, V=128,
                         dtype=torch.bfloat16, init_std=0.1, backward=True),
}


def varlen_lengths(count: int, lo: int, hi: int, target: int, seed: int = 0):
    """Sequence lengths, i.i.d. uniform integers on [lo, hi].

    Tries seeds seed, seed+1, ... and keeps the first draw whose total lies
    within 10% of `target`. Returns (lengths, seed_used).
    """
    s = seed
    while True:
        rng = np.random.default_rng(s)
        lens = rng.integers(lo, hi + 1, size=count)
        if abs(int(lens.sum()) - target) <= 0.1 * target:
            return [int(x) for x in lens], s
        s += 1


def _normal(gen, shape):
    return torch.randn(shape, generator=gen, dtype=torch.float32)


def make_inputs(w: Workload | str, seed: int = 0, T: Optional[int] = None,
                H: Optional[int] = None, lengths: Optional[list] = None,
                dtype: Optional[torch.dtype] = None) -> dict:
    """Draw one batch of inputs for workload `w` (CPU tensors).

    `T`, `H`, `lengths` and `dtype` override the workload's sizes, which tests
    use to get small cases with the same distributions.

    Returns a dict with q, k, v (input dtype, [B,T,H,K|V]), g, beta
    (fp32 [B,T,H]), initial_state (fp32 [N,H,V,K] or None), cu_seqlens
    (int32 [N+1] or None), d_o and d_final_state (backward workloads only),
    head_scale (fp32 [H]) and meta (a dict describing the draw).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    H = w.H if H is None else H
    dtype = w.dtype if dtype is None else dtype
    meta = {"workload": w.name, "seed": seed}
    cu = None
    if w.varlen_count or lengths is not None:
        if lengths is None:
            lengths, lseed = varlen_lengths(w.varlen_count, *w.varlen_range,
                                            w.varlen_total, seed)
            meta["length_seed"] = lseed
        B, Tt = 1, int(sum(lengths))
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
        nseq = len(lengths)
        meta["lengths"] = list(lengths)
    else:
        B = w.B
        Tt = w.T if T is None else T
        nseq = B
    K, V = w.K, w.V
    gen = torch.Generator().manual_seed(seed)
    if w.head_scale_range is not None:
        lo, hi = w.head_scale_range
        s_h = lo + (hi - lo) * torch.rand(H, generator=gen, dtype=torch.float32)
    else:
        s_h = torch.ones(H, dtype=torch.float32)
    q = _normal(gen, (B, Tt, H, K))
    q = q / q.norm(dim=-1, keepdim=True)
    q = q.to(dtype)
    k = _normal(gen, (B, Tt, H, K))
    k = k / k.norm(dim=-1, keepdim=True)
    k = k.to(dtype)
    v = _normal(gen, (B, Tt, H, V)).to(dtype)
    beta = torch.sigmoid(_normal(gen, (B, Tt, H)))
    g = -torch.nn.functional.softplus(_normal(gen, (B, Tt, H))) * 0.1 * s_h
    g = g.to(torch.float32).contiguous()
    init = None
    if w.init_std is not None:
        init = _normal(gen, (nseq, H, V, K)) * w.init_std
    out = dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=init,
               cu_seqlens=cu, head_scale=s_h, meta=meta)
    if w.backward:
        out["d_o"] = _normal(gen, (B, Tt, H, V)).to(dtype)
        out["d_final_state"] = _normal(gen, (nseq, H, V, K)) * 0.1
    return out
