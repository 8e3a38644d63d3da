"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no attention arithmetic: it only draws random tensors.
Both sides of every parity check consume the exact bytes produced here.

Recipe (the pages' workload is "LLaMA-shaped" random tensors of fixed
length; the handbook page "Context parallelism: Ring Attention and
Ulysses", section "Which operations split directly", draws its test data
with ``torch.manual_seed(0)`` followed by three ``torch.randn(S, H, D)``
calls for q, k and v):

* a CPU ``torch.Generator`` seeded with ``seed`` draws q, k, v in that
  order as float32 N(0, 1);
* for bf16 inputs the float32 draws are cast with ``Tensor.to`` (round to
  nearest even);
* k and v may have fewer heads than q (grouped-query attention).

With the defaults ``(S=32, H=8, D=16, seed=0)`` this reproduces the
handbook's ``make_qkv()`` exactly.
"""
from __future__ import annotations

import hashlib

import torch


def make_qkv(S: int = 32, H: int = 8, D: int = 16, seed: int = 0,
             dtype: torch.dtype = torch.float32, Hkv: int | None = None):
    """Return CPU tensors q [S,H,D], k [S,Hkv,D], v [S,Hkv,D] of ``dtype``."""
    Hkv = H if Hkv is None else Hkv
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn(S, H, D, generator=g, dtype=torch.float32)
    k = torch.randn(S, Hkv, D, generator=g, dtype=torch.float32)
    v = torch.randn(S, Hkv, D, generator=g, dtype=torch.float32)
    if dtype != torch.float32:
        q, k, v = q.to(dtype), k.to(dtype), v.to(dtype)
    return q, k, v


def sha256_of(*tensors: torch.Tensor) -> str:
    """Digest of the raw bytes of ``tensors`` (recorded next to results)."""
    h = hashlib.sha256()
    for t in tensors:
        t = t.contiguous()
        h.update(t.view(torch.uint8).numpy().tobytes() if t.dtype == torch.bfloat16
                 else t.numpy().tobytes())
    return h.hexdigest()


def sample_rows(n_total: int, n_sample: int, seed: int = 1) -> torch.Tensor:
    """Sorted, distinct row indices in [0, n_total): the first and last rows,
    plus seeded uniform draws.  Used to pick the outputs that the oracle
    recomputes one by one at full sizes."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    n_sample = min(n_sample, n_total)
    picks = {0, n_total - 1}
    if n_sample > len(picks):
        extra = torch.randperm(n_total, generator=g)[: n_sample].tolist()
        for r in extra:
            if len(picks) >= n_sample:
                break
            picks.add(int(r))
    return torch.tensor(sorted(picks), dtype=torch.int64)
