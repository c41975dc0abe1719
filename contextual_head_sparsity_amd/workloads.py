"""Seeded synthetic decode workloads for Selective Head Attention (SHA).

This module only draws inputs: shapes, seeded random tensors, index tensors
and the output sentinel.  It contains none of the attention arithmetic, so it
can feed both the HIP path and the fp64 oracle without coupling them.

Shapes follow the models the Polar Sparsity pages evaluate (papernotes.org
notes, 实验关键数据 tables; atlas.scime.ai summary, "Key results"): OPT-6.7B,
OPT-66B (batch 64, sequence length 1920), LLaMA-2-7B and LLaMA-3.1-70B (GQA,
62.5% group density).  Real activations are not available, so Q/K/V are
i.i.d. N(0, 1) draws of those shapes, rounded once to the storage dtype.

Layouts (row-major, contiguous), as in the Require line of Algorithm 1 on the
reproducibility page (ri.k117.org, "Pseudocode"):
    q, o : [B, H, 1, d]
    k, v : [B, H_kv, Nkv, d]
    batch_head_index / batch_group_index : [B, top_k] int32
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# Output prefill: quiet NaNs with a non-canonical payload, so that any stray
# write (even of a NaN) to an inactive slot changes the bits.
SENTINEL_BITS = {"f32": 0x7FC5A5A5, "f16": 0x7E5A, "bf16": 0x7FDA}
_BITS_VIEW = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode-layer call: shapes, dtype and the index sampling recipe."""

    name: str
    B: int
    H: int          # query heads
    H_kv: int       # KV heads (== H for MHA)
    d: int
    Nkv: int
    top_k: int      # active heads (MHA) or active KV groups (GQA) per row
    dtype: str      # "f32" | "f16" | "bf16"
    gqa: bool = False
    sampling: str = "uniform"   # "uniform" | "zipf"
    zipf_s: float = 1.1
    value_scale: float = 1.0
    seed: int = 0

    @property
    def G(self) -> int:
        return self.H // self.H_kv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def units(self) -> int:
        """(b, slot) pairs, each one flash-decoding stream over Nkv keys."""
        return self.B * self.top_k

    @property
    def active_kv_bytes(self) -> int:
        """K+V bytes of the active heads (groups): the algorithmic traffic."""
        return self.units * 2 * self.Nkv * self.d * self.elem_bytes

    @property
    def dense_kv_bytes(self) -> int:
        return self.B * self.H_kv * 2 * self.Nkv * self.d * self.elem_bytes

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five decode configurations (tiny case first; the OPT-66B layer is the
# headline measurement).
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", B=2, H=4, H_kv=4, d=64, Nkv=64, top_k=2,
                         dtype="f32", seed=1),
    "opt6.7b_f16": Workload("opt6.7b_f16", B=16, H=32, H_kv=32, d=128, Nkv=1024,
                            top_k=16, dtype="f16", seed=2),
    "opt66b_f16": Workload("opt66b_f16", B=64, H=72, H_kv=72, d=128, Nkv=1920,
                           top_k=22, dtype="f16", sampling="zipf", seed=3),
    "llama2_7b_bf16": Workload("llama2_7b_bf16", B=128, H=32, H_kv=32, d=128,
                               Nkv=4096, top_k=16, dtype="bf16",
                               value_scale=0.5, seed=4),
    "llama3.1_70b_gqa_bf16": Workload("llama3.1_70b_gqa_bf16", B=64, H=64, H_kv=8,
                                      d=128, Nkv=8192, top_k=5, dtype="bf16",
                                      gqa=True, seed=5),
}
HEADLINE = "opt66b_f16"


def sample_index(w: Workload) -> np.ndarray:
    """Per-row active heads (or KV groups), distinct and sorted, int32 [B, top_k].

    uniform: each row draws top_k of the candidates without replacement.
    zipf:    head popularity w_h ~ (rank_h + 1)^-s over a seeded random ranking
             of the heads; each row draws top_k distinct heads by successive
             weighted draws.  (The pages give no popularity model; this one
             only makes some heads busier than others.)
    """
    rng = np.random.default_rng(2000 + w.seed)
    n = w.H_kv if w.gqa else w.H
    if not (1 <= w.top_k <= n):
        raise ValueError(f"top_k={w.top_k} outside [1, {n}]")
    out = np.empty((w.B, w.top_k), dtype=np.int32)
    if w.sampling == "uniform":
        for b in range(w.B):
            out[b] = np.sort(rng.choice(n, w.top_k, replace=False))
    elif w.sampling == "zipf":
        rank = rng.permutation(n)
        p = (rank + 1.0) ** (-w.zipf_s)
        p = p / p.sum()
        for b in range(w.B):
            out[b] = np.sort(rng.choice(n, w.top_k, replace=False, p=p))
    else:
        raise ValueError(w.sampling)
    return out


def _randn(shape, gen: torch.Generator, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32, device=device)


def make_qkv(w: Workload, device="cpu", seed_offset: int = 0):
    """Seeded q, k, v in the workload dtype on `device`.

    Drawn in fp32 in the order q, k, v, multiplied by value_scale and rounded
    (round-to-nearest-even) to the storage dtype once.  On a CUDA device the
    draw uses the device generator: values differ from a CPU draw of the same
    seed but are equally deterministic, and both sides of a comparison always
    read the same rounded tensors.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 + w.seed + 7919 * seed_offset)
    dt = DTYPES[w.dtype]
    shapes = ((w.B, w.H, 1, w.d), (w.B, w.H_kv, w.Nkv, w.d), (w.B, w.H_kv, w.Nkv, w.d))
    out = []
    for shp in shapes:
        t = _randn(shp, gen, device)
        if w.value_scale != 1.0:
            t.mul_(w.value_scale)
        out.append(t.to(dt) if dt != torch.float32 else t)
        del t
    return tuple(out)


def sentinel_like(w: Workload, device="cpu") -> torch.Tensor:
    """Output buffer [B, H, 1, d] prefilled with the sentinel NaN payload."""
    bits = torch.full((w.B, w.H, 1, w.d), SENTINEL_BITS[w.dtype] if w.dtype == "f32"
                      else _as_signed16(SENTINEL_BITS[w.dtype]),
                      dtype=_BITS_VIEW[w.dtype], device=device)
    return bits.view(DTYPES[w.dtype])


def raw_bits(t: torch.Tensor) -> torch.Tensor:
    """Integer view of a float tensor's storage (for bit-exact comparisons)."""
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def _as_signed16(x: int) -> int:
    return x - 0x10000 if x >= 0x8000 else x


def make_workload(w: Workload, device="cpu", seed_offset: int = 0):
    """Everything one call needs: q, k, v, index (int32, on device), o (sentinel)."""
    q, k, v = make_qkv(w, device, seed_offset)
    idx = torch.from_numpy(sample_index(w)).to(device)
    o = sentinel_like(w, device)
    return q, k, v, idx, o


# ---------------------------------------------------------------------------
# Selective MLP workloads (OPT MLP shapes: d model width, D = 4 d neurons)
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class MlpWorkload:
    """One selective-MLP layer call: batch rows each activating k_row neurons."""

    name: str
    B: int
    d: int
    D: int
    k_row: int        # neurons each row's router activates
    dtype: str        # "f16" | "bf16"
    seed: int = 0

    def with_(self, **kw) -> "MlpWorkload":
        return dataclasses.replace(self, **kw)

    @property
    def weight_bytes_per_neuron(self) -> int:
        return 2 * self.d * 2      # one W1^T row and one W2^T row, 16-bit


MLP_WORKLOADS = {
    "tiny_mlp_bf16": MlpWorkload("tiny_mlp_bf16", B=3, d=256, D=1000, k_row=50, dtype="bf16", seed=11),
    "opt6.7b_mlp_f16": MlpWorkload("opt6.7b_mlp_f16", B=16, d=4096, D=16384, k_row=1638,
                                   dtype="f16", seed=12),
    "opt66b_mlp_bf16": MlpWorkload("opt66b_mlp_bf16", B=64, d=9216, D=36864, k_row=3686,
                                   dtype="bf16", seed=13),
}


def sample_row_neurons(w: MlpWorkload) -> np.ndarray:
    """Each row's active neurons (a router's per-row top-k), int32 [B, k_row],
    distinct per row, drawn uniformly without replacement from seed."""
    rng = np.random.default_rng(3000 + w.seed)
    return np.stack([np.sort(rng.choice(w.D, w.k_row, replace=False))
                     for _ in range(w.B)]).astype(np.int32)


def make_mlp(w: MlpWorkload, device="cpu"):
    """x [B, d] ~ N(0, 1); w1t ~ N(0, 1/d) and w2t ~ N(0, 1/D), both [D, d]
    (neuron-major), so activations and outputs are O(1); rounded once."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(4000 + w.seed)
    dt = DTYPES[w.dtype]
    x = _randn((w.B, w.d), gen, device).to(dt)
    w1t = _randn((w.D, w.d), gen, device).mul_(1.0 / math.sqrt(w.d)).to(dt)
    w2t = _randn((w.D, w.d), gen, device).mul_(1.0 / math.sqrt(w.D)).to(dt)
    rows = torch.from_numpy(sample_row_neurons(w)).to(device)
    return x, w1t, w2t, rows
