"""fp64 CPU oracle for Selective Head Attention (SHA) decode.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The HIP library never
calls it and shares no code with it; it reads nothing from the HIP path.

What it computes (the plain definition, written out):
  * Per (batch row b, head h) the decode attention of one query vector,
        O[b, h] = softmax(s * q K^T) V,
    where q = Q[b, h, 0, :], K = K[b, g], V = V[b, g] over all Nkv keys and
    s is the score scale.  Definition: papernotes.org notes on Polar Sparsity,
    方法详解 > 关键设计 > "Attention Head 稀疏性", the attention equation
    softmax(Q K^T / sqrt(d_h)) V per batch row and head.
  * Only the heads listed in batch_head_index[b, :] are computed and written;
    every other output slot is left as it was.  papernotes.org notes,
    "Selective Head Attention (SHA) Kernel" (the kernel takes a batch head
    index tensor and only reads/writes active heads); reproducibility page
    (ri.k117.org), "Pseudocode", Algorithm 1 (each unit resolves its (b, k)
    pair to head_idx and writes O[b, head_idx, 0, :]).
  * GQA: papernotes.org notes, SHA Kernel bullets (GQA models are made
    sparse per KV group); atlas.scime.ai summary, "Approach" (routers pick top-k heads
    or GQA groups).  batch_group_index selects KV groups; all G = H/H_kv
    query heads of a selected group are computed against that group's K/V.

Algorithm 1's tiled online softmax reaches exactly this value (up to rounding
order); it is the method's way of streaming, not a different result, so the
oracle does not tile.  It uses a two-pass softmax (max, then exp/sum) in
fp64 per (b, h).

Readings where the pages are silent (each also checked by the tests):
  * scale: the call passes a float32 scale; the oracle uses float64 of that
    float32 value (Algorithm 1 fixes s = 1/sqrt(d); callers pass that).
  * an index entry outside [0, H) (or [0, H_kv) for groups) is skipped: no
    read, no write.
  * GQA head <-> group mapping is contiguous: group g owns query heads
    g*G .. g*G+G-1; with H_kv < H in the head-indexed call, head h reads KV
    head h // G.
  * duplicate entries in a row compute the same head twice (same value).
  * Nkv must be >= 1 (an empty key set has no softmax).
  * Per-row cache lengths (optional seqlens[B]): row b attends to its first
    min(seqlens[b], Nkv) keys; a row whose length is <= 0 has no keys and its
    active heads get an all-zero output (the empty weighted sum).
"""
from __future__ import annotations

import numpy as np

try:  # torch is only needed to widen bfloat16 tensors (exact conversion).
    import torch
except ImportError:  # pragma: no cover
    torch = None


def to_f64(x) -> np.ndarray:
    """Exact widening of an f16/bf16/f32/f64 array or CPU tensor to float64."""
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.float64).numpy()
    a = np.asarray(x)
    if a.dtype.kind != "f":
        raise TypeError(f"expected a floating array, got {a.dtype}")
    return a.astype(np.float64)


def _scale64(scale: float) -> float:
    # The call site passes a float32 scale; use exactly that value in fp64.
    return float(np.float64(np.float32(scale)))


def _check_shapes(Q, K, V, idx, gqa: bool):
    if Q.ndim != 4 or Q.shape[2] != 1:
        raise ValueError(f"q must be [B, H, 1, d], got {Q.shape}")
    if K.ndim != 4 or V.shape != K.shape:
        raise ValueError(f"k, v must be [B, H_kv, Nkv, d], got {K.shape} {V.shape}")
    B, H, _, d = Q.shape
    Bk, H_kv, Nkv, dk = K.shape
    if Bk != B or dk != d:
        raise ValueError("q and k/v disagree on B or d")
    if H_kv < 1 or H % H_kv != 0:
        raise ValueError(f"H={H} is not a multiple of H_kv={H_kv}")
    if Nkv < 1 or d < 1:
        raise ValueError("Nkv and d must be >= 1")
    if idx.ndim != 2 or idx.shape[0] != B:
        raise ValueError(f"index must be [B, top_k], got {idx.shape}")
    top_k = idx.shape[1]
    limit = H_kv if gqa else H
    if not (1 <= top_k <= limit):
        raise ValueError(f"top_k={top_k} outside [1, {limit}]")
    return B, H, H_kv, Nkv, d, top_k


def attend_one(q: np.ndarray, K: np.ndarray, V: np.ndarray, s: float) -> np.ndarray:
    """softmax(s * q K^T) V for one query vector, fp64, two-pass softmax.

    q: [d], K: [Nkv, d], V: [Nkv, d]  ->  [d]
    """
    scores = s * (K @ q)                 # [Nkv]
    m = scores.max()
    p = np.exp(scores - m)
    return (p @ V) / p.sum()


def _prefill(o_in, shape):
    if o_in is None:
        return np.full(shape, np.nan)
    o = to_f64(o_in).copy()
    if o.shape != shape:
        raise ValueError(f"o must be {shape}, got {o.shape}")
    return o


def _row_lengths(seqlens, B, Nkv):
    if seqlens is None:
        return [Nkv] * B
    L = np.asarray(seqlens.cpu() if torch is not None and isinstance(seqlens, torch.Tensor)
                   else seqlens).reshape(-1)
    if L.shape[0] != B:
        raise ValueError("seqlens must have B entries")
    return [int(min(max(int(x), 0), Nkv)) for x in L]


def _attend_prefix(q, K, V, s, n):
    """attend_one over the first n keys; n == 0 gives zeros."""
    if n == 0:
        return np.zeros(V.shape[1])
    return attend_one(q, K[:n], V[:n], s)


def sha_decode_ref(q, k, v, batch_head_index, scale, o_in=None, seqlens=None):
    """Head-indexed SHA decode in fp64.

    Returns (O, written): O is [B, H, 1, d] float64 holding o_in (widened;
    NaN where o_in is None) at untouched slots; written is a [B, H] bool mask
    of the slots the call computes.
    """
    Q, K, V = to_f64(q), to_f64(k), to_f64(v)
    idx = np.asarray(batch_head_index.cpu() if torch is not None and
                     isinstance(batch_head_index, torch.Tensor) else batch_head_index)
    B, H, H_kv, Nkv, d, top_k = _check_shapes(Q, K, V, idx, gqa=False)
    G = H // H_kv
    s = _scale64(scale)
    lens = _row_lengths(seqlens, B, Nkv)
    O = _prefill(o_in, Q.shape)
    written = np.zeros((B, H), dtype=bool)
    for b in range(B):
        for kk in range(top_k):
            h = int(idx[b, kk])
            if h < 0 or h >= H:
                continue
            g = h // G
            O[b, h, 0, :] = _attend_prefix(Q[b, h, 0, :], K[b, g], V[b, g], s, lens[b])
            written[b, h] = True
    return O, written


def sha_decode_gqa_ref(q, k, v, batch_group_index, scale, o_in=None, seqlens=None):
    """Group-indexed (GQA group sparsity) SHA decode in fp64.

    batch_group_index[b, :] lists active KV groups; every query head
    g*G .. g*G+G-1 of an active group g is computed.  Returns (O, written)
    as sha_decode_ref does.
    """
    Q, K, V = to_f64(q), to_f64(k), to_f64(v)
    gidx = np.asarray(batch_group_index.cpu() if torch is not None and
                      isinstance(batch_group_index, torch.Tensor) else batch_group_index)
    B, H, H_kv, Nkv, d, top_k = _check_shapes(Q, K, V, gidx, gqa=True)
    G = H // H_kv
    s = _scale64(scale)
    lens = _row_lengths(seqlens, B, Nkv)
    O = _prefill(o_in, Q.shape)
    written = np.zeros((B, H), dtype=bool)
    for b in range(B):
        for kk in range(top_k):
            g = int(gidx[b, kk])
            if g < 0 or g >= H_kv:
                continue
            for j in range(G):
                h = g * G + j
                O[b, h, 0, :] = _attend_prefix(Q[b, h, 0, :], K[b, g], V[b, g], s, lens[b])
                written[b, h] = True
    return O, written


def sha_units_ref(q_rows, k_slabs, v_slabs, scale) -> np.ndarray:
    """Sampled-unit form: q_rows [n, d], k_slabs/v_slabs [n, Nkv, d] -> [n, d].

    Used where only a sample of a large call's units is checked: the caller
    gathers the (q, K, V) of each sampled unit; the arithmetic per unit is
    attend_one.
    """
    qs, Ks, Vs = to_f64(q_rows), to_f64(k_slabs), to_f64(v_slabs)
    s = _scale64(scale)
    return np.stack([attend_one(qs[i], Ks[i], Vs[i], s) for i in range(qs.shape[0])])
