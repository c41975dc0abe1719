"""fp64 CPU oracle for the attention router of Polar Sparsity.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the HIP library never
calls it and shares no code with it.

What it computes (the plain definition, written out):
  * The attention router is one fully connected layer on the token's hidden
    state whose per-request top-k picks the active heads (or, for GQA
    models, KV groups): papernotes.org notes on Polar Sparsity, 损失函数 /
    训练策略 (attention router: a single FC layer, supervised by the top-k of
    the per-head attention-output norm); atlas.scime.ai summary, "Approach"
    (routers pick top-k attention heads or GQA groups per request).
        scores = x W^T + b,   x [B, d], W [H, d] (one row per head), b [H]
        index[b] = the top_k heads with the largest scores, ascending order
  * The index feeds the selective head attention as batch_head_index.

Readings where the pages are silent:
  * Ties are broken toward the lower head index; a NaN score ranks like -inf.
    The selected heads are returned in ascending head order (the attention
    result does not depend on the order).
  * The bias is optional (None = no bias).
"""
from __future__ import annotations

import numpy as np

from .sha_oracle import to_f64


def router_scores_ref(x, w, bias=None) -> np.ndarray:
    """scores = x W^T + b in fp64; x [B, d], w [H, d], bias [H] or None."""
    X, W = to_f64(x), to_f64(w)
    if X.ndim != 2 or W.ndim != 2 or X.shape[1] != W.shape[1]:
        raise ValueError("x [B, d] and w [H, d] required")
    s = X @ W.T
    if bias is not None:
        s = s + to_f64(bias)[None, :]
    return s


def topk_ref(scores, top_k: int) -> np.ndarray:
    """Per row, the top_k largest entries (ties -> lower index, NaN as -inf),
    returned as ascending indices, int64 [B, top_k]."""
    S = np.asarray(scores, dtype=np.float64)
    B, H = S.shape
    if not (0 <= top_k <= H):
        raise ValueError("top_k outside [0, H]")
    out = np.empty((B, top_k), dtype=np.int64)
    for b in range(B):
        key = [(-np.inf if np.isnan(v) else v) for v in S[b]]
        # rank by (score descending, index ascending)
        order = sorted(range(H), key=lambda h: (-key[h], h))
        out[b] = np.sort(order[:top_k])
    return out


def router_topk_ref(x, w, bias, top_k: int):
    """(index [B, top_k] ascending, scores [B, H]) of the attention router."""
    s = router_scores_ref(x, w, bias)
    return topk_ref(s, top_k), s
