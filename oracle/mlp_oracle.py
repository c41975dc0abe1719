"""fp64 CPU oracle for the selective MLP ("Selective GEMM") of Polar Sparsity.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the HIP library never
calls it and shares no code with it.

What it computes (the plain definition, written out):
  * MLP over the batch union of active neurons (papernotes.org notes on
    Polar Sparsity, 方法详解 > 关键设计 > "MLP 层动态稀疏", the equation
    MLP_{S_B}(x) = sigma(x W_{1,S_B}) W_{2,S_B}^T):
        y = relu(x W1[:, S]) W2[:, S]^T
    for x [B, d], W1, W2 [d, D] and S a subset of the D hidden neurons.
  * S_B is the union, over the rows of the batch, of each row's active
    neurons (same passage: the union of all sequences' active neurons).

Readings where the pages are silent:
  * sigma is ReLU: the pages apply the selective MLP to OPT models (atlas.
    scime.ai summary, "Approach"), whose MLP activation is ReLU; no bias terms
    appear in the equation and none are added.
  * Storage is neuron-major: w1t = W1^T and w2t = W2^T, both [D, d], so that
    neuron j's input weights and output weights are each one contiguous row.
    In this notation y = relu(x w1t[S]^T) w2t[S].
  * A row's neuron list, and the selection itself, may hold -1 (or any entry
    outside [0, D)) as padding; such entries are skipped.  The union is
    returned sorted ascending.
"""
from __future__ import annotations

import numpy as np

from .sha_oracle import to_f64


def _as_np_int(a) -> np.ndarray:
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a)


def mlp_union_ref(row_neurons, D: int) -> np.ndarray:
    """Sorted union of the valid entries of row_neurons [B, k] (int), in [0, D)."""
    rows = _as_np_int(row_neurons)
    if rows.ndim != 2:
        raise ValueError("row_neurons must be [B, k]")
    seen = set()
    for b in range(rows.shape[0]):
        for j in rows[b]:
            j = int(j)
            if 0 <= j < D:
                seen.add(j)
    return np.array(sorted(seen), dtype=np.int64)


def selective_mlp_ref(x, w1t, w2t, sel) -> np.ndarray:
    """y = relu(x w1t[sel]^T) w2t[sel] in fp64; x [B, d], w1t/w2t [D, d], sel [n]."""
    X = to_f64(x)
    W1t, W2t = to_f64(w1t), to_f64(w2t)
    S = _as_np_int(sel).astype(np.int64).reshape(-1)
    if X.ndim != 2 or W1t.ndim != 2 or W2t.shape != W1t.shape or W1t.shape[1] != X.shape[1]:
        raise ValueError("x [B, d], w1t / w2t [D, d] required")
    D = W1t.shape[0]
    S = S[(S >= 0) & (S < D)]               # padding entries select nothing
    if S.size == 0:
        return np.zeros((X.shape[0], X.shape[1]))
    H = np.maximum(X @ W1t[S].T, 0.0)      # [B, n]: sigma(x W1[:, S])
    return H @ W2t[S]                        # [B, d]: ... W2[:, S]^T
