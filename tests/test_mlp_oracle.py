"""Pins for the fp64 selective-MLP oracle (CPU): a library MLP for the dense
case, hand-derived closed forms, brute force, the exactness premise of
contextual sparsity (a selection that covers every positively activated
neuron reproduces the dense MLP), invariants, and planted mistakes."""
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle.mlp_oracle as mo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "selective_mlp_cases.json")
REAL = types.SimpleNamespace(mlp=mo.selective_mlp_ref, union=mo.mlp_union_ref)


def _rand(rng, B, d, D):
    return (rng.standard_normal((B, d)), rng.standard_normal((D, d)) / math.sqrt(d),
            rng.standard_normal((D, d)) / math.sqrt(D))


def pin_dense_equals_torch_mlp(impl):
    rng = np.random.default_rng(41)
    for B, d, D in [(3, 8, 20), (1, 16, 5), (5, 4, 33)]:
        x, w1t, w2t = _rand(rng, B, d, D)
        y = impl.mlp(x, w1t, w2t, np.arange(D))
        X, W1t, W2t = (torch.from_numpy(a) for a in (x, w1t, w2t))
        ref = torch.nn.functional.linear(torch.relu(torch.nn.functional.linear(X, W1t)), W2t.T)
        np.testing.assert_allclose(y, ref.numpy(), rtol=0, atol=1e-12)


def pin_golden(impl):
    g = json.load(open(GOLDEN))
    for case in g["mlp_cases"]:
        for name, sel in case["selections"].items():
            y = impl.mlp(np.array(case["x"]), np.array(case["w1t"]), np.array(case["w2t"]),
                         np.array(sel["sel"], dtype=np.int64))
            np.testing.assert_allclose(y, np.array(sel["y"]), rtol=0, atol=1e-13,
                                       err_msg=f"{case['name']}/{name}")
    for case in g["union_cases"]:
        got = impl.union(np.array(case["rows"]), case["D"])
        assert list(got) == case["union"], case["name"]


def _brute(x, w1t, w2t, sel):
    B, d = len(x), len(x[0])
    y = [[0.0] * d for _ in range(B)]
    for b in range(B):
        for j in sel:
            h = max(math.fsum(x[b][t] * w1t[j][t] for t in range(d)), 0.0)
            for t in range(d):
                y[b][t] += h * w2t[j][t]
    return y


def pin_brute_force(impl):
    rng = np.random.default_rng(42)
    x, w1t, w2t = _rand(rng, 3, 5, 9)
    sel = np.array([7, 0, 4, 2])
    ref = _brute(x.tolist(), w1t.tolist(), w2t.tolist(), sel.tolist())
    np.testing.assert_allclose(impl.mlp(x, w1t, w2t, sel), ref, rtol=0, atol=1e-12)


def pin_cover_of_active_neurons_is_exact(impl):
    """If S holds every neuron that is positive for some row, the selective
    MLP equals the dense one (the other neurons contribute relu = 0)."""
    rng = np.random.default_rng(43)
    x, w1t, w2t = _rand(rng, 4, 12, 40)
    w1t[::3] -= 5.0 * np.abs(w1t[::3]).sum(1, keepdims=True)  # some neurons never fire
    x = np.abs(x)
    pre = x @ w1t.T
    active = np.nonzero((pre > 0).any(axis=0))[0]
    assert 0 < len(active) < 40
    dense = impl.mlp(x, w1t, w2t, np.arange(40))
    np.testing.assert_allclose(impl.mlp(x, w1t, w2t, active), dense, rtol=0, atol=1e-12)
    # and dropping one active neuron changes the result
    assert not np.allclose(impl.mlp(x, w1t, w2t, active[1:]), dense, rtol=0, atol=1e-9)


def pin_invariants(impl):
    rng = np.random.default_rng(44)
    x, w1t, w2t = _rand(rng, 3, 6, 15)
    sel = rng.permutation(15)[:8]
    y = impl.mlp(x, w1t, w2t, sel)
    # selection order does not matter
    np.testing.assert_allclose(impl.mlp(x, w1t, w2t, sel[::-1].copy()), y, rtol=0, atol=1e-13)
    # positive homogeneity in x (relu(c z) = c relu(z), c > 0)
    np.testing.assert_allclose(impl.mlp(2.5 * x, w1t, w2t, sel), 2.5 * y, rtol=0, atol=1e-12)
    # linear in the output weights
    w2b = rng.standard_normal(w2t.shape)
    np.testing.assert_allclose(impl.mlp(x, w1t, 2 * w2t - w2b, sel),
                               2 * y - impl.mlp(x, w1t, w2b, sel), rtol=0, atol=1e-12)
    # empty selection gives zeros
    assert np.array_equal(impl.mlp(x, w1t, w2t, np.array([], dtype=np.int64)), np.zeros((3, 6)))


def pin_union(impl):
    rng = np.random.default_rng(45)
    rows = rng.integers(-3, 30, size=(6, 5))
    got = impl.union(rows, 25)
    want = sorted({int(v) for v in rows.ravel() if 0 <= v < 25})
    assert list(got) == want
    assert list(impl.union(np.full((2, 3), -1), 8)) == []


def pin_padding_entries_select_nothing(impl):
    """Entries outside [0, D) (-1, D, D + 7) select no neuron: the result
    equals the call on the filtered list, and a selection of padding alone
    gives zeros.  The last neuron fires for every row here, so reading -1 as
    neuron D - 1 would change the result."""
    rng = np.random.default_rng(46)
    D = 12
    x, w1t, w2t = _rand(rng, 3, 5, D)
    x = np.abs(x)
    w1t[D - 1] = np.abs(w1t[D - 1]) + 0.5
    valid = np.array([4, 0, 9, 2])
    padded = np.array([-1, 4, D, 0, 9, -1, D + 7, 2])
    np.testing.assert_allclose(impl.mlp(x, w1t, w2t, padded), impl.mlp(x, w1t, w2t, valid),
                               rtol=0, atol=1e-14)
    assert np.array_equal(impl.mlp(x, w1t, w2t, np.array([-1, D, D + 7])), np.zeros((3, 5)))
    ref = _brute(x.tolist(), w1t.tolist(), w2t.tolist(), valid.tolist())
    np.testing.assert_allclose(impl.mlp(x, w1t, w2t, padded), ref, rtol=0, atol=1e-12)


PINS = [pin_dense_equals_torch_mlp, pin_golden, pin_brute_force,
        pin_cover_of_active_neurons_is_exact, pin_invariants, pin_union,
        pin_padding_entries_select_nothing]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_mlp_oracle_pin(pin):
    pin(REAL)


def _mutant_mlp(kind):
    def mlp(x, w1t, w2t, sel):
        X, W1t, W2t = (np.asarray(a, dtype=np.float64) for a in (x, w1t, w2t))
        S = np.asarray(sel, dtype=np.int64).reshape(-1)
        if kind == "ignores_selection":
            S = np.arange(W1t.shape[0])
        if kind == "padding_wraps":
            S = S[S < W1t.shape[0]]          # -1 kept: numpy reads it as neuron D - 1
        elif kind == "padding_clamped":
            S = np.clip(S, 0, W1t.shape[0] - 1)
        elif kind != "ignores_selection":
            S = S[(S >= 0) & (S < W1t.shape[0])]
        if S.size == 0:
            return np.zeros((X.shape[0], X.shape[1]))
        pre = X @ W1t[S].T
        if kind == "no_relu":
            H = pre
        elif kind == "abs_instead_of_relu":
            H = np.abs(pre)
        else:
            H = np.maximum(pre, 0.0)
        if kind == "w1_for_output":
            return H @ W1t[S]
        if kind == "relu_after_output":
            return np.maximum(pre @ W2t[S], 0.0)
        if kind == "selects_output_by_position":
            return H @ W2t[: len(S)]
        return H @ W2t[S]
    return mlp


def _mutant_union(kind):
    def union(rows, D):
        rows = np.asarray(rows)
        vals = [int(v) for v in rows.ravel()]
        if kind == "keeps_padding":
            return np.array(sorted(set(v for v in vals if v < D)))
        if kind == "first_row_only":
            return np.array(sorted(set(v for v in rows[0] if 0 <= v < D)))
        if kind == "not_deduplicated":
            return np.array(sorted(v for v in vals if 0 <= v < D))
        return mo.mlp_union_ref(rows, D)
    return union


MLP_MUTANTS = ["ignores_selection", "no_relu", "abs_instead_of_relu", "w1_for_output",
               "relu_after_output", "selects_output_by_position", "padding_wraps",
               "padding_clamped"]
UNION_MUTANTS = ["keeps_padding", "first_row_only", "not_deduplicated"]


@pytest.mark.parametrize("kind", MLP_MUTANTS + UNION_MUTANTS)
def test_planted_mlp_mistake_is_caught(kind):
    if kind in MLP_MUTANTS:
        impl = types.SimpleNamespace(mlp=_mutant_mlp(kind), union=mo.mlp_union_ref)
    else:
        impl = types.SimpleNamespace(mlp=mo.selective_mlp_ref, union=_mutant_union(kind))
    failed = []
    for pin in PINS:
        try:
            pin(impl)
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every pin"
