"""Pins for the fp64 attention-router oracle (CPU): torch linear / topk as
library routines, closed forms, the definition of top-k checked by brute
force, invariants, and planted mistakes."""
import types

import numpy as np
import pytest
import torch

import oracle.router_oracle as ro

REAL = types.SimpleNamespace(scores=ro.router_scores_ref, topk=ro.topk_ref)


def pin_scores_equal_torch_linear(impl):
    rng = np.random.default_rng(51)
    x, w, b = rng.standard_normal((5, 12)), rng.standard_normal((7, 12)), rng.standard_normal(7)
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b))
    np.testing.assert_allclose(impl.scores(x, w, b), ref.numpy(), rtol=0, atol=1e-13)
    ref0 = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w))
    np.testing.assert_allclose(impl.scores(x, w, None), ref0.numpy(), rtol=0, atol=1e-13)


def pin_topk_equals_torch_topk(impl):
    rng = np.random.default_rng(52)
    s = rng.standard_normal((6, 40))
    for k in (1, 5, 22, 40):
        ref = torch.topk(torch.from_numpy(s), k, dim=1).indices.sort(dim=1).values.numpy()
        assert np.array_equal(impl.topk(s, k), ref)


def pin_closed_forms(impl):
    x = np.array([[1.0, 0.0], [0.0, 2.0]])
    w = np.array([[1.0, 0.0], [3.0, 0.0], [2.0, 0.0], [0.0, 1.0]])
    s = impl.scores(x, w, np.array([0.0, 0.0, 0.0, 0.5]))
    np.testing.assert_allclose(s, [[1, 3, 2, 0.5], [0, 0, 0, 2.5]], rtol=0, atol=0)
    assert impl.topk(s, 2).tolist() == [[1, 2], [0, 3]]      # row 1: tie 0,0,0 -> lowest index
    assert impl.topk(np.zeros((1, 5)), 3).tolist() == [[0, 1, 2]]
    assert impl.topk(np.array([[np.nan, 1.0, -np.inf, 2.0]]), 2).tolist() == [[1, 3]]
    assert impl.topk(s, 0).shape == (2, 0)


def pin_topk_definition(impl):
    """Brute force: exactly k picks, each picked score >= each unpicked one."""
    rng = np.random.default_rng(53)
    s = np.round(rng.standard_normal((8, 17)), 1)   # many ties
    for k in (1, 4, 9, 17):
        idx = impl.topk(s, k)
        for b in range(8):
            picked = set(int(i) for i in idx[b])
            assert len(picked) == k and list(idx[b]) == sorted(picked)
            rest = [h for h in range(17) if h not in picked]
            if picked and rest:
                lo = min(s[b, h] for h in picked)
                hi = max(s[b, h] for h in rest)
                assert lo >= hi
                # among equal scores at the boundary, lower indices are picked first
                for h in rest:
                    if s[b, h] == lo:
                        assert all(p < h for p in picked if s[b, p] == lo)


def pin_invariants(impl):
    rng = np.random.default_rng(54)
    x, w = rng.standard_normal((4, 9)), rng.standard_normal((11, 9))
    base = impl.topk(impl.scores(x, w, None), 4)
    assert np.array_equal(impl.topk(impl.scores(x, w, np.full(11, 3.0)), 4), base)  # shift
    assert np.array_equal(impl.topk(impl.scores(2.0 * x, w, None), 4), base)          # scale


PINS = [pin_scores_equal_torch_linear, pin_topk_equals_torch_topk, pin_closed_forms,
        pin_topk_definition, pin_invariants]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_router_oracle_pin(pin):
    pin(REAL)


def _mut_topk(kind):
    def topk(scores, k):
        S = np.asarray(scores, dtype=np.float64)
        out = []
        for row in S:
            key = [(-np.inf if np.isnan(v) else v) for v in row]
            if kind == "smallest":
                order = sorted(range(len(row)), key=lambda h: (key[h], h))
            elif kind == "ties_to_higher":
                order = sorted(range(len(row)), key=lambda h: (-key[h], -h))
            else:
                order = sorted(range(len(row)), key=lambda h: (-key[h], h))
            sel = order[:k]
            out.append(sel if kind == "score_order" else sorted(sel))
        return np.array(out, dtype=np.int64).reshape(len(S), k)
    return topk


def _mut_scores(kind):
    def scores(x, w, bias=None):
        X, W = np.asarray(x, float), np.asarray(w, float)
        s = X @ W.T
        if kind == "bias_ignored":
            return s
        if kind == "bias_subtracted" and bias is not None:
            return s - np.asarray(bias)[None, :]
        return s if bias is None else s + np.asarray(bias)[None, :]
    return scores


@pytest.mark.parametrize("kind", ["smallest", "ties_to_higher", "score_order", "bias_ignored",
                                  "bias_subtracted"])
def test_planted_router_mistake_is_caught(kind):
    if kind in ("bias_ignored", "bias_subtracted"):
        impl = types.SimpleNamespace(scores=_mut_scores(kind), topk=ro.topk_ref)
    else:
        impl = types.SimpleNamespace(scores=ro.router_scores_ref, topk=_mut_topk(kind))
    failed = []
    for pin in PINS:
        try:
            pin(impl)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every pin"
