"""Pins for the fp64 oracle, checked before the oracle is trusted (CPU only).

Every pin compares the oracle with something other than itself: a library
routine (torch scaled_dot_product_attention in fp64), hand-derived closed
forms (tests/golden), brute force with a differently arranged softmax, and
invariants the definition implies.  The mutation test at the end plants
plausible mistakes in copies of the oracle and checks that each one trips at
least one pin, so the pins are known to have teeth.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle.sha_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")

REAL = types.SimpleNamespace(mha=so.sha_decode_ref, gqa=so.sha_decode_gqa_ref)


def _rand(rng, B, H, H_kv, Nkv, d, scale_q=1.0):
    q = rng.standard_normal((B, H, 1, d)) * scale_q
    k = rng.standard_normal((B, H_kv, Nkv, d))
    v = rng.standard_normal((B, H_kv, Nkv, d))
    return q, k, v


def _sorted_rows(rng, B, n, top_k):
    return np.stack([np.sort(rng.choice(n, top_k, replace=False)) for _ in range(B)]).astype(np.int32)


# ----------------------------------------------------------------------------
# pins: each takes an implementation and raises AssertionError on mismatch
# ----------------------------------------------------------------------------

def pin_dense_equals_sdpa(impl):
    """top_k = H with index arange(H) is plain dense attention: compare with
    torch's scaled_dot_product_attention in fp64 (a library routine)."""
    rng = np.random.default_rng(11)
    for (B, H, H_kv, Nkv, d) in [(2, 4, 4, 7, 8), (3, 6, 2, 5, 4), (1, 2, 1, 33, 16)]:
        q, k, v = _rand(rng, B, H, H_kv, Nkv, d)
        s = float(np.float32(0.37))
        idx = np.tile(np.arange(H, dtype=np.int32), (B, 1))
        O, written = impl.mha(q, k, v, idx, s)
        G = H // H_kv
        kk = torch.from_numpy(k).repeat_interleave(G, dim=1)
        vv = torch.from_numpy(v).repeat_interleave(G, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), kk, vv, scale=s).numpy()
        assert written.all()
        np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def pin_single_key_returns_v(impl):
    """Nkv = 1: the only weight is exp(0)/exp(0) = 1, so O = V[b, g, 0] exactly."""
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 2, 4, 2, 1, 8)
    idx = np.array([[3, 0], [1, 2]], dtype=np.int32)
    O, _ = impl.mha(q, k, v, idx, 0.25)
    for b in range(2):
        for h in idx[b]:
            assert np.array_equal(O[b, h, 0], v[b, h // 2, 0]), (b, h)


def pin_uniform_scores_give_mean(impl):
    """q = 0, or all keys equal, makes every score equal: O = mean of V rows."""
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 2, 3, 3, 9, 5)
    q[:, 1] = 0.0
    k[:, 2] = k[:, 2, :1]          # every key row of head 2 equal
    idx = np.array([[1, 2], [2, 1]], dtype=np.int32)
    O, _ = impl.mha(q, k, v, idx, 0.7)
    for b in range(2):
        for h in (1, 2):
            np.testing.assert_allclose(O[b, h, 0], v[b, h].mean(axis=0), rtol=0, atol=1e-13)


def _brute_force_one(q, K, V, s):
    """Weights as 1 / sum_j exp(S_j - S_i): a different arrangement of the
    softmax than max-shift + normalise, in pure Python."""
    n, d = len(K), len(q)
    S = [s * math.fsum(q[t] * K[i][t] for t in range(d)) for i in range(n)]
    w = [1.0 / math.fsum(math.exp(S[j] - S[i]) for j in range(n)) for i in range(n)]
    return [math.fsum(w[i] * V[i][t] for i in range(n)) for t in range(d)]


def pin_brute_force(impl):
    rng = np.random.default_rng(14)
    for (B, H, H_kv, Nkv, d, top_k) in [(2, 4, 4, 8, 8, 2), (2, 4, 2, 5, 3, 3), (1, 3, 3, 1, 2, 1)]:
        q, k, v = _rand(rng, B, H, H_kv, Nkv, d, scale_q=2.0)
        idx = _sorted_rows(rng, B, H, top_k)
        s = float(np.float32(1.0 / math.sqrt(d)))
        O, written = impl.mha(q, k, v, idx, s)
        G = H // H_kv
        for b in range(B):
            for h in range(H):
                if h in idx[b]:
                    ref = _brute_force_one(q[b, h, 0].tolist(), k[b, h // G].tolist(),
                                           v[b, h // G].tolist(), s)
                    np.testing.assert_allclose(O[b, h, 0], ref, rtol=0, atol=1e-12)
                else:
                    assert not written[b, h]


def pin_head_order_invariant(impl):
    """Permuting the entries of an index row changes nothing (bitwise)."""
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 3, 6, 6, 10, 4)
    idx = _sorted_rows(rng, 3, 6, 4)
    perm = idx[:, ::-1].copy()
    O1, w1 = impl.mha(q, k, v, idx, 0.5)
    O2, w2 = impl.mha(q, k, v, perm, 0.5)
    assert np.array_equal(w1, w2)
    assert np.array_equal(O1[w1], O2[w2])


def pin_key_permutation_invariant(impl):
    """Permuting K and V rows jointly along Nkv leaves O unchanged."""
    rng = np.random.default_rng(16)
    q, k, v = _rand(rng, 2, 4, 4, 17, 6)
    idx = _sorted_rows(rng, 2, 4, 3)
    p = rng.permutation(17)
    O1, w = impl.mha(q, k, v, idx, 0.4)
    O2, _ = impl.mha(q, k[:, :, p], v[:, :, p], idx, 0.4)
    np.testing.assert_allclose(O1[w], O2[w], rtol=0, atol=1e-13)


def pin_key_shift_invariant(impl):
    """K + 1 u^T adds s q.u to every score of a head: softmax unchanged."""
    rng = np.random.default_rng(17)
    q, k, v = _rand(rng, 2, 4, 4, 12, 6)
    idx = _sorted_rows(rng, 2, 4, 2)
    u = rng.standard_normal(6) * 3.0
    O1, w = impl.mha(q, k, v, idx, 0.3)
    O2, _ = impl.mha(q, k + u, v, idx, 0.3)
    np.testing.assert_allclose(O1[w], O2[w], rtol=0, atol=1e-12)


def pin_value_affine(impl):
    """O(a V + 1 c^T) = a O(V) + c: the weights sum to one."""
    rng = np.random.default_rng(18)
    q, k, v = _rand(rng, 2, 4, 4, 9, 5)
    idx = _sorted_rows(rng, 2, 4, 2)
    c = rng.standard_normal(5)
    O1, w = impl.mha(q, k, v, idx, 0.6)
    O2, _ = impl.mha(q, k, -2.5 * v + c, idx, 0.6)
    np.testing.assert_allclose(O2[w], (-2.5 * O1 + c)[w], rtol=0, atol=1e-12)


def pin_sparse_subset_of_dense(impl):
    """An active head's output does not depend on which other heads are active."""
    rng = np.random.default_rng(19)
    q, k, v = _rand(rng, 3, 5, 5, 8, 4)
    idx = _sorted_rows(rng, 3, 5, 2)
    dense = np.tile(np.arange(5, dtype=np.int32), (3, 1))
    Os, w = impl.mha(q, k, v, idx, 0.5)
    Od, _ = impl.mha(q, k, v, dense, 0.5)
    assert w.sum() == 3 * 2
    assert np.array_equal(Os[w], Od[w])


def pin_gqa_equals_repeated_mha(impl):
    """Group g computed with its shared K/V equals head-level attention on K/V
    repeated G times along the head axis (query heads g*G .. g*G+G-1)."""
    rng = np.random.default_rng(20)
    B, H, H_kv, Nkv, d = 3, 8, 2, 11, 4
    G = H // H_kv
    q, k, v = _rand(rng, B, H, H_kv, Nkv, d)
    gidx = np.array([[1], [0], [1]], dtype=np.int32)
    Og, wg = impl.gqa(q, k, v, gidx, 0.5)
    heads = np.stack([np.arange(g * G, g * G + G) for g in gidx[:, 0]]).astype(np.int32)
    kk, vv = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    Om, wm = impl.mha(q, kk, vv, heads, 0.5)
    assert np.array_equal(wg, wm)
    np.testing.assert_allclose(Og[wg], Om[wm], rtol=0, atol=1e-14)


def pin_large_scores_stable(impl):
    """Scores far beyond exp's range: finite output tending to V at the argmax."""
    rng = np.random.default_rng(21)
    q, k, v = _rand(rng, 2, 3, 3, 16, 8)
    idx = _sorted_rows(rng, 2, 3, 2)
    O, w = impl.mha(q * 1e4, k, v, idx, 1.0)
    assert np.isfinite(O[w]).all()
    for b in range(2):
        for h in idx[b]:
            S = k[b, h] @ q[b, h, 0]
            np.testing.assert_allclose(O[b, h, 0], v[b, h, np.argmax(S)], rtol=0, atol=1e-9)


def pin_untouched_and_padding(impl):
    """Slots not listed keep the prefill; -1 and out-of-range entries are skipped."""
    rng = np.random.default_rng(22)
    q, k, v = _rand(rng, 2, 4, 4, 5, 3)
    prefill = rng.standard_normal((2, 4, 1, 3))
    idx = np.array([[-1, 2], [4, 0]], dtype=np.int32)
    O, w = impl.mha(q, k, v, idx, 0.5, o_in=prefill)
    expect_w = np.zeros((2, 4), bool)
    expect_w[0, 2] = expect_w[1, 0] = True
    assert np.array_equal(w, expect_w)
    assert np.array_equal(O[~w], prefill[~w])
    gidx = np.array([[7], [-3]], dtype=np.int32)
    Og, wg = impl.gqa(q, k[:, :2], v[:, :2], gidx, 0.5, o_in=prefill)
    assert not wg.any() and np.array_equal(Og, prefill)


def _load_golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def pin_golden_closed_forms(impl):
    for case in _load_golden():
        q, k, v = (np.array(case[x], dtype=np.float64) for x in ("q", "k", "v"))
        idx = np.array(case["index"], dtype=np.int32)
        prefill = np.full(q.shape, 123.0)
        fn = impl.gqa if case["kind"] == "gqa" else impl.mha
        O, w = fn(q, k, v, idx, case["scale"], o_in=prefill)
        for key, val in case["expected"].items():
            b, h = map(int, key.split(","))
            assert w[b, h], (case["name"], key)
            np.testing.assert_allclose(O[b, h, 0], val, rtol=0, atol=1e-13,
                                       err_msg=case["name"])
        for key in case["untouched"]:
            b, h = map(int, key.split(","))
            assert not w[b, h] and np.all(O[b, h] == 123.0), (case["name"], key)


def pin_seqlens(impl):
    """Per-row cache lengths: the same as slicing each row's K/V to its
    length; full length is the default; length 1 gives V[0]; <= 0 gives zeros."""
    rng = np.random.default_rng(23)
    q, k, v = _rand(rng, 4, 4, 2, 20, 6)
    idx = np.array([[0, 3], [1, 2], [3, 0], [2, 1]], dtype=np.int32)
    lens = np.array([20, 7, 1, 0])
    O, w = impl.mha(q, k, v, idx, 0.4, seqlens=lens)
    O_full, _ = impl.mha(q, k, v, idx, 0.4)
    assert np.array_equal(O[0], O_full[0], equal_nan=True)
    for b, n in ((1, 7),):
        Ob, _ = impl.mha(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], idx[b:b + 1], 0.4)
        np.testing.assert_allclose(O[b], Ob[0], rtol=0, atol=1e-14)
    for h in idx[2]:
        assert np.array_equal(O[2, h, 0], v[2, h // 2, 0])
    for h in idx[3]:
        assert np.array_equal(O[3, h, 0], np.zeros(6))
    # lengths are clamped to [0, Nkv]
    Oc, _ = impl.mha(q, k, v, idx, 0.4, seqlens=np.array([99, 7, 1, -5]))
    assert np.array_equal(Oc, O, equal_nan=True)
    # group form: lengths apply to every head of the group
    gidx = np.array([[1], [0], [1], [0]], dtype=np.int32)
    Og, wg = impl.gqa(q, k, v, gidx, 0.4, seqlens=np.array([20, 7, 1, 0]))
    Om, _ = impl.mha(q, k, v, np.array([[2, 3], [0, 1], [2, 3], [0, 1]], dtype=np.int32), 0.4,
                     seqlens=np.array([20, 7, 1, 0]))
    np.testing.assert_allclose(Og[wg], Om[wg], rtol=0, atol=1e-14)


PINS = [pin_seqlens, pin_dense_equals_sdpa, pin_single_key_returns_v, pin_uniform_scores_give_mean,
        pin_brute_force, pin_head_order_invariant, pin_key_permutation_invariant,
        pin_key_shift_invariant, pin_value_affine, pin_sparse_subset_of_dense,
        pin_gqa_equals_repeated_mha, pin_large_scores_stable, pin_untouched_and_padding,
        pin_golden_closed_forms]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(REAL)


# ----------------------------------------------------------------------------
# Algorithm 1 as written (tiled online softmax, normalising every tile) in
# fp64 reaches the oracle's two-pass result: the method is exact.
# ----------------------------------------------------------------------------

def _algorithm1_one(q, K, V, s, Bc):
    Nkv = K.shape[0]
    O_acc, l_acc, m_acc = np.zeros(V.shape[1]), 0.0, -np.inf
    for start in range(0, Nkv, Bc):
        Kj, Vj = K[start:start + Bc], V[start:start + Bc]
        Sj = s * (Kj @ q)
        mj = Sj.max()
        Pj = np.exp(Sj - mj)
        lj = Pj.sum()
        m_new = max(m_acc, mj)
        alpha, beta = math.exp(m_acc - m_new), math.exp(mj - m_new)
        l_new = alpha * l_acc + beta * lj
        O_acc = (alpha * l_acc * O_acc + beta * (Pj @ Vj)) / l_new
        l_acc, m_acc = l_new, m_new
    return O_acc


@pytest.mark.parametrize("Bc", [1, 3, 16, 64])
def test_algorithm1_tiling_reaches_definition(Bc):
    rng = np.random.default_rng(30 + Bc)
    q, k, v = _rand(rng, 2, 4, 4, 50, 8, scale_q=3.0)
    idx = _sorted_rows(rng, 2, 4, 2)
    O, w = so.sha_decode_ref(q, k, v, idx, 0.35)
    s = float(np.float32(0.35))
    for b in range(2):
        for h in idx[b]:
            np.testing.assert_allclose(_algorithm1_one(q[b, h, 0], k[b, h], v[b, h], s, Bc),
                                       O[b, h, 0], rtol=0, atol=1e-13)


def test_input_validation():
    q, k, v = _rand(np.random.default_rng(0), 1, 4, 3, 4, 2)
    with pytest.raises(ValueError):
        so.sha_decode_ref(q, k, v, np.zeros((1, 1), np.int32), 1.0)    # 4 % 3 != 0
    q, k, v = _rand(np.random.default_rng(0), 1, 4, 4, 0, 2)
    with pytest.raises(ValueError):
        so.sha_decode_ref(q, k, v, np.zeros((1, 1), np.int32), 1.0)    # Nkv = 0
    q, k, v = _rand(np.random.default_rng(0), 1, 4, 4, 3, 2)
    with pytest.raises(ValueError):
        so.sha_decode_ref(q, k, v, np.zeros((1, 5), np.int32), 1.0)    # top_k > H
    with pytest.raises(ValueError):
        so.sha_decode_gqa_ref(q, k[:, :2], v[:, :2], np.zeros((1, 3), np.int32), 1.0)


def test_widening_bf16_f16_exact():
    """to_f64 widens f16/bf16 storage exactly (checked against bit patterns)."""
    bits = np.array([0x3F80, 0xC040, 0x0001, 0x7F7F], dtype=np.uint16).view(np.int16)
    t = torch.from_numpy(bits).view(torch.bfloat16)
    assert so.to_f64(t).tolist() == [1.0, -3.0, 2.0 ** -133, 3.3895313892515355e38]
    h = np.array([0x3C00, 0x0001, 0x7BFF], dtype=np.uint16).view(np.float16)
    assert so.to_f64(h).tolist() == [1.0, 2.0 ** -24, 65504.0]


# ----------------------------------------------------------------------------
# Mutation check: plausible oracle mistakes must each fail some pin.
# ----------------------------------------------------------------------------

def _mutant_attend(kind):
    def attend(q, K, V, s):
        if kind == "no_scale":
            sc = K @ q
        elif kind == "inverse_scale":
            sc = (K @ q) / s
        else:
            sc = s * (K @ q)
        if kind == "drop_last_key":
            sc, K, V = sc[:-1], K[:-1], V[:-1]
        m = sc.max()
        p = np.exp(sc) if kind == "no_max_shift" else np.exp(sc - m)
        if kind == "pv_uses_k":
            return (p @ K) / p.sum()
        if kind == "divide_by_nkv":
            return (p @ V) / len(p)
        if kind == "transposed_scores":
            # q read against the wrong operand orientation (columns of K).
            sc2 = s * (K[:, ::-1] @ q)
            p2 = np.exp(sc2 - sc2.max())
            return (p2 @ V) / p2.sum()
        return (p @ V) / p.sum()
    return attend


def _mutant_mha(kind):
    def mha(q, k, v, idx, scale, o_in=None, seqlens=None):
        Q, K, V = so.to_f64(q), so.to_f64(k), so.to_f64(v)
        idx = np.asarray(idx)
        B, H = Q.shape[:2]
        H_kv = K.shape[1]
        G = H // H_kv
        s = float(np.float32(scale))
        O = np.full(Q.shape, np.nan) if o_in is None else so.to_f64(o_in).copy()
        w = np.zeros((B, H), bool)
        for b in range(B):
            for kk in range(idx.shape[1]):
                h = int(idx[b, kk])
                if kind == "slot_as_head":
                    h = kk
                if kind != "no_skip" and (h < 0 or h >= H):
                    continue
                h = h % H
                g = h % H_kv if kind == "gqa_modulo" else h // G
                n = K.shape[2] if seqlens is None else max(0, min(int(seqlens[b]), K.shape[2]))
                O[b, h, 0] = so.attend_one(Q[b, h, 0], K[b, g, :n], V[b, g, :n], s) if n else 0.0
                w[b, h] = True
        return O, w
    return mha


def _mutant_gqa(kind):
    def gqa(q, k, v, gidx, scale, o_in=None, seqlens=None):
        Q, K, V = so.to_f64(q), so.to_f64(k), so.to_f64(v)
        gidx = np.asarray(gidx)
        B, H = Q.shape[:2]
        H_kv = K.shape[1]
        G = H // H_kv
        s = float(np.float32(scale))
        O = np.full(Q.shape, np.nan) if o_in is None else so.to_f64(o_in).copy()
        w = np.zeros((B, H), bool)
        for b in range(B):
            for kk in range(gidx.shape[1]):
                g = int(gidx[b, kk])
                if g < 0 or g >= H_kv:
                    continue
                heads = [g] if kind == "gqa_first_head_only" else (
                    [g + j * H_kv for j in range(G)] if kind == "gqa_strided_heads"
                    else [g * G + j for j in range(G)])
                n = K.shape[2] if seqlens is None else max(0, min(int(seqlens[b]), K.shape[2]))
                for h in heads:
                    O[b, h, 0] = so.attend_one(Q[b, h, 0], K[b, g, :n], V[b, g, :n], s) if n else 0.0
                    w[b, h] = True
        return O, w
    return gqa


ATTEND_MUTANTS = ["no_scale", "inverse_scale", "drop_last_key", "no_max_shift",
                  "pv_uses_k", "divide_by_nkv", "transposed_scores"]
INDEX_MUTANTS = ["slot_as_head", "no_skip", "gqa_modulo"]
GQA_MUTANTS = ["gqa_first_head_only", "gqa_strided_heads"]


def _pins_failed(impl, monkeypatch=None):
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("kind", ATTEND_MUTANTS + INDEX_MUTANTS + GQA_MUTANTS)
def test_planted_mistake_is_caught(kind, monkeypatch):
    if kind in ATTEND_MUTANTS:
        monkeypatch.setattr(so, "attend_one", _mutant_attend(kind))
        impl = types.SimpleNamespace(mha=so.sha_decode_ref, gqa=so.sha_decode_gqa_ref)
    elif kind in INDEX_MUTANTS:
        impl = types.SimpleNamespace(mha=_mutant_mha(kind), gqa=so.sha_decode_gqa_ref)
    else:
        impl = types.SimpleNamespace(mha=so.sha_decode_ref, gqa=_mutant_gqa(kind))
    failed = _pins_failed(impl)
    assert failed, f"mutant {kind} passed every pin"


# ----------------------------------------------------------------------------
# Sampled-unit form (sha_units_ref): the checker of the full-size GPU tests.
# Pinned against the whole-call oracle at the same slots (bitwise: the same
# definition evaluated on the same widened operands), closed forms and brute
# force; planted mistakes must each fail.
# ----------------------------------------------------------------------------

def _gather_units(q, k, v, slots, G):
    qs = np.stack([q[b, h, 0] for b, h in slots])
    ks = np.stack([k[b, h // G] for b, h in slots])
    vs = np.stack([v[b, h // G] for b, h in slots])
    return qs, ks, vs


def upin_equals_whole_call(units):
    """Gathered (q, K, V) of active slots give bitwise the whole-call result,
    for f32-exact and f16-rounded operands and a scale that float32 rounds."""
    rng = np.random.default_rng(61)
    for (B, H, H_kv, Nkv, d, top_k) in [(3, 6, 3, 13, 8, 2), (2, 4, 4, 40, 16, 4)]:
        q, k, v = _rand(rng, B, H, H_kv, Nkv, d, scale_q=2.0)
        q, k, v = (torch.from_numpy(a).to(torch.float16) for a in (q, k, v))
        idx = _sorted_rows(rng, B, H, top_k)
        scale = 0.1  # not a float32 value: both forms must round it alike
        O, w = so.sha_decode_ref(q, k, v, idx, scale)
        slots = [tuple(x) for x in np.argwhere(w)]
        got = units(*_gather_units(q.numpy(), k.numpy(), v.numpy(), slots, H // H_kv), scale)
        assert got.shape == (len(slots), d)
        for i, (b, h) in enumerate(slots):
            assert np.array_equal(got[i], O[b, h, 0]), (b, h)


def upin_closed_forms(units):
    """One key gives that key's value row; equal scores give the mean row."""
    rng = np.random.default_rng(62)
    qs, ks, vs = rng.standard_normal((3, 5)), rng.standard_normal((3, 1, 5)), rng.standard_normal((3, 1, 5))
    assert np.array_equal(units(qs, ks, vs, 0.5), vs[:, 0])
    ks = rng.standard_normal((3, 7, 5))
    vs = rng.standard_normal((3, 7, 5))
    qz = np.zeros((3, 5))
    np.testing.assert_allclose(units(qz, ks, vs, 0.5), vs.mean(axis=1), rtol=0, atol=1e-14)


def upin_brute_force(units):
    rng = np.random.default_rng(63)
    qs, ks, vs = rng.standard_normal((4, 6)) * 2, rng.standard_normal((4, 9, 6)), rng.standard_normal((4, 9, 6))
    s = float(np.float32(0.3))
    got = units(qs, ks, vs, s)
    for i in range(4):
        ref = _brute_force_one(qs[i].tolist(), ks[i].tolist(), vs[i].tolist(), s)
        np.testing.assert_allclose(got[i], ref, rtol=0, atol=1e-12)


UNIT_PINS = [upin_equals_whole_call, upin_closed_forms, upin_brute_force]


@pytest.mark.parametrize("pin", UNIT_PINS, ids=lambda p: p.__name__)
def test_units_oracle_pin(pin):
    pin(so.sha_units_ref)


def _mutant_units(kind):
    def units(q_rows, k_slabs, v_slabs, scale):
        qs, Ks, Vs = so.to_f64(q_rows), so.to_f64(k_slabs), so.to_f64(v_slabs)
        s = float(scale) if kind == "unrounded_scale" else float(np.float32(scale))
        n = qs.shape[0]
        out = []
        for i in range(n):
            j = 0 if kind == "first_unit_only" else i
            K, V = (Vs[j], Ks[j]) if kind == "k_v_swapped" else (Ks[j], Vs[j])
            out.append(so.attend_one(qs[i], K, V, s))
        res = np.stack(out)
        return res[::-1].copy() if kind == "reversed_order" else res
    return units


@pytest.mark.parametrize("kind", ["unrounded_scale", "first_unit_only", "k_v_swapped",
                                  "reversed_order"])
def test_planted_units_mistake_is_caught(kind):
    failed = []
    for pin in UNIT_PINS:
        try:
            pin(_mutant_units(kind))
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every pin"
