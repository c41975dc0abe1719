"""Selective MLP on the GPU against the fp64 oracle (through the C ABI).

Tolerance (derived from the arithmetic): the inputs are exact 16-bit values,
products and sums are fp32, relu(x W1[:, S]) is rounded once to the 16-bit
type and y once more.  Each rounding is at most u relative (u = 2^-8 for
bf16, 2^-11 for f16), so |y_gpu - y| <= 4 u max(1, max|y|) with a wide margin
for the O(1) activations these inputs produce.
"""
import numpy as np
import pytest
import torch

import contextual_head_sparsity_amd as sha
from contextual_head_sparsity_amd import workloads as wl
from oracle import mlp_union_ref, selective_mlp_ref

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
U = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def say(m):
    print(m, flush=True)


def _tol(dtype, ref):
    return 4 * U[dtype] * max(1.0, float(np.abs(ref).max()))


def _run(x, w1t, w2t, sel, n_sel, n_max=None):
    y = sha.selective_mlp(x, w1t, w2t, sel, n_sel, n_max=n_max)
    torch.cuda.synchronize()
    return y.cpu().double().numpy()


@pytest.mark.parametrize("B,k,D", [(1, 5, 100), (7, 40, 1000), (64, 300, 5000), (3, 0, 10),
                                   (5, 33, 40000), (9, 500, 100000), (64, 3686, 36864),
                                   (2, 70000, 65537), (16, 1638, 16384), (16, 4096, 65536),
                                   (16, 4097, 65536), (1, 1, 1), (3, 7, 65536), (8, 3686, 36864)])
def test_union_matches_oracle(B, k, D):
    say(f"[mlp] union B={B} k={k} D={D}")
    rng = np.random.default_rng(B * 1000 + k)
    rows = rng.integers(-2, D + 3, size=(B, k)).astype(np.int32)
    sel, n_sel = sha.mlp_union(torch.from_numpy(rows).to(DEV), D)
    torch.cuda.synchronize()
    want = mlp_union_ref(rows, D)
    n = int(n_sel.item())
    assert n == len(want)
    assert np.array_equal(sel[:n].cpu().numpy(), want)


def test_union_rows_not_16_byte_aligned():
    """Row lists need only 4-byte alignment (here 4 bytes past a 16-byte
    boundary)."""
    say("[mlp] union, rows at a 4-byte offset")
    rng = np.random.default_rng(77)
    B, k, D = 6, 301, 5000
    flat = torch.from_numpy(rng.integers(-2, D + 3, size=B * k + 1).astype(np.int32)).to(DEV)
    rows = flat[1:].view(B, k)
    assert rows.data_ptr() % 16 == 4
    sel, n_sel = sha.mlp_union(rows, D)
    torch.cuda.synchronize()
    want = mlp_union_ref(rows.cpu().numpy(), D)
    n = int(n_sel.item())
    assert n == len(want)
    assert np.array_equal(sel[:n].cpu().numpy(), want)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,d,D,k_row", [(1, 256, 300, 20), (3, 256, 1000, 50), (64, 512, 2000, 100),
                                         (70, 256, 700, 30), (5, 768, 4096, 400)])
def test_selective_mlp_union_pipeline(dtype, B, d, D, k_row):
    """router rows -> union on device -> selective MLP; compare with the oracle."""
    say(f"[mlp] pipeline {dtype} B={B} d={d} D={D} k_row={k_row}")
    w = wl.MlpWorkload("t", B=B, d=d, D=D, k_row=k_row, dtype=dtype, seed=B + d)
    x, w1t, w2t, rows = wl.make_mlp(w, "cpu")
    sel, n_sel = sha.mlp_union(rows.to(DEV), D)
    got = _run(x.to(DEV), w1t.to(DEV), w2t.to(DEV), sel, n_sel)
    S = mlp_union_ref(rows, D)
    ref = selective_mlp_ref(x, w1t, w2t, S)
    err = float(np.abs(got - ref).max())
    say(f"   n_sel={len(S)} max_err={err:.3e} tol={_tol(dtype, ref):.3e}")
    assert err <= _tol(dtype, ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_selection_edge_cases(dtype):
    say(f"[mlp] edge cases {dtype}")
    w = wl.MlpWorkload("t", B=5, d=256, D=600, k_row=10, dtype=dtype, seed=7)
    x, w1t, w2t, _ = wl.make_mlp(w, "cpu")
    xd, w1d, w2d = x.to(DEV), w1t.to(DEV), w2t.to(DEV)
    # empty selection -> zeros
    sel = torch.zeros(64, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    assert np.array_equal(_run(xd, w1d, w2d, sel, cnt), np.zeros((5, 256)))
    # padding (-1, >= D) inside the counted entries contributes nothing;
    # the device count limits which entries are read; unsorted order is fine
    entries = np.array([599, -1, 3, 1000, 250, 7, 42, 599], dtype=np.int32)
    sel = torch.from_numpy(np.concatenate([entries, np.full(56, 5, np.int32)])).to(DEV)
    cnt = torch.tensor([len(entries)], dtype=torch.int32, device=DEV)
    got = _run(xd, w1d, w2d, sel, cnt, n_max=64)
    ref = selective_mlp_ref(x, w1t, w2t, entries)
    assert float(np.abs(got - ref).max()) <= _tol(dtype, ref)
    # a device count above n_max is clamped to n_max
    cnt = torch.tensor([1000], dtype=torch.int32, device=DEV)
    got = _run(xd, w1d, w2d, sel, cnt, n_max=10)
    ref = selective_mlp_ref(x, w1t, w2t, sel[:10].cpu().numpy())
    assert float(np.abs(got - ref).max()) <= _tol(dtype, ref)


def test_dense_selection_and_determinism():
    say("[mlp] dense + determinism")
    w = wl.MlpWorkload("t", B=64, d=512, D=3000, k_row=3000, dtype="bf16", seed=3)
    x, w1t, w2t, _ = wl.make_mlp(w, "cpu")
    sel = torch.arange(3000, dtype=torch.int32, device=DEV)
    cnt = torch.tensor([3000], dtype=torch.int32, device=DEV)
    g1 = _run(x.to(DEV), w1t.to(DEV), w2t.to(DEV), sel, cnt)
    g2 = _run(x.to(DEV), w1t.to(DEV), w2t.to(DEV), sel, cnt)
    assert np.array_equal(g1, g2)
    dense = torch.nn.functional.linear(
        torch.relu(torch.nn.functional.linear(x.double(), w1t.double())), w2t.double().T).numpy()
    assert float(np.abs(g1 - dense).max()) <= _tol("bf16", dense)


@pytest.mark.parametrize("name", ["opt6.7b_mlp_f16", "opt66b_mlp_bf16"])
def test_full_size_sampled_rows(name):
    """Full OPT MLP shapes on the GPU; the oracle checks a sample of rows."""
    w = wl.MLP_WORKLOADS[name]
    say(f"[mlp] full size {name}")
    x, w1t, w2t, rows = wl.make_mlp(w, DEV)
    sel, n_sel = sha.mlp_union(rows, w.D)
    y = sha.selective_mlp(x, w1t, w2t, sel, n_sel)
    torch.cuda.synchronize()
    n = int(n_sel.item())
    S = sel[:n].cpu().numpy()
    assert np.array_equal(S, mlp_union_ref(rows.cpu(), w.D))
    pick = np.random.default_rng(w.seed).choice(w.B, size=min(4, w.B), replace=False)
    ref = selective_mlp_ref(x[pick].cpu(), w1t.cpu(), w2t.cpu(), S)
    got = y[pick].cpu().double().numpy()
    err = float(np.abs(got - ref).max())
    say(f"   union={n}/{w.D} max_err={err:.3e}")
    assert err <= _tol(w.dtype, ref)
    assert torch.isfinite(y).all()
