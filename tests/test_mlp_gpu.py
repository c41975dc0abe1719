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
                                   (16, 4097, 65536), (1, 1, 1), (3, 7, 65536), (8, 3686, 36864),
                                   (2, 4096, 262144), (1, 8193, 262144), (2, 100, 262145),
                                   (1, 8192, 300000), (4, 2048, 1000)])
@pytest.mark.parametrize("path", ["auto", "three_kernels"])
def test_union_matches_oracle(B, k, D, path, monkeypatch):
    """Unions of at most 8192 entries and 2^18 neurons run in one workgroup
    unless SHA_MLP_UNION_SMALL=0; larger ones (entries or neurons) always take
    the three-kernel path."""
    if path == "three_kernels":
        monkeypatch.setenv("SHA_MLP_UNION_SMALL", "0")
    say(f"[mlp] union B={B} k={k} D={D} {path}")
    rng = np.random.default_rng(B * 1000 + k)
    rows = rng.integers(-2, D + 3, size=(B, k)).astype(np.int32)
    sel, n_sel = sha.mlp_union(torch.from_numpy(rows).to(DEV), D)
    torch.cuda.synchronize()
    want = mlp_union_ref(rows, D)
    n = int(n_sel.item())
    assert n == len(want)
    assert np.array_equal(sel[:n].cpu().numpy(), want)


@pytest.mark.parametrize("B,d,D,k_row", [(1, 4096, 16384, 1638), (16, 1024, 3000, 200),
                                         (40, 512, 2000, 150), (70, 512, 900, 60),
                                         (5, 768, 1000, 100)])
def test_down_waves_agree(B, d, D, k_row, monkeypatch):
    """The 4-wave (256-column) and 8-wave (512-column) down workgroups give
    bit-identical outputs at the same split count (each output sums the
    same neuron chunks in the same order) and both match the oracle; a width
    that is not a multiple of 512 keeps the 4-wave form."""
    say(f"[mlp] down waves B={B} d={d} D={D} k_row={k_row}")
    w = wl.MlpWorkload("t", B=B, d=d, D=D, k_row=k_row, dtype="bf16", seed=B * 5 + d)
    x, w1t, w2t, rows = wl.make_mlp(w, "cpu")
    sel, n_sel = sha.mlp_union(rows.to(DEV), D)
    ref = selective_mlp_ref(x, w1t, w2t, mlp_union_ref(rows, D))
    xd, w1d, w2d = x.to(DEV), w1t.to(DEV), w2t.to(DEV)
    outs = {}
    for splits in ("3", None):
        for waves in ("4", "8"):
            monkeypatch.setenv("SHA_MLP_DN_WAVES", waves)
            if splits:
                monkeypatch.setenv("SHA_MLP_DN_SPLITS", splits)
            else:
                monkeypatch.delenv("SHA_MLP_DN_SPLITS", raising=False)
            y = sha.selective_mlp(xd, w1d, w2d, sel, n_sel, n_max=sel.numel())
            torch.cuda.synchronize()
            err = float(np.abs(y.cpu().double().numpy() - ref).max())
            assert err <= _tol("bf16", ref), (waves, splits, err)
            outs[(splits, waves)] = y.cpu()
    assert torch.equal(wl.raw_bits(outs[("3", "4")]), wl.raw_bits(outs[("3", "8")]))


@pytest.mark.parametrize("B,d,D,k_row", [(1, 4096, 16384, 1638), (16, 1024, 3000, 200),
                                         (5, 768, 1000, 100), (16, 4096, 16384, 1638),
                                         (20, 1024, 3000, 150), (32, 512, 2500, 80),
                                         (17, 4096, 16384, 1638)])
def test_up_shared_x_agrees(B, d, D, k_row, monkeypatch):
    """Batches of at most 32 rows (one or two batch blocks): the up workgroup
    with x shared through LDS gives bit-identical outputs to the one whose
    waves each load all of their x, and both match the oracle."""
    say(f"[mlp] up shared x B={B} d={d} D={D} k_row={k_row}")
    w = wl.MlpWorkload("t", B=B, d=d, D=D, k_row=k_row, dtype="f16", seed=B * 11 + d)
    x, w1t, w2t, rows = wl.make_mlp(w, "cpu")
    sel, n_sel = sha.mlp_union(rows.to(DEV), D)
    ref = selective_mlp_ref(x, w1t, w2t, mlp_union_ref(rows, D))
    xd, w1d, w2d = x.to(DEV), w1t.to(DEV), w2t.to(DEV)
    outs = {}
    for mode in ("0", "2"):
        monkeypatch.setenv("SHA_MLP_UP_XLDS", mode)
        y = sha.selective_mlp(xd, w1d, w2d, sel, n_sel, n_max=sel.numel())
        torch.cuda.synchronize()
        err = float(np.abs(y.cpu().double().numpy() - ref).max())
        assert err <= _tol("f16", ref), (mode, err)
        outs[mode] = y.cpu()
    assert torch.equal(wl.raw_bits(outs["0"]), wl.raw_bits(outs["2"]))


@pytest.mark.parametrize("B,d,D,k_row", [(64, 1024, 36864, 3686), (40, 512, 2000, 150),
                                         (70, 256, 900, 60), (33, 768, 5000, 40),
                                         (40, 256, 100, 30)])
def test_up_tiles_agree(B, d, D, k_row, monkeypatch):
    """Full batch tiles: 128- and 144-neuron up workgroups give bit-identical
    outputs at the same K split count (per neuron the same stages in the
    same order) and both match the oracle; the shapes include selections
    whose last 144-neuron tile runs past the padding."""
    say(f"[mlp] up tiles B={B} d={d} D={D} k_row={k_row}")
    w = wl.MlpWorkload("t", B=B, d=d, D=D, k_row=k_row, dtype="bf16", seed=B * 13 + d)
    x, w1t, w2t, rows = wl.make_mlp(w, "cpu")
    sel, n_sel = sha.mlp_union(rows.to(DEV), D)
    ref = selective_mlp_ref(x, w1t, w2t, mlp_union_ref(rows, D))
    xd, w1d, w2d = x.to(DEV), w1t.to(DEV), w2t.to(DEV)
    outs = {}
    for splits in ("2", None):
        for tile in ("128", "144"):
            monkeypatch.setenv("SHA_MLP_UP_TILE", tile)
            if splits:
                monkeypatch.setenv("SHA_MLP_UP_SPLITS", splits)
            else:
                monkeypatch.delenv("SHA_MLP_UP_SPLITS", raising=False)
            y = sha.selective_mlp(xd, w1d, w2d, sel, n_sel, n_max=sel.numel())
            torch.cuda.synchronize()
            err = float(np.abs(y.cpu().double().numpy() - ref).max())
            assert err <= _tol("bf16", ref), (tile, splits, err)
            outs[(splits, tile)] = y.cpu()
    assert torch.equal(wl.raw_bits(outs[("2", "128")]), wl.raw_bits(outs[("2", "144")]))


@pytest.mark.parametrize("B,d,D,k_row", [(64, 1024, 36864, 3686), (40, 512, 2000, 150),
                                         (70, 256, 900, 60), (33, 768, 5000, 40),
                                         (40, 256, 100, 30), (128, 1024, 4000, 300)])
def test_up_k_groups_agree(B, d, D, k_row, monkeypatch):
    """Full batch tiles: the 512-thread up workgroup that splits K between
    its two halves and sums them on chip gives bit-identical outputs to two
    K splits summed by the finalize (same halves, same order), for 128- and
    144-neuron tiles, with one or two batch tiles and a single stage per
    half (d = 256), and matches the oracle."""
    say(f"[mlp] up K groups B={B} d={d} D={D} k_row={k_row}")
    w = wl.MlpWorkload("t", B=B, d=d, D=D, k_row=k_row, dtype="bf16", seed=B * 29 + d)
    x, w1t, w2t, rows = wl.make_mlp(w, "cpu")
    sel, n_sel = sha.mlp_union(rows.to(DEV), D)
    ref = selective_mlp_ref(x, w1t, w2t, mlp_union_ref(rows, D))
    xd, w1d, w2d = x.to(DEV), w1t.to(DEV), w2t.to(DEV)
    for tile in ("128", "144"):
        outs = {}
        monkeypatch.setenv("SHA_MLP_UP_TILE", tile)
        for kg in ("1", "2"):
            monkeypatch.setenv("SHA_MLP_UP_KG", kg)
            if kg == "1":
                monkeypatch.setenv("SHA_MLP_UP_SPLITS", "2")
            else:
                monkeypatch.delenv("SHA_MLP_UP_SPLITS", raising=False)
            y = sha.selective_mlp(xd, w1d, w2d, sel, n_sel, n_max=sel.numel())
            torch.cuda.synchronize()
            err = float(np.abs(y.cpu().double().numpy() - ref).max())
            assert err <= _tol("bf16", ref), (tile, kg, err)
            outs[kg] = y.cpu()
        assert torch.equal(wl.raw_bits(outs["1"]), wl.raw_bits(outs["2"])), tile


@pytest.mark.parametrize("B,d,D,k_row,splits", [(16, 4096, 16384, 1638, None),
                                                (8, 9216, 36864, 3686, None),
                                                (20, 1024, 3000, 200, "2"), (5, 768, 1000, 100, "3"),
                                                (30, 768, 5000, 300, "4"), (1, 512, 700, 650, "4"),
                                                (12, 256, 2000, 150, "2")])
def test_down_folds_up_finalize_agree(B, d, D, k_row, splits, monkeypatch):
    """One or two batch blocks with 2-4 up K splits: the down projection
    summing the up partials itself gives bit-identical outputs to the up
    finalize followed by the down projection (4- and 8-wave down
    workgroups, selections ending inside a chunk) and matches the oracle."""
    say(f"[mlp] folded up finalize B={B} d={d} D={D} k_row={k_row} splits={splits}")
    w = wl.MlpWorkload("t", B=B, d=d, D=D, k_row=k_row, dtype="f16", seed=B * 37 + d)
    x, w1t, w2t, rows = wl.make_mlp(w, "cpu")
    sel, n_sel = sha.mlp_union(rows.to(DEV), D)
    ref = selective_mlp_ref(x, w1t, w2t, mlp_union_ref(rows, D))
    xd, w1d, w2d = x.to(DEV), w1t.to(DEV), w2t.to(DEV)
    if splits:
        monkeypatch.setenv("SHA_MLP_UP_SPLITS", splits)
    outs = {}
    for fold in ("0", "1"):
        monkeypatch.setenv("SHA_MLP_FUSE_UP", fold)
        y = sha.selective_mlp(xd, w1d, w2d, sel, n_sel, n_max=sel.numel())
        torch.cuda.synchronize()
        err = float(np.abs(y.cpu().double().numpy() - ref).max())
        assert err <= _tol("f16", ref), (fold, err)
        outs[fold] = y.cpu()
    assert torch.equal(wl.raw_bits(outs["0"]), wl.raw_bits(outs["1"]))


@pytest.mark.parametrize("B,d,D,k_row", [(32, 1024, 36864, 3686), (24, 512, 36864, 3000),
                                         (20, 256, 36864, 2000), (17, 768, 40000, 3000),
                                         (30, 512, 3000, 200)])
def test_full_tiles_for_two_blocks_agree(B, d, D, k_row, monkeypatch):
    """Batches of 17-32 rows computed as two batch blocks or as the whole
    64-row tile (the plan's choice when the two-K-group up form then fills
    the chip; padding rows repeat row B - 1 and are never stored) give
    bit-identical outputs (per neuron and output the same K stages, splits
    and chunks in the same order) and match the oracle."""
    say(f"[mlp] full tiles for two blocks B={B} d={d} D={D} k_row={k_row}")
    w = wl.MlpWorkload("t", B=B, d=d, D=D, k_row=k_row, dtype="bf16", seed=B * 31 + d)
    x, w1t, w2t, rows = wl.make_mlp(w, "cpu")
    sel, n_sel = sha.mlp_union(rows.to(DEV), D)
    ref = selective_mlp_ref(x, w1t, w2t, mlp_union_ref(rows, D))
    xd, w1d, w2d = x.to(DEV), w1t.to(DEV), w2t.to(DEV)
    outs = {}
    for bb in ("2", "4", None):
        if bb:
            monkeypatch.setenv("SHA_MLP_BB", bb)
        else:
            monkeypatch.delenv("SHA_MLP_BB", raising=False)
        y = sha.selective_mlp(xd, w1d, w2d, sel, n_sel, n_max=sel.numel())
        torch.cuda.synchronize()
        err = float(np.abs(y.cpu().double().numpy() - ref).max())
        assert err <= _tol("bf16", ref), (bb, err)
        outs[bb] = y.cpu()
    assert torch.equal(wl.raw_bits(outs["2"]), wl.raw_bits(outs["4"]))
    assert torch.equal(wl.raw_bits(outs["2"]), wl.raw_bits(outs[None]))


@pytest.mark.parametrize("B,d,D,k_row,waves", [(64, 1024, 3000, 200, "8"), (64, 768, 3000, 200, "4"),
                                               (70, 512, 2000, 150, "8"), (16, 4096, 16384, 1638, "8"),
                                               (20, 1024, 1500, 60, "8"), (5, 768, 1000, 100, "4")])
def test_down_staged_partials_agree(B, d, D, k_row, waves, monkeypatch):
    """The down kernel's split partials stored through LDS as whole-row
    pieces give bit-identical outputs to the direct stores (4- and 8-wave
    workgroups, one to four batch blocks, two batch tiles, partial rows past
    B) and match the oracle."""
    say(f"[mlp] staged partials B={B} d={d} D={D} k_row={k_row} waves={waves}")
    w = wl.MlpWorkload("t", B=B, d=d, D=D, k_row=k_row, dtype="bf16", seed=B * 19 + d)
    x, w1t, w2t, rows = wl.make_mlp(w, "cpu")
    sel, n_sel = sha.mlp_union(rows.to(DEV), D)
    ref = selective_mlp_ref(x, w1t, w2t, mlp_union_ref(rows, D))
    xd, w1d, w2d = x.to(DEV), w1t.to(DEV), w2t.to(DEV)
    monkeypatch.setenv("SHA_MLP_DN_WAVES", waves)
    monkeypatch.setenv("SHA_MLP_DN_SPLITS", "3")
    outs = {}
    for stage in ("0", "1"):
        monkeypatch.setenv("SHA_MLP_DN_STAGE", stage)
        y = sha.selective_mlp(xd, w1d, w2d, sel, n_sel, n_max=sel.numel())
        torch.cuda.synchronize()
        err = float(np.abs(y.cpu().double().numpy() - ref).max())
        assert err <= _tol("bf16", ref), (stage, err)
        outs[stage] = y.cpu()
    assert torch.equal(wl.raw_bits(outs["0"]), wl.raw_bits(outs["1"]))


@pytest.mark.parametrize("B,d,D,k_row,tile", [(64, 1024, 36864, 3686, "144"), (64, 1024, 3000, 200, "128"),
                                              (70, 512, 2000, 150, "144"), (40, 256, 100, 30, "144"),
                                              (33, 768, 5000, 40, "128")])
def test_up_staged_partials_agree(B, d, D, k_row, tile, monkeypatch):
    """Full batch tiles: the up kernel's K-split partials stored through LDS
    as whole-row pieces give bit-identical outputs to the direct stores
    (128- and 144-neuron tiles, a last tile past the padding, two batch
    tiles, rows past B) and match the oracle."""
    say(f"[mlp] up staged partials B={B} d={d} D={D} k_row={k_row} tile={tile}")
    w = wl.MlpWorkload("t", B=B, d=d, D=D, k_row=k_row, dtype="bf16", seed=B * 23 + d)
    x, w1t, w2t, rows = wl.make_mlp(w, "cpu")
    sel, n_sel = sha.mlp_union(rows.to(DEV), D)
    ref = selective_mlp_ref(x, w1t, w2t, mlp_union_ref(rows, D))
    xd, w1d, w2d = x.to(DEV), w1t.to(DEV), w2t.to(DEV)
    monkeypatch.setenv("SHA_MLP_UP_TILE", tile)
    monkeypatch.setenv("SHA_MLP_UP_SPLITS", "2")
    outs = {}
    for stage in ("0", "1"):
        monkeypatch.setenv("SHA_MLP_UP_STAGE", stage)
        y = sha.selective_mlp(xd, w1d, w2d, sel, n_sel, n_max=sel.numel())
        torch.cuda.synchronize()
        err = float(np.abs(y.cpu().double().numpy() - ref).max())
        assert err <= _tol("bf16", ref), (stage, err)
        outs[stage] = y.cpu()
    assert torch.equal(wl.raw_bits(outs["0"]), wl.raw_bits(outs["1"]))


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
                                         (70, 256, 700, 30), (5, 768, 4096, 400),
                                         (17, 256, 800, 40), (20, 256, 1500, 60),
                                         (32, 512, 2500, 80), (40, 256, 900, 50)])
def test_selective_mlp_union_pipeline(dtype, B, d, D, k_row):
    """router rows -> union on device -> selective MLP; compare with the oracle.
    Batches of 1-16, 17-32 and 33+ rows run the kernels' 1, 2 and 4 batch-block
    forms (70 rows: two batch tiles)."""
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


@pytest.mark.parametrize("B,D", [(64, 36864), (24, 36864), (8, 36864), (40, 600)])
def test_selection_edge_cases_every_plan(B, D):
    """The edge cases above under each planned form: n_max = D = 36864 at
    B = 64 and 24 takes 256 up workgroups with two K groups (B = 24 as a
    whole 64-row tile), B = 8 the folded up finalize; B = 40 with a small D
    the four-wave form with K splits.  An empty selection gives zeros and
    padding entries inside a short count contribute nothing."""
    say(f"[mlp] edge cases under the plan for B={B} D={D}")
    w = wl.MlpWorkload("t", B=B, d=256, D=D, k_row=10, dtype="bf16", seed=B + 11)
    x, w1t, w2t, _ = wl.make_mlp(w, "cpu")
    xd, w1d, w2d = x.to(DEV), w1t.to(DEV), w2t.to(DEV)
    sel = torch.zeros(D, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    assert np.array_equal(_run(xd, w1d, w2d, sel, cnt, n_max=D), np.zeros((B, 256)))
    entries = np.array([D - 1, -1, 3, D + 5, 250, 7, 42, D - 1, 599], dtype=np.int32)
    sel = torch.from_numpy(np.concatenate([entries, np.full(D - len(entries), 5, np.int32)])).to(DEV)
    cnt = torch.tensor([len(entries)], dtype=torch.int32, device=DEV)
    got = _run(xd, w1d, w2d, sel, cnt, n_max=D)
    ref = selective_mlp_ref(x, w1t, w2t, entries)
    assert float(np.abs(got - ref).max()) <= _tol("bf16", ref)


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
