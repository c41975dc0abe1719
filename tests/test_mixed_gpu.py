"""Seeded sweep of decode calls that mix the features the other GPU tests
take one at a time: head-indexed calls with shared KV heads and group calls
with G from 1 to 32, d = 64 / 128, all three element types, cache lengths
from 1 to 3000 keys (ragged per row or not), contiguous, [B, Nkv, H_kv, d]
strided and paged caches, library-planned and forced split counts, and index
rows holding padding (-1, out of range) and repeated entries.  Each call is
compared with the fp64 oracle on the same inputs (active slots within the
dtype tolerance, inactive slots bit-identical to their prefill) and run twice
for bitwise determinism.  Rows past a row's length are NaN in the cache, so
a read beyond it shows.  Two smaller sweeps do the same for the selective MLP
(batch rows over one to three 64-row tiles, widths and neuron counts across
the 128-neuron and 256-column tiles, empty and padded selections) and the
router (1-1024 heads, ragged hidden widths, top_k from 0 to H; the K-split
form forced too wherever the shape has one), with the tolerances of their
own GPU test files."""
import os

import numpy as np
import pytest
import torch

import contextual_head_sparsity_amd as sha
from contextual_head_sparsity_amd import workloads as wl
from oracle import sha_decode_gqa_ref, sha_decode_ref

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import DEV, TOL, bnhd, paged, ragged, say

# SHA_MIXED_CASES / _MLP / _ROUTER widen a sweep for a one-off longer check.
N_CASES = int(os.environ.get("SHA_MIXED_CASES", 48))


def _case(i):
    rng = np.random.default_rng(9100 + i)
    dtype = ("f32", "f16", "bf16")[int(rng.integers(3))]
    gqa = bool(rng.integers(2))
    d = (64, 128)[int(rng.integers(2))]
    B = int(rng.integers(1, 7))
    Nkv = max(1, int(np.exp(rng.uniform(0.0, np.log(3000.0)))))
    if gqa:
        H_kv = int(rng.integers(1, 9))
        G = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 17, 32]))
        H, n_sel = H_kv * G, H_kv
    else:
        H = int(rng.integers(1, 25))
        H_kv = int(rng.choice([x for x in (1, 2, 3, 4, H) if H % x == 0]))
        n_sel = H
    top_k = int(rng.integers(1, n_sel + 1))
    idx = np.stack([rng.permutation(n_sel)[:top_k] for _ in range(B)]).astype(np.int32)
    if top_k >= 2 and rng.integers(2):        # padding: -1 and an id past the range
        idx[0, -1] = -1
        idx[-1, 0] = n_sel
    if top_k >= 3 and rng.integers(2):        # a repeated entry
        idx[B // 2, 1] = idx[B // 2, 2]
    layout = ("contig", "bnhd", "paged16", "paged64")[int(rng.integers(4))]
    lens = rng.integers(-2, Nkv + 40, size=B).astype(np.int32) if rng.integers(2) else None
    nsplit = int(rng.choice([0, 1, 2, 3, 7, 16]))
    w = wl.Workload(f"mixed{i}", B=B, H=H, H_kv=H_kv, d=d, Nkv=Nkv, top_k=top_k, dtype=dtype,
                    gqa=gqa, seed=300 + i)
    return w, torch.from_numpy(idx), layout, lens, nsplit


def _run(w, q, kd, vd, bt, idx, o, lens, nsplit):
    out = o.to(DEV)
    sl = torch.from_numpy(lens).to(DEV) if lens is not None else None
    if bt is not None:
        sha.sha_decode_paged(q.to(DEV), kd, vd, bt, idx.to(DEV), w.Nkv, seqlens=sl, gqa=w.gqa,
                             scale=w.scale, out=out, nsplit=nsplit)
    else:
        fn = sha.sha_decode_gqa if w.gqa else sha.sha_decode
        fn(q.to(DEV), kd, vd, idx.to(DEV), scale=w.scale, out=out, nsplit=nsplit, seqlens=sl)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("i", range(N_CASES))
def test_mixed_features(i):
    w, idx, layout, lens, nsplit = _case(i)
    say(f"[mixed {i}] {w.dtype} gqa={w.gqa} B={w.B} H={w.H} H_kv={w.H_kv} d={w.d} "
        f"Nkv={w.Nkv} top_k={w.top_k} layout={layout} ragged={lens is not None} nsplit={nsplit}")
    q, k, v, _, o = wl.make_workload(w, "cpu")
    if lens is not None:
        k, v = ragged(w, k, v, lens)
    bt = None
    if layout == "bnhd":
        kd, vd = bnhd(k), bnhd(v)
    elif layout.startswith("paged"):
        kd, vd, bt = paged(w, k, v, int(layout[5:]), "nphd", seed=i)
    else:
        kd, vd = k.to(DEV), v.to(DEV)
    got = _run(w, q, kd, vd, bt, idx, o, lens, nsplit)
    ref_fn = sha_decode_gqa_ref if w.gqa else sha_decode_ref
    ref, written = ref_fn(q, k, v, idx, w.scale, seqlens=lens)
    g64 = got.cpu().to(torch.float64).numpy()
    assert np.isfinite(g64[written]).all(), "non-finite output in an active slot"
    err = float(np.max(np.abs(g64[written] - ref[written]))) if written.any() else 0.0
    assert err <= TOL[w.dtype], f"max abs error {err:.3e}"
    wt = torch.from_numpy(written)
    assert torch.equal(wl.raw_bits(got.cpu())[~wt], wl.raw_bits(o)[~wt]), "an inactive slot changed"
    again = _run(w, q, kd, vd, bt, idx, o, lens, nsplit)
    assert torch.equal(wl.raw_bits(again), wl.raw_bits(got)), "two runs differ"
    say(f"   max abs error {err:.2e}")


# ---------------------------------------------------------------------------
# selective MLP and router: seeded shapes across their tile boundaries
# ---------------------------------------------------------------------------

N_MLP = int(os.environ.get("SHA_MIXED_MLP", 24))
U16 = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def _mlp_case(i):
    rng = np.random.default_rng(9500 + i)
    dtype = ("bf16", "f16")[int(rng.integers(2))]
    B = int(rng.integers(1, 141))                       # 1-3 tiles of 64 rows
    d = int(rng.choice([256, 512, 768, 1280, 2048]))
    D = max(1, int(np.exp(rng.uniform(0.0, np.log(12000.0)))))
    k_row = int(rng.integers(0, min(D, 800) + 1))
    pad = bool(rng.integers(2))
    return wl.MlpWorkload(f"mixed_mlp{i}", B=B, d=d, D=D, k_row=k_row, dtype=dtype, seed=60 + i), pad


def _mlp_splits(i):
    """Forced split counts for some cases (0: the planner's), from their own
    seed so the shapes above do not depend on them."""
    rng = np.random.default_rng(9600 + i)
    return int(rng.choice([0, 0, 1, 2, 3, 8])), int(rng.choice([0, 0, 1, 2, 5]))


@pytest.mark.parametrize("i", range(N_MLP))
def test_mixed_selective_mlp(i, monkeypatch):
    """Batches of 1-140 rows (every batch-block form, 1-3 batch tiles), with
    the planner's split counts and down workgroup form or forced ones
    (SHA_MLP_UP_SPLITS / SHA_MLP_DN_SPLITS / SHA_MLP_DN_WAVES /
    SHA_MLP_UP_TILE / SHA_MLP_UP_KG / SHA_MLP_BB / SHA_MLP_FUSE_UP, read by
    the library on every call)."""
    from oracle import mlp_union_ref, selective_mlp_ref
    w, pad = _mlp_case(i)
    us, ds = _mlp_splits(i)
    rw = np.random.default_rng(9700 + i)
    waves = int(rw.choice([0, 0, 4]))
    tile = int(rw.choice([0, 0, 128, 144]))
    kg = int(np.random.default_rng(9800 + i).choice([0, 0, 1, 2]))
    if kg:
        monkeypatch.setenv("SHA_MLP_UP_KG", str(kg))
    bb = int(np.random.default_rng(10000 + i).choice([0, 0, 0, 2, 4]))
    if bb:
        monkeypatch.setenv("SHA_MLP_BB", str(bb))
    fold = int(np.random.default_rng(10100 + i).choice([1, 1, 0]))
    monkeypatch.setenv("SHA_MLP_FUSE_UP", str(fold))
    if tile:
        monkeypatch.setenv("SHA_MLP_UP_TILE", str(tile))
    if waves:
        monkeypatch.setenv("SHA_MLP_DN_WAVES", str(waves))
    if us:
        monkeypatch.setenv("SHA_MLP_UP_SPLITS", str(us))
    if ds:
        monkeypatch.setenv("SHA_MLP_DN_SPLITS", str(ds))
    say(f"[mixed mlp {i}] {w.dtype} B={w.B} d={w.d} D={w.D} k_row={w.k_row} pad={pad} "
        f"up_splits={us or 'plan'} dn_splits={ds or 'plan'} dn_waves={waves or 'plan'} "
        f"up_tile={tile or 'plan'} up_kg={kg or 'plan'} bb={bb or 'plan'} fold={fold}")
    x, w1t, w2t, rows = wl.make_mlp(w, "cpu")
    if pad and w.k_row > 0:                            # entries outside [0, D) are skipped
        rows = rows.clone()
        rows[0, 0] = -1
        rows[-1, -1] = w.D
    sel, n_sel = sha.mlp_union(rows.to(DEV), w.D)
    y = sha.selective_mlp(x.to(DEV), w1t.to(DEV), w2t.to(DEV), sel, n_sel)
    torch.cuda.synchronize()
    S = mlp_union_ref(rows.numpy(), w.D)
    assert int(n_sel.item()) == len(S)
    assert np.array_equal(sel[:len(S)].cpu().numpy(), S)
    ref = selective_mlp_ref(x, w1t, w2t, S)
    got = y.cpu().double().numpy()
    tol = 4 * U16[w.dtype] * max(1.0, float(np.abs(ref).max()))
    err = float(np.abs(got - ref).max())
    assert err <= tol, f"max abs error {err:.3e} > {tol:.3e}"
    y2 = sha.selective_mlp(x.to(DEV), w1t.to(DEV), w2t.to(DEV), sel, n_sel)
    assert torch.equal(y2, y), "two runs differ"
    say(f"   |S|={len(S)} max abs error {err:.2e} (tol {tol:.2e})")


N_ROUTER = int(os.environ.get("SHA_MIXED_ROUTER", 24))


def _router_case(i):
    rng = np.random.default_rng(9700 + i)
    dtype = ("f32", "f16", "bf16")[int(rng.integers(3))]
    B = int(rng.integers(1, 201))
    H = max(1, int(np.exp(rng.uniform(0.0, np.log(1024.0)))))
    unit = 4 if dtype == "f32" else 8
    d = unit * int(rng.integers(1, 1500 // unit * 8 + 1))
    k = int(rng.integers(0, H + 1))
    bias = bool(rng.integers(2))
    B = min(B, max(1, 2_000_000 // (H * max(k, 1))))   # keeps the per-row set check short
    return dtype, B, d, H, k, bias


@pytest.mark.parametrize("i", range(N_ROUTER))
def test_mixed_router(i):
    from test_router_gpu import _check, _inputs
    dtype, B, d, H, k, bias = _router_case(i)
    say(f"[mixed router {i}] {dtype} B={B} d={d} H={H} k={k} bias={bias}")
    x, w, b = _inputs(B, d, H, dtype, seed=800 + i, bias=bias)
    bd = b.to(DEV) if b is not None else None
    idx, sc = sha.router_topk(x.to(DEV), w.to(DEV), k, bias=bd)
    torch.cuda.synchronize()
    exact = _check(x, w, b, k, idx, sc)
    say(f"   rows with an exact set check: {exact}/{B}")
    if sha.router_workspace_bytes(B, d, H, x.dtype, split=True) > 0:
        # the K-split form forced on the same case
        idx2, sc2 = sha.router_topk(x.to(DEV), w.to(DEV), k, bias=bd, split=True)
        torch.cuda.synchronize()
        _check(x, w, b, k, idx2, sc2)
        say("   K-split form checked too")
