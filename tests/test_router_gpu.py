"""Attention router on the GPU against the fp64 oracle, and router -> SHA
decode end to end (through the C ABI).

Scores: fp32 accumulation of exact 16-bit products; the bound is
|s_gpu - s| <= 1e-4 * (1 + sum_k |x_k w_k|).  The top-k is a discrete
decision taken on fp32 scores, so it is compared for what is unique: every
picked head scores (in fp64) at least as high as every unpicked one up to the
score tolerance, and where the fp64 gap at the boundary exceeds that
tolerance the picked set equals the oracle's exactly.
"""
import numpy as np
import pytest
import torch

import contextual_head_sparsity_amd as sha
from contextual_head_sparsity_amd import workloads as wl
from oracle import router_scores_ref, sha_decode_gqa_ref, sha_decode_ref, to_f64, topk_ref

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def say(m):
    print(m, flush=True)


def _inputs(B, d, H, dtype, seed, bias=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, d, generator=g).to(DT[dtype])
    w = (torch.randn(H, d, generator=g) / d ** 0.5).to(DT[dtype])
    b = torch.randn(H, generator=g) * 0.1 if bias else None
    return x, w, b


def _check(x, w, b, k, idx_gpu, sc_gpu):
    ref = router_scores_ref(x, w, b)
    mag = np.abs(to_f64(x)) @ np.abs(to_f64(w)).T + 1.0
    tol = 1e-4 * mag
    sc = sc_gpu.cpu().double().numpy()
    assert np.all(np.abs(sc - ref) <= tol), float(np.max(np.abs(sc - ref) / tol))
    got = idx_gpu.cpu().numpy()
    want = topk_ref(ref, k)
    B, H = ref.shape
    exact = 0
    for r in range(B):
        picked = list(got[r])
        assert picked == sorted(set(picked)) and len(picked) == k
        assert all(0 <= h < H for h in picked)
        rest = [h for h in range(H) if h not in picked]
        if picked and rest:
            assert min(ref[r, picked]) >= max(ref[r, rest]) - 2 * tol[r].max()
            order = np.sort(ref[r])[::-1]
            if k < H and order[k - 1] - order[k] > 2 * tol[r].max():
                assert picked == list(want[r])
                exact += 1
        else:
            assert picked == list(want[r])
            exact += 1
    return exact


# The shapes take both heads-per-workgroup choices of the scores kernel (4,
# and 2 when B * ceil(H / 4) is below the CU count), head counts that leave a
# partial head group, hidden sizes whose last 64-piece block is ragged, and
# more blocks than the workgroup has waves.
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("B,d,H,k", [(1, 64, 8, 3), (64, 9216, 72, 22), (16, 4096, 32, 16),
                                     (5, 8192, 8, 5), (3, 512, 1000, 300), (7, 256, 64, 64),
                                     (2, 128, 40, 0), (4, 256, 200, 50), (3, 320, 300, 100),
                                     (2, 8, 1024, 1000), (50, 1000, 37, 9), (9, 2056, 13, 4),
                                     (3, 33000, 5, 2)])
def test_router_matches_oracle(dtype, B, d, H, k):
    say(f"[router] {dtype} B={B} d={d} H={H} k={k}")
    x, w, b = _inputs(B, d, H, dtype, seed=B * 7 + H)
    idx, sc = sha.router_topk(x.to(DEV), w.to(DEV), k, bias=b.to(DEV))
    torch.cuda.synchronize()
    exact = _check(x, w, b, k, idx, sc)
    say(f"   rows with an exact set check: {exact}/{B}")


def test_router_ties_and_nan():
    """Equal scores pick the lowest heads; NaN scores rank last."""
    x = torch.ones(2, 64, dtype=torch.float16)
    w = torch.zeros(10, 64, dtype=torch.float16)
    w[7] = 1.0                                   # head 7 scores 64, the rest 0
    b = torch.zeros(10)
    b[3] = float("nan")
    idx, sc = sha.router_topk(x.to(DEV), w.to(DEV), 4, bias=b.to(DEV))
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == [[0, 1, 2, 7], [0, 1, 2, 7]]
    assert torch.isnan(sc[:, 3]).all()


def test_router_feeds_sha_decode():
    """x -> router -> batch_head_index -> SHA decode, all on the device,
    against the oracle pipeline (OPT-66B head count, reduced batch)."""
    say("[router] pipeline into sha_decode")
    w_ = wl.WORKLOADS["opt66b_f16"].with_(B=4, Nkv=777)
    q, k, v, _, o = wl.make_workload(w_, "cpu")
    x, wr, br = _inputs(w_.B, 1024, w_.H, "f16", seed=5)
    idx, sc = sha.router_topk(x.to(DEV), wr.to(DEV), w_.top_k, bias=br.to(DEV))
    od = o.to(DEV)
    sha.sha_decode(q.to(DEV), k.to(DEV), v.to(DEV), idx, scale=w_.scale, out=od)
    torch.cuda.synchronize()
    _check(x, wr, br, w_.top_k, idx, sc)
    ref, written = sha_decode_ref(q, k, v, idx.cpu(), w_.scale)
    g = od.cpu().double().numpy()
    assert float(np.abs(g[written] - ref[written]).max()) <= 2e-3
    assert torch.equal(wl.raw_bits(od.cpu())[torch.from_numpy(~written)],
                       wl.raw_bits(o)[torch.from_numpy(~written)])


def test_group_router_feeds_gqa_decode():
    say("[router] group pipeline into sha_decode_gqa")
    w_ = wl.WORKLOADS["llama3.1_70b_gqa_bf16"].with_(B=3, Nkv=600)
    q, k, v, _, o = wl.make_workload(w_, "cpu")
    x, wr, br = _inputs(w_.B, 2048, w_.H_kv, "bf16", seed=6)
    gidx, _ = sha.router_topk(x.to(DEV), wr.to(DEV), w_.top_k, bias=br.to(DEV))
    od = o.to(DEV)
    sha.sha_decode_gqa(q.to(DEV), k.to(DEV), v.to(DEV), gidx, scale=w_.scale, out=od)
    torch.cuda.synchronize()
    ref, written = sha_decode_gqa_ref(q, k, v, gidx.cpu(), w_.scale)
    g = od.cpu().double().numpy()
    assert float(np.abs(g[written] - ref[written]).max()) <= 1e-2
