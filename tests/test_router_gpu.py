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
ROUTER_CHUNK = 256   # hidden elements per K-split partial


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


@pytest.mark.parametrize("split", [False, True])
def test_router_ties_and_nan(split):
    """Equal scores pick the lowest heads; NaN scores rank last (one-pass and
    K-split forms)."""
    x = torch.ones(2, 64, dtype=torch.float16)
    w = torch.zeros(10, 64, dtype=torch.float16)
    w[7] = 1.0                                   # head 7 scores 64, the rest 0
    b = torch.zeros(10)
    b[3] = float("nan")
    idx, sc = sha.router_topk(x.to(DEV), w.to(DEV), 4, bias=b.to(DEV), split=split)
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


def test_router_consecutive_calls_and_streams():
    """Consecutive calls of growing and shrinking batches and widths, on the
    current stream and on a side stream, all match the oracle."""
    side = torch.cuda.Stream(device=DEV)
    for i, (B, d, H, k, st) in enumerate([(3, 256, 72, 22, None), (5000, 128, 72, 22, None),
                                          (64, 9216, 72, 22, None), (7, 512, 40, 8, side),
                                          (4100, 64, 13, 4, side), (3, 12288, 9, 4, side),
                                          (2, 64, 8, 3, None)]):
        say(f"[router] counters call {i}: B={B} d={d} H={H} k={k} side={st is not None}")
        x, w, b = _inputs(B, d, H, "bf16", seed=100 + i)
        xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
        if st is not None:
            st.wait_stream(torch.cuda.current_stream())
        idx, sc = sha.router_topk(xd, wd, k, bias=bd, stream=st)
        torch.cuda.synchronize()
        _check(x, w, b, k, idx, sc)


@pytest.mark.parametrize("split", [None, True])
@pytest.mark.parametrize("warm", [False, True])
def test_router_graph_replays(warm, split):
    """A router call captured in a graph, on a fresh or an already used
    stream: each replay (with eager router calls on the same stream in
    between) matches the eager result bit for bit and the oracle; the
    K-split form's temporary workspace is captured with the call."""
    say(f"[router] graph replays warm={warm} split={split}")
    B, d, H, k = 48, 2048, 72, 22
    x, w, b = _inputs(B, d, H, "f16", seed=7)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    sc = torch.empty((B, H), dtype=torch.float32, device=DEV)
    if warm:
        sha.router_topk(xd, wd, k, bias=bd, index=idx, scores=sc, stream=s, split=split)
        s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        sha.router_topk(xd, wd, k, bias=bd, index=idx, scores=sc, stream=s, split=split)
    torch.cuda.synchronize()
    x2, w2, b2 = _inputs(B, d, H, "f16", seed=8)
    eager_idx, eager_sc = None, None
    for rep in range(3):
        idx.fill_(-1)
        sc.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check(x, w, b, k, idx, sc)
        if eager_idx is None:
            eager_idx, eager_sc = sha.router_topk(xd, wd, k, bias=bd, stream=s, split=split)
            s.synchronize()
        assert torch.equal(idx, eager_idx) and torch.equal(sc, eager_sc)
        # other work on the captured stream between replays
        i2, s2 = sha.router_topk(x2.to(DEV), w2.to(DEV), k, bias=b2.to(DEV), stream=s,
                                 split=split)
        s.synchronize()
        _check(x2, w2, b2, k, i2, s2)


# The K-split form (16-bit, H <= 128, B <= 4096): row blocks of 16 with a
# ragged last block, head blocks of 16 with a partial last block (1 ... 8
# blocks), hidden widths whose last 256-element chunk is partial (down to one
# 8-element piece), one chunk only, top_k = 0 (scores only), and the largest
# shape it takes (4096 rows x 128 heads).
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("B,d,H,k", [(64, 9216, 72, 22), (16, 4096, 32, 16), (128, 4096, 32, 16),
                                     (64, 8192, 8, 5), (17, 520, 128, 40), (1, 8, 1, 1),
                                     (33, 1032, 65, 64), (5, 512, 17, 0), (300, 2056, 100, 7),
                                     (4096, 64, 8, 2), (4096, 264, 128, 64)])
def test_router_split_form_matches_oracle(dtype, B, d, H, k):
    say(f"[router split] {dtype} B={B} d={d} H={H} k={k}")
    dt = DT[dtype]
    need = sha.router_workspace_bytes(B, d, H, dt, split=True)
    assert need == (B * -(-d // ROUTER_CHUNK) * H * 4 + 255) // 256 * 256
    x, w, b = _inputs(B, d, H, dtype, seed=B * 11 + H + d)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)   # contents do not matter
    idx, sc = sha.router_topk(xd, wd, k, bias=bd, workspace=ws, split=True)
    torch.cuda.synchronize()
    _check(x, w, b, k, idx, sc)
    # the same inputs again: the same bits (fixed summation order)
    idx2, sc2 = sha.router_topk(xd, wd, k, bias=bd, split=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(sc, sc2)
    # the one-pass kernels agree with the oracle too
    idx1, sc1 = sha.router_topk(xd, wd, k, bias=bd, split=False)
    torch.cuda.synchronize()
    _check(x, w, b, k, idx1, sc1)


def test_router_split_raw_entry_points():
    """sha_router_topk_ex through the C ABI: an explicit workspace gives the
    binding's result; a short one is refused before any launch and leaves the
    outputs untouched; no workspace runs the one-pass kernels."""
    say("[router split] raw C ABI")
    L = sha.lib()
    B, d, H, k = 24, 3072, 72, 22
    x, w, b = _inputs(B, d, H, "f16", seed=77)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    need = L.sha_router_split_bytes(B, d, H, 1)
    assert need == B * 12 * H * 4
    assert L.sha_router_workspace_bytes(B, d, H, 1) == 0     # below 2^24 multiply-adds
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    idx = torch.full((B, k), -7, dtype=torch.int32, device=DEV)
    sc = torch.full((B, H), 3.0, dtype=torch.float32, device=DEV)
    s = torch.cuda.current_stream(DEV).cuda_stream
    st = L.sha_router_topk_ex(xd.data_ptr(), wd.data_ptr(), bd.data_ptr(), B, d, H, k,
                              idx.data_ptr(), sc.data_ptr(), s, 1, ws.data_ptr(), need - 4)
    torch.cuda.synchronize()
    assert st == 4 and (idx == -7).all() and (sc == 3.0).all()
    st = L.sha_router_topk_ex(xd.data_ptr(), wd.data_ptr(), bd.data_ptr(), B, d, H, k,
                              idx.data_ptr(), sc.data_ptr(), s, 1, ws.data_ptr(), need)
    torch.cuda.synchronize()
    assert st == 0
    _check(x, w, b, k, idx, sc)
    bidx, bsc = sha.router_topk(xd, wd, k, bias=bd, split=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, bidx) and torch.equal(sc, bsc)
    st = L.sha_router_topk(xd.data_ptr(), wd.data_ptr(), bd.data_ptr(), B, d, H, k,
                           idx.data_ptr(), sc.data_ptr(), s, 1)
    torch.cuda.synchronize()
    assert st == 0
    _check(x, w, b, k, idx, sc)
