"""Streams and graph capture through the C ABI and the binding (GPU).

* A call on a stream other than the current one, while the current stream
  is still busy: the binding makes its temporaries (the int32 index copy,
  the zero-filled output, the workspace) on the call's stream, so the result
  matches the fp64 oracle.
* Host tensors passed where the library expects device memory (outputs,
  index and count buffers, workspaces) are refused by the binding.
* The internal-workspace entry points on a stream under capture: a call
  that would have to grow the workspace returns SHA_ERR_WORKSPACE and
  enqueues nothing; once the workspace exists, the call is captured and
  every replay matches the eager result bit for bit.
"""
import numpy as np
import pytest
import torch

import contextual_head_sparsity_amd as sha
from contextual_head_sparsity_amd import _binding as bd
from contextual_head_sparsity_amd import workloads as wl
from oracle import mlp_union_ref, router_scores_ref, selective_mlp_ref, sha_decode_ref, topk_ref

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import DEV, TOL, check_full, say

SHA_ERR_WORKSPACE = 4


def _busy(n=6):
    """Queue a few milliseconds of work on the current stream."""
    a = torch.randn(4096, 4096, device=DEV)
    for _ in range(n):
        a = a @ a
        a = a / a.abs().amax()
    return a


def _case(B=4, Nkv=3000, seed=3):
    w = wl.WORKLOADS["opt66b_f16"].with_(B=B, Nkv=Nkv, seed=seed)
    return (w, *wl.make_workload(w, "cpu"))


def test_decode_on_a_side_stream_while_current_is_busy():
    say("[streams] decode on a side stream")
    w, q, k, v, idx, o = _case()
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    idx64 = idx.to(torch.int64).to(DEV)            # converted by the binding, on the side stream
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    junk = _busy()
    out = sha.sha_decode(qd, kd, vd, idx64, scale=w.scale, nsplit=3, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    # out=None: zero-filled on the side stream, only the selected slots written
    ref, written = sha_decode_ref(q, k, v, idx, w.scale)
    got = out.cpu().double().numpy()
    err = float(np.max(np.abs(got[written] - ref[written])))
    assert err <= TOL["f16"], err
    assert np.all(got[~written] == 0.0)


def test_mlp_and_router_on_a_side_stream():
    say("[streams] selective MLP and router on a side stream")
    mw = wl.MlpWorkload("side", B=5, d=256, D=700, k_row=40, dtype="bf16", seed=9)
    x, w1t, w2t, rows = wl.make_mlp(mw, DEV)
    rows64 = rows.to(torch.int64)
    rw = torch.randn(24, 256, device=DEV).to(torch.bfloat16)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    junk = _busy()
    sel, n_sel = sha.mlp_union(rows64, mw.D, stream=side)
    y = sha.selective_mlp(x, w1t, w2t, sel, n_sel, stream=side)
    index, scores = sha.router_topk(x, rw, 5, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    S = mlp_union_ref(rows.cpu(), mw.D)
    n = int(n_sel.item())
    assert n == len(S) and np.array_equal(sel[:n].cpu().numpy(), S)
    ref = selective_mlp_ref(x.cpu(), w1t.cpu(), w2t.cpu(), S)
    u = 2.0 ** -8                                  # bf16 unit roundoff
    assert np.all(np.abs(y.cpu().double().numpy() - ref) <= 4 * u * np.maximum(1.0, np.abs(ref)))
    sref = router_scores_ref(x.cpu(), rw.cpu(), None)
    tol = 1e-4 * (1.0 + np.abs(x.cpu().double().numpy()) @ np.abs(rw.cpu().double().numpy()).T)
    assert np.all(np.abs(scores.cpu().double().numpy() - sref) <= tol)
    # the selection is exactly the top 5 of the scores the kernel computed
    assert np.array_equal(index.cpu().numpy(), topk_ref(scores.cpu(), 5))


def test_selective_mlp_rejects_n_max_beyond_selection():
    mw = wl.MlpWorkload("nmax", B=2, d=256, D=300, k_row=4, dtype="f16", seed=1)
    x, w1t, w2t, rows = wl.make_mlp(mw, DEV)
    sel = torch.zeros(8, dtype=torch.int32, device=DEV)
    n_sel = torch.full((1,), 8, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="n_max"):
        sha.selective_mlp(x, w1t, w2t, sel, n_sel, n_max=9)


def test_binding_rejects_host_buffers():
    """Every output, index and workspace argument the binding passes to the
    library as a device address must be a tensor on the call's device: a
    host tensor is refused with ValueError before the library enqueues
    anything, and the device outputs stay as they were."""
    say("[binding] host buffers refused")
    host = torch.empty(1 << 20, dtype=torch.uint8)
    w, q, k, v, idx, o = _case(B=2, Nkv=3000)
    qd, kd, vd, idd = q.to(DEV), k.to(DEV), v.to(DEV), idx.to(DEV)
    assert sha.workspace_bytes(2, w.H, w.H_kv, 3000, w.d, w.top_k, dtype=qd.dtype, nsplit=4) > 0
    od = torch.full_like(qd, 5.0)
    with pytest.raises(ValueError, match="out"):
        sha.sha_decode(qd, kd, vd, idd, out=o)
    with pytest.raises(ValueError, match="workspace"):
        sha.sha_decode(qd, kd, vd, idd, out=od, nsplit=4, workspace=host)
    with pytest.raises(ValueError, match="device"):
        sha.sha_decode(qd, k, vd, idd, out=od)
    with pytest.raises(ValueError, match="seqlens"):
        sha.sha_decode(qd, kd, vd, idd, out=od,
                       seqlens=torch.full((2,), 64, dtype=torch.int32))
    torch.cuda.synchronize()
    assert (od == 5.0).all()
    # router: index, scores, bias, workspace
    x = torch.randn(64, 9216, device=DEV).half()
    rw = torch.randn(72, 9216, device=DEV).half()
    idx_d = torch.full((64, 22), -5, dtype=torch.int32, device=DEV)
    sc_d = torch.full((64, 72), 7.0, device=DEV)
    for kw, what in [(dict(index=torch.empty(64, 22, dtype=torch.int32)), "index"),
                     (dict(scores=torch.empty(64, 72)), "scores"),
                     (dict(bias=torch.zeros(72)), "bias"),
                     (dict(workspace=host, index=idx_d, scores=sc_d), "workspace")]:
        with pytest.raises(ValueError, match=what):
            sha.router_topk(x, rw, 22, **kw)
    torch.cuda.synchronize()
    assert (idx_d == -5).all() and (sc_d == 7.0).all()
    # union and selective MLP: sel, n_sel, out, workspace
    mw = wl.MlpWorkload("host", B=2, d=256, D=300, k_row=4, dtype="f16", seed=1)
    xm, w1t, w2t, rows = wl.make_mlp(mw, DEV)
    sel, n_sel = sha.mlp_union(rows, mw.D)
    for kw, what in [(dict(sel=torch.empty(8, dtype=torch.int32)), "sel"),
                     (dict(n_sel=torch.empty(1, dtype=torch.int32)), "n_sel"),
                     (dict(workspace=host), "workspace")]:
        with pytest.raises(ValueError, match=what):
            sha.mlp_union(rows, mw.D, **kw)
    y = torch.full_like(xm, 3.0)
    for args, kw, what in [((sel.cpu(), n_sel), {}, "sel"), ((sel, n_sel.cpu()), {}, "n_sel"),
                           ((sel, n_sel), dict(out=torch.empty(2, 256, dtype=torch.half)), "out"),
                           ((sel, n_sel), dict(out=y, workspace=host), "workspace")]:
        with pytest.raises(ValueError, match=what):
            sha.selective_mlp(xm, w1t, w2t, *args, **kw)
    torch.cuda.synchronize()
    assert (y == 3.0).all()


def test_internal_workspace_under_capture():
    say("[streams] internal workspace under graph capture")
    L = bd.lib()
    w, q, k, v, idx, o = _case(B=2, Nkv=6000, seed=5)
    qd, kd, vd, idd = q.to(DEV), k.to(DEV), v.to(DEV), idx.to(DEV)
    ns = bd.plan_nsplit(w.B, w.H, w.H_kv, w.Nkv, w.d, w.top_k, False, q.dtype)
    assert ns > 1                                  # the call needs a workspace
    sentinel = o.to(DEV)
    s = torch.cuda.Stream()                        # no workspace on this stream yet

    def call(out, stream):
        return L.sha_decode_f16(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), idd.data_ptr(),
                                w.B, w.H, w.H_kv, w.Nkv, w.d, w.top_k, w.scale, out.data_ptr(),
                                stream.cuda_stream)

    # Cold: the workspace would have to be allocated while capturing.
    oc = sentinel.clone()
    torch.cuda.synchronize()
    g0 = torch.cuda.CUDAGraph()
    with _nowarn():                                # torch warns that the graph is empty
        with torch.cuda.graph(g0, stream=s):
            st = call(oc, s)
    assert st == SHA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(wl.raw_bits(oc), wl.raw_bits(sentinel))   # nothing ran
    # Warm: one eager call on the stream grows its workspace; capture then works.
    oe = sentinel.clone()
    with torch.cuda.stream(s):
        assert call(oe, s) == 0
    s.synchronize()
    check_full(False, q, k, v, idx, w.scale, o, oe.cpu(), TOL["f16"])
    og = sentinel.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        assert call(og, s) == 0
    for rep in range(3):
        og.copy_(sentinel)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(wl.raw_bits(og), wl.raw_bits(oe)), f"replay {rep}"
        junk = torch.randn(1 << 20, device=DEV).cumsum(0)   # unrelated work between replays
        del junk


class _nowarn:
    def __enter__(self):
        import warnings
        self._c = warnings.catch_warnings()
        self._c.__enter__()
        warnings.simplefilter("ignore")

    def __exit__(self, *exc):
        return self._c.__exit__(*exc)
