"""sha_decode_noalloc (the decode entry point that allocates nothing) through
the C ABI, against the explicit-workspace entry points on the same inputs:
two calls in a row, the second smaller, both with KV splits (so both use the
library's fixed scratch array), bit for bit against sha_decode_gqa_ex /
sha_decode_ex at the same split count and within tolerance of the fp64
oracle; unselected slots keep their sentinel bits.  A call whose partials do
not fit the array returns SHA_ERR_WORKSPACE and leaves the output untouched."""
import ctypes

import numpy as np
import pytest
import torch

from contextual_head_sparsity_amd import _binding as bd
from contextual_head_sparsity_amd import workloads as wl

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import DEV, TOL, check_full, say

SCRATCH_BYTES = 8 << 20          # SHA_NOALLOC_SCRATCH_BYTES
SHA_ERR_WORKSPACE = 4
DT = {"f32": 0, "f16": 1, "bf16": 2}


def _ptrs(*ts):
    return [t.data_ptr() for t in ts]


def _run_pair(w, nsplit):
    """(no-alloc output, explicit-workspace output) for one workload."""
    L = bd.lib()
    q, k, v, idx, o = wl.make_workload(w, "cpu")
    qd, kd, vd, idd = q.to(DEV), k.to(DEV), v.to(DEV), idx.to(DEV)
    o1, o2 = o.to(DEV), o.to(DEV)
    stream = torch.cuda.current_stream().cuda_stream
    ns = L.sha_plan_nsplit(w.B, w.H, w.H_kv, w.Nkv, w.d, w.top_k, int(w.gqa), DT[w.dtype], 0) \
        if nsplit == 0 else nsplit
    need = L.sha_workspace_bytes(w.B, w.H, w.H_kv, w.Nkv, w.d, w.top_k, int(w.gqa),
                                 DT[w.dtype], ns, 0)
    assert 0 < need <= SCRATCH_BYTES, need        # split: the scratch array is used
    st = L.sha_decode_noalloc(*_ptrs(qd, kd, vd, idd), w.B, w.H, w.H_kv, w.Nkv, w.d, w.top_k,
                              w.scale, o1.data_ptr(), stream, DT[w.dtype], int(w.gqa), nsplit)
    assert st == 0, bd.STATUS.get(st, st)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    fn = L.sha_decode_gqa_ex if w.gqa else L.sha_decode_ex
    st = fn(*_ptrs(qd, kd, vd, idd), w.B, w.H, w.H_kv, w.Nkv, w.d, w.top_k, w.scale,
            o2.data_ptr(), stream, DT[w.dtype], ns, ws.data_ptr(), need)
    assert st == 0, bd.STATUS.get(st, st)
    torch.cuda.synchronize()
    return (q, k, v, idx, o), o1, o2


def test_noalloc_matches_explicit_workspace_twice():
    cases = [
        # a LLaMA-3.1-70B-shaped group layer at 3 forced splits
        (wl.WORKLOADS["llama3.1_70b_gqa_bf16"].with_(B=8, Nkv=4096), 3),
        # then a smaller head-indexed call at its planned split
        (wl.WORKLOADS["opt66b_f16"].with_(B=2, Nkv=3000, top_k=5), 0),
    ]
    for w, nsplit in cases:
        say(f"[noalloc] {w.name} B={w.B} Nkv={w.Nkv} gqa={w.gqa} nsplit={nsplit}")
        (q, k, v, idx, o), o1, o2 = _run_pair(w, nsplit)
        assert torch.equal(wl.raw_bits(o1), wl.raw_bits(o2)), "differs from the workspace form"
        check_full(w.gqa, q, k, v, idx, w.scale, o, o1.cpu(), TOL[w.dtype])


def test_noalloc_rejects_partials_beyond_the_array():
    """8 rows x 8 groups x 8 heads x 64 splits of 130 floats need 17 MB of
    partials.  The buffers are real and of the stated shape, so even a call
    that got past the check would stay in bounds."""
    say("[noalloc] size limit")
    L = bd.lib()
    B, H, H_kv, Nkv, d, top_k = 8, 64, 8, 8192, 128, 8
    need = L.sha_workspace_bytes(B, H, H_kv, Nkv, d, top_k, 1, DT["bf16"], 64, 0)
    assert need > SCRATCH_BYTES
    q = torch.zeros(B, H, 1, d, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(B, H_kv, Nkv, d, dtype=torch.bfloat16, device=DEV)
    idx = torch.arange(H_kv, dtype=torch.int32, device=DEV).repeat(B, 1)
    o = torch.full((B, H, 1, d), 7.0, dtype=torch.bfloat16, device=DEV)
    st = L.sha_decode_noalloc(*_ptrs(q, k, k, idx), B, H, H_kv, Nkv, d, top_k, 0.1,
                              o.data_ptr(), torch.cuda.current_stream().cuda_stream,
                              DT["bf16"], 1, 64)
    assert st == SHA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
