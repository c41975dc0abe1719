"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching a device (CPU only: no compute calls)."""
import ctypes
import os
import re

import pytest

from contextual_head_sparsity_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sha.h")

pytestmark = pytest.mark.skipif(not os.path.exists(bd.LIB_PATH),
                                reason="libsha.so not built (run __graft_entry__.build())")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sha_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported_and_bound():
    names = _declared_functions()
    assert len(names) == 30, names
    L = ctypes.CDLL(bd.LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
    assert set(names) == set(bd.SIGNATURES), "binding and header disagree"
    bd.lib()


def test_status_strings_and_version():
    L = bd.lib()
    for code, name in bd.STATUS.items():
        assert L.sha_status_string(code).decode() == name
    assert re.fullmatch(r"\d+\.\d+\.\d+", L.sha_version().decode())


A16 = 0x10000       # a fake, 16-byte aligned "device" address: never dereferenced
ARGS = dict(B=2, H=4, H_kv=4, Nkv=64, d=64, top_k=2)


def _decode(fn="sha_decode_ex", q=A16, k=A16, v=A16, idx=A16, o=A16, scale=0.125, dtype=0,
            nsplit=1, ws=None, ws_bytes=0, **kw):
    a = dict(ARGS, **kw)
    L = bd.lib()
    base = (q, k, v, idx, a["B"], a["H"], a["H_kv"], a["Nkv"], a["d"], a["top_k"], scale, o, None)
    if fn in ("sha_decode_ex", "sha_decode_gqa_ex"):
        return getattr(L, fn)(*base, dtype, nsplit, ws, ws_bytes)
    if fn in ("sha_decode", "sha_decode_gqa"):
        return getattr(L, fn)(*base, dtype)
    return getattr(L, fn)(*base)


@pytest.mark.parametrize("kw,expect", [
    (dict(Nkv=0), 1), (dict(B=-1), 1), (dict(top_k=-1), 1), (dict(H=4, H_kv=3), 1),
    (dict(top_k=5), 1), (dict(H_kv=0), 1), (dict(d=96), 2), (dict(d=256), 2), (dict(dtype=7), 2),
    (dict(q=None), 1), (dict(o=None), 1), (dict(idx=None), 1), (dict(scale=float("nan")), 1),
    (dict(scale=float("inf")), 1), (dict(k=A16 + 8), 3), (dict(o=A16 + 2), 3), (dict(idx=A16 + 2), 3),
    (dict(nsplit=-1), 1),
])
def test_host_validation_errors(kw, expect):
    assert _decode(**kw) == expect


def test_empty_calls_are_noops():
    # B == 0 or top_k == 0: nothing to read or write, null pointers allowed.
    assert _decode(B=0, q=None, k=None, v=None, idx=None, o=None) == 0
    assert _decode(top_k=0, q=None, k=None, v=None, idx=None, o=None) == 0
    assert _decode(fn="sha_decode_gqa_ex", top_k=0, H=8, H_kv=2, q=None, k=None, v=None,
                   idx=None, o=None) == 0


def test_gqa_validation():
    assert _decode(fn="sha_decode_gqa_ex", H=8, H_kv=2, top_k=3) == 1   # top_k > H_kv
    assert _decode(fn="sha_decode_gqa_ex", H=130, H_kv=2, top_k=1) == 2  # group of 65 heads


def test_typed_entry_points_validate():
    for fn in ("sha_decode_f32", "sha_decode_f16", "sha_decode_bf16", "sha_decode_gqa_f32",
               "sha_decode_gqa_f16", "sha_decode_gqa_bf16", "sha_decode", "sha_decode_gqa"):
        assert _decode(fn=fn, Nkv=0) == 1
        assert _decode(fn=fn, d=80) == 2


def test_workspace_errors():
    # A split call needs a workspace: missing or short -> SHA_ERR_WORKSPACE.
    need = bd.lib().sha_workspace_bytes(2, 4, 4, 64, 64, 2, 0, 0, 4, 256)
    assert need > 0
    assert _decode(nsplit=4) == 4
    assert _decode(nsplit=4, ws=A16, ws_bytes=need - 1) == 4
    assert _decode(nsplit=4, ws=A16 + 4, ws_bytes=need) == 3


def test_planner_and_workspace_accounting():
    L = bd.lib()
    # Head-indexed: about one workgroup per CU.  The OPT-66B layer (1408
    # units) and a 256-unit layer need no split; 64 units split 4 ways; a
    # single short row is capped so that no split is shorter than 512 keys.
    assert L.sha_plan_nsplit(64, 72, 72, 1920, 128, 22, 0, 1, 256) == 1
    assert L.sha_plan_nsplit(16, 32, 32, 1024, 128, 16, 0, 1, 256) == 1
    assert L.sha_plan_nsplit(4, 32, 32, 4096, 128, 16, 0, 1, 256) == 4
    assert L.sha_plan_nsplit(1, 32, 32, 4096, 128, 16, 0, 1, 256) == 8
    # Group (matrix-core) kernel: round model of the grid.  The LLaMA-3.1-70B
    # layer (320 units, more than one workgroup per CU) takes 2-wave
    # workgroups, 4 per CU, and splits 2 ways (640 workgroups, one round);
    # 512 units keep 4-wave workgroups and fill one round unsplit; 128 rows of
    # 1 K keys (640 units) take 2-wave workgroups unsplit; 8 units split down
    # to the 512-key minimum.
    assert L.sha_plan_nsplit(64, 64, 8, 8192, 128, 5, 1, 2, 256) == 2
    assert L.sha_plan_nsplit(64, 64, 8, 8192, 128, 8, 1, 2, 256) == 1
    assert L.sha_plan_nsplit(128, 64, 8, 1024, 128, 5, 1, 2, 256) == 1
    assert L.sha_plan_nsplit(2, 64, 8, 8192, 128, 4, 1, 2, 256) == 16
    # The f32 group kernel (vector ALUs) keeps the one-workgroup-per-CU rule.
    assert L.sha_plan_nsplit(64, 64, 8, 8192, 128, 5, 1, 0, 256) == 1
    # Workspace: per (unit, head, split) d fp32 partial outputs + (m, l).
    ns = 4
    ws = L.sha_workspace_bytes(4, 32, 32, 4096, 128, 16, 0, 1, 0, 256)
    n = 4 * 16 * ns
    assert ws == (n * 128 * 4 + 255) // 256 * 256 + n * 8
    assert L.sha_workspace_bytes(16, 32, 32, 1024, 128, 16, 0, 1, 1, 256) == 0
    # GQA accounting counts every query head of a group.
    n = 64 * 5 * 8 * 3
    assert L.sha_workspace_bytes(64, 64, 8, 8192, 128, 5, 1, 2, 3, 256) == \
        (n * 128 * 4 + 255) // 256 * 256 + n * 8
    # Split count never exceeds Nkv, invalid arguments plan to 0.
    assert L.sha_plan_nsplit(1, 4, 4, 1, 64, 1, 0, 0, 256) == 1
    assert L.sha_plan_nsplit(1, 4, 4, 0, 64, 1, 0, 0, 256) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 2, 1, 64)
    k = torch.zeros(1, 2, 8, 64)
    with pytest.raises(ValueError):
        bd.sha_decode(q, k, k, torch.zeros(1, 1, dtype=torch.int32))


def test_mlp_host_validation():
    L = bd.lib()
    P = A16
    # union: bad sizes, null outputs, workspace
    big = 1 << 20
    assert L.sha_mlp_union(P, 2, 3, 0, P, P, None, P, big) == 1
    assert L.sha_mlp_union(P, -1, 3, 10, P, P, None, P, big) == 1
    assert L.sha_mlp_union(P, 2, 3, 10, None, P, None, P, big) == 1
    assert L.sha_mlp_union(None, 2, 3, 10, P, P, None, P, big) == 1
    assert L.sha_mlp_union(P + 2, 2, 3, 10, P, P, None, P, big) == 3
    assert L.sha_mlp_union_workspace_bytes(1000) == 1024           # one flag byte per neuron
    assert L.sha_mlp_union_workspace_bytes(36864) == 36864
    assert L.sha_mlp_union(P, 2, 3, 1000, P, P, None, P, 1023) == 4
    assert L.sha_mlp_union(P, 2, 3, 1000, P, P, None, None, big) == 4

    def mlp(x=P, w1=P, w2=P, sel=P, n=P, n_max=64, B=4, d=256, D=1000, y=P, dtype=2, ws=P,
            wsb=1 << 30):
        return L.sha_selective_mlp(x, w1, w2, sel, n, n_max, B, d, D, y, None, dtype, ws, wsb)

    assert mlp(d=200) == 2            # d must be a multiple of 256
    assert mlp(D=262144, d=8192, n_max=64) == 2   # a 4 GiB weight matrix
    assert mlp(dtype=0) == 2          # f32 has no matrix-core path here
    assert mlp(n_max=1001) == 1       # n_max > D
    assert mlp(B=-1) == 1
    assert mlp(B=0, x=None, w1=None, w2=None, sel=None, n=None, y=None) == 0   # empty call
    assert mlp(sel=None) == 1
    assert mlp(x=P + 8) == 3
    assert mlp(ws=None) == 4
    # grids past 2^31 - 1 workgroups are refused before any launch: 65535
    # batch tiles x 32769 up-projection neuron tiles of a 256-wide MLP
    assert mlp(B=65535 * 64, d=256, D=32769 * 128, n_max=32769 * 128) == 1
    assert mlp(B=65535 * 64, d=256, D=32768 * 128, n_max=32768 * 128) == 4   # fits: workspace next
    need = L.sha_selective_mlp_workspace_bytes(4, 256, 1000, 64, 256)
    assert need > 0 and mlp(wsb=need - 1) == 4


def test_mlp_workspace_accounting():
    L = bd.lib()
    # OPT-66B MLP, all 36864 neurons selected, 64 rows, 256 CUs: H (64 x 36864
    # 16-bit) and the down projection's fp32 partials over 14 neuron splits
    # (18 column blocks of 512 x 14 ~ one workgroup per CU).  The up
    # projection takes 256 workgroups of 144 neurons with two K groups each
    # (one round at one per CU), so it has no K-split partials.
    ws = L.sha_selective_mlp_workspace_bytes(64, 9216, 36864, 36864, 256)
    assert ws == 64 * 36864 * 2 + 14 * 64 * 9216 * 4
    # 21120 padded neurons (165 workgroups): 3 K splits (3072-element ranges)
    ws = L.sha_selective_mlp_workspace_bytes(8, 9216, 36864, 21033, 256)
    assert ws == 64 * 21120 * 2 + 3 * 64 * 21120 * 4 + 14 * 64 * 9216 * 4
    # a 64-neuron selection (one 128-neuron workgroup) splits the up
    # projection's K 8 ways (1152-element ranges) and keeps a single down split
    ws = L.sha_selective_mlp_workspace_bytes(64, 9216, 36864, 64, 256)
    assert ws == 64 * 128 * 2 + 8 * 64 * 128 * 4
    # 24 rows of the OPT-66B MLP: the whole 64-row tile with two K groups
    # (no up partials), as at 64 rows
    ws = L.sha_selective_mlp_workspace_bytes(24, 9216, 36864, 36864, 256)
    assert ws == 64 * 36864 * 2 + 14 * 64 * 9216 * 4
    # 32 rows of the OPT-6.7B MLP: 128 tiles cannot fill the chip at one
    # workgroup per CU, so two batch blocks with 4 up K splits (and the
    # down projection's 8 column blocks x 32 neuron splits)
    ws = L.sha_selective_mlp_workspace_bytes(32, 4096, 16384, 16384, 256)
    assert ws == 64 * 16384 * 2 + 4 * 64 * 16384 * 4 + 32 * 64 * 4096 * 4


def test_router_host_validation():
    L = bd.lib()
    P = A16

    def r(x=P, w=P, bias=None, B=4, d=256, H=72, k=22, idx=P, sc=P, dtype=1):
        return L.sha_router_topk(x, w, bias, B, d, H, k, idx, sc, None, dtype)

    assert r(k=73) == 1 and r(k=-1) == 1 and r(H=0) == 1 and r(d=0) == 1
    assert r(H=1025) == 2 and r(d=252) == 2 and r(dtype=5) == 2
    assert r(B=0, x=None, w=None, idx=None, sc=None) == 0
    assert r(sc=None) == 1 and r(idx=None) == 1
    assert r(x=P + 8) == 3 and r(idx=P + 2) == 3 and r(bias=P + 2) == 3
    # the scores grid: B * ceil(H / 2) workgroups, at most 2^22
    assert r(B=(1 << 22) // 36 + 1) == 1 and r(B=(1 << 22) // 36, x=None) == 1
    assert r(B=1 << 22, H=1, k=1, x=None) == 1 and r(B=(1 << 22) + 1, H=1, k=1) == 1


def test_router_workspace_accounting_and_validation():
    """The K-split form's workspace: one fp32 partial per (row, 512 hidden
    elements, head), 256-byte rounded; 0 for shapes without the form.  Errors
    are raised on the host before any launch (fake device addresses)."""
    L = bd.lib()
    P = A16
    sb, wsb = L.sha_router_split_bytes, L.sha_router_workspace_bytes
    assert sb(64, 9216, 72, 1) == 64 * 36 * 72 * 4
    assert sb(16, 4096, 32, 2) == 16 * 16 * 32 * 4
    assert sb(3, 264, 5, 1) == (3 * 2 * 5 * 4 + 255) // 256 * 256     # ragged last chunk
    assert sb(4096, 512, 128, 2) == 4096 * 2 * 128 * 4
    for args in [(64, 9216, 72, 0),       # f32: one-pass only
                 (64, 9216, 129, 1),      # more than 128 heads
                 (4097, 512, 8, 1),       # more than 4096 rows
                 (0, 512, 8, 1), (4, 12, 8, 1), (4, 512, 8, 7),
                 (4096, (1 << 30) + 8, 8, 1)]:   # hidden width past 2^30
        assert sb(*args) == 0 and wsb(*args) == 0, args
    # the library's pick: the split form from 2^24 multiply-adds per call
    assert wsb(64, 9216, 72, 1) == sb(64, 9216, 72, 1)          # OPT-66B layer
    assert wsb(128, 4096, 32, 2) == sb(128, 4096, 32, 2)        # exactly 2^24
    assert wsb(127, 4096, 32, 2) == 0 and wsb(16, 4096, 32, 1) == 0 and wsb(64, 8192, 8, 2) == 0

    def r(ws=P, ws_bytes=1 << 20, B=4, d=256, H=72, k=22, dtype=1, x=P):
        return L.sha_router_topk_ex(x, P, None, B, d, H, k, P, P, None, dtype, ws, ws_bytes)

    # the binding's helper: the library's pick, any eligible shape, or none
    f16 = bd.torch.float16
    assert bd.router_workspace_bytes(64, 9216, 72, f16) == wsb(64, 9216, 72, 1) > 0
    assert bd.router_workspace_bytes(16, 4096, 32, f16) == 0
    assert bd.router_workspace_bytes(16, 4096, 32, f16, split=True) == sb(16, 4096, 32, 1) > 0
    assert bd.router_workspace_bytes(64, 9216, 72, f16, split=False) == 0
    assert bd.router_workspace_bytes(64, 9216, 72, bd.torch.float32, split=True) == 0

    need = sb(4, 256, 72, 1)
    assert r(ws_bytes=need - 1) == 4 and r(ws=P + 8) == 3
    assert r(k=73) == 1 and r(x=P + 8) == 3 and r(B=0, x=None, ws=None) == 0
    # shapes without the split form ignore the workspace, even a short one
    assert r(ws_bytes=0, H=200, x=P + 8) == 3 and r(ws_bytes=0, dtype=0, x=P + 4) == 3


def _kv_layout(**kw):
    # contiguous [B, H_kv, Nkv, d] strides of ARGS (d = 64, Nkv = 64, H_kv = 4)
    f = dict(k_batch_stride=4 * 64 * 64, k_head_stride=64 * 64, k_row_stride=64,
             v_batch_stride=4 * 64 * 64, v_head_stride=64 * 64, v_row_stride=64)
    f.update(kw)
    return bd.KvLayout(**f)


def _decode_kv(lay, fn="sha_decode_kv", dtype=1, nsplit=1, **kw):
    a = dict(ARGS, **kw)
    return getattr(bd.lib(), fn)(A16, A16, A16, A16, a["B"], a["H"], a["H_kv"], a["Nkv"], a["d"],
                                 a["top_k"], 0.125, A16, None, dtype, ctypes.byref(lay), nsplit,
                                 None, 0)


@pytest.mark.parametrize("kw,expect", [
    (dict(k_row_stride=4), 3),              # 8 bytes: rows not 16-byte aligned (f16)
    (dict(v_head_stride=64 * 64 + 4), 3),
    (dict(k_batch_stride=-64), 1),
    (dict(seqlens=A16 + 2), 3),
    (dict(block_table=A16, page_size=24, block_table_stride=4, num_pages=8), 1),   # not a power of 2
    (dict(block_table=A16, page_size=8, block_table_stride=8, num_pages=8), 1),    # below 16
    (dict(block_table=A16, page_size=16, block_table_stride=3, num_pages=8), 1),   # 64 keys need 4 pages
    (dict(block_table=A16, page_size=16, block_table_stride=4, num_pages=0), 1),
    (dict(block_table=A16 + 2, page_size=16, block_table_stride=4, num_pages=8), 3),
])
def test_kv_layout_validation(kw, expect):
    assert _decode_kv(_kv_layout(**kw)) == expect
    assert _decode_kv(_kv_layout(**kw), fn="sha_decode_gqa_kv", H=8, H_kv=4) == expect


def test_kv_layout_limits_and_workspace():
    L = bd.lib()
    # f32 rows need 4-element (16-byte) strides; f16 needs 8 (the f32 case
    # is checked through the workspace query, which launches nothing).
    assert L.sha_workspace_bytes_kv(2, 4, 4, 64, 64, 2, 0, 0, 4, 256,
                                    ctypes.byref(_kv_layout(k_row_stride=68))) > 0
    assert L.sha_workspace_bytes_kv(2, 4, 4, 64, 64, 2, 0, 1, 4, 256,
                                    ctypes.byref(_kv_layout(k_row_stride=68))) == 0
    # Paged caches keep each split within 1024 pages: a 64-split cap.
    huge = 64 * 1024 * 16 + 1
    lay = _kv_layout(block_table=A16, page_size=16, block_table_stride=huge, num_pages=8)
    assert _decode_kv(lay, Nkv=huge) == 2
    # Paged split geometry: chunks are whole pages, and a row longer than
    # 1024 pages forces a split even when one is requested.
    lay = _kv_layout(block_table=A16, page_size=16, block_table_stride=2048, num_pages=8)
    ws = L.sha_workspace_bytes_kv(2, 4, 4, 20000, 64, 2, 0, 1, 1, 256, ctypes.byref(lay))
    n = 2 * 2 * 2
    assert ws == (n * 64 * 4 + 255) // 256 * 256 + n * 8
    lay = _kv_layout(block_table=A16, page_size=256, block_table_stride=16, num_pages=8)
    ws = L.sha_workspace_bytes_kv(2, 4, 4, 4096, 64, 2, 0, 1, 5, 256, ctypes.byref(lay))
    n = 2 * 2 * 4            # chunk 820 -> 1024 keys (4 pages): 4 splits
    assert ws == (n * 64 * 4 + 255) // 256 * 256 + n * 8
    # No layout: same accounting as sha_workspace_bytes.
    assert L.sha_workspace_bytes_kv(4, 32, 32, 4096, 128, 16, 0, 1, 0, 256, None) == \
        L.sha_workspace_bytes(4, 32, 32, 4096, 128, 16, 0, 1, 0, 256)
    # Invalid layouts account to 0.
    assert L.sha_workspace_bytes_kv(2, 4, 4, 64, 64, 2, 0, 1, 4, 256,
                                    ctypes.byref(_kv_layout(k_row_stride=3))) == 0


def test_step_host_validation():
    """sha_step_create rejects bad configurations before any device work."""
    L = bd.lib()
    h = ctypes.c_void_p()

    def create(n_layers=1, dense=0, index=A16, **kw):
        cfg = dict(B=2, H=4, H_kv=4, Nkv=64, d=64, top_k=2, gqa=0, scale=0.125, dtype=1,
                   router_d=64, mlp_d=0, mlp_D=0, mlp_k=0)
        cfg.update(kw)
        arr = (bd.StepLayer * max(n_layers, 1))()
        for lay in arr:
            lay.dense, lay.index, lay.router_scores = dense, index, A16
        return L.sha_step_create(ctypes.byref(bd.StepConfig(**cfg)), arr, n_layers, 1,
                                 ctypes.byref(h))

    assert create(n_layers=0) == 1
    assert create(B=0) == 1
    assert create(top_k=0) == 1
    assert create(H=4, H_kv=3) == 1          # invalid attention shape (planner says 0)
    assert create(index=None) == 1           # a sparse layer needs its router output
    assert h.value is None
    assert L.sha_step_create(None, None, 1, 1, ctypes.byref(h)) == 1
    assert L.sha_step_run(None, None) == 1
    assert L.sha_step_destroy(None) == 1


def test_read_probe_library():
    """The benchmark's read-bandwidth probe loads and rejects bad arguments
    before launching anything."""
    path = os.path.join(os.path.dirname(bd.LIB_PATH), "libsha_probe.so")
    assert os.path.exists(path)
    P = ctypes.CDLL(path)
    P.sha_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p]
    EINVAL = -1
    assert P.sha_probe_read(None, 1 << 20, 4, A16, None) == EINVAL
    assert P.sha_probe_read(A16, 1 << 20, 4, None, None) == EINVAL
    assert P.sha_probe_read(A16, 1 << 20, 0, A16, None) == EINVAL
    assert P.sha_probe_read(A16, (1 << 20) + 16, 4, A16, None) == EINVAL   # not whole 32 KiB steps
    assert P.sha_probe_read(A16 + 8, 1 << 20, 4, A16, None) == EINVAL      # misaligned


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No fallback: without libsha.so every entry point raises."""
    monkeypatch.setattr(bd, "LIB_PATH", str(tmp_path / "libsha.so"))
    monkeypatch.setattr(bd, "_lib", None)
    with pytest.raises(ImportError):
        bd.lib()
    with pytest.raises(ImportError):
        bd.plan_nsplit(1, 4, 4, 64, 64, 1)
    with pytest.raises(ImportError):
        bd.workspace_bytes(1, 4, 4, 64, 64, 1)
    with pytest.raises(ImportError):
        bd.selective_mlp_workspace_bytes(1, 256, 512, 64)


@pytest.mark.parametrize("header", ["sha.h", "sha_probe.h"])
def test_headers_compile_as_c(header, tmp_path):
    """The boundary is a C ABI: each public header compiles as C11, and no
    diagnostic (with -Wall -Wextra -pedantic) points into it."""
    import shutil
    import subprocess
    cc = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(cc):
        cc = shutil.which("clang")
    if cc is None:
        pytest.skip("no clang to compile C with")
    src = tmp_path / "use.c"
    src.write_text(f'#include "{header}"\nint main(void) {{ return 0; }}\n')
    r = subprocess.run([cc, "-x", "c", "-std=c11", "-Wall", "-Wextra", "-pedantic",
                        "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                        "-D__HIP_PLATFORM_AMD__", "-fsyntax-only", str(src)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    ours = [ln for ln in r.stderr.splitlines()
            if os.path.join("include", header) in ln and ("warning" in ln or "error" in ln)]
    assert not ours, ours
