"""ctypes binding over libsha.so (include/sha.h): argument marshalling only.

Tensors are PyTorch device tensors (PyTorch supplies device memory and the
stream); every arithmetic step runs in the library's HIP kernels.  There is
no fallback: if libsha.so is missing or fails to load, calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsha.so")

SHA_F32, SHA_F16, SHA_BF16 = 0, 1, 2
_DT = {torch.float32: SHA_F32, torch.float16: SHA_F16, torch.bfloat16: SHA_BF16}
STATUS = {0: "SHA_OK", 1: "SHA_ERR_INVALID_ARG", 2: "SHA_ERR_UNSUPPORTED",
          3: "SHA_ERR_MISALIGNED", 4: "SHA_ERR_WORKSPACE", 5: "SHA_ERR_HIP"}



class KvLayout(ctypes.Structure):
    """sha_kv_layout: element strides, per-row lengths and the page table."""
    _fields_ = [("k_batch_stride", ctypes.c_int64), ("k_head_stride", ctypes.c_int64),
                ("k_row_stride", ctypes.c_int64), ("v_batch_stride", ctypes.c_int64),
                ("v_head_stride", ctypes.c_int64), ("v_row_stride", ctypes.c_int64),
                ("seqlens", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("block_table_stride", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


class StepConfig(ctypes.Structure):
    """sha_step_config."""
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("H_kv", ctypes.c_int),
                ("Nkv", ctypes.c_int), ("d", ctypes.c_int), ("top_k", ctypes.c_int),
                ("gqa", ctypes.c_int), ("scale", ctypes.c_float), ("dtype", ctypes.c_int),
                ("router_d", ctypes.c_int), ("mlp_d", ctypes.c_int), ("mlp_D", ctypes.c_int),
                ("mlp_k", ctypes.c_int)]


class StepLayer(ctypes.Structure):
    """sha_step_layer."""
    _fields_ = [("router_x", ctypes.c_void_p), ("router_w", ctypes.c_void_p),
                ("router_bias", ctypes.c_void_p), ("router_scores", ctypes.c_void_p),
                ("index", ctypes.c_void_p), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("kv", ctypes.POINTER(KvLayout)), ("dense", ctypes.c_int),
                ("mlp_x", ctypes.c_void_p), ("mlp_w1t", ctypes.c_void_p),
                ("mlp_w2t", ctypes.c_void_p), ("mlp_y", ctypes.c_void_p),
                ("mlp_rows", ctypes.c_void_p)]


# (name, restype, argtypes) for every symbol include/sha.h declares.
_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_L = ctypes.POINTER(KvLayout)
_DECODE_ARGS = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P]
SIGNATURES = {
    "sha_decode_f32": (_I, _DECODE_ARGS),
    "sha_decode_f16": (_I, _DECODE_ARGS),
    "sha_decode_bf16": (_I, _DECODE_ARGS),
    "sha_decode": (_I, _DECODE_ARGS + [_I]),
    "sha_decode_gqa_f32": (_I, _DECODE_ARGS),
    "sha_decode_gqa_f16": (_I, _DECODE_ARGS),
    "sha_decode_gqa_bf16": (_I, _DECODE_ARGS),
    "sha_decode_gqa": (_I, _DECODE_ARGS + [_I]),
    "sha_decode_ex": (_I, _DECODE_ARGS + [_I, _I, _P, _S]),
    "sha_decode_gqa_ex": (_I, _DECODE_ARGS + [_I, _I, _P, _S]),
    "sha_decode_noalloc": (_I, _DECODE_ARGS + [_I, _I, _I]),
    "sha_decode_kv": (_I, _DECODE_ARGS + [_I, _L, _I, _P, _S]),
    "sha_decode_gqa_kv": (_I, _DECODE_ARGS + [_I, _L, _I, _P, _S]),
    "sha_workspace_bytes_kv": (_S, [_I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _L]),
    "sha_plan_nsplit": (_I, [_I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "sha_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "sha_mlp_union_workspace_bytes": (_S, [_I]),
    "sha_mlp_union": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _S]),
    "sha_selective_mlp_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "sha_selective_mlp": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _P, _S]),
    "sha_router_topk": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _I]),
    "sha_router_split_bytes": (_S, [_I, _I, _I, _I]),
    "sha_router_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "sha_router_topk_ex": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _I, _P, _S]),
    "sha_step_create": (_I, [ctypes.POINTER(StepConfig), ctypes.POINTER(StepLayer), _I, _I,
                             ctypes.POINTER(ctypes.c_void_p)]),
    "sha_step_run": (_I, [_P, _P]),
    "sha_step_destroy": (_I, [_P]),
    "sha_status_string": (ctypes.c_char_p, [_I]),
    "sha_last_hip_error": (_I, []),
    "sha_version": (ctypes.c_char_p, []),
}


class ShaError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        msg = f"{where}: {STATUS.get(status, status)}"
        if status == 5:
            msg += f" (hipError_t {hip_error})"
        super().__init__(msg)
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libsha.so (built in-tree by contextual_head_sparsity_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m contextual_head_sparsity_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(st: int, where: str):
    if st != 0:
        raise ShaError(st, where, lib().sha_last_hip_error())


def plan_nsplit(B, H, H_kv, Nkv, d, top_k, gqa=False, dtype=torch.float16, num_cus=0) -> int:
    return lib().sha_plan_nsplit(B, H, H_kv, Nkv, d, top_k, int(gqa), _DT[dtype], num_cus)


def workspace_bytes(B, H, H_kv, Nkv, d, top_k, gqa=False, dtype=torch.float16, nsplit=0,
                    num_cus=0) -> int:
    return lib().sha_workspace_bytes(B, H, H_kv, Nkv, d, top_k, int(gqa), _DT[dtype], nsplit,
                                     num_cus)


def workspace_bytes_paged(B, H, H_kv, Nkv, d, top_k, gqa=False, dtype=torch.float16, nsplit=0,
                          page_size=16, num_cus=0) -> int:
    """Workspace of a paged call (its split geometry follows the page size).
    Host-only query: the block-table address below is never dereferenced."""
    n_pages = (Nkv + page_size - 1) // page_size
    lay = KvLayout(0, 0, 8, 0, 0, 8)
    lay.block_table, lay.block_table_stride, lay.page_size, lay.num_pages = 16, n_pages, page_size, 1
    return lib().sha_workspace_bytes_kv(B, H, H_kv, Nkv, d, top_k, int(gqa), _DT[dtype], nsplit,
                                        num_cus, ctypes.byref(lay))


def _stream_for(dev, stream):
    return torch.cuda.current_stream(dev) if stream is None else stream


def _on(t, dev, name):
    """t must be a tensor on device dev (a host tensor's address would reach
    a kernel as a device address)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != dev:
        raise ValueError(f"{name} must be a tensor on {dev}")
    return t


def _workspace(ws, need, dev):
    """The caller's workspace (a contiguous tensor on dev), or a new one when
    none is given or it is shorter than need bytes."""
    if ws is not None:
        _on(ws, dev, "workspace")
        if not ws.is_contiguous():
            raise ValueError("workspace must be contiguous")
        if ws.numel() * ws.element_size() >= need:
            return ws
    return torch.empty(max(need, 1), dtype=torch.uint8, device=dev)


def _prepare(q, k, v, index, scale, out, gqa, paged=False):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    for name, t in (("k", k), ("v", v)):
        if t.stride(3) != 1:
            raise ValueError(f"{name}: the head dimension must be unit-stride")
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one of float32 / float16 / bfloat16")
    B, H, one, d = q.shape
    if one != 1:
        raise ValueError("q must be [B, H, 1, d]")
    Bk, H_kv, Nkv, dk = k.shape
    if dk != d or v.shape != k.shape or (not paged and Bk != B):
        raise ValueError("k, v must be [B, H_kv, Nkv, d] (paged: [num_pages, H_kv, page, d]) "
                         "matching q")
    if index.dim() != 2 or index.shape[0] != B:
        raise ValueError("index must be [B, top_k]")
    if index.device != q.device:
        raise ValueError("index must be on the same device as q")
    if index.dtype != torch.int32:
        index = index.to(torch.int32)
    index = index.contiguous()
    top_k = index.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.zeros_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    return B, H, H_kv, Nkv, d, top_k, index, float(scale), out


def _layout(k, v, seqlens, block_table, B, Nkv):
    """KvLayout from the K/V views' strides (None for the plain contiguous call)."""
    if seqlens is None and block_table is None and k.is_contiguous() and v.is_contiguous():
        return None, ()
    keep = []
    lay = KvLayout(k.stride(0), k.stride(1), k.stride(2), v.stride(0), v.stride(1), v.stride(2))
    if seqlens is not None:
        seqlens = _dev_i32(_on(seqlens, k.device, "seqlens"), "seqlens")
        if seqlens.numel() != B:
            raise ValueError("seqlens must hold B entries")
        lay.seqlens = seqlens.data_ptr()
        keep.append(seqlens)
    if block_table is not None:
        bt = _dev_i32(_on(block_table, k.device, "block_table"), "block_table")
        if bt.dim() != 2 or bt.shape[0] != B:
            raise ValueError("block_table must be [B, max_pages]")
        lay.block_table = bt.data_ptr()
        lay.block_table_stride = bt.shape[1]
        lay.page_size = k.shape[2]
        lay.num_pages = k.shape[0]
        keep.append(bt)
    return lay, keep


def _call(gqa, q, k, v, index, scale, out, nsplit, workspace, stream, seqlens=None,
          block_table=None, Nkv=None):
    paged = block_table is not None
    if isinstance(q, torch.Tensor) and q.is_cuda:
        stream = _stream_for(q.device, stream)
    # Every temporary (index copy, zero-filled out, workspace) is made on the
    # call's stream, so the kernel sees it ready and the allocator does not
    # hand its memory to other streams while the kernel may still read it.
    with torch.cuda.stream(stream) if stream is not None else _nullctx():
        B, H, H_kv, Nk, d, top_k, index, scale, out = _prepare(q, k, v, index, scale, out, gqa,
                                                               paged)
        if paged:
            if Nkv is None:
                raise ValueError("a paged call needs Nkv (the longest row)")
        else:
            Nkv = Nk
        lay, keep = _layout(k, v, seqlens, block_table, B, Nkv)
        L = lib()
        dt = _DT[q.dtype]
        lp = ctypes.byref(lay) if lay is not None else None
        need = L.sha_workspace_bytes_kv(B, H, H_kv, Nkv, d, top_k, int(gqa), dt, nsplit, 0, lp)
        workspace = _workspace(workspace, need, q.device) if need else None
        ws_ptr = workspace.data_ptr() if need else None
        with torch.cuda.device(q.device):
            if lay is None:
                name = "sha_decode_gqa_ex" if gqa else "sha_decode_ex"
                st = getattr(L, name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), index.data_ptr(),
                                      B, H, H_kv, Nkv, d, top_k, scale, out.data_ptr(),
                                      stream.cuda_stream, dt, nsplit, ws_ptr, need)
            else:
                name = "sha_decode_gqa_kv" if gqa else "sha_decode_kv"
                st = getattr(L, name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), index.data_ptr(),
                                      B, H, H_kv, Nkv, d, top_k, scale, out.data_ptr(),
                                      stream.cuda_stream, dt, lp, nsplit, ws_ptr, need)
        del keep
    _check(st, name)
    return out


class _nullctx:
    def __enter__(self):
        return None

    def __exit__(self, *exc):
        return False


def sha_decode(q, k, v, batch_head_index, scale=None, out=None, nsplit=0, workspace=None,
               stream=None, seqlens=None):
    """Head-indexed SHA decode; returns `out` (allocated zeroed when None).

    q [B, H, 1, d] contiguous; k/v [B, H_kv, Nkv, d], any strides with a
    unit-stride last dimension (e.g. a [B, Nkv, H_kv, d] cache viewed with
    permute(0, 2, 1, 3)); batch_head_index [B, top_k]; seqlens [B] (optional)
    limits row b to its first seqlens[b] keys.  Slots of `out` not named by
    the index are left untouched.

    stream (default: the current stream) runs the call; the inputs must be
    ready on it, as for any operation on that stream.  workspace: a device
    tensor for the split partials (allocated on the stream when None or too
    small).
    """
    return _call(False, q, k, v, batch_head_index, scale, out, nsplit, workspace, stream, seqlens)


def sha_decode_gqa(q, k, v, batch_group_index, scale=None, out=None, nsplit=0, workspace=None,
                   stream=None, seqlens=None):
    """Group-indexed (GQA group sparsity) SHA decode; see sha_decode."""
    return _call(True, q, k, v, batch_group_index, scale, out, nsplit, workspace, stream, seqlens)


def sha_decode_paged(q, k_pages, v_pages, block_table, index, Nkv, seqlens=None, gqa=False,
                     scale=None, out=None, nsplit=0, workspace=None, stream=None):
    """SHA decode over a paged cache.

    k_pages / v_pages: [num_pages, H_kv, page_size, d] views of the page pool
    (any strides, unit-stride last dimension; a [num_pages, page_size, H_kv,
    d] pool is passed as pool.permute(0, 2, 1, 3)).  block_table [B,
    max_pages] int32: row b's key r is on page block_table[b, r // page_size].
    Nkv: the longest row; seqlens [B] optional.  gqa selects group indexing.
    """
    return _call(gqa, q, k_pages, v_pages, index, scale, out, nsplit, workspace, stream, seqlens,
                 block_table, Nkv)


# ---------------------------------------------------------------------------
# selective MLP
# ---------------------------------------------------------------------------

def _dev_i32(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != torch.int32:
        t = t.to(torch.int32)
    return t.contiguous()


def mlp_union(row_neurons, D, sel=None, n_sel=None, stream=None, workspace=None):
    """Sorted union of the rows' neuron lists (entries outside [0, D) skipped),
    on the device: returns (sel [min(D, B*k)] int32, n_sel [1] int32).
    Runs on `stream` (default: the current stream); temporaries are made there."""
    if not isinstance(row_neurons, torch.Tensor) or not row_neurons.is_cuda:
        raise ValueError("row_neurons must be a device tensor")
    stream = _stream_for(row_neurons.device, stream)
    with torch.cuda.stream(stream):
        rows = _dev_i32(row_neurons, "row_neurons")
        if rows.dim() != 2:
            raise ValueError("row_neurons must be [B, k]")
        B, k = rows.shape
        cap = max(1, min(D, B * k))
        if sel is None:
            sel = torch.empty(cap, dtype=torch.int32, device=rows.device)
        elif (_on(sel, rows.device, "sel").numel() < cap or sel.dtype != torch.int32
              or not sel.is_contiguous()):
            raise ValueError(f"sel must be a contiguous int32 tensor of >= {cap} entries")
        if n_sel is None:
            n_sel = torch.empty(1, dtype=torch.int32, device=rows.device)
        elif (_on(n_sel, rows.device, "n_sel").numel() < 1 or n_sel.dtype != torch.int32
              or not n_sel.is_contiguous()):
            raise ValueError("n_sel must be a contiguous int32 tensor of >= 1 entry")
        need = lib().sha_mlp_union_workspace_bytes(D)
        workspace = _workspace(workspace, need, rows.device)
        with torch.cuda.device(rows.device):
            st = lib().sha_mlp_union(rows.data_ptr(), B, k, D, sel.data_ptr(), n_sel.data_ptr(),
                                     stream.cuda_stream, workspace.data_ptr(), need)
    _check(st, "sha_mlp_union")
    return sel, n_sel


def selective_mlp_workspace_bytes(B, d, D, n_max, num_cus=0) -> int:
    return lib().sha_selective_mlp_workspace_bytes(B, d, D, n_max, num_cus)


def selective_mlp(x, w1t, w2t, sel, n_sel, n_max=None, out=None, workspace=None, stream=None):
    """y = relu(x w1t[S]^T) w2t[S], S = sel[:n_sel] (device count).

    x [B, d]; w1t, w2t [D, d] (neuron-major: W1^T and W2^T); f16 or bf16.
    n_max bounds the count (default: sel.numel()); sel must hold at least
    n_max entries.  Runs on `stream` (default: the current stream).
    """
    for name, t in (("x", x), ("w1t", w1t), ("w2t", w2t)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
            raise ValueError(f"{name} must be a contiguous 2-D device tensor")
    if x.dtype not in (torch.float16, torch.bfloat16) or w1t.dtype != x.dtype or w2t.dtype != x.dtype:
        raise ValueError("x, w1t, w2t must share float16 or bfloat16")
    B, d = x.shape
    D = w1t.shape[0]
    if w1t.shape != (D, d) or w2t.shape != (D, d):
        raise ValueError("w1t and w2t must be [D, d]")
    if w1t.device != x.device or w2t.device != x.device:
        raise ValueError("x, w1t, w2t must be on one device")
    stream = _stream_for(x.device, stream)
    with torch.cuda.stream(stream):
        sel = _dev_i32(_on(sel, x.device, "sel"), "sel")
        n_sel = _dev_i32(_on(n_sel, x.device, "n_sel"), "n_sel")
        if n_sel.numel() < 1:
            raise ValueError("n_sel must hold the count")
        if n_max is None:
            n_max = min(sel.numel(), D)
        if n_max > sel.numel():
            raise ValueError(f"n_max = {n_max} exceeds the {sel.numel()} entries of sel")
        if out is None:
            out = torch.empty_like(x)
        elif (_on(out, x.device, "out").shape != x.shape or out.dtype != x.dtype
              or not out.is_contiguous()):
            raise ValueError("out must be a contiguous tensor like x")
        L = lib()
        need = L.sha_selective_mlp_workspace_bytes(B, d, D, n_max, 0)
        workspace = _workspace(workspace, need, x.device)
        with torch.cuda.device(x.device):
            st = L.sha_selective_mlp(x.data_ptr(), w1t.data_ptr(), w2t.data_ptr(), sel.data_ptr(),
                                     n_sel.data_ptr(), n_max, B, d, D, out.data_ptr(),
                                     stream.cuda_stream, _DT[x.dtype], workspace.data_ptr(), need)
    _check(st, "sha_selective_mlp")
    return out


# ---------------------------------------------------------------------------
# attention router
# ---------------------------------------------------------------------------

def router_workspace_bytes(B, d, H, dtype, split=None) -> int:
    """Workspace bytes of the router's K-split form: where the library picks
    it (split=None), for any shape that has it (True), or 0 (False)."""
    if split is False:
        return 0
    fn = lib().sha_router_split_bytes if split else lib().sha_router_workspace_bytes
    return fn(B, d, H, _DT[dtype])


def router_topk(x, w, top_k, bias=None, index=None, scores=None, stream=None, workspace=None,
                split=None):
    """Attention router on the device: scores = x w^T (+ bias), the top_k heads
    per row in ascending order.  x [B, d], w [H, d] (f32 / f16 / bf16), bias
    [H] fp32.  Returns (index [B, top_k] int32, scores [B, H] fp32).  Runs on
    `stream` (default: the current stream).  split=None takes the K-split
    form where the library finds it faster, True wherever the shape has one,
    False never; it runs in `workspace` (a device byte tensor) or a
    temporary one."""
    for name, t in (("x", x), ("w", w)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
            raise ValueError(f"{name} must be a contiguous 2-D device tensor")
    if x.dtype not in _DT or w.dtype != x.dtype:
        raise ValueError("x and w must share float32 / float16 / bfloat16")
    B, d = x.shape
    H = w.shape[0]
    if w.shape[1] != d:
        raise ValueError("w must be [H, d]")
    if w.device != x.device:
        raise ValueError("x and w must be on one device")
    stream = _stream_for(x.device, stream)
    with torch.cuda.stream(stream):
        if bias is not None:
            if _on(bias, x.device, "bias").dtype != torch.float32 or bias.numel() != H:
                raise ValueError("bias must be a float32 device tensor of H entries")
            bias = bias.contiguous()
        if index is None:
            index = torch.empty((B, top_k), dtype=torch.int32, device=x.device)
        elif _on(index, x.device, "index").dtype != torch.int32 or not index.is_contiguous() or \
                tuple(index.shape) != (B, top_k):
            raise ValueError("index must be a contiguous int32 [B, top_k] tensor")
        if scores is None:
            scores = torch.empty((B, H), dtype=torch.float32, device=x.device)
        elif _on(scores, x.device, "scores").dtype != torch.float32 or \
                not scores.is_contiguous() or tuple(scores.shape) != (B, H):
            raise ValueError("scores must be a contiguous float32 [B, H] tensor")
        need = router_workspace_bytes(B, d, H, x.dtype, split)
        if need > 0:
            workspace = _workspace(workspace, need, x.device)
        with torch.cuda.device(x.device):
            st = lib().sha_router_topk_ex(x.data_ptr(), w.data_ptr(),
                                          bias.data_ptr() if bias is not None else None, B, d, H,
                                          top_k, index.data_ptr(), scores.data_ptr(),
                                          stream.cuda_stream, _DT[x.dtype],
                                          workspace.data_ptr() if need > 0 else None, need)
    _check(st, "sha_router_topk_ex")
    return index, scores


# ---------------------------------------------------------------------------
# multi-layer decode step (optionally one HIP graph)
# ---------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else t.data_ptr()


def _step_check(i, L, B, top_k, n_sel):
    def need(name, dtype, shape=None):
        t = L.get(name)
        if t is None:
            return
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dtype \
                or not t.is_contiguous() or (shape is not None and tuple(t.shape) != shape):
            want = f"contiguous {dtype} device tensor" + (f" of shape {shape}" if shape else "")
            raise ValueError(f"layer {i}: {name} must be a {want}")
    need("seqlens", torch.int32, (B,))
    need("block_table", torch.int32)
    if L.get("block_table") is not None and L["block_table"].dim() != 2:
        raise ValueError(f"layer {i}: block_table must be [B, max_pages]")
    if not L.get("dense", False):
        need("index", torch.int32, (B, top_k))
        need("router_scores", torch.float32, (B, n_sel))


class DecodeStep:
    """n layers of router -> selective head attention (-> selective MLP),
    created once and run many times (sha_step_create / sha_step_run).

    layers: list of dicts with device tensors under the sha_step_layer field
    names (router_x, router_w, router_bias, router_scores, index, q, k, v, o,
    dense, mlp_x, mlp_w1t, mlp_w2t, mlp_y, mlp_rows) and optionally
    seqlens (per-row key counts) and block_table (a paged layer: k/v are
    [num_pages, H_kv, page, d] views of page pools and block_table is the
    [B, max_pages] int32 table, as for sha_decode_paged; Nkv is then the
    longest row).
    The tensors are referenced for the life of the step: refresh their
    contents in place between runs.  A tensor the step would otherwise have
    to copy (seqlens or block_table not contiguous int32, index not
    contiguous int32 [B, top_k], router_scores not contiguous float32
    [B, H] -- [B, H_kv] for group layers) is rejected with ValueError, since
    in-place refreshes of the original would never reach the copy.
    """

    def __init__(self, B, H, H_kv, Nkv, d, top_k, dtype, layers, gqa=False, scale=None,
                 router_d=0, mlp_d=0, mlp_D=0, mlp_k=0, use_graph=True):
        self._handle = None
        self._keep = []
        cfg = StepConfig(B, H, H_kv, Nkv, d, top_k, int(gqa),
                         float(scale if scale is not None else 1.0 / math.sqrt(d)), _DT[dtype],
                         router_d, mlp_d, mlp_D, mlp_k)
        arr = (StepLayer * len(layers))()
        n_sel = H_kv if gqa else H
        for i, L in enumerate(layers):
            _step_check(i, L, B, top_k, n_sel)
            for name in ("router_x", "router_w", "router_bias", "router_scores", "index", "q",
                         "k", "v", "o", "mlp_x", "mlp_w1t", "mlp_w2t", "mlp_y", "mlp_rows"):
                t = L.get(name)
                if t is not None:
                    if not isinstance(t, torch.Tensor) or not t.is_cuda or \
                            t.device != layers[0]["q"].device:
                        raise ValueError(f"layer {i}: {name} must be a tensor on the device of "
                                         "layer 0's q")
                    self._keep.append(t)
                setattr(arr[i], name, _ptr(t))
            arr[i].dense = int(bool(L.get("dense", False)))
            k, v, sl, bt = L["k"], L["v"], L.get("seqlens"), L.get("block_table")
            if sl is not None or bt is not None or not (k.is_contiguous() and v.is_contiguous()):
                lay, keep = _layout(k, v, sl, bt, B, Nkv)
                self._keep += [lay] + list(keep)
                arr[i].kv = ctypes.pointer(lay)
        self._keep.append(arr)
        h = ctypes.c_void_p()
        _check(lib().sha_step_create(ctypes.byref(cfg), arr, len(layers), int(use_graph),
                                     ctypes.byref(h)), "sha_step_create")
        self._handle = h

    def run(self, stream=None):
        if self._handle is None:
            raise RuntimeError("step is closed")
        if stream is None:
            stream = torch.cuda.current_stream()
        _check(lib().sha_step_run(self._handle, stream.cuda_stream), "sha_step_run")

    def close(self):
        if self._handle is not None:
            torch.cuda.synchronize()
            lib().sha_step_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
