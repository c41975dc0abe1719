"""Multi-layer decode step on the GPU (sha_step_* through the C ABI).

A step strings router -> selective head attention -> selective MLP over
several layers, layer 0 dense, and may run as one captured HIP graph.  Every
run is compared bit for bit with the same calls made one by one, and every
layer's attention output is checked against the fp64 oracle on the index
the step's own router wrote (all heads for the dense layer), with that
layer's per-row lengths and page layout.  Graph replays are interleaved with
in-place input updates (queries, router inputs, MLP rows and the per-row
lengths), other device work and synchronisations, and every replay is
checked.
"""
import numpy as np
import pytest
import torch

import contextual_head_sparsity_amd as sha
from contextual_head_sparsity_amd import workloads as wl
from oracle import sha_decode_gqa_ref, sha_decode_ref

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import DEV, TOL, say


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _to_pages(k, v, P, seed):
    """The rows of k/v [B, H_kv, Nkv, d] scattered into pools of P-row pages
    [num_pages, H_kv, P, d] in a seeded page order, and the block table."""
    B, H_kv, Nkv, d = k.shape
    npg = (Nkv + P - 1) // P
    perm = torch.randperm(B * npg, generator=torch.Generator().manual_seed(seed)).reshape(B, npg)
    kp = torch.zeros(B * npg, H_kv, P, d, dtype=k.dtype, device=DEV)
    vp = torch.zeros_like(kp)
    for b in range(B):
        for j in range(npg):
            r0, r1 = j * P, min((j + 1) * P, Nkv)
            kp[perm[b, j], :, :r1 - r0] = k[b, :, r0:r1]
            vp[perm[b, j], :, :r1 - r0] = v[b, :, r0:r1]
    return kp, vp, perm.to(torch.int32).to(DEV)


def _layers(cfg, n_layers, mlp, seed, seqlens_layer=None, paged=None):
    B, H, H_kv, d, Nkv = cfg["B"], cfg["H"], cfg["H_kv"], cfg["d"], cfg["Nkv"]
    dt = cfg["dtype"]
    nh = H_kv if cfg["gqa"] else H
    g = _gen(seed)
    out = []
    for l in range(n_layers):
        w = wl.Workload("step", B=B, H=H, H_kv=H_kv, d=d, Nkv=Nkv, top_k=cfg["top_k"],
                        dtype=cfg["dname"], gqa=cfg["gqa"], seed=seed + l)
        q, k, v = wl.make_qkv(w, DEV)
        # k_ref / v_ref: the contiguous cache the oracle reads (the step
        # never looks at these keys).
        L = dict(q=q, k=k, v=v, o=wl.sentinel_like(w, DEV), dense=(l == 0), k_ref=k, v_ref=v)
        if l == seqlens_layer:
            L["k"] = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
            L["v"] = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
            L["seqlens"] = torch.randint(0, Nkv + 1, (B,), generator=g, device=DEV,
                                         dtype=torch.int32)
        if paged is not None and l == paged[0]:
            L["k"], L["v"], L["block_table"] = _to_pages(k, v, paged[1], seed=seed + l)
        if l > 0:
            L["router_x"] = torch.randn(B, cfg["router_d"], generator=g, device=DEV).to(dt)
            L["router_w"] = torch.randn(nh, cfg["router_d"], generator=g, device=DEV).to(dt)
            L["router_bias"] = torch.randn(nh, generator=g, device=DEV)
            L["router_scores"] = torch.empty(B, nh, device=DEV)
            L["index"] = torch.empty(B, cfg["top_k"], dtype=torch.int32, device=DEV)
        if mlp:
            md, mD, mk = mlp
            mw = wl.MlpWorkload("step", B=B, d=md, D=mD, k_row=mk, dtype=cfg["dname"],
                                seed=seed + 100 + l)
            x, w1t, w2t, rows = wl.make_mlp(mw, DEV)
            L.update(mlp_x=x, mlp_w1t=w1t, mlp_w2t=w2t, mlp_rows=rows,
                     mlp_y=torch.full_like(x, float("nan")))
        out.append(L)
    return out


def _eager(cfg, layers, mlp):
    """The step's calls one by one through the per-call entry points."""
    B = cfg["B"]
    nh = cfg["H_kv"] if cfg["gqa"] else cfg["H"]
    fn = sha.sha_decode_gqa if cfg["gqa"] else sha.sha_decode
    res = []
    for L in layers:
        r = {}
        if L["dense"]:
            idx = torch.arange(nh, dtype=torch.int32, device=DEV).repeat(B, 1)
        else:
            idx, sc = sha.router_topk(L["router_x"], L["router_w"], cfg["top_k"],
                                      bias=L["router_bias"])
            r["index"], r["router_scores"] = idx, sc
        o = wl.sentinel_like(wl.Workload("s", B=B, H=cfg["H"], H_kv=cfg["H_kv"], d=cfg["d"],
                                         Nkv=cfg["Nkv"], top_k=1, dtype=cfg["dname"]), DEV)
        if "block_table" in L:
            r["o"] = sha.sha_decode_paged(L["q"], L["k"], L["v"], L["block_table"], idx,
                                          cfg["Nkv"], gqa=cfg["gqa"], scale=cfg["scale"], out=o,
                                          seqlens=L.get("seqlens"))
        else:
            r["o"] = fn(L["q"], L["k"], L["v"], idx, scale=cfg["scale"], out=o,
                        seqlens=L.get("seqlens"))
        if mlp:
            md, mD, mk = mlp
            sel, n_sel = sha.mlp_union(L["mlp_rows"], mD)
            r["mlp_y"] = sha.selective_mlp(L["mlp_x"], L["mlp_w1t"], L["mlp_w2t"], sel, n_sel,
                                           n_max=min(B * mk, mD))
        res.append(r)
    torch.cuda.synchronize()
    return res


def _compare(layers, ref):
    for l, (L, r) in enumerate(zip(layers, ref)):
        for name, t in r.items():
            got = L[name]
            if got.dtype.is_floating_point:
                same = torch.equal(wl.raw_bits(got) if got.dtype != torch.float32
                                   else got.view(torch.int32),
                                   wl.raw_bits(t) if t.dtype != torch.float32
                                   else t.view(torch.int32))
            else:
                same = torch.equal(got, t)
            assert same, f"layer {l}: {name} differs from the per-call result"


def _reset_outputs(cfg, layers):
    for L in layers:
        L["o"].copy_(wl.sentinel_like(wl.Workload("s", B=cfg["B"], H=cfg["H"], H_kv=cfg["H_kv"],
                                                  d=cfg["d"], Nkv=cfg["Nkv"], top_k=1,
                                                  dtype=cfg["dname"]), DEV))
        if "mlp_y" in L:
            L["mlp_y"].fill_(float("nan"))
        if "index" in L:
            L["index"].fill_(-5)


def _refresh_inputs(layers, seed):
    g = _gen(seed)
    for L in layers:
        L["q"].copy_(torch.randn(L["q"].shape, generator=g, device=DEV).to(L["q"].dtype))
        if "router_x" in L:
            L["router_x"].copy_(torch.randn(L["router_x"].shape, generator=g, device=DEV)
                                .to(L["router_x"].dtype))
        if "mlp_x" in L:
            L["mlp_x"].copy_(torch.randn(L["mlp_x"].shape, generator=g, device=DEV)
                             .to(L["mlp_x"].dtype))
            D = L["mlp_w1t"].shape[0]
            L["mlp_rows"].copy_(torch.randint(-1, D, L["mlp_rows"].shape, generator=g,
                                              device=DEV, dtype=torch.int32))
        if "seqlens" in L:
            n = L["k_ref"].shape[2]
            L["seqlens"].copy_(torch.randint(0, n + 1, L["seqlens"].shape, generator=g,
                                             device=DEV, dtype=torch.int32))


def _check_oracle(cfg, layers, sentinel_bits):
    """Each layer's o against the fp64 oracle on the index the step used."""
    ref_fn = sha_decode_gqa_ref if cfg["gqa"] else sha_decode_ref
    nh = cfg["H_kv"] if cfg["gqa"] else cfg["H"]
    for l, L in enumerate(layers):
        if L["dense"]:
            idx = np.tile(np.arange(nh, dtype=np.int32), (cfg["B"], 1))
        else:
            idx = L["index"].cpu().numpy()
        sl = L.get("seqlens")
        O, written = ref_fn(L["q"].cpu(), L["k_ref"].cpu(), L["v_ref"].cpu(), idx, cfg["scale"],
                            seqlens=None if sl is None else sl.cpu())
        if L["dense"]:
            assert written.all()
        got = L["o"].cpu()
        g64 = got.double().numpy()
        assert np.isfinite(g64[written]).all(), f"layer {l}: non-finite active output"
        err = float(np.max(np.abs(g64[written] - O[written])))
        assert err <= TOL[cfg["dname"]], f"layer {l}: max abs error {err:.3e}"
        w = torch.from_numpy(written)
        assert torch.equal(wl.raw_bits(got)[~w], sentinel_bits[~w]), \
            f"layer {l}: an unselected slot changed"


# (config, MLP (d, D, k per row) or None, layer with per-row lengths, (paged
# layer, page rows) or None)
CASES = {
    "opt_mha_f16_mlp": (dict(B=8, H=8, H_kv=8, d=128, Nkv=300, top_k=3, gqa=False,
                             dtype=torch.float16, dname="f16", router_d=256),
                        (256, 1024, 64), None, (2, 16)),
    "gqa_bf16_ragged": (dict(B=4, H=16, H_kv=4, d=128, Nkv=700, top_k=2, gqa=True,
                             dtype=torch.bfloat16, dname="bf16", router_d=512),
                        None, 2, (1, 64)),
    "mha_f32_d64": (dict(B=3, H=6, H_kv=6, d=64, Nkv=2100, top_k=2, gqa=False,
                         dtype=torch.float32, dname="f32", router_d=128),
                    None, 1, None),
    # B * H * router_d = 2^24: the router takes its K-split form, its partials
    # in the step's attention workspace
    "mha_bf16_split_router": (dict(B=64, H=8, H_kv=8, d=64, Nkv=130, top_k=3, gqa=False,
                                   dtype=torch.bfloat16, dname="bf16", router_d=32768),
                              None, 2, None),
}


@pytest.mark.parametrize("use_graph", [True, False])
@pytest.mark.parametrize("case", list(CASES))
def test_step_matches_per_call(case, use_graph):
    cfg, mlp, sl_layer, paged = CASES[case]
    cfg = dict(cfg, scale=1.0 / np.sqrt(cfg["d"]))
    say(f"[step] {case} graph={use_graph}")
    n_layers = 3
    layers = _layers(cfg, n_layers, mlp, seed=17, seqlens_layer=sl_layer, paged=paged)
    md, mD, mk = mlp if mlp else (0, 0, 0)
    step = sha.DecodeStep(cfg["B"], cfg["H"], cfg["H_kv"], cfg["Nkv"], cfg["d"], cfg["top_k"],
                          cfg["dtype"], layers, gqa=cfg["gqa"], scale=cfg["scale"],
                          router_d=cfg["router_d"], mlp_d=md, mlp_D=mD, mlp_k=mk,
                          use_graph=use_graph)
    sentinel_bits = wl.raw_bits(wl.sentinel_like(
        wl.Workload("s", B=cfg["B"], H=cfg["H"], H_kv=cfg["H_kv"], d=cfg["d"], Nkv=cfg["Nkv"],
                    top_k=1, dtype=cfg["dname"]), "cpu"))
    try:
        for rep in range(3):
            _reset_outputs(cfg, layers)
            torch.cuda.synchronize()
            step.run()
            torch.cuda.synchronize()
            _check_oracle(cfg, layers, sentinel_bits)
            ref = _eager(cfg, layers, mlp)
            _compare(layers, ref)
            # in-place refresh plus unrelated device work before the next run
            _refresh_inputs(layers, seed=100 + rep)
            torch.cuda.synchronize()
            junk = torch.randn(1 << 20, device=DEV).cumsum(0)
            del junk
    finally:
        step.close()


def test_step_rejects_tensors_it_would_copy():
    """The step keeps pointers to its inputs: tensors the binding would have
    to convert (so that in-place refreshes would never reach the step) are
    rejected instead."""
    cfg = dict(CASES["gqa_bf16_ragged"][0])
    cfg["scale"] = 1.0 / np.sqrt(cfg["d"])
    layers = _layers(cfg, 2, None, seed=5, seqlens_layer=1)
    args = (cfg["B"], cfg["H"], cfg["H_kv"], cfg["Nkv"], cfg["d"], cfg["top_k"], cfg["dtype"])
    kw = dict(gqa=True, scale=cfg["scale"], router_d=cfg["router_d"])
    bad = [("seqlens", layers[1]["seqlens"].to(torch.int64)),
           ("index", layers[1]["index"].to(torch.int64)),
           ("index", layers[1]["index"][:, :1].contiguous()),
           ("router_scores", layers[1]["router_scores"].to(torch.float16)),
           ("router_scores", layers[1]["router_scores"].t().contiguous().t())]
    for name, t in bad:
        L1 = dict(layers[1], **{name: t})
        with pytest.raises(ValueError, match=name):
            sha.DecodeStep(*args, [layers[0], L1], **kw)
