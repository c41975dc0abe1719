"""KV cache layouts and per-row cache lengths on the GPU (through the C ABI):
strided views ([B, Nkv, H_kv, d] caches), ragged seqlens and paged pools,
each against the fp64 oracle with the same lengths, plus exact properties
(bitwise equality with the contiguous call where the arithmetic order is the
same, untouched inactive slots, no read past a row's length or outside its
pages)."""
import numpy as np
import pytest
import torch

import contextual_head_sparsity_amd as sha
from contextual_head_sparsity_amd import workloads as wl
from oracle import sha_decode_gqa_ref, sha_decode_ref, sha_units_ref

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import DEV, TOL, bnhd as _bnhd, paged as _paged, ragged as _ragged, say, \
        written_mask


def _case(dtype, gqa, B=4, Nkv=300, d=128, seed=11):
    if gqa:
        w = wl.Workload("kv", B=B, H=16, H_kv=2, d=d, Nkv=Nkv, top_k=1, dtype=dtype, gqa=True,
                        seed=seed)
    else:
        w = wl.Workload("kv", B=B, H=8, H_kv=8, d=d, Nkv=Nkv, top_k=3, dtype=dtype, seed=seed)
    q, k, v, idx, o = wl.make_workload(w, "cpu")
    return w, q, k, v, idx, o


def _check(w, q, k, v, idx, o_before, got, seqlens=None):
    ref_fn = sha_decode_gqa_ref if w.gqa else sha_decode_ref
    ref, written = ref_fn(q, k, v, idx, w.scale, seqlens=seqlens)
    g = got.cpu()
    g64 = g.to(torch.float64).numpy()
    assert np.isfinite(g64[written]).all(), "non-finite output in an active slot"
    err = float(np.max(np.abs(g64[written] - ref[written])))
    assert err <= TOL[w.dtype], f"max abs error {err:.3e}"
    wt = torch.from_numpy(written)
    assert torch.equal(wl.raw_bits(g)[~wt], wl.raw_bits(o_before)[~wt]), "an inactive slot changed"
    return err


def _call(w, q, k, v, idx, o, **kw):
    fn = sha.sha_decode_gqa if w.gqa else sha.sha_decode
    out = o.to(DEV)
    fn(q.to(DEV), k, v, idx.to(DEV), scale=w.scale, out=out, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("gqa", [False, True])
@pytest.mark.parametrize("nsplit", [1, 3, 0])
def test_strided_bnhd_cache(dtype, gqa, nsplit):
    say(f"[kv] strided dtype={dtype} gqa={gqa} nsplit={nsplit}")
    w, q, k, v, idx, o = _case(dtype, gqa)
    got = _call(w, q, _bnhd(k), _bnhd(v), idx, o, nsplit=nsplit)
    _check(w, q, k, v, idx, o, got)
    # Same arithmetic order as the contiguous call: identical bits.
    ref = _call(w, q, k.to(DEV), v.to(DEV), idx, o, nsplit=nsplit)
    assert torch.equal(wl.raw_bits(got), wl.raw_bits(ref))
    # K and V with different layouts in one call.
    mixed = _call(w, q, _bnhd(k), v.to(DEV), idx, o, nsplit=nsplit)
    assert torch.equal(wl.raw_bits(mixed), wl.raw_bits(ref))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("gqa", [False, True])
@pytest.mark.parametrize("nsplit", [1, 4, 0])
def test_ragged_seqlens(dtype, gqa, nsplit):
    say(f"[kv] seqlens dtype={dtype} gqa={gqa} nsplit={nsplit}")
    w, q, k, v, idx, o = _case(dtype, gqa, B=7, Nkv=300)
    lens = np.array([300, 0, 1, 17, 160, 999, -4], dtype=np.int32)
    k, v = _ragged(w, k, v, lens)
    sl = torch.from_numpy(lens).to(DEV)
    got = _call(w, q, k.to(DEV), v.to(DEV), idx, o, nsplit=nsplit, seqlens=sl)
    _check(w, q, k, v, idx, o, got, seqlens=lens)
    # Empty rows (length 0 or negative) get exact zeros in their active slots.
    written = written_mask(idx.numpy(), w.H, w.H_kv, w.gqa)
    for b in (1, 6):
        assert torch.count_nonzero(got[b][torch.from_numpy(written[b]).to(DEV)]) == 0
    # Strided and ragged together.
    got2 = _call(w, q, _bnhd(k), _bnhd(v), idx, o, nsplit=nsplit, seqlens=sl)
    assert torch.equal(wl.raw_bits(got2), wl.raw_bits(got))


def _call_paged(w, q, kp, vp, bt, idx, o, **kw):
    out = o.to(DEV)
    sha.sha_decode_paged(q.to(DEV), kp, vp, bt, idx.to(DEV), w.Nkv, gqa=w.gqa, scale=w.scale,
                         out=out, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("gqa", [False, True])
@pytest.mark.parametrize("P,pool", [(16, "nphd"), (64, "nhpd"), (256, "nphd")])
def test_paged_cache(dtype, gqa, P, pool):
    say(f"[kv] paged dtype={dtype} gqa={gqa} P={P} pool={pool}")
    w, q, k, v, idx, o = _case(dtype, gqa, B=5, Nkv=700)
    kp, vp, bt = _paged(w, k, v, P, pool, seed=P)
    for nsplit in (1, 3, 0):
        got = _call_paged(w, q, kp, vp, bt, idx, o, nsplit=nsplit)
        _check(w, q, k, v, idx, o, got)
    lens = np.array([700, 0, 1, 333, 2000], dtype=np.int32)
    got = _call_paged(w, q, kp, vp, bt, idx, o, seqlens=torch.from_numpy(lens).to(DEV))
    _check(w, q, k, v, idx, o, got, seqlens=lens)


@pytest.mark.parametrize("gqa", [False, True])
def test_paged_bitwise_equals_contiguous(gqa):
    """16-row pages keep the contiguous split geometry, so the bits agree."""
    say(f"[kv] paged == contiguous gqa={gqa}")
    w, q, k, v, idx, o = _case("bf16", gqa, B=3, Nkv=1000)
    kp, vp, bt = _paged(w, k, v, 16, "nphd", seed=5)
    for nsplit in (1, 3):
        got = _call_paged(w, q, kp, vp, bt, idx, o, nsplit=nsplit)
        ref = _call(w, q, k.to(DEV), v.to(DEV), idx, o, nsplit=nsplit)
        assert torch.equal(wl.raw_bits(got), wl.raw_bits(ref))


def test_long_paged_rows_force_splits():
    """A row longer than 1024 pages is split even when one split is asked."""
    say("[kv] 1024-page split limit")
    w, q, k, v, idx, o = _case("f16", False, B=1, Nkv=16 * 1024 + 40, d=64, seed=3)
    kp, vp, bt = _paged(w, k, v, 16, "nphd", seed=9, extra=0)
    got = _call_paged(w, q, kp, vp, bt, idx, o, nsplit=1)
    _check(w, q, k, v, idx, o, got)


def _sampled_ragged(w, q, k, v, idx, lens, o_bits, got, n, seed):
    G = w.G
    written = written_mask(idx.cpu().numpy(), w.H, w.H_kv, w.gqa)
    wt = torch.from_numpy(written).to(DEV)
    assert torch.equal(wl.raw_bits(got)[~wt], o_bits[~wt]), "an inactive slot changed"
    assert torch.isfinite(got[wt]).all()
    rng = np.random.default_rng(seed)
    active = np.argwhere(written)
    pick = active[rng.choice(len(active), size=min(n, len(active)), replace=False)]
    err = 0.0
    for b, h in pick:
        m = max(0, min(int(lens[b]), w.Nkv))
        gotv = got[b, h, 0].cpu().to(torch.float64).numpy()
        if m == 0:
            assert not np.any(gotv)
            continue
        ref = sha_units_ref(q[b, h, 0][None].cpu(), k[b, h // G, :m][None].cpu(),
                            v[b, h // G, :m][None].cpu(), w.scale)[0]
        err = max(err, float(np.max(np.abs(gotv - ref))))
    assert err <= TOL[w.dtype], f"max abs error {err:.3e} on sampled slots"
    return err


def test_full_size_opt66b_bnhd_ragged():
    """The OPT-66B decode layer with a [B, Nkv, H, d] cache and ragged rows."""
    w = wl.WORKLOADS["opt66b_f16"]
    say(f"[kv] full size {w.name} bnhd + ragged seqlens")
    q, k, v, idx, o = wl.make_workload(w, DEV)
    lens = np.random.default_rng(5).integers(0, w.Nkv + 1, size=w.B).astype(np.int32)
    lens[:3] = [0, 1, w.Nkv]
    kb, vb = _bnhd(k), _bnhd(v)
    bits = wl.raw_bits(o).clone()
    fn_out = sha.sha_decode(q, kb, vb, idx, scale=w.scale, out=o,
                            seqlens=torch.from_numpy(lens).to(DEV))
    torch.cuda.synchronize()
    err = _sampled_ragged(w, q, k, v, idx, lens, bits, fn_out, 48, 1)
    say(f"   max_err={err:.3e}")


def test_full_size_llama70b_paged():
    """The LLaMA-3.1-70B GQA layer from a 64-row-page pool (group sparsity)."""
    w = wl.WORKLOADS["llama3.1_70b_gqa_bf16"]
    say(f"[kv] full size {w.name} paged P=64")
    q, k, v, idx, o = wl.make_workload(w, DEV)
    P = 64
    npg = w.Nkv // P
    perm = torch.from_numpy(np.random.default_rng(7).permutation(w.B * npg).astype(np.int32))
    bt = perm.view(w.B, npg).to(DEV)
    # pool [num_pages, P, H_kv, d]: page bt[b, j] holds rows j*P .. j*P+P-1 of row b
    kpool = torch.empty((w.B * npg, P, w.H_kv, w.d), dtype=k.dtype, device=DEV)
    vpool = torch.empty_like(kpool)
    src_k = k.view(w.B, w.H_kv, npg, P, w.d).permute(0, 2, 3, 1, 4).reshape(-1, P, w.H_kv, w.d)
    src_v = v.view(w.B, w.H_kv, npg, P, w.d).permute(0, 2, 3, 1, 4).reshape(-1, P, w.H_kv, w.d)
    kpool[bt.view(-1).long()] = src_k
    vpool[bt.view(-1).long()] = src_v
    del src_k, src_v
    lens = np.random.default_rng(8).integers(1, w.Nkv + 1, size=w.B).astype(np.int32)
    bits = wl.raw_bits(o).clone()
    sha.sha_decode_paged(q, kpool.permute(0, 2, 1, 3), vpool.permute(0, 2, 1, 3), bt, idx, w.Nkv,
                         seqlens=torch.from_numpy(lens).to(DEV), gqa=True, scale=w.scale, out=o)
    torch.cuda.synchronize()
    err = _sampled_ragged(w, q, k, v, idx, lens, bits, o, 48, 2)
    say(f"   max_err={err:.3e}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("gqa", [False, True])
def test_d64_strided_and_paged(dtype, gqa):
    """Head dimension 64 (half-width rows) through the strided and paged
    layouts, with ragged lengths, split and unsplit."""
    say(f"[kv] d=64 dtype={dtype} gqa={gqa}")
    w, q, k, v, idx, o = _case(dtype, gqa, B=4, Nkv=900, d=64, seed=13)
    lens = np.array([900, 1, 450, 0], dtype=np.int32)
    lens_d = torch.from_numpy(lens).to(DEV)
    for nsplit in (1, 3):
        got = _call(w, q, _bnhd(k), _bnhd(v), idx, o, nsplit=nsplit, seqlens=lens_d)
        _check(w, q, k, v, idx, o, got, seqlens=lens)
        kp, vp, bt = _paged(w, k, v, 32, "nphd", seed=3)
        got = _call_paged(w, q, kp, vp, bt, idx, o, nsplit=nsplit, seqlens=lens_d)
        _check(w, q, k, v, idx, o, got, seqlens=lens)
