"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and compare with the fp64 oracle element by element."""
import math

import numpy as np
import torch

import contextual_head_sparsity_amd as sha
from contextual_head_sparsity_amd import workloads as wl
from oracle import sha_decode_gqa_ref, sha_decode_ref, sha_units_ref

# Max abs error on active heads for N(0, 1) inputs, per element type.
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
TOL_T = {torch.float32: 1e-5, torch.float16: 2e-3, torch.bfloat16: 1e-2}

DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def run_gpu(gqa, q, k, v, idx, scale, o, nsplit=0, workspace=None):
    fn = sha.sha_decode_gqa if gqa else sha.sha_decode
    fn(q, k, v, idx, scale=scale, out=o, nsplit=nsplit, workspace=workspace)
    torch.cuda.synchronize()
    return o


def check_full(gqa, q, k, v, idx, scale, o_before, o_after, tol):
    """Whole-call comparison: every slot, with the oracle on the CPU."""
    ref_fn = sha_decode_gqa_ref if gqa else sha_decode_ref
    ref, written = ref_fn(q.cpu(), k.cpu(), v.cpu(), idx.cpu(), scale)
    got = o_after.cpu()
    g64 = got.to(torch.float64).numpy()
    w = written
    assert np.isfinite(g64[w]).all(), "non-finite output in an active slot"
    err = float(np.max(np.abs(g64[w] - ref[w]))) if w.any() else 0.0
    assert err <= tol, f"max abs error {err:.3e} > {tol}"
    wt = torch.from_numpy(w)
    assert torch.equal(wl.raw_bits(got)[~wt], wl.raw_bits(o_before.cpu())[~wt]), \
        "an inactive slot changed"
    return err, written


def written_mask(idx_cpu: np.ndarray, H: int, H_kv: int, gqa: bool) -> np.ndarray:
    B = idx_cpu.shape[0]
    G = H // H_kv
    w = np.zeros((B, H), bool)
    for b in range(B):
        for e in idx_cpu[b]:
            if gqa:
                if 0 <= e < H_kv:
                    w[b, e * G:(e + 1) * G] = True
            elif 0 <= e < H:
                w[b, e] = True
    return w


def check_sampled(gqa, q, k, v, idx, scale, o_before_bits, o_after, tol, n_samples, seed):
    """Full-size comparison: a seeded sample of active (b, h) slots against the
    oracle computed unit by unit, plus whole-tensor properties (every active
    slot finite, every inactive slot bit-identical to its prefill)."""
    B, H = q.shape[:2]
    H_kv = k.shape[1]
    G = H // H_kv
    idx_cpu = idx.cpu().numpy()
    w = written_mask(idx_cpu, H, H_kv, gqa)
    wt = torch.from_numpy(w).to(o_after.device)
    bits = wl.raw_bits(o_after)
    assert torch.equal(bits[~wt], o_before_bits[~wt]), "an inactive slot changed"
    assert torch.isfinite(o_after[wt]).all(), "non-finite output in an active slot"
    rng = np.random.default_rng(seed)
    active = np.argwhere(w)
    pick = active[rng.choice(len(active), size=min(n_samples, len(active)), replace=False)]
    qs = torch.stack([q[b, h, 0] for b, h in pick]).cpu()
    ks = torch.stack([k[b, h // G] for b, h in pick]).cpu()
    vs = torch.stack([v[b, h // G] for b, h in pick]).cpu()
    ref = sha_units_ref(qs, ks, vs, scale)
    got = torch.stack([o_after[b, h, 0] for b, h in pick]).cpu().to(torch.float64).numpy()
    err = float(np.max(np.abs(got - ref)))
    assert err <= tol, f"max abs error {err:.3e} > {tol} on sampled slots"
    return err


def bnhd(t):
    """The same values stored as [B, Nkv, H_kv, d], viewed as [B, H_kv, Nkv, d]."""
    return t.to(DEV).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


def ragged(w, k, v, lens):
    """Rows past each row's length are NaN, so any read of them would show."""
    k, v = k.clone(), v.clone()
    for b, n in enumerate(lens):
        n = max(0, min(int(n), w.Nkv))
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    return k, v


def paged(w, k, v, P, pool="nphd", seed=0, extra=3):
    """Scatter the rows of k/v into a page pool in a seeded page order.

    Unused pages and the tail of each row's last page are NaN, and the block
    table entries past a row's pages hold a huge id, so a read outside a
    row's keys would show up as NaN."""
    B, H_kv, Nkv, d = k.shape
    npg = math.ceil(Nkv / P)
    num_pages = B * npg + extra
    perm = np.random.default_rng(seed).permutation(num_pages)[:B * npg].reshape(B, npg)
    shape = (num_pages, P, H_kv, d) if pool == "nphd" else (num_pages, H_kv, P, d)
    kp = torch.full(shape, float("nan"), dtype=k.dtype)
    vp = torch.full(shape, float("nan"), dtype=v.dtype)
    for b in range(B):
        for j in range(npg):
            r0, r1 = j * P, min((j + 1) * P, Nkv)
            if pool == "nphd":
                kp[perm[b, j], :r1 - r0] = k[b, :, r0:r1].transpose(0, 1)
                vp[perm[b, j], :r1 - r0] = v[b, :, r0:r1].transpose(0, 1)
            else:
                kp[perm[b, j], :, :r1 - r0] = k[b, :, r0:r1]
                vp[perm[b, j], :, :r1 - r0] = v[b, :, r0:r1]
    bt = np.full((B, npg + 2), 10 ** 9, dtype=np.int32)
    bt[:, :npg] = perm
    kd, vd = kp.to(DEV), vp.to(DEV)
    if pool == "nphd":
        kd, vd = kd.permute(0, 2, 1, 3), vd.permute(0, 2, 1, 3)
    return kd, vd, torch.from_numpy(bt).to(DEV)


def check_every_slot(gqa, q, k, v, idx, scale, o_before_bits, o_after, tol):
    """Full-size comparison of every active slot, one batch row at a time so
    that host memory holds one row's selected K/V: the row's selected heads
    (or groups, with their G query heads) are gathered on the device into a
    compact problem with index 0 .. top_k-1 and run through the whole-call
    oracle; plus whole-tensor properties (inactive slots bit-identical to
    their prefill, active slots finite).  Returns (max abs error, slots)."""
    B, H = q.shape[:2]
    H_kv = k.shape[1]
    G = H // H_kv
    idx_cpu = idx.cpu().numpy()
    w = written_mask(idx_cpu, H, H_kv, gqa)
    wt = torch.from_numpy(w).to(o_after.device)
    assert torch.equal(wl.raw_bits(o_after)[~wt], o_before_bits[~wt]), "an inactive slot changed"
    assert torch.isfinite(o_after[wt]).all(), "non-finite output in an active slot"
    err, slots = 0.0, 0
    for b in range(B):
        sel = [int(e) for e in idx_cpu[b] if 0 <= e < (H_kv if gqa else H)]
        if not sel:
            continue
        if gqa:
            heads = [g * G + j for g in sel for j in range(G)]
            kv_rows = sel
        else:
            heads = sel
            kv_rows = [h // G for h in sel]
        dev_h = torch.tensor(heads, device=q.device)
        dev_g = torch.tensor(kv_rows, device=q.device)
        qc = q[b].index_select(0, dev_h).unsqueeze(0).cpu()         # [1, n_heads, 1, d]
        kc = k[b].index_select(0, dev_g).unsqueeze(0).cpu()         # [1, n_kv, Nkv, d]
        vc = v[b].index_select(0, dev_g).unsqueeze(0).cpu()
        if gqa:
            compact = np.arange(len(sel), dtype=np.int32)[None, :]
            ref, written = sha_decode_gqa_ref(qc, kc, vc, compact, scale)
        else:
            # head j of the compact problem reads KV row j (H_kv = H there)
            compact = np.arange(len(sel), dtype=np.int32)[None, :]
            ref, written = sha_decode_ref(qc, kc, vc, compact, scale)
        assert written.all()
        got = o_after[b].index_select(0, dev_h).cpu().to(torch.float64).numpy()
        err = max(err, float(np.max(np.abs(got - ref[0]))))
        slots += len(set(heads))
    assert err <= tol, f"max abs error {err:.3e} > {tol}"
    assert slots == int(w.sum())
    return err, slots
