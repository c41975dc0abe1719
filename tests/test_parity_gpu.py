"""HIP path vs the fp64 oracle on the five decode workloads (GPU).

Two sizes per workload: a reduced batch the oracle checks completely
(several tiles, a ragged key tail, splits), and the full size, where every
active slot is compared with the oracle (run one batch row at a time) and
every inactive slot is checked bit for bit.  Tolerances are
the max abs errors for N(0, 1) inputs: 1e-5 (f32), 2e-3 (f16), 1e-2 (bf16).
Every inactive slot must keep the sentinel NaN payload bit for bit.
"""
import pytest
import torch

from contextual_head_sparsity_amd import workloads as wl

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import DEV, TOL, check_every_slot, check_full, check_sampled, run_gpu, say


REDUCED = {
    "tiny_f32": dict(),
    "opt6.7b_f16": dict(B=3, Nkv=1024 + 37),
    "opt66b_f16": dict(B=3, Nkv=1920),
    "llama2_7b_bf16": dict(B=2, Nkv=4096 - 5),
    "llama3.1_70b_gqa_bf16": dict(B=2, Nkv=2048 + 77),
}


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
@pytest.mark.parametrize("nsplit", [0, 1, 3])
def test_reduced_full_compare(name, nsplit):
    w = wl.WORKLOADS[name].with_(**REDUCED[name])
    say(f"[parity reduced] {name} B={w.B} Nkv={w.Nkv} nsplit={nsplit}")
    q, k, v, idx, o = wl.make_workload(w, "cpu")
    before = o.clone()
    od = o.to(DEV)
    run_gpu(w.gqa, q.to(DEV), k.to(DEV), v.to(DEV), idx.to(DEV), w.scale, od, nsplit=nsplit)
    err, _ = check_full(w.gqa, q, k, v, idx, w.scale, before, od, TOL[w.dtype])
    say(f"   max_err={err:.3e}")


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_full_size_every_slot(name):
    """The workload at its full size, in the launch configuration the
    benchmark times (planned split count): every active slot against the
    oracle, no sampling."""
    w = wl.WORKLOADS[name]
    say(f"[parity full] {name} B={w.B} H={w.H} H_kv={w.H_kv} Nkv={w.Nkv} top_k={w.top_k}")
    q, k, v, idx, o = wl.make_workload(w, DEV)
    before_bits = wl.raw_bits(o).clone()
    run_gpu(w.gqa, q, k, v, idx, w.scale, o)
    err, slots = check_every_slot(w.gqa, q, k, v, idx, w.scale, before_bits, o, TOL[w.dtype])
    say(f"   every active slot ({slots}): max_err={err:.3e}")
    del q, k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("gqa,dtype", [(False, "f16"), (True, "bf16")])
@pytest.mark.parametrize("nsplit", [0, 64])
def test_long_context(gqa, dtype, nsplit):
    """A 128 K-key cache with few units: the planner splits up to its cap
    (64 splits of 2048 keys for the head kernel), every active slot is
    checked against the oracle, and inactive slots keep their bits."""
    if gqa:
        w = wl.Workload("long", B=2, H=16, H_kv=2, d=128, Nkv=131072, top_k=1, dtype=dtype,
                        gqa=True, seed=21)
    else:
        w = wl.Workload("long", B=2, H=4, H_kv=4, d=128, Nkv=131072, top_k=2, dtype=dtype,
                        seed=21)
    say(f"[parity long] gqa={gqa} {dtype} Nkv={w.Nkv} nsplit={nsplit}")
    q, k, v, idx, o = wl.make_workload(w, DEV)
    before_bits = wl.raw_bits(o).clone()
    run_gpu(w.gqa, q, k, v, idx, w.scale, o, nsplit=nsplit)
    n_active = w.B * w.top_k * (w.H // w.H_kv if gqa else 1)
    err = check_sampled(w.gqa, q, k, v, idx, w.scale, before_bits, o, TOL[w.dtype],
                        n_samples=n_active, seed=w.seed)
    say(f"   max_err={err:.3e}")
    del q, k, v
    torch.cuda.empty_cache()
