"""Host-side checks of the seeded workload generator (CPU only)."""
import numpy as np
import torch

from contextual_head_sparsity_amd import workloads as wl


def test_index_rows_distinct_sorted_in_range():
    for w in wl.WORKLOADS.values():
        idx = wl.sample_index(w)
        n = w.H_kv if w.gqa else w.H
        assert idx.shape == (w.B, w.top_k) and idx.dtype == np.int32
        assert (idx >= 0).all() and (idx < n).all()
        assert (np.diff(idx, axis=1) > 0).all()          # sorted and distinct
        assert np.array_equal(idx, wl.sample_index(w))   # seeded


def test_zipf_popularity_is_skewed():
    w = wl.WORKLOADS["opt66b_f16"]
    counts = np.bincount(wl.sample_index(w).ravel(), minlength=w.H)
    assert counts.max() == w.B            # the most popular heads appear in every row
    assert counts.min() < w.B // 4        # unpopular heads are rare


def test_sentinel_bits_and_qkv_seeded():
    w = wl.WORKLOADS["tiny_f32"]
    for dt in ("f32", "f16", "bf16"):
        ww = w.with_(dtype=dt)
        o = wl.sentinel_like(ww)
        bits = wl.raw_bits(o).flatten()[0].item() & (0xFFFFFFFF if dt == "f32" else 0xFFFF)
        assert bits == wl.SENTINEL_BITS[dt]
        assert torch.isnan(o).all()
        q1, k1, v1 = wl.make_qkv(ww)
        q2, k2, v2 = wl.make_qkv(ww)
        assert torch.equal(wl.raw_bits(k1), wl.raw_bits(k2))
        assert q1.dtype == wl.DTYPES[dt] and k1.shape == (w.B, w.H_kv, w.Nkv, w.d)


def test_byte_accounting():
    w = wl.WORKLOADS["opt66b_f16"]
    assert w.units == 1408
    assert w.active_kv_bytes == 1408 * 2 * 1920 * 128 * 2 == 1_384_120_320
    g = wl.WORKLOADS["llama3.1_70b_gqa_bf16"]
    assert g.G == 8 and g.active_kv_bytes == 64 * 5 * 2 * 8192 * 128 * 2
