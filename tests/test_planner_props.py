"""Properties of the host planners over random shapes (CPU, no device).

The split planner must keep every split inside [1, 64], never cut a row into
splits shorter than its 512-key minimum unless the row is shorter than that,
and its workspace query must match the partial buffer layout for the split
count it plans; a paged cache forces enough splits that no split stages more
than 1024 page ids.  The selective-MLP workspace must cover H and stay within
its split bounds.
"""
import ctypes
import os

import pytest
from hypothesis import given, settings, strategies as st

from contextual_head_sparsity_amd import _binding as bd

pytestmark = pytest.mark.skipif(not os.path.exists(bd.LIB_PATH),
                                reason="libsha.so not built (run __graft_entry__.build())")


def _r256(x):
    return (x + 255) // 256 * 256


def _partials(n, d):
    return _r256(n * d * 4) + n * 8 if n else 0


shape = st.tuples(
    st.integers(1, 256),                      # B
    st.integers(1, 64),                       # H_kv
    st.sampled_from([1, 2, 4, 8, 16, 32]),    # G = H / H_kv
    st.integers(1, 200_000),                  # Nkv
    st.sampled_from([64, 128]),               # d
    st.integers(0, 2),                        # dtype (f32, f16, bf16)
    st.booleans(),                            # group-indexed
    st.sampled_from([80, 256, 304]),          # CUs
    st.integers(1, 64),                       # top_k (clipped below)
)


@settings(max_examples=400, deadline=None)
@given(shape)
def test_split_plan_bounds_and_workspace(s):
    assert "SHA_NSPLIT" not in os.environ
    B, H_kv, G, Nkv, d, dt, gqa, cus, k = s
    H = H_kv * G
    top_k = min(k, H_kv if gqa else H)
    L = bd.lib()
    ns = L.sha_plan_nsplit(B, H, H_kv, Nkv, d, top_k, int(gqa), dt, cus)
    assert 1 <= ns <= 64
    assert ns == 1 or Nkv // ns >= 512                # no split shorter than 512 keys
    heads = G if (gqa and G > 1) else 1
    ws = L.sha_workspace_bytes(B, H, H_kv, Nkv, d, top_k, int(gqa), dt, 0, cus)
    assert ws == (_partials(B * top_k * heads * ns, d) if ns > 1 else 0)


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 64), st.integers(20_000, 400_000), st.sampled_from([16, 32, 64]),
       st.booleans())
def test_paged_caches_force_enough_splits(B, Nkv, P, gqa):
    # every split stages at most 1024 page ids: ns >= ceil(Nkv / (1024 P))
    H_kv, G, d, top_k = 2, 8, 128, 1
    H = H_kv * G
    L = bd.lib()
    pages = (Nkv + P - 1) // P
    lay = bd.KvLayout(0, 0, 0, 0, 0, 0)
    lay.k_batch_stride, lay.k_head_stride, lay.k_row_stride = P * H_kv * d, P * d, d
    lay.v_batch_stride, lay.v_head_stride, lay.v_row_stride = P * H_kv * d, P * d, d
    lay.block_table = 0x10000
    lay.block_table_stride = pages
    lay.page_size = P
    lay.num_pages = B * pages
    heads = G if gqa else 1
    min_ns = -(-Nkv // (1024 * P))
    ws = L.sha_workspace_bytes_kv(B, H, H_kv, Nkv, d, top_k, int(gqa), 2, 1, 256,
                                  ctypes.byref(lay))
    n = B * top_k * heads
    # an explicit request of one split is raised to the page-staging minimum
    assert ws == (_partials(n * min_ns, d) if min_ns > 1 else 0)


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 512), st.sampled_from([256, 1024, 4096, 9216]), st.integers(1, 40_000),
       st.floats(0.0, 1.0), st.sampled_from([80, 256, 304]))
def test_mlp_workspace_covers_h_within_split_bounds(B, d, D, frac, cus):
    n_max = max(0, min(D, int(D * frac)))
    L = bd.lib()
    ws = L.sha_selective_mlp_workspace_bytes(B, d, D, n_max, cus)
    b_pad = (B + 63) // 64 * 64
    n_pad = (max(n_max, 1) + 127) // 128 * 128
    h = _r256(b_pad * n_pad * 2)
    assert ws % 256 == 0 and ws >= h
    assert ws <= h + _r256(8 * b_pad * n_pad * 4) + _r256(64 * b_pad * d * 4)
