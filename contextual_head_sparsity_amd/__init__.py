"""Selective Head Attention (SHA) decode for AMD Instinct MI355X (gfx950).

The compute runs in hand-written HIP kernels behind a C ABI (include/sha.h);
this package is a thin binding over that library plus the seeded workload
generator.  The library is loaded on first use and a missing build is an
error: there is no CPU fallback.
"""
from . import workloads

_BINDING_NAMES = ("sha_decode", "sha_decode_gqa", "sha_decode_paged", "KvLayout", "DecodeStep",
                  "ShaError", "lib", "plan_nsplit", "workspace_bytes", "workspace_bytes_paged",
                  "router_topk", "router_workspace_bytes", "mlp_union", "selective_mlp",
                  "selective_mlp_workspace_bytes")

__all__ = ["workloads", *_BINDING_NAMES]


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
