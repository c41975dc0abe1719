"""fp64 CPU oracles for SHA decode, the attention router and the selective MLP:
test infrastructure only.

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the HIP library and its Python binding never do.
"""
from .mlp_oracle import mlp_union_ref, selective_mlp_ref
from .router_oracle import router_scores_ref, router_topk_ref, topk_ref
from .sha_oracle import (attend_one, sha_decode_gqa_ref, sha_decode_ref,
                         sha_units_ref, to_f64)

__all__ = ["attend_one", "sha_decode_ref", "sha_decode_gqa_ref", "sha_units_ref", "to_f64",
           "mlp_union_ref", "selective_mlp_ref", "router_scores_ref", "router_topk_ref",
           "topk_ref"]
