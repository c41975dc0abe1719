"""fp64 CPU oracle for SHA decode: test infrastructure only.

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the HIP library and its Python binding never do.
"""
from .sha_oracle import (attend_one, sha_decode_gqa_ref, sha_decode_ref,
                         sha_units_ref, to_f64)

__all__ = ["attend_one", "sha_decode_ref", "sha_decode_gqa_ref", "sha_units_ref", "to_f64"]
