"""CPU float64 oracle for split-KV paged decode attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the GPU library.  It shares
no code with the HIP path; both take their inputs from ``workloads``.
"""

from .reference import (SPLIT_ALIGN, attend, decode_reference, gather, kv_head_of,
                        merge_reference, prefix_split_bounds, softmax_weights, split_bounds,
                        split_reference, to_f64, visible_keys)

__all__ = ["SPLIT_ALIGN", "attend", "decode_reference", "gather", "kv_head_of",
           "merge_reference", "prefix_split_bounds", "softmax_weights", "split_bounds",
           "split_reference", "to_f64", "visible_keys"]
