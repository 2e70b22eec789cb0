"""Split-KV paged decode attention for MI355X (gfx950).

The compute runs in libsplitkv.so (HIP kernels behind the C ABI of
include/attn_decode.h); this package is its ctypes binding plus helpers that
fill the shape descriptor from torch tensors.
"""

from ._lib import (ATTN_BF16, ATTN_EHIP, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EWORKSPACE, ATTN_F32, ATTN_OK,
                   ATTN_PLAN_FUSED_MERGE, ATTN_PLAN_NO_XCD_REMAP, ATTN_PLAN_POLICY_P2, ATTN_PLAN_PRIVATE_PAGES,
                   ATTN_PLAN_SHARED_PASS, ATTN_VARIANT_MFMA, ATTN_VARIANT_VALU, EXPORTED, LIB_PATH,
                   NOALLOC_SCRATCH_BYTES, SHARED_PASS_MIN_ROWS, AttnDecodeDesc, AttnDecodeError, AttnDecodePlan,
                   AttnDecodePrefixPlan, attn_decode_last_error, attn_decode_merge, attn_decode_partials,
                   attn_decode_plan, attn_decode_plan_lens, attn_decode_plan_prefix, attn_decode_run,
                   attn_decode_run_noalloc, attn_decode_run_prefix, attn_decode_split_range,
                   attn_decode_workspace_init, attn_decode_workspace_layout, lib, make_desc)
from .tensors import desc_from_tensors, make_desc_from_tensors

__all__ = [n for n in dir() if not n.startswith("_")]
