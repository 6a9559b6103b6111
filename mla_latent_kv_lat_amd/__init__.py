"""MI355X-native MLA absorbed decode.

The product is libmla.so (HIP kernels for gfx950 behind the C ABI in
include/mla.h).  This package is its thin Python binding plus a helper that
runs the calls of one decode step on caller-owned torch tensors, and the
cache-append producer that writes each new token's cache row, the MHA-form
prefill calls and the output-side absorption (fused W_O W_UV).
"""

from .binding import (BF16, F32, FLAG_GENERIC, FP8_E4M3, TILE_TOKENS, MLAAppendDims, MLADims,
                      MLAError, append_dims, dims, mla_kv_append, mla_kv_append_noalloc,
                      mla_kv_append_workspace_bytes,
                      mla_absorb_q, mla_combine, mla_combine_out_proj, mla_decode_attn,
                      mla_fuse_out_weight, mla_fused_out_weight_bytes, mla_num_splits_hint,
                      mla_out_proj, mla_out_proj_fused,
                      mla_out_proj_fused_workspace_bytes, mla_prefill_attn, mla_prefill_expand, mla_split_plan,
                      mla_workspace_bytes, mla_workspace_elems)
from .step import DecodeStep

__all__ = [
    "BF16", "F32", "FLAG_GENERIC", "FP8_E4M3", "TILE_TOKENS", "MLAAppendDims", "MLADims", "MLAError",
    "append_dims", "dims", "mla_kv_append", "mla_kv_append_noalloc", "mla_kv_append_workspace_bytes",
    "mla_absorb_q", "mla_combine", "mla_combine_out_proj", "mla_decode_attn",
    "mla_fuse_out_weight", "mla_fused_out_weight_bytes", "mla_num_splits_hint", "mla_out_proj",
    "mla_out_proj_fused", "mla_out_proj_fused_workspace_bytes",
    "mla_prefill_attn", "mla_prefill_expand", "mla_split_plan", "mla_workspace_bytes",
    "mla_workspace_elems", "DecodeStep",
]
