"""CPU oracle for MLA absorbed decode -- test infrastructure only.

Only the test suite, the smoke check in __graft_entry__ and the cpu_baseline
leg of bench.py may import this package.  The product path (the HIP library
and its Python binding) never imports, calls or links anything here.
"""

from .mla_oracle import (
    bf16_to_f64,
    cache_f64,
    e4m3_to_f64,
    fuse_out_weight,
    kv_append,
    kv_cache_bytes_per_token,
    mla_absorbed,
    mla_decode,
    mla_expand,
    out_proj_fused,
    rms_norm,
    rope_interleaved,
    stored_to_f64,
)

__all__ = [
    "bf16_to_f64",
    "cache_f64",
    "e4m3_to_f64",
    "fuse_out_weight",
    "kv_append",
    "kv_cache_bytes_per_token",
    "mla_absorbed",
    "mla_decode",
    "mla_expand",
    "out_proj_fused",
    "rms_norm",
    "rope_interleaved",
    "stored_to_f64",
]
