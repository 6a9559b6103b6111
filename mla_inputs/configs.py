"""Workload shapes for MLA decode.

The DeepSeek-V3 attention shape (128 heads, latent width 512, decoupled RoPE
width 64, per-head no-position query/key width 128, value width 128) comes from
"Model Architecture Driving Inference Systems ... MLA Matrix Absorption"
(section 2.1 and the table in section 2.4) and from "Multi-Head Latent
Attention (MLA): Mathematical Foundations ..." (the architectural comparison
list and the reference module's defaults).  Page size 64 tokens: the same
first page, section 4.1.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass

BLOCK_TOKENS = 64


@dataclass(frozen=True)
class MLAConfig:
    name: str
    batch: int
    q_len: int
    heads: int
    d_nope: int
    d_rope: int
    d_latent: int
    d_v: int
    seq_len: int = 0            # fixed cached length per sequence (0: ragged)
    len_lo: int = 0             # ragged lengths ~ integer U{len_lo..len_hi}
    len_hi: int = 0
    paged: bool = False         # paged pool in 64-token blocks + block_table
    q_dtype: str = "bf16"       # 'f32' | 'bf16': queries, weights, outputs
    kv_dtype: str = "bf16"      # 'f32' | 'bf16' | 'fp8'
    causal: bool = False        # bottom-right causal mask among the q_len queries
    query_in_cache: bool = False  # query i sits at position len-q_len+i (else len+i)
    rope_base: float = 10000.0
    outlier_frac: float = 0.0   # fraction of rows scaled by outlier_scale
    outlier_scale: float = 8.0
    weight_std: float = 0.0     # 0: 1/sqrt(d_latent)
    seed: int = 20261203

    @property
    def row_width(self) -> int:
        return self.d_latent + self.d_rope

    @property
    def max_seq_len(self) -> int:
        return self.seq_len if self.seq_len else self.len_hi

    @property
    def ragged(self) -> bool:
        return self.seq_len == 0

    @property
    def softmax_scale(self) -> float:
        # 1/sqrt(d_nope + d_rope): the scale of the score definition on the
        # first page, section 3.1.
        return float((self.d_nope + self.d_rope) ** -0.5)

    @property
    def w_std(self) -> float:
        return self.weight_std if self.weight_std else float(self.d_latent ** -0.5)

    def storage_bytes_per_token(self) -> int:
        """Bytes one cached token occupies (row plus its scale for fp8)."""
        el = {"f32": 4, "bf16": 2, "fp8": 1}[self.kv_dtype]
        return self.row_width * el + (4 if self.kv_dtype == "fp8" else 0)


def scaled(cfg: MLAConfig, **kw) -> MLAConfig:
    """A copy of ``cfg`` with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(cfg, **kw)


_DSV3 = dict(heads=128, d_nope=128, d_rope=64, d_latent=512, d_v=128)

CONFIGS = {
    # batch 1, 4 heads, latent 32, rope 16, nope 32, v 32, 64 cached tokens,
    # fp32; query at position 64, keys at 0..63; scale 1/sqrt(48).
    "tiny_f32": MLAConfig(
        name="tiny_f32", batch=1, q_len=1, heads=4, d_nope=32, d_rope=16,
        d_latent=32, d_v=32, seq_len=64, q_dtype="f32", kv_dtype="f32",
        seed=20261203),
    # DeepSeek-V3 shaped layer, bf16, batch 16, contiguous 4096-token cache.
    "dsv3_b16_l4k": MLAConfig(
        name="dsv3_b16_l4k", batch=16, q_len=1, seq_len=4096, seed=20261204,
        **_DSV3),
    # batch 64, ragged lengths U{1024..8192}, paged 64-token blocks.
    "dsv3_b64_ragged_paged": MLAConfig(
        name="dsv3_b64_ragged_paged", batch=64, q_len=1, len_lo=1024,
        len_hi=8192, paged=True, seed=20261205, **_DSV3),
    # batch 4, 131072 tokens each, 1% of rows scaled x8.
    "long_b4_l128k": MLAConfig(
        name="long_b4_l128k", batch=4, q_len=1, seq_len=131072,
        outlier_frac=0.01, outlier_scale=8.0, seed=20261206, **_DSV3),
    # fp8 E4M3 cache with per-token fp32 scale, batch 128, 16384 tokens,
    # 2 query tokens per sequence under a causal mask between them.
    "fp8_b128_l16k_q2": MLAConfig(
        name="fp8_b128_l16k_q2", batch=128, q_len=2, seq_len=16384,
        kv_dtype="fp8", causal=True, query_in_cache=True, seed=20261207,
        **_DSV3),
    # Headline shape: batch 64, 8192 tokens each, paged 64-token blocks.
    "dsv3_b64_l8k_paged": MLAConfig(
        name="dsv3_b64_l8k_paged", batch=64, q_len=1, seq_len=8192,
        paged=True, seed=20261208, **_DSV3),
    # Multi-token decode on the headline shape (two new tokens per sequence,
    # e.g. one speculative or multi-token-prediction draft): both queries are
    # in the cache and the second also sees the first (causal).
    "dsv3_b64_l8k_paged_mtp2": MLAConfig(
        name="dsv3_b64_l8k_paged_mtp2", batch=64, q_len=2, seq_len=8192,
        paged=True, causal=True, query_in_cache=True, seed=20261209, **_DSV3),
}

HEADLINE = "dsv3_b64_l8k_paged"

# Prefill (MHA form): every cached token of a sequence is also a query token
# of its prompt, under the causal mask.  Kept apart from the decode
# workloads: it runs the prefill calls, not the decode step.
PREFILL_CONFIGS = {
    # batch 4 prompts of 4096 tokens, paged 64-token blocks.
    "prefill_b4_s4k": MLAConfig(
        name="prefill_b4_s4k", batch=4, q_len=4096, seq_len=4096, paged=True,
        causal=True, query_in_cache=True, seed=20261210, **_DSV3),
}

# Output-side absorption: the latent outputs of one decode step's query
# tokens projected through the pre-fused W_O W_UV to the DeepSeek-V3 hidden
# width 7168 (batch 64 with one or two query tokens per sequence).
OUT_FUSED_CONFIGS = {
    "out_fused_dsv3_m64": dict(m=64, heads=128, d_model=7168, d_v=128, seed=20261470),
    "out_fused_dsv3_m128": dict(m=128, heads=128, d_model=7168, d_v=128, seed=20261471),
}
