"""Upload generated inputs to GPU memory as torch tensors (data movement only)."""

from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import torch


def _t(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)          # uint8 codes
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_device(inp, device="cuda") -> SimpleNamespace:
    """Torch tensors of every input of one decode step.

    ``latent`` and ``rope`` are views into the same fused row pool
    (row stride d_latent + d_rope), ``rope`` starting d_latent elements in.
    """
    c = inp.cfg
    pool = inp.pool()
    rows = _t(pool.rows, c.kv_dtype, device)
    return SimpleNamespace(
        q_nope=_t(inp.q_nope, c.q_dtype, device),
        q_rope=_t(inp.q_rope, c.q_dtype, device),
        positions=torch.from_numpy(inp.positions).to(device),
        w_uk=_t(inp.w_uk, c.q_dtype, device),
        w_uv=_t(inp.w_uv, c.q_dtype, device),
        rows=rows,
        latent=rows[:, : c.d_latent],
        rope=rows[:, c.d_latent:],
        kv_row_stride=c.row_width,
        kv_scale=None if pool.kv_scale is None else torch.from_numpy(pool.kv_scale).to(device),
        seq_lens=torch.from_numpy(inp.seq_lens).to(device),
        block_table=None if pool.block_table is None else torch.from_numpy(pool.block_table).to(device),
        max_blocks_per_seq=pool.max_blocks_per_seq,
        max_seq_len=pool.max_seq_len,
        causal=int(c.causal),
        softmax_scale=inp.softmax_scale,
        rope_base=inp.rope_base,
    )
